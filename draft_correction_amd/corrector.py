"""Thin ctypes binding of libcorrector.so with the C-ABI's names.

Argument marshalling only: tensors are passed as device pointers, strides in
elements, and the current torch stream as the hipStream_t.  Every step of the
computation runs in the HIP kernels of the library.  Loading fails loudly if
the library has not been built; there is no fallback path.
"""

from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcorrector.so")

VARIANTS = {"mlp": 0, "cosine": 1}
DTYPES = {"bf16": 0, "f32": 1}
STATUS = {0: "CORR_OK", 1: "CORR_E_NULL", 2: "CORR_E_SHAPE", 3: "CORR_E_UNSUPPORTED",
          4: "CORR_E_ALIGN", 5: "CORR_E_WORKSPACE", 6: "CORR_E_HIP", 7: "CORR_E_HANDLE"}

# exported symbols declared in include/corrector.h
SYMBOLS = ("corrector_create", "corrector_destroy", "corrector_workspace_bytes",
           "corrector_topk", "corrector_topk_softmax", "corrector_score", "corrector_walk", "corrector_run",
           "corrector_run_static", "corrector_intermediates", "corrector_set_timing", "corrector_kernel_times",
           "corrector_status_string", "corrector_table_bytes", "corrector_fold_table",
           "corrector_use_table")


class CorrectorDesc(C.Structure):
    _fields_ = [("vocab", C.c_int64), ("slots", C.c_int32), ("k", C.c_int32),
                ("d_hidden", C.c_int32), ("d_embed", C.c_int32), ("r", C.c_int32),
                ("mlp_hidden", C.c_int32), ("d_vec", C.c_int32), ("variant", C.c_int32),
                ("logits_dtype", C.c_int32), ("max_requests", C.c_int32),
                ("ln_eps", C.c_float), ("sigma", C.c_float), ("path_rule", C.c_int32),
                ("path_lambda", C.c_float), ("beam_width", C.c_int32), ("succ_top_m", C.c_int32)]

PATH_RULES = {"greedy": 0, "global_sum": 1, "geometric": 2, "beam": 3}


WEIGHT_FIELDS = ("embed", "w_cand", "w_ctx", "w_fuse", "w_pair", "ln_gamma", "ln_beta", "w1",
                 "b1", "w2", "b2", "w_out", "w_in")


class CorrectorWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in WEIGHT_FIELDS]


class CorrectorError(RuntimeError):
    def __init__(self, call: str, code: int):
        super().__init__("%s failed: %s (%d)" % (call, STATUS.get(code, "?"), code))
        self.code = code


_lib = None


def load(path: str = LIB_PATH):
    """Load libcorrector.so (raises if it is missing: build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libcorrector.so is not built (%s); run draft_correction_amd.build" % path)
    lib = C.CDLL(path)
    P, I32, I64, SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    lib.corrector_create.argtypes = [C.POINTER(CorrectorDesc), C.POINTER(CorrectorWeights), C.POINTER(P)]
    lib.corrector_create.restype = C.c_int
    lib.corrector_destroy.argtypes = [P]
    lib.corrector_destroy.restype = None
    lib.corrector_workspace_bytes.argtypes = [P, I32]
    lib.corrector_workspace_bytes.restype = SZ
    lib.corrector_topk.argtypes = [P, I32, P, I64, I64, P, P, P, SZ, P]
    lib.corrector_topk_softmax.argtypes = [P, I32, P, I64, I64, P, P, P, P, P, SZ, P]
    lib.corrector_score.argtypes = [P, I32, P, P, P, I64, I64, P, P, SZ, P]
    lib.corrector_walk.argtypes = [P, I32, P, P, P, P, P]
    lib.corrector_run.argtypes = [P, I32, P, I64, I64, P, I64, I64, P, P, P, P, P, P, SZ, P]
    lib.corrector_run_static.argtypes = [P, I32, P, I64, I64, P, I64, I64, P, P, P, P, P, P]
    lib.corrector_intermediates.argtypes = [P, I32, P, SZ, P, P, P, P]
    lib.corrector_set_timing.argtypes = [P, C.c_int]
    lib.corrector_kernel_times.argtypes = [P, P, P, C.c_int]
    lib.corrector_table_bytes.argtypes = [P]
    lib.corrector_table_bytes.restype = SZ
    lib.corrector_fold_table.argtypes = [P, P, P]
    lib.corrector_use_table.argtypes = [P, P]
    lib.corrector_status_string.argtypes = [C.c_int]
    lib.corrector_status_string.restype = C.c_char_p
    for fn in ("corrector_topk", "corrector_topk_softmax", "corrector_score", "corrector_walk", "corrector_run",
               "corrector_run_static", "corrector_intermediates", "corrector_set_timing", "corrector_kernel_times",
               "corrector_fold_table", "corrector_use_table"):
        getattr(lib, fn).restype = C.c_int
    _lib = lib
    return lib


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ok(call, rc):
    if rc != 0:
        raise CorrectorError(call, rc)


def make_desc(cfg: dict, max_requests: int) -> CorrectorDesc:
    return CorrectorDesc(cfg["V"], cfg["B"], cfg["K"], cfg["d"], cfg["de"], cfg["r"],
                         cfg.get("h", 0), cfg.get("dvec", 0), VARIANTS[cfg["variant"]],
                         DTYPES[cfg["logits_dtype"]], max_requests, cfg.get("ln_eps", 1e-5),
                         cfg.get("sigma", 1.0), PATH_RULES[cfg.get("path_rule", "greedy")],
                         cfg.get("path_lambda", 0.75), cfg.get("beam_width", 4), cfg.get("succ_top_m", 0))


class Corrector:
    """A corrector handle.  ``weights`` maps field names to device tensors
    (bfloat16 matrices may be given as int16/uint16/bfloat16 tensors of bits)
    that must stay alive as long as the handle."""

    def __init__(self, cfg: dict, weights: dict, max_requests: int):
        self.lib = load()
        self.cfg = dict(cfg)
        self.desc = make_desc(cfg, max_requests)
        self._weights = {k: v for k, v in weights.items() if v is not None}
        cw = CorrectorWeights(*[_p(self._weights.get(n)) for n in WEIGHT_FIELDS])
        h = C.c_void_p()
        _ok("corrector_create", self.lib.corrector_create(C.byref(self.desc), C.byref(cw), C.byref(h)))
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            self.lib.corrector_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, n: int) -> int:
        return int(self.lib.corrector_workspace_bytes(self.h, n))

    def new_workspace(self, n: int, device="cuda") -> torch.Tensor:
        return torch.empty(max(self.workspace_bytes(n), 1), dtype=torch.uint8, device=device)

    def topk(self, n, logits, req_stride, slot_stride, ids, vals, ws, offset: int = 0, stream=None):
        base = _p(logits) + offset * logits.element_size()
        _ok("corrector_topk", self.lib.corrector_topk(self.h, n, base, req_stride, slot_stride,
                                                      _p(ids), _p(vals), _p(ws), ws.numel(),
                                                      _stream(stream)))

    def topk_softmax(self, n, logits, req_stride, slot_stride, ids, vals, logz, ws, conf=None,
                     offset: int = 0, stream=None):
        base = _p(logits) + offset * logits.element_size()
        _ok("corrector_topk_softmax", self.lib.corrector_topk_softmax(
            self.h, n, base, req_stride, slot_stride, _p(ids), _p(vals), _p(logz), _p(conf), _p(ws),
            ws.numel(), _stream(stream)))

    def score(self, n, ids, vals, hidden, h_req_stride, h_slot_stride, scores, ws, offset: int = 0,
              stream=None):
        base = _p(hidden) + offset * hidden.element_size()
        _ok("corrector_score", self.lib.corrector_score(self.h, n, _p(ids), _p(vals), base,
                                                        h_req_stride, h_slot_stride, _p(scores),
                                                        _p(ws), ws.numel(), _stream(stream)))

    def walk(self, n, scores, ids, tokens, choice=None, stream=None):
        _ok("corrector_walk", self.lib.corrector_walk(self.h, n, _p(scores), _p(ids), _p(tokens),
                                                      _p(choice), _stream(stream)))

    def run(self, n, logits, l_req_stride, l_slot_stride, hidden, h_req_stride, h_slot_stride,
            tokens, ws, choice=None, ids=None, vals=None, scores=None, l_offset: int = 0,
            h_offset: int = 0, stream=None):
        lb = _p(logits) + l_offset * logits.element_size()
        hb = _p(hidden) + h_offset * hidden.element_size()
        _ok("corrector_run", self.lib.corrector_run(self.h, n, lb, l_req_stride, l_slot_stride, hb,
                                                    h_req_stride, h_slot_stride, _p(tokens),
                                                    _p(choice), _p(ids), _p(vals), _p(scores),
                                                    _p(ws), ws.numel(), _stream(stream)))

    def run_static(self, n, logits, l_req_stride, l_slot_stride, hidden, h_req_stride, h_slot_stride,
                   tokens, choice=None, ids=None, vals=None, scores=None, l_offset: int = 0,
                   h_offset: int = 0, stream=None):
        """corrector_run_static: the library's own static workspace (no allocation)."""
        lb = _p(logits) + l_offset * logits.element_size()
        hb = _p(hidden) + h_offset * hidden.element_size()
        _ok("corrector_run_static", self.lib.corrector_run_static(
            self.h, n, lb, l_req_stride, l_slot_stride, hb, h_req_stride, h_slot_stride, _p(tokens), _p(choice),
            _p(ids), _p(vals), _p(scores), _stream(stream)))

    def intermediates(self, n, ws, z=None, g=None, s=None, stream=None):
        _ok("corrector_intermediates", self.lib.corrector_intermediates(
            self.h, n, _p(ws), ws.numel(), _p(z), _p(g), _p(s), _stream(stream)))

    def table_bytes(self) -> int:
        return int(self.lib.corrector_table_bytes(self.h))

    def fold_table(self, table, stream=None):
        _ok("corrector_fold_table", self.lib.corrector_fold_table(self.h, _p(table), _stream(stream)))

    def use_table(self, table):
        self._table = table  # keep the buffer alive while attached
        _ok("corrector_use_table", self.lib.corrector_use_table(self.h, _p(table)))

    def set_timing(self, enabled: bool):
        _ok("corrector_set_timing", self.lib.corrector_set_timing(self.h, 1 if enabled else 0))

    def kernel_times(self):
        cap = 12
        ms = (C.c_float * cap)()
        names = (C.c_char_p * cap)()
        k = self.lib.corrector_kernel_times(self.h, ms, names, cap)
        if k < 0:
            raise CorrectorError("corrector_kernel_times", -k)
        return [(names[i].decode(), float(ms[i])) for i in range(min(k, cap))]
