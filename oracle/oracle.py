"""ctypes wrapper of the C oracle (``oracle.c``), NumPy arrays in and out.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Argument marshalling
only: every step of the computation is in ``oracle.c``.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A prebuilt variant of the same source (the sanitizer build of the tests) is
# loaded instead when this names it; it is then never rebuilt here.
_LIB_OVERRIDE = os.environ.get("DRAFT_ORACLE_LIB")

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc into ``liboracle.so`` next to it."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Desc(C.Structure):
    _fields_ = [("V", C.c_int64), ("B", C.c_int32), ("K", C.c_int32), ("d", C.c_int32),
                ("de", C.c_int32), ("r", C.c_int32), ("h", C.c_int32), ("dvec", C.c_int32),
                ("variant", C.c_int32), ("logits_dtype", C.c_int32),
                ("eps", C.c_double), ("sigma", C.c_double), ("top_m", C.c_int32)]


class _Weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("embed", "w_cand", "w_ctx", "w_fuse", "w_pair", "w1", "w_out", "w_in",
                 "gamma", "beta", "b1", "w2", "b2")]


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = C.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = C.CDLL(_LIB)
        P = C.c_void_p
        lib.oracle_param_count.restype = C.c_int64
        lib.oracle_param_count.argtypes = [P]
        lib.oracle_topk_row.argtypes = [P, C.c_int, C.c_int64, C.c_int32, P, P]
        lib.oracle_topk.argtypes = [P, C.c_int32, P, C.c_int64, C.c_int64, P, P]
        lib.oracle_log_normaliser_row.argtypes = [P, C.c_int, C.c_int64, P]
        lib.oracle_log_normaliser.argtypes = [P, C.c_int32, P, C.c_int64, C.c_int64, P]
        lib.oracle_represent.argtypes = [P, P, C.c_int32, P, P, C.c_int64, C.c_int64, P, P, P, P]
        lib.oracle_score.argtypes = [P, P, C.c_int32, P, P, P, P, P]
        lib.oracle_walk.argtypes = [P, C.c_int32, P, P, P, P]
        lib.oracle_viterbi.argtypes = [P, C.c_int32, P, P, C.c_double, P, P, P]
        lib.oracle_beam.argtypes = [P, C.c_int32, P, P, C.c_int32, P, P, P]
        lib.oracle_accepted.argtypes = [C.c_int32, C.c_int32, P, P, P]
        lib.oracle_layernorm.argtypes = [P, C.c_int, C.c_double, P, P]
        lib.oracle_gelu.restype = C.c_double
        lib.oracle_gelu.argtypes = [C.c_double]
        lib.oracle_set_threads.argtypes = [C.c_int]
        lib.oracle_get_threads.restype = C.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError("oracle %s failed with code %d" % (what, rc))


@dataclass
class OracleDesc:
    V: int
    B: int
    K: int
    d: int
    de: int
    r: int
    h: int
    dvec: int
    variant: str = "mlp"
    logits_dtype: str = "bf16"
    eps: float = 1e-5
    sigma: float = 1.0
    top_m: int = 0

    @classmethod
    def from_config(cls, cfg: dict) -> "OracleDesc":
        return cls(V=cfg["V"], B=cfg["B"], K=cfg["K"], d=cfg["d"], de=cfg["de"], r=cfg["r"],
                   h=cfg["h"], dvec=cfg["dvec"], variant=cfg["variant"],
                   logits_dtype=cfg["logits_dtype"], eps=cfg["ln_eps"], sigma=cfg["sigma"],
                   top_m=cfg.get("succ_top_m", 0))

    def c(self) -> _Desc:
        return _Desc(self.V, self.B, self.K, self.d, self.de, self.r, self.h, self.dvec,
                     0 if self.variant == "mlp" else 1,
                     0 if self.logits_dtype == "bf16" else 1, self.eps, self.sigma, self.top_m)


class _Keep:
    """Holds converted arrays alive while a call is in flight."""

    def __init__(self):
        self.items = []

    def arr(self, a, dtype):
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=dtype)
        self.items.append(a)
        return a


def _weights(w: dict, embed, keep: _Keep) -> _Weights:
    cw = _Weights()
    for name, key, dt in (("embed", None, np.uint16), ("w_cand", "w_cand", np.uint16),
                          ("w_ctx", "w_ctx", np.uint16), ("w_fuse", "w_fuse", np.uint16),
                          ("w_pair", "w_pair", np.uint16), ("w1", "w1", np.uint16),
                          ("w_out", "w_out", np.uint16), ("w_in", "w_in", np.uint16),
                          ("gamma", "ln_gamma", np.float32), ("beta", "ln_beta", np.float32),
                          ("b1", "b1", np.float32), ("w2", "w2", np.float32),
                          ("b2", "b2", np.float32)):
        src = embed if name == "embed" else w.get(key)
        a = keep.arr(src, dt)
        setattr(cw, name, None if a is None else a.ctypes.data)
    return cw


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


def param_count(desc: OracleDesc) -> int:
    d = desc.c()
    return int(_load().oracle_param_count(C.byref(d)))


def gelu(t: float) -> float:
    return float(_load().oracle_gelu(float(t)))


def layernorm(x, eps: float, gamma=None, beta=None) -> np.ndarray:
    keep = _Keep()
    y = np.array(x, dtype=np.float64, copy=True)
    g = keep.arr(gamma, np.float32)
    b = keep.arr(beta, np.float32)
    _load().oracle_layernorm(_ptr(y), y.size, float(eps), _ptr(g), _ptr(b))
    return y


def topk_row(row, K: int):
    """Top-K of one row (float32 array, or uint16 array of bfloat16 bits)."""
    row = np.ascontiguousarray(row)
    dt = 0 if row.dtype == np.uint16 else 1
    if dt == 1:
        row = np.ascontiguousarray(row, dtype=np.float32)
    ids = np.empty(K, np.int32)
    vals = np.empty(K, np.float64)
    _check(_load().oracle_topk_row(_ptr(row), dt, row.size, K, _ptr(ids), _ptr(vals)), "topk_row")
    return ids, vals


def topk(desc: OracleDesc, logits, n: int, req_stride: int, slot_stride: int, offset: int = 0):
    """Top-K of every drafted slot; ``offset`` (elements) skips the anchor row."""
    dt = np.uint16 if desc.logits_dtype == "bf16" else np.float32
    flat = np.ascontiguousarray(logits, dtype=dt).reshape(-1)
    ids = np.empty((n, desc.B, desc.K), np.int32)
    vals = np.empty((n, desc.B, desc.K), np.float64)
    d = desc.c()
    base = flat[offset:]
    _check(_load().oracle_topk(C.byref(d), n, _ptr(base), req_stride, slot_stride,
                               _ptr(ids), _ptr(vals)), "topk")
    return ids, vals


def log_normaliser_row(row) -> float:
    """log sum_v exp(l_v) of one row (float32 array, or uint16 array of bfloat16 bits)."""
    row = np.ascontiguousarray(row)
    dt = 0 if row.dtype == np.uint16 else 1
    if dt == 1:
        row = np.ascontiguousarray(row, dtype=np.float32)
    out = np.empty(1, np.float64)
    _check(_load().oracle_log_normaliser_row(_ptr(row), dt, row.size, _ptr(out)), "log_normaliser_row")
    return float(out[0])


def log_normaliser(desc: OracleDesc, logits, n: int, req_stride: int, slot_stride: int, offset: int = 0):
    """log Z of every drafted slot row, [n][B]; rows addressed as in topk."""
    dt = np.uint16 if desc.logits_dtype == "bf16" else np.float32
    flat = np.ascontiguousarray(logits, dtype=dt).reshape(-1)
    logz = np.empty((n, desc.B), np.float64)
    d = desc.c()
    _check(_load().oracle_log_normaliser(C.byref(d), n, _ptr(flat[offset:]), req_stride, slot_stride,
                                         _ptr(logz)), "log_normaliser")
    return logz


CONF_FIELDS = ("logprob", "prob", "gap", "rank", "top")


def confidence(vals, logz) -> np.ndarray:
    """The five confidence scalars of every candidate (LiLiCorr appendix A,
    Architecture), read from the drafter's distribution at its slot:
    vals [..., K] are the candidates' logits in top-K order and logz [...] the
    slot's log-normaliser.  Last axis, in CONF_FIELDS order:
      logprob  l - log Z;
      prob     exp(l - log Z);
      gap      log-prob of the slot's most likely token minus the candidate's
               (>= 0; the most likely token is rank 0 of the top-K);
      rank     the candidate's rank r in 0..K-1 scaled to [0, 1] as r / (K-1)
               (0 when K = 1);
      top      1 for rank 0, else 0.
    """
    vals = np.asarray(vals, dtype=np.float64)
    logz = np.asarray(logz, dtype=np.float64)
    K = vals.shape[-1]
    # an infinite logit over an infinite log Z gives a NaN log-probability
    # (inf - inf), as the definition does; numpy's warning is not needed
    with np.errstate(invalid="ignore"):
        logp = vals - logz[..., None]
    out = np.empty(vals.shape + (5,))
    out[..., 0] = logp
    out[..., 1] = np.exp(logp)
    out[..., 2] = logp[..., :1] - logp
    out[..., 3] = np.arange(K) / max(K - 1, 1)
    out[..., 4] = (np.arange(K) == 0)
    return out


def represent(desc: OracleDesc, weights: dict, embed, ids, hidden, n: int,
              h_req_stride: int, h_slot_stride: int, offset: int = 0):
    """Steps (2)-(3): b, g, z and the pair states s."""
    keep = _Keep()
    cw = _weights(weights, embed, keep)
    flat = np.ascontiguousarray(hidden, dtype=np.uint16).reshape(-1)[offset:]
    ids = keep.arr(ids, np.int32)
    B, K, r = desc.B, desc.K, desc.r
    b = np.empty((n, B, K, r))
    g = np.empty((n, B, r))
    z = np.empty((n, B, K, r))
    s = np.empty((n, max(B - 1, 0), r))
    d = desc.c()
    _check(_load().oracle_represent(C.byref(d), C.byref(cw), n, _ptr(ids), _ptr(flat),
                                    h_req_stride, h_slot_stride, _ptr(b), _ptr(g), _ptr(z),
                                    _ptr(s)), "represent")
    return dict(b=b, g=g, z=z, s=s)


def score(desc: OracleDesc, weights: dict, vals, z, s, n: int):
    """Step (4) (or the cosine variant): delta and S, [n][B-1][K][K]."""
    keep = _Keep()
    cw = _weights(weights, None, keep)
    vals = keep.arr(vals, np.float64)
    z = keep.arr(z, np.float64)
    s = keep.arr(s, np.float64)
    B, K = desc.B, desc.K
    delta = np.empty((n, max(B - 1, 0), K, K))
    S = np.empty((n, max(B - 1, 0), K, K))
    d = desc.c()
    _check(_load().oracle_score(C.byref(d), C.byref(cw), n, _ptr(vals), _ptr(z), _ptr(s),
                                _ptr(delta), _ptr(S)), "score")
    return delta, S


def walk(desc: OracleDesc, scores, ids, n: int):
    """Step (5): tokens [n][B] and candidate choices [n][B]."""
    keep = _Keep()
    scores = keep.arr(scores, np.float64)
    ids = keep.arr(ids, np.int32)
    tokens = np.empty((n, desc.B), np.int32)
    choice = np.empty((n, desc.B), np.int32)
    d = desc.c()
    _check(_load().oracle_walk(C.byref(d), n, _ptr(scores), _ptr(ids), _ptr(tokens),
                               _ptr(choice)), "walk")
    return tokens, choice


def viterbi(desc: OracleDesc, scores, ids, n: int, lam: float = 1.0):
    """Global-Sum path rule (lam = 1): tokens [n][B], choices [n][B] and the
    summed transition score [n] of the best path (slot 1 fixed at rank 0).
    With lam < 1, pair p's term is weighted by lam**p (the Geometric rule as
    read here) and total is the weighted sum."""
    keep = _Keep()
    scores = keep.arr(scores, np.float64)
    ids = keep.arr(ids, np.int32)
    tokens = np.empty((n, desc.B), np.int32)
    choice = np.empty((n, desc.B), np.int32)
    total = np.empty(n, np.float64)
    d = desc.c()
    _check(_load().oracle_viterbi(C.byref(d), n, _ptr(scores), _ptr(ids), float(lam), _ptr(tokens),
                                  _ptr(choice), _ptr(total)), "viterbi")
    return tokens, choice, total


def beam(desc: OracleDesc, scores, ids, n: int, width: int):
    """Beam search of the given width over float32 scores (summed transition
    score, slot 1 at rank 0): tokens [n][B], choices [n][B] and the chosen
    path's float32 score [n]."""
    keep = _Keep()
    scores = keep.arr(scores, np.float32)
    ids = keep.arr(ids, np.int32)
    tokens = np.empty((n, desc.B), np.int32)
    choice = np.empty((n, desc.B), np.int32)
    total = np.empty(n, np.float32)
    d = desc.c()
    _check(_load().oracle_beam(C.byref(d), n, _ptr(scores), _ptr(ids), int(width), _ptr(tokens), _ptr(choice),
                               _ptr(total)), "beam")
    return tokens, choice, total


def accepted_lengths(tokens, targets) -> np.ndarray:
    """Greedy-verifier accepted prefix length per block."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    targets = np.ascontiguousarray(targets, dtype=np.int32)
    n, B = tokens.shape
    acc = np.empty(n, np.int32)
    _check(_load().oracle_accepted(n, B, _ptr(tokens), _ptr(targets), _ptr(acc)), "accepted")
    return acc


def run(cfg_or_desc, inputs: dict, n: int | None = None, first: int = 0):
    """One full pass over blocks [first, first+n) of a generated input set.

    ``inputs`` is the dict from ``workload.gen_inputs``: logits [n][B+1][V]
    and hidden [n][B+1][d] with the anchor at position 0 of each block.
    """
    desc = cfg_or_desc if isinstance(cfg_or_desc, OracleDesc) else OracleDesc.from_config(cfg_or_desc)
    logits, hidden = inputs["logits"], inputs["hidden"]
    ntot = logits.shape[0]
    n = ntot - first if n is None else n
    V, d = logits.shape[2], hidden.shape[2]
    lg = logits[first:first + n]
    hd = hidden[first:first + n]
    ids, vals = topk(desc, lg, n, (desc.B + 1) * V, V, offset=V)
    rep = represent(desc, inputs["weights"], inputs["embed"], ids, hd, n,
                    (desc.B + 1) * d, d, offset=d)
    delta, S = score(desc, inputs["weights"], vals, rep["z"], rep["s"], n)
    tokens, choice = walk(desc, S, ids, n)
    return dict(ids=ids, vals=vals, delta=delta, scores=S, tokens=tokens, choice=choice, **rep)
