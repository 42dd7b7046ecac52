"""CPU checks of the C-ABI boundary: the library loads, exports every call the
header declares, and rejects bad arguments on the host before anything is
enqueued (no call here reaches a kernel, so no GPU is needed)."""

import ctypes as C
import os
import re

import pytest

from draft_correction_amd import corrector as corr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "corrector.h")

FAKE = 0x10000  # a 64 KiB-aligned fake device address; never dereferenced here


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(corr.LIB_PATH):
        from draft_correction_amd import build
        build.build()
    return corr.load()


def declared_calls():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|void|size_t|const char \*)\s*\*?\s*(corrector_\w+)\s*\(",
                                 text, re.M)))


def test_exports_every_declared_call(lib):
    names = declared_calls()
    assert len(names) >= 10
    assert set(names) == set(corr.SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def _desc(**kw):
    base = dict(vocab=151936, slots=15, k=16, d_hidden=4096, d_embed=4096, r=128, mlp_hidden=256,
                d_vec=128, variant=0, logits_dtype=0, max_requests=32, ln_eps=1e-5, sigma=1.0,
                path_rule=0, path_lambda=0.75, beam_width=4, succ_top_m=0)
    base.update(kw)
    return corr.CorrectorDesc(*[base[f] for f, _ in corr.CorrectorDesc._fields_])


def _weights(**kw):
    w = {n: FAKE for n in corr.WEIGHT_FIELDS}
    w.update(kw)
    return corr.CorrectorWeights(*[w[n] for n in corr.WEIGHT_FIELDS])


def _create(lib, d, w):
    h = C.c_void_p()
    rc = lib.corrector_create(C.byref(d), C.byref(w), C.byref(h))
    return rc, h


def test_create_and_workspace(lib):
    rc, h = _create(lib, _desc(), _weights())
    assert rc == 0 and h.value
    ws1 = lib.corrector_workspace_bytes(h, 1)
    ws32 = lib.corrector_workspace_bytes(h, 32)
    assert 0 < ws1 < ws32
    assert lib.corrector_workspace_bytes(h, 33) == 0
    assert lib.corrector_workspace_bytes(h, -1) == 0
    lib.corrector_destroy(h)


@pytest.mark.parametrize("field,value,code", [
    ("vocab", 0, 2), ("k", 0, 2), ("k", 65, 2), ("slots", 0, 2), ("d_hidden", 100, 2),
    ("d_embed", 0, 2), ("r", 96, 3), ("mlp_hidden", 8, 3), ("mlp_hidden", 512, 3),
    ("variant", 2, 3), ("logits_dtype", 5, 3), ("max_requests", 0, 2), ("ln_eps", 0.0, 2),
    ("path_rule", 4, 3), ("path_rule", -1, 3), ("succ_top_m", -1, 2), ("succ_top_m", 17, 2),
])
def test_create_rejects_bad_desc(lib, field, value, code):
    rc, h = _create(lib, _desc(**{field: value}), _weights())
    assert rc == code and not h.value


def test_create_accepts_every_path_rule(lib):
    for rule in (0, 1, 2, 3):
        rc, h = _create(lib, _desc(path_rule=rule), _weights())
        assert rc == 0 and h.value
        lib.corrector_destroy(h)


def test_geometric_lambda_range(lib):
    for lam in (0.0, -0.5, 1.5, float("nan"), float("inf")):
        rc, h = _create(lib, _desc(path_rule=2, path_lambda=lam), _weights())
        assert rc == 2 and not h.value, lam
    for lam in (1e-3, 1.0):
        rc, h = _create(lib, _desc(path_rule=2, path_lambda=lam), _weights())
        assert rc == 0
        lib.corrector_destroy(h)
    for width, code in ((0, 2), (5, 2), (-1, 2), (1, 0), (4, 0)):
        rc, h = _create(lib, _desc(path_rule=3, beam_width=width), _weights())
        assert rc == code, width
        if rc == 0:
            lib.corrector_destroy(h)
    # the other rules ignore lambda
    rc, h = _create(lib, _desc(path_rule=1, path_lambda=0.0), _weights())
    assert rc == 0
    lib.corrector_destroy(h)


def test_create_rejects_k_above_v(lib):
    rc, _ = _create(lib, _desc(vocab=8, k=9), _weights())
    assert rc == 2


def test_create_checks_weights(lib):
    assert _create(lib, _desc(), _weights(w1=None))[0] == 1
    assert _create(lib, _desc(), _weights(embed=None))[0] == 1
    assert _create(lib, _desc(variant=1), _weights(w_in=None))[0] == 1
    rc, h = _create(lib, _desc(variant=1), _weights(w_pair=None, w1=None, b1=None, w2=None, b2=None))
    assert rc == 0
    lib.corrector_destroy(h)
    assert _create(lib, _desc(), _weights(w_cand=FAKE + 2))[0] == 4
    h = C.c_void_p()
    assert lib.corrector_create(None, C.byref(_weights()), C.byref(h)) == 1


def test_calls_validate_before_launch(lib):
    rc, h = _create(lib, _desc(max_requests=4), _weights())
    assert rc == 0
    need = lib.corrector_workspace_bytes(h, 4)
    # n = 0 is a no-op even with null pointers
    assert lib.corrector_topk(h, 0, None, 0, 0, None, None, None, 0, None) == 0
    assert lib.corrector_run(h, 0, None, 0, 0, None, 0, 0, None, None, None, None, None, None, 0, None) == 0
    # too many requests
    assert lib.corrector_topk(h, 5, FAKE, 16 * 151936, 151936, FAKE, FAKE, FAKE, need, None) == 2
    # null logits / outputs
    assert lib.corrector_topk(h, 1, None, 0, 0, FAKE, FAKE, FAKE, need, None) == 1
    assert lib.corrector_topk(h, 1, FAKE, 0, 0, None, FAKE, FAKE, need, None) == 1
    # misaligned pointer and stride (bf16: 8 elements per 16 bytes)
    assert lib.corrector_topk(h, 1, FAKE + 2, 0, 151936, FAKE, FAKE, FAKE, need, None) == 4
    assert lib.corrector_topk(h, 1, FAKE, 0, 151937, FAKE, FAKE, FAKE, need, None) == 4
    # negative strides
    assert lib.corrector_topk(h, 1, FAKE, -8, 8, FAKE, FAKE, FAKE, need, None) == 2
    # workspace too small / missing / misaligned
    assert lib.corrector_topk(h, 4, FAKE, 16 * 151936, 151936, FAKE, FAKE, FAKE, need - 1, None) == 5
    assert lib.corrector_topk(h, 1, FAKE, 16 * 151936, 151936, FAKE, FAKE, None, need, None) == 1
    assert lib.corrector_topk(h, 1, FAKE, 16 * 151936, 151936, FAKE, FAKE, FAKE + 4, need, None) == 4
    # fused top-K + normalisation: logz required, conf optional; same checks as top-K
    assert lib.corrector_topk_softmax(h, 1, FAKE, 16 * 151936, 151936, FAKE, FAKE, None, None, FAKE, need,
                                      None) == 1
    assert lib.corrector_topk_softmax(h, 5, FAKE, 16 * 151936, 151936, FAKE, FAKE, FAKE, None, FAKE, need,
                                      None) == 2
    assert lib.corrector_topk_softmax(h, 1, FAKE + 2, 0, 151936, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == 4
    assert lib.corrector_topk_softmax(h, 4, FAKE, 16 * 151936, 151936, FAKE, FAKE, FAKE, None, FAKE, need - 1,
                                      None) == 5
    assert lib.corrector_topk_softmax(h, 0, None, 0, 0, None, None, None, None, None, 0, None) == 0
    # score: hidden alignment, null scores
    assert lib.corrector_score(h, 1, FAKE, FAKE, FAKE + 2, 0, 4096, FAKE, FAKE, need, None) == 4
    assert lib.corrector_score(h, 1, FAKE, FAKE, FAKE, 0, 4096, None, FAKE, need, None) == 1
    # walk: null tokens
    assert lib.corrector_walk(h, 1, FAKE, FAKE, None, None, None) == 1
    # run: tokens required
    assert lib.corrector_run(h, 1, FAKE, 16 * 151936, 151936, FAKE, 16 * 4096, 4096, None, None,
                             None, None, None, FAKE, need, None) == 1
    lib.corrector_destroy(h)


def test_destroyed_and_null_handles(lib):
    assert lib.corrector_topk(None, 1, FAKE, 0, 0, FAKE, FAKE, FAKE, 1 << 30, None) == 7
    assert lib.corrector_topk_softmax(None, 1, FAKE, 0, 0, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == 7
    assert lib.corrector_workspace_bytes(None, 1) == 0
    lib.corrector_destroy(None)


def test_status_strings(lib):
    for code in range(8):
        assert lib.corrector_status_string(code)
    assert lib.corrector_status_string(99) == b"unknown status"
