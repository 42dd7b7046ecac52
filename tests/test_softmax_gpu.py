"""Fused top-K and vocabulary-wide normalisation (corrector_topk_softmax) on
the GPU against the oracle: top-K ids and values bit-exact and identical to
corrector_topk's, log Z within the float32 bound below, the five confidence
scalars within the bounds that follow from it.  Workload-sized batches
(Zipf-like bf16 logits, V = 151936, K = 16 and 32) and edge rows: ragged
vocabularies, K = 1 and K = V, rows of -inf, a single finite logit, ties,
values near the float32 and bfloat16 maxima, float32 and bf16 rows.

Tolerance of log Z (float32 arithmetic): each chunk of 6144 (bf16) or 3072
(float32) logits is summed as exp(l - m) with m the lane maximum, every term
within a few ulp, then lanes, chunks and the row are combined by sums of at
most 96, 64 and ~50 terms; the relative error of the sum stays below
~1e-5 and log turns it into an absolute error of the same size.  Rounding
log Z itself to float32 adds 2^-24 |log Z|.  The gate is
|log Z_gpu - log Z| <= 2e-5 + 2^-22 |log Z|.
"""

import numpy as np
import pytest
import torch

import oracle
from draft_correction_amd import device
from workload import config, f32_to_bf16_bits, gen_weights
from workload.gen import gen_logits

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def logz_tol(lz):
    lz = np.asarray(lz, dtype=np.float64)
    return 2e-5 + 2.0 ** -22 * np.abs(np.where(np.isfinite(lz), lz, 0.0))


def check_softmax(ids, vals, logz, conf, want_ids, want_vals, want_logz, where=""):
    """Gates of the fused call against the oracle's top-K, log Z and scalars."""
    np.testing.assert_array_equal(ids, want_ids, err_msg="ids " + where)
    np.testing.assert_array_equal(vals.astype(np.float64), want_vals, err_msg="vals " + where)
    lz = logz.astype(np.float64)
    fin = np.isfinite(want_logz)
    np.testing.assert_array_equal(lz[~fin], want_logz[~fin], err_msg="log Z (-inf rows) " + where)
    err = np.abs(lz[fin] - want_logz[fin])
    tol = logz_tol(want_logz[fin])
    assert (err <= tol).all(), "log Z %s: worst %.3g (tol %.3g)" % (where, err.max(), tol[np.argmax(err - tol)])
    if conf is None:
        return
    # scalars from the oracle's values and log Z; the GPU's log-prob may differ
    # by its log Z error plus the rounding of l - log Z
    want = oracle.confidence(want_vals, want_logz)
    c = conf.astype(np.float64)
    dl = logz_tol(want_logz)[..., None] + 2.0 ** -23 * np.abs(np.nan_to_num(want[..., 0], posinf=0, neginf=0))
    ok = np.isfinite(want[..., 0])
    np.testing.assert_array_equal(c[..., 0][~ok], want[..., 0][~ok], err_msg="log-prob (non-finite) " + where)
    assert (np.abs(c[..., 0][ok] - want[..., 0][ok]) <= dl[ok]).all(), "log-prob " + where
    # probability: relative error of exp from the log-prob error, plus float32 rounding
    # (a probability of exactly 0, a -inf candidate, must be 0: its bound is 0,
    # not 0 * inf where log Z's bound is huge)
    with np.errstate(over="ignore", invalid="ignore"):
        pt = np.where(want[..., 1] == 0, 0.0, want[..., 1] * (np.expm1(dl) + 2.0 ** -21))
    np.testing.assert_array_equal(np.isnan(c[..., 1]), np.isnan(want[..., 1]), err_msg="prob NaN " + where)
    m = ~np.isnan(want[..., 1])
    assert (np.abs(c[..., 1] - want[..., 1])[m] <= pt[m]).all(), "prob " + where
    # gap: one float32 subtraction of two float32-exact logits
    g = want[..., 2]
    gm = np.isfinite(g)
    assert (np.abs(c[..., 2][gm] - g[gm]) <= 2.0 ** -23 * np.abs(g[gm])).all(), "gap " + where
    np.testing.assert_array_equal(c[..., 2][~gm], g[~gm], err_msg="gap (non-finite) " + where)
    # rank: one correctly rounded float32 division; top flag exact
    np.testing.assert_allclose(c[..., 3], want[..., 3], rtol=2.0 ** -23, atol=0, err_msg="rank " + where)
    np.testing.assert_array_equal(c[..., 4], want[..., 4], err_msg="top flag " + where)


# ----------------------------------------------------------- workloads --

def _topk_corrector(cfg):
    """A handle for the top-K calls only: the widths of the later steps are
    shrunk (top-K reads none of their weights) and the embedding is zero."""
    small = dict(cfg, d=64, de=64, r=16, h=32, dvec=16)
    emb = np.zeros((cfg["V"], 64), np.uint16)
    return device.make_corrector(small, dict(weights=device.weights_to_device(gen_weights(small), emb)),
                                 max_requests=cfg["n"])


def _fused(corr, cfg, logits_dev, n, conf=True):
    B, K = cfg["B"], cfg["K"]
    st = device.strides(cfg)
    ids = torch.empty((n, B, K), dtype=torch.int32, device="cuda")
    vals = torch.empty((n, B, K), dtype=torch.float32, device="cuda")
    logz = torch.empty((n, B), dtype=torch.float32, device="cuda")
    cf = torch.empty((n, B, K, 5), dtype=torch.float32, device="cuda") if conf else None
    corr.topk_softmax(n, logits_dev, st["l_req"], st["l_slot"], ids, vals, logz, corr.new_workspace(n), conf=cf,
                      offset=st["l_off"])
    torch.cuda.synchronize()
    return (ids.cpu().numpy(), vals.cpu().numpy(), logz.cpu().numpy(),
            cf.cpu().numpy() if conf else None)


@pytest.mark.parametrize("name", ["tiny", "b1", "b32", "stress"])
def test_workload_rows(name):
    """Every drafted row of the workload's logits (anchor rows skipped by the
    strides); ids and values also equal corrector_topk's."""
    _log("topk_softmax %s" % name)
    cfg = config(name)
    logits = gen_logits(cfg)
    n, B, K, V = cfg["n"], cfg["B"], cfg["K"], cfg["V"]
    corr = _topk_corrector(cfg)
    t = device.tensor(logits)
    ids, vals, logz, conf = _fused(corr, cfg, t, n)
    st = device.strides(cfg)
    ids2 = torch.empty((n, B, K), dtype=torch.int32, device="cuda")
    vals2 = torch.empty((n, B, K), dtype=torch.float32, device="cuda")
    corr.topk(n, t, st["l_req"], st["l_slot"], ids2, vals2, corr.new_workspace(n), offset=st["l_off"])
    torch.cuda.synchronize()
    corr.close()
    np.testing.assert_array_equal(ids, ids2.cpu().numpy())
    np.testing.assert_array_equal(vals, vals2.cpu().numpy())
    d = oracle.OracleDesc.from_config(cfg)
    want_ids, want_vals = oracle.topk(d, logits, n, (B + 1) * V, V, offset=V)
    want_logz = oracle.log_normaliser(d, logits, n, (B + 1) * V, V, offset=V)
    check_softmax(ids, vals, logz, conf, want_ids, want_vals, want_logz, name)


def test_conf_is_optional():
    _log("topk_softmax without conf")
    cfg = config("b1")
    logits = device.tensor(gen_logits(cfg))
    corr = _topk_corrector(cfg)
    a = _fused(corr, cfg, logits, 1, conf=False)
    b = _fused(corr, cfg, logits, 1, conf=True)
    corr.close()
    for u, v in zip(a[:3], b[:3]):
        np.testing.assert_array_equal(u, v)


# ----------------------------------------------------------------- edges --

def _run(rows_f32, K, dtype):
    """rows_f32: [n][B][V] float32 values (bf16-rounded when dtype is bf16)."""
    n, B, V = rows_f32.shape
    cfg = config("tiny", V=V, K=K, logits_dtype=dtype, n=n, B=B)
    emb = np.zeros((V, cfg["de"]), np.uint16)
    corr = device.make_corrector(cfg, dict(weights=device.weights_to_device(gen_weights(cfg), emb)),
                                 max_requests=n)
    host = f32_to_bf16_bits(rows_f32).reshape(rows_f32.shape) if dtype == "bf16" else rows_f32.astype(np.float32)
    per = 8 if dtype == "bf16" else 4          # keep every row start 16-byte aligned
    Vp = (V + per - 1) // per * per
    buf = np.zeros((n, B, Vp), host.dtype)
    buf[..., :V] = host
    t = device.tensor(buf)
    ids = torch.empty((n, B, K), dtype=torch.int32, device="cuda")
    vals = torch.empty((n, B, K), dtype=torch.float32, device="cuda")
    logz = torch.empty((n, B), dtype=torch.float32, device="cuda")
    conf = torch.empty((n, B, K, 5), dtype=torch.float32, device="cuda")
    corr.topk_softmax(n, t, B * Vp, Vp, ids, vals, logz, corr.new_workspace(n), conf=conf)
    torch.cuda.synchronize()
    corr.close()
    want_ids = np.empty((n, B, K), np.int32)
    want_vals = np.empty((n, B, K))
    want_logz = np.empty((n, B))
    for i in range(n):
        for s in range(B):
            want_ids[i, s], want_vals[i, s] = oracle.topk_row(host[i, s], K)
            want_logz[i, s] = oracle.log_normaliser_row(host[i, s])
    check_softmax(ids.cpu().numpy(), vals.cpu().numpy(), logz.cpu().numpy(), conf.cpu().numpy(),
                  want_ids, want_vals, want_logz, "%s V=%d K=%d" % (dtype, V, K))


@pytest.mark.parametrize("V,K", [(1, 1), (7, 7), (64, 64), (1003, 5), (6144, 16), (6145, 1), (8193, 64),
                                 (151936, 32)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_and_extreme_k(V, K, dtype):
    _log("softmax ragged V=%d K=%d %s" % (V, K, dtype))
    g = np.random.default_rng(V * 7 + K)
    rows = (g.normal(size=(2, 3, V)) * 3).astype(np.float32)
    rows[1, 2] += 40.0                            # a shifted row
    _run(rows, K, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_infinities_ties_and_extremes(dtype):
    _log("softmax extremes %s" % dtype)
    V = 20000
    rows = np.zeros((1, 6, V), np.float32)
    rows[0, 0] = -np.inf                          # no finite logit: log Z = -inf
    rows[0, 1] = -np.inf
    rows[0, 1, 12345] = 3.25                      # one finite logit: log Z = 3.25, p = 1
    rows[0, 2] = 1.5                              # all equal: log Z = 1.5 + log V
    big = np.float32(3.0e38) if dtype == "f32" else np.float32(3.3e38)
    rows[0, 3] = -np.inf
    rows[0, 3, ::1000] = big                      # near the maximum: exp(l) alone would overflow
    rows[0, 4] = np.random.default_rng(1).normal(size=V).astype(np.float32) - 80.0   # far below zero
    rows[0, 5] = np.random.default_rng(2).choice(np.array([0.0, -0.0, -np.inf, 1.0], np.float32), size=V)
    _run(rows, 16, dtype)
    _run(rows[:, :, :7], 7, dtype)                # K = V with -inf candidates
