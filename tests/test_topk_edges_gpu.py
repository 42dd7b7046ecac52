"""Top-K edge cases on the GPU through corrector_topk, exact against the
oracle: heavy ties (a whole row of equal values forces the tie-overflow
path), signed zeros and -inf, K = V, ragged vocabularies that end inside a
16-byte vector and inside a chunk, K = 1 and K = 64, float32 and bf16 rows."""

import numpy as np
import pytest
import torch

import oracle
from draft_correction_amd import device
from workload import config, f32_to_bf16_bits, gen_weights

pytestmark = pytest.mark.gpu


def _corrector(V, K, dtype, n):
    cfg = config("tiny", V=V, K=K, logits_dtype=dtype, n=n, B=3)
    w = gen_weights(cfg)
    emb = np.zeros((V, cfg["de"]), np.uint16)
    dev = dict(weights=device.weights_to_device(w, emb))
    return cfg, device.make_corrector(cfg, dev, max_requests=n)


def _run(rows_f32, K, dtype):
    """rows_f32: [n][B][V] float32 values (bf16-rounded when dtype is bf16)."""
    n, B, V = rows_f32.shape
    cfg, corr = _corrector(V, K, dtype, n)
    if dtype == "bf16":
        host = f32_to_bf16_bits(rows_f32).reshape(rows_f32.shape)
    else:
        host = rows_f32.astype(np.float32)
    # pad each row to a 16-byte multiple so every row start stays aligned
    esz = 2 if dtype == "bf16" else 4
    per = 16 // esz
    Vp = (V + per - 1) // per * per
    buf = np.zeros((n, B, Vp), host.dtype)
    buf[..., :V] = host
    t = device.tensor(buf)
    ids = torch.empty((n, B, K), dtype=torch.int32, device="cuda")
    vals = torch.empty((n, B, K), dtype=torch.float32, device="cuda")
    ws = corr.new_workspace(n)
    corr.topk(n, t, B * Vp, Vp, ids, vals, ws)
    torch.cuda.synchronize()
    ids, vals = ids.cpu().numpy(), vals.cpu().numpy()
    corr.close()
    for i in range(n):
        for s in range(B):
            oi, ov = oracle.topk_row(host[i, s], K)
            np.testing.assert_array_equal(ids[i, s], oi, err_msg="row %d/%d" % (i, s))
            np.testing.assert_array_equal(vals[i, s].astype(np.float64), ov)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_all_equal_rows(dtype):
    print("all-equal rows", dtype, flush=True)
    rows = np.full((2, 3, 20000), 1.5, np.float32)
    rows[1, 2, :] = -0.0
    rows[1, 1, ::2] = 0.0
    rows[1, 1, 1::2] = -0.0
    _run(rows, 16, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_signed_zero_and_inf(dtype):
    print("signed zero / inf", dtype, flush=True)
    g = np.random.default_rng(0)
    rows = g.choice(np.array([0.0, -0.0, -np.inf, 1.0, -1.0], np.float32), size=(1, 3, 9000))
    _run(rows.astype(np.float32), 32, dtype)


@pytest.mark.parametrize("V,K", [(1, 1), (7, 7), (64, 64), (8193, 64), (8200, 1), (1003, 5),
                                 (16384 + 3, 17), (151936, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_and_extreme_k(V, K, dtype):
    print("ragged V=%d K=%d %s" % (V, K, dtype), flush=True)
    g = np.random.default_rng(V * 131 + K)
    rows = g.normal(size=(1, 3, V)).astype(np.float32)
    if V > 10:
        rows[0, 1, g.integers(0, V, size=V // 4)] = 2.5   # many ties near the top
    _run(rows, K, dtype)


def test_low_entropy_and_duplicates_bf16():
    print("coarse bf16 values", flush=True)
    g = np.random.default_rng(5)
    rows = np.round(g.normal(size=(2, 3, 40000)) * 2) / 2   # few distinct values
    _run(rows.astype(np.float32), 16, "bf16")
