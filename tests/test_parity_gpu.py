"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Every configuration runs the whole pass (corrector_run) and compares top-K
(exact), the intermediates z / g / s, the transition scores (S and Delta
gates) and the walk (teacher forced), as described in tests/parity.py.
Each configuration also runs with the zero-initialised output layer (walk
and S exact) and with a walk-stress output layer (w2 ~ N(0, 1)) so that the
walk leaves rank 0 often enough to be tested.
"""

import numpy as np
import pytest

import parity as P

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ tiny --

@pytest.mark.parametrize("head", ["normal", "zero", "stress"])
@pytest.mark.parametrize("ties", [False, True])
def test_tiny(head, ties):
    _log("tiny head=%s ties=%s" % (head, ties))
    x = P.inputs("tiny", head=head, ties=ties)
    gpu = P.gpu_run(x)
    ora = P.oracle_run(x)
    P.check_all(gpu, ora, "tiny/%s" % head, exact_walk=(head == "zero"))
    if head == "zero":
        want = np.broadcast_to(gpu["vals"][:, 1:, None, :], gpu["scores"].shape)
        np.testing.assert_array_equal(gpu["scores"], want)
        assert (gpu["choice"] == 0).all()


@pytest.mark.parametrize("B,n", [(2, 3), (4, 2), (7, 2)])
def test_tiny_pair_counts(B, n):
    """1, 3 and 6 adjacent pairs per request (the MLP kernel takes the pairs
    of a request two at a time; an odd count leaves a single last pair), and
    several requests per call."""
    _log("tiny B=%d n=%d" % (B, n))
    x = P.inputs("tiny", head="stress", B=B, n=n)
    gpu = P.gpu_run(x)
    ora = P.oracle_run(x)
    P.check_all(gpu, ora, "tiny/B=%d/n=%d" % (B, n))


@pytest.mark.parametrize("r", [32, 64])
def test_tiny_rep_widths(r):
    """Representation widths r = 32 and 64 (the other compiled instances of
    the candidate and MLP kernels)."""
    _log("tiny r=%d" % r)
    x = P.inputs("tiny", head="stress", r=r, n=2, B=4)
    gpu = P.gpu_run(x)
    ora = P.oracle_run(x)
    P.check_all(gpu, ora, "tiny/r=%d" % r)


@pytest.mark.parametrize("K", [1, 4, 5, 8, 13])
def test_tiny_small_k(K):
    """K = 1 (one candidate per slot: every pair a single transition, the walk
    fixed), odd K below 16 (the last predecessor and successor tasks of the
    K <= 16 MLP consumers cut short), and K = 4 and 8 (the per-pair finishing
    step with rows of one and two lanes)."""
    _log("tiny K=%d" % K)
    x = P.inputs("tiny", head="stress", K=K, n=2, B=4)
    gpu = P.gpu_run(x)
    ora = P.oracle_run(x)
    P.check_all(gpu, ora, "tiny/K=%d" % K)


@pytest.mark.parametrize("K", [37, 64])
def test_tiny_wide_k(K):
    """K = 37 (three 16-row tiles, the last ragged, in the MLP's U | V
    products; odd logit rows) and K = 64 (four tiles)."""
    _log("tiny K=%d" % K)
    x = P.inputs("tiny", head="stress", K=K, n=2, B=4)
    gpu = P.gpu_run(x)
    ora = P.oracle_run(x)
    P.check_all(gpu, ora, "tiny/K=%d" % K)


@pytest.mark.parametrize("h,K", [(80, 16), (208, 16), (80, 37), (208, 37)])
def test_tiny_mlp_widths(h, K):
    """MLP hidden widths whose last block of 64 units is partial (h = 80: 64 +
    16; h = 208: three full blocks + 16), in both MLP kernels (K <= 16 and
    K > 16): the finishing step sums several block partials, one of them from
    a block whose producer tiles and consumer units are cut at h."""
    _log("tiny h=%d K=%d" % (h, K))
    x = P.inputs("tiny", head="stress", h=h, K=K, n=2, B=4)
    gpu = P.gpu_run(x)
    ora = P.oracle_run(x)
    P.check_all(gpu, ora, "tiny/h=%d/K=%d" % (h, K))


@pytest.mark.parametrize("de", [96, 1056, 2080])
def test_tiny_embed_widths(de):
    """Candidate projections whose k-split ends in a half 64-deep slab (d_e =
    96: one split; 1056: one split of 16.5 slabs; 2080: two splits of 1056 and
    1024), over a ragged last tile of gathered rows (n B K = 60)."""
    _log("tiny d_e=%d" % de)
    x = P.inputs("tiny", head="stress", de=de, n=3, B=5)
    gpu = P.gpu_run(x)
    ora = P.oracle_run(x)
    P.check_all(gpu, ora, "tiny/de=%d" % de)


@pytest.mark.parametrize("sigma", [1.0, 8.0])
def test_tiny_cosine(sigma):
    _log("tiny cosine sigma=%g" % sigma)
    x = P.inputs("tiny", variant="cosine", sigma=sigma)
    gpu = P.gpu_run(x)
    ora = P.oracle_run(x)
    P.check_all(gpu, ora, "tiny-cos", variant="cosine")


# ---------------------------------------------------- Qwen3-8B shape, n=1 --

@pytest.mark.parametrize("head", ["normal", "zero", "stress"])
def test_b1(head):
    _log("b1 head=%s" % head)
    x = P.inputs("b1", head=head)
    gpu = P.gpu_run(x)
    ora = P.oracle_run(x)
    steps, exempt, moved = P.check_all(gpu, ora, "b1/%s" % head, exact_walk=(head == "zero"))
    _log("  walk steps %d exempt %d moved %d" % (steps, exempt, moved))


# ------------------------------------------------------------- batch 32 --

@pytest.mark.parametrize("head", ["normal", "stress"])
def test_b32(head):
    _log("b32 head=%s" % head)
    x = P.inputs("b32", head=head)
    gpu = P.gpu_run(x)
    ora = P.oracle_run(x)
    steps, exempt, moved = P.check_all(gpu, ora, "b32/%s" % head)
    _log("  walk steps %d exempt %d moved %d" % (steps, exempt, moved))
    if head == "stress":
        assert moved > steps // 10


@pytest.mark.parametrize("K", [4, 8])
def test_b32_small_k(K):
    """K = 4 and 8 at the batch-32 shape over 8 blocks (112 pairs): the
    warp-specialised MLP with each pair's finishing step and the request's
    walk in its tail, on score rows of one and two lanes; each request run
    alone (the per-(pair, 16 units) MLP form) gives the same bits."""
    _log("b32 K=%d n=8" % K)
    x = P.inputs("b32", head="stress", K=K)
    gpu = P.gpu_run(x, n=8)
    ora = P.oracle_run(x, n=8)
    steps, exempt, moved = P.check_all(gpu, ora, "b32/K=%d" % K)
    _log("  walk steps %d exempt %d moved %d" % (steps, exempt, moved))
    assert moved > 0
    for i in (0, 7):
        one = P.gpu_run(x, n=1, first=i)
        sub = P.select(gpu, i, 1)
        for k in ("ids", "vals", "scores", "tokens", "choice", "z", "s", "g"):
            np.testing.assert_array_equal(one[k], sub[k], err_msg="K=%d request %d alone: %s" % (K, i, k))


@pytest.mark.parametrize("n,first", [(6, 5), (3, 20)])
def test_b32_mid_batch(n, first):
    """Middle batch sizes, between the batch-1 and batch-32 forms: n = 6 puts
    the candidate kernel in groups of 8 (1440 candidates) and n = 3 in groups
    of 4; the small GEMM forms and the warp-specialised MLP (more than 256
    pair-block groups) run on uneven runs of pairs."""
    _log("b32 mid batch n=%d first=%d" % (n, first))
    x = P.inputs("b32", head="stress")
    gpu = P.gpu_run(x, n=n, first=first)
    ora = P.oracle_run(x, n=n, first=first)
    steps, exempt, moved = P.check_all(gpu, ora, "b32/n=%d" % n)
    _log("  walk steps %d exempt %d moved %d" % (steps, exempt, moved))
    full = P.gpu_run(x)
    sub = P.select(full, first, n)
    for k in ("ids", "vals", "scores", "tokens", "choice", "z", "s", "g"):
        np.testing.assert_array_equal(gpu[k], sub[k], err_msg="n=%d against the batch of 32: %s" % (n, k))


def test_b32_batch_invariance_and_determinism():
    _log("b32 batch invariance")
    x = P.inputs("b32")
    full = P.gpu_run(x)
    again = P.gpu_run(x)
    for k in ("ids", "vals", "scores", "tokens", "choice", "z"):
        np.testing.assert_array_equal(full[k], again[k], err_msg="rerun " + k)
    for i in (0, 17, 31):
        one = P.gpu_run(x, n=1, first=i)
        sub = P.select(full, i, 1)
        for k in ("ids", "vals", "scores", "tokens", "choice", "z", "s", "g"):
            np.testing.assert_array_equal(one[k], sub[k], err_msg="request %d alone: %s" % (i, k))


@pytest.mark.parametrize("name,n", [("b32", 32), ("b32", 1), ("tiny", 1)])
def test_tokens_only(name, n):
    """corrector_run with only the token output given (choice, ids, values and
    scores left to the workspace): the same tokens as a run that asks for
    every output."""
    _log("tokens only %s n=%d" % (name, n))
    import torch
    from draft_correction_amd import device
    x = P.inputs(name, head="stress")
    cfg = x["cfg"]
    full = P.gpu_run(x, n=n)
    dev = P.dev_inputs(x)
    corr = device.make_corrector(cfg, dev, max_requests=n)
    ws = corr.new_workspace(n)
    st = device.strides(cfg)
    tokens = torch.full((n, cfg["B"]), -1, dtype=torch.int32, device="cuda")
    corr.run(n, dev["logits"], st["l_req"], st["l_slot"], dev["hidden"], st["h_req"], st["h_slot"], tokens, ws,
             l_offset=st["l_off"], h_offset=st["h_off"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(tokens.cpu().numpy(), full["tokens"])
    corr.close()


def test_workspace_reuse_across_calls():
    """One workspace serves a sequence of calls with different request counts
    and repeated calls: each call's outputs equal those of a fresh workspace
    (no state carries over from one call to the next)."""
    _log("workspace reuse across calls")
    from draft_correction_amd import device
    for name, head in (("b32", "stress"), ("cosine", "normal")):
        x = P.inputs(name, head=head)
        cfg = x["cfg"]
        corr = device.make_corrector(cfg, P.dev_inputs(x), max_requests=cfg["n"])
        ws = corr.new_workspace(cfg["n"])
        for n, first, reps in ((cfg["n"], 0, 3), (1, 17, 2), (5, 3, 1), (cfg["n"], 0, 1), (2, 30, 2)):
            got = P.gpu_run(x, n=n, first=first, reps=reps, corr=corr, ws=ws)
            want = P.gpu_run(x, n=n, first=first)
            # the cosine variant has no pair state s (its intermediate is not written)
            keys = ("ids", "vals", "scores", "tokens", "choice", "z", "g") + (("s",) if cfg["variant"] == "mlp" else ())
            for k in keys:
                np.testing.assert_array_equal(got[k], want[k], err_msg="%s n=%d first=%d: %s" % (name, n, first, k))
        corr.close()


# ------------------------------------------------------ Global-Sum path --

@pytest.mark.parametrize("rule", ["global_sum", "geometric", "beam"])
@pytest.mark.parametrize("name,head", [("tiny", "normal"), ("tiny", "zero"), ("tiny", "stress"), ("b1", "stress"),
                                       ("b1", "zero"), ("b32", "stress"), ("cosine", "normal")])
def test_global_sum_path(name, head, rule):
    """corrector_run with the Global-Sum path rule (LiLiCorr appendix E) or the
    Geometric rule (lambda = 0.75, read as a discounted sum): the same scores
    as the walk configuration, a path that is optimal for them."""
    _log("%s %s head=%s" % (rule, name, head))
    lam = 0.75 if rule == "geometric" else 1.0
    x = P.inputs(name, head=head, path_rule=rule, path_lambda=lam, beam_width=3)
    n = 4 if name == "cosine" else None   # the cosine oracle on a sample of requests
    gpu = P.gpu_run(x, n=n)
    ora = P.oracle_run(x, n=n)
    P.check_topk(gpu, ora, name)
    P.check_scores(gpu, ora, name)
    if rule == "beam":
        P.check_beam(gpu, x["cfg"], "%s/%s" % (name, head))
        diverged = P.check_beam_bound(gpu, ora, x["cfg"], "%s/%s" % (name, head))
        _log("  beams that differ from the oracle's (each within the score error): %d" % diverged)
        if head == "zero":
            assert (gpu["choice"] == 0).all()
            assert diverged == 0
        return
    near = P.check_global_sum(gpu, ora, x["cfg"], "%s/%s/%s" % (rule, name, head), exact=(head == "zero"), lam=lam)
    if head == "zero":
        assert (gpu["choice"] == 0).all()
    _log("  near-tie paths: %d" % near)


# ------------------------------------------- top-m successor sparsification --

@pytest.mark.parametrize("name,head,m", [("tiny", "stress", 2), ("b1", "stress", 8), ("b32", "normal", 8),
                                         ("b32", "stress", 4), ("cosine", "normal", 8)])
def test_top_m_successors(name, head, m):
    """Only the first m successors of each pair are scored (the rest are -inf);
    the kept scores pass the usual gates and the walk never leaves them."""
    _log("top-m %s head=%s m=%d" % (name, head, m))
    x = P.inputs(name, head=head, succ_top_m=m)
    n = 4 if name == "cosine" else None
    gpu = P.gpu_run(x, n=n)
    ora = P.oracle_run(x, n=n)
    P.check_topk(gpu, ora, name)
    assert np.isneginf(gpu["scores"][..., m:]).all()
    kept_g = dict(gpu, scores=gpu["scores"][..., :m], vals=gpu["vals"][..., :m])
    kept_o = dict(ora, scores=ora["scores"][..., :m], delta=ora["delta"][..., :m])
    P.check_scores(kept_g, kept_o, "%s/m=%d" % (name, m))
    P.check_walk(gpu, ora, "%s/m=%d" % (name, m))
    assert (gpu["choice"][:, 1:] < m).all()


# ---------------------------------------------------------------- cosine --

@pytest.mark.parametrize("sigma", [1.0, 8.0])
def test_cosine_b32(sigma):
    """Every request of the batch against the oracle.  The walk must leave
    rank 0 somewhere: on these inputs the oracle's walk departs in about 3 %
    of the steps at sigma = 1 and about 19 % at sigma = 8."""
    _log("cosine b32 sigma=%g" % sigma)
    x = P.inputs("cosine", sigma=sigma)
    gpu = P.gpu_run(x)
    ora = P.oracle_run(x)
    steps, exempt, moved = P.check_all(gpu, ora, "cosine", variant="cosine")
    _log("  walk steps %d exempt %d moved %d" % (steps, exempt, moved))
    assert moved > 0
    if sigma == 8.0:
        assert moved > steps // 20
    bound = np.abs(gpu["scores"] - gpu["vals"][:, 1:, None, :])
    assert (bound <= sigma * (1 + 1e-5)).all()


# ---------------------------------------------------------------- stress --

@pytest.mark.parametrize("head", ["normal", "stress"])
def test_stress(head):
    """The full stress batch (256 requests, K = 32, d = 5120): top-K of every
    row exactly, everything else on sampled requests (one per entropy tier and
    a few more).  The walk-stress head (w2 ~ N(0, 1)) makes the K = 32 walk
    leave rank 0, which the normal head almost never does."""
    _log("stress n=256 K=32 d=5120 head=%s" % head)
    x = P.inputs("stress", head=head)
    gpu = P.gpu_run(x)
    cfg = x["cfg"]
    if head == "normal":
        ids, vals = P.oracle.topk(P.oracle.OracleDesc.from_config(cfg), x["logits"], cfg["n"],
                                  (cfg["B"] + 1) * cfg["V"], cfg["V"], offset=cfg["V"])
        P.check_topk(gpu, dict(ids=ids, vals=vals), "stress")
    total_moved = 0
    for i in (0, 77, 128, 200, 255):
        ora = P.oracle_run(x, n=1, first=i)
        steps, exempt, moved = P.check_all(P.select(gpu, i, 1), ora, "stress/%s/%d" % (head, i))
        total_moved += moved
    _log("  sampled walk steps moved from rank 0: %d" % total_moved)
    if head == "stress":
        assert total_moved > 0


def test_long_runs():
    """Many requests at K = 16 and the full hidden width (400 blocks of a small
    vocabulary and d): the K <= 16 MLP's workgroups then take runs of 64 pairs,
    the most one holds (more workgroups than CUs), across request boundaries.
    Sampled requests against the oracle, the first and last included, with the
    walk-stress head so the walk moves."""
    _log("long runs n=400 K=16 h=256")
    x = P.inputs("b1", head="stress", n=400, V=4096, d=64, de=64)
    gpu = P.gpu_run(x)
    total_moved = 0
    for i in (0, 1, 63, 64, 199, 398, 399):
        ora = P.oracle_run(x, n=1, first=i)
        steps, exempt, moved = P.check_all(P.select(gpu, i, 1), ora, "long runs/%d" % i)
        total_moved += moved
    assert total_moved > 0


# ---------------------------------------------------- folded projection --

@pytest.mark.parametrize("name,head", [("tiny", "stress"), ("b1", "stress"), ("b32", "normal"),
                                       ("b32", "stress")])
def test_folded_table(name, head):
    """corrector_fold_table + corrector_use_table: the candidate projection reads
    rows of E W_cand^T; every gate as for the per-pass projection."""
    _log("folded %s head=%s" % (name, head))
    x = P.inputs(name, head=head)
    gpu = P.gpu_run(x, fold=True)
    ora = P.oracle_run(x)
    P.check_all(gpu, ora, "folded/%s/%s" % (name, head))


def test_folded_cosine():
    _log("folded cosine")
    x = P.inputs("cosine", sigma=8.0)
    gpu = P.gpu_run(x, fold=True)
    ora = P.oracle_run(x, n=1, first=7)
    P.check_all(P.select(gpu, 7, 1), ora, "folded-cos", variant="cosine")


def test_fold_table_rows():
    """Rows of the folded table against a plain float64 product E[v] W_cand^T."""
    import torch
    from draft_correction_amd import device
    from workload import bf16_bits_to_f32
    x = P.inputs("b1")
    cfg = x["cfg"]
    dev = P.dev_inputs(x)
    corr = device.make_corrector(cfg, dev)
    table = torch.empty(corr.table_bytes() // 4, dtype=torch.float32, device="cuda")
    corr.fold_table(table)
    torch.cuda.synchronize()
    T = table.view(cfg["V"], cfg["r"]).cpu().numpy()
    corr.close()
    rows = np.array([0, 1, 4095, 4096, 77777, cfg["V"] - 1])
    E = bf16_bits_to_f32(x["embed"][rows]).astype(np.float64).reshape(len(rows), cfg["de"])
    W = bf16_bits_to_f32(x["weights"]["w_cand"]).astype(np.float64).reshape(cfg["r"], cfg["de"])
    want = E @ W.T
    np.testing.assert_allclose(T[rows], want, rtol=1e-4, atol=1e-5 * np.abs(want).max())
