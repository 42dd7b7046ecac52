"""corrector_walk on caller-supplied scores, on the GPU, against the oracle,
for every path rule: the prefix-first walk (DCOCO method details step (5))
and the beam search (widths 1, 2, 4; float32 extension sums on both sides)
exactly, and the Global-Sum (LiLiCorr appendix E, Eq. 12) and Geometric
(lambda = 0.75, a discounted sum) paths as optimal for the scores given.

Shapes cover one-wave groups of 16 predecessors with a ragged last group
(K = 37), K = 1, B = 1 and 2, and scores too large for one workgroup's LDS
(B = K = 64: 1 MB per request), which the path kernel reads from memory
instead of staging.  Integer-valued scores force ties.
"""

import numpy as np
import pytest
import torch

import oracle
from draft_correction_amd import device
from workload import config, gen_weights

pytestmark = pytest.mark.gpu

LAM = {"greedy": 1.0, "global_sum": 1.0, "geometric": 0.75, "beam1": 1.0, "beam2": 1.0, "beam4": 1.0}


def _walk(S, ids, rule):
    n, Bm1, K, _ = S.shape
    B = Bm1 + 1
    width = int(rule[4:]) if rule.startswith("beam") else 4
    cfg = config("tiny", B=B, K=K, V=max(1000, K), n=n, path_rule="beam" if rule.startswith("beam") else rule,
                 path_lambda=LAM[rule], beam_width=width)
    emb = np.zeros((cfg["V"], cfg["de"]), np.uint16)
    corr = device.make_corrector(cfg, dict(weights=device.weights_to_device(gen_weights(cfg), emb)), max_requests=n)
    tokens = torch.empty((n, B), dtype=torch.int32, device="cuda")
    choice = torch.empty((n, B), dtype=torch.int32, device="cuda")
    s = torch.from_numpy(np.ascontiguousarray(S, dtype=np.float32)).cuda()
    i = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    corr.walk(n, s if Bm1 > 0 else None, i, tokens, choice)
    torch.cuda.synchronize()
    corr.close()
    return tokens.cpu().numpy(), choice.cpu().numpy(), cfg


def _weighted(S, choice, lam):
    n, P = S.shape[0], S.shape[1]
    i = np.arange(n)[:, None]
    p = np.arange(P)[None, :]
    return (S[i, p, choice[:, :-1], choice[:, 1:]] * lam ** np.arange(P)[None, :]).sum(axis=1)


def _check(S, ids, rule, where, ties=False):
    tokens, choice, cfg = _walk(S, ids, rule)
    n, B = choice.shape
    desc = oracle.OracleDesc.from_config(cfg)
    S64 = S.astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(tokens, np.take_along_axis(ids, choice[:, :, None], 2)[:, :, 0],
                                  err_msg="tokens follow the choices " + where)
    assert (choice[:, 0] == 0).all()
    if rule.startswith("beam"):
        want_t, want_c, _ = oracle.beam(desc, S.astype(np.float32), ids, n, int(rule[4:]))
        np.testing.assert_array_equal(choice, want_c, err_msg="beam " + where)
        np.testing.assert_array_equal(tokens, want_t, err_msg="beam tokens " + where)
        return
    if rule == "greedy":
        want_t, want_c = oracle.walk(desc, S64, ids, n)
        np.testing.assert_array_equal(choice, want_c, err_msg="walk " + where)
        np.testing.assert_array_equal(tokens, want_t, err_msg="walk tokens " + where)
        return
    lam = LAM[rule]
    _, want_c, want_tot = oracle.viterbi(desc, S64, ids, n, lam=lam)
    if B < 2:
        np.testing.assert_array_equal(choice, want_c)
        return
    # float32 sums on the GPU: the same path, or one within rounding of the optimum
    scale = max(1.0, float(np.abs(S64).max()))
    got = _weighted(S64, choice, lam)
    assert (np.abs(got - want_tot) <= 1e-5 * (B - 1) * scale).all(), "%s: not optimal" % where
    # Continuous scores: near-ties that rounding may resolve either way are
    # rare, as long as every pair's weight lam^p stays well above float32
    # resolution of the total (at lam = 0.75 and B = 64 the last pairs weigh
    # ~1e-8 and the GPU can only be optimal to rounding there).
    if not ties and lam ** (B - 2) >= 1e-3:
        same = (choice == want_c).all(axis=1)
        assert same.mean() >= 0.6, "%s: %d of %d paths differ" % (where, (~same).sum(), n)


@pytest.mark.parametrize("rule", ["greedy", "global_sum", "geometric", "beam1", "beam2", "beam4"])
@pytest.mark.parametrize("B,K", [(15, 16), (15, 37), (5, 1), (1, 8), (2, 64), (64, 64)])
def test_walk_rules(rule, B, K):
    print("walk %s B=%d K=%d" % (rule, B, K), flush=True)
    g = np.random.default_rng(B * 100 + K)
    n = 8 if B * K * K <= 64 * 64 * 16 else 3
    S = g.normal(size=(n, B - 1, K, K)).astype(np.float32)
    ids = g.integers(0, 1000, size=(n, B, K)).astype(np.int32)
    _check(S, ids, rule, "normal %s B=%d K=%d" % (rule, B, K))
    # integer scores: ties everywhere (the walk resolves them to the lowest
    # index, exactly; the dynamic programs return an optimal path)
    S = g.integers(-2, 3, size=(n, B - 1, K, K)).astype(np.float32)
    _check(S, ids, rule, "ties %s B=%d K=%d" % (rule, B, K), ties=True)


@pytest.mark.parametrize("rule", ["global_sum", "geometric", "beam1", "beam2", "beam4"])
def test_k16_forms_match_general(rule):
    """For K <= 16 the dynamic program and the beam search run in forms that
    spread a pair's work over all 64 lanes; they must choose exactly what the
    general forms choose.  The same scores padded with a 17th candidate whose
    scores are all -inf (which no path can use) go through the general forms:
    the choices must be identical, on continuous scores and on tie-heavy
    integer scores."""
    print("K=16 forms against K=17 %s" % rule, flush=True)
    g = np.random.default_rng(1616)
    n, B, K = 8, 15, 16
    ids = g.integers(0, 1000, size=(n, B, K)).astype(np.int32)
    ids17 = np.concatenate([ids, np.zeros((n, B, 1), np.int32)], axis=2)
    for kind in ("normal", "ties"):
        S = (g.normal(size=(n, B - 1, K, K)) if kind == "normal"
             else g.integers(-2, 3, size=(n, B - 1, K, K))).astype(np.float32)
        S17 = np.full((n, B - 1, K + 1, K + 1), -np.inf, np.float32)
        S17[:, :, :K, :K] = S
        t16, c16, _ = _walk(S, ids, rule)
        t17, c17, _ = _walk(S17, ids17, rule)
        np.testing.assert_array_equal(c16, c17, err_msg="%s %s" % (rule, kind))
        np.testing.assert_array_equal(t16, t17, err_msg="%s %s tokens" % (rule, kind))
