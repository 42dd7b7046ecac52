"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against what the pages or the mathematics fix:
library routines on special cases (NumPy lexsort, torch CPU linear /
layer_norm / gelu / normalize in float64), brute force on tiny inputs, closed
forms, invariants, and the numbers the pages print.  A plausible mistake in
the oracle (a dropped term, a swapped concatenation block, a wrong sign, a
transposed operand, a reversed tie rule) fails at least one of them.
"""

import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workload import bf16_bits_to_f32, config, f32_to_bf16_bits, gen_inputs, gen_targets

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _t(bits):
    """bfloat16 bits -> float64 torch tensor."""
    return torch.from_numpy(bf16_bits_to_f32(bits).astype(np.float64).reshape(np.shape(bits)))


def _lexsort_topk(values, K):
    values = np.asarray(values, dtype=np.float64)
    ids = np.arange(values.size)
    order = np.lexsort((ids, -values))  # value descending, then id ascending
    return order[:K].astype(np.int32), values[order[:K]]


# ----------------------------------------------------------------- counts --

def test_param_count_matches_page():
    g = _golden("dcoco_counts.json")
    q = g["qwen3_8b"]
    desc = oracle.OracleDesc(V=151936, B=q["B"], K=q["K"], d=q["d"], de=q["de"], r=q["r"],
                             h=q["h"], dvec=128)
    assert oracle.param_count(desc) == g["param_count"]
    assert 3 * q["r"] + 2 == g["mlp_input_width"]


def test_transition_and_node_counts():
    g = _golden("dcoco_counts.json")
    cfg = config("tiny", B=g["qwen3_8b"]["B"], K=g["qwen3_8b"]["K"], V=200)
    x = gen_inputs(cfg)
    r = oracle.run(cfg, x)
    assert r["ids"][0].size == g["nodes_per_block"]
    assert r["scores"][0].size == g["transitions_per_block"]


def test_every_parameter_tensor_is_used():
    """Perturbing any single parameter tensor changes the scores: no term dropped."""
    cfg = config("tiny")
    x = gen_inputs(cfg)
    base = oracle.run(cfg, x)["scores"]
    for name in ("w_cand", "w_ctx", "w_fuse", "w_pair", "w1", "ln_gamma", "ln_beta",
                 "b1", "w2", "b2"):
        y = dict(x)
        w = {k: v.copy() for k, v in x["weights"].items()}
        if w[name].dtype == np.uint16:
            f = bf16_bits_to_f32(w[name]).reshape(w[name].shape) * np.float32(1.5)
            w[name] = f32_to_bf16_bits(f).reshape(w[name].shape)
        else:
            w[name] = (w[name] * np.float32(1.5) + np.float32(0.05)).astype(np.float32)
        y["weights"] = w
        assert not np.allclose(oracle.run(cfg, y)["scores"], base, rtol=0, atol=1e-9), name
    # the embedding table and the hidden states feed the scores too
    y = dict(x)
    y["hidden"] = x["hidden"].copy()
    y["hidden"][0, 2, 5] ^= 0x0100
    assert not np.allclose(oracle.run(cfg, y)["scores"], base, rtol=0, atol=1e-9)


# ----------------------------------------------------------------- top-K --

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_topk_matches_lexsort(dtype):
    g = np.random.default_rng(7)
    for trial in range(40):
        V = int(g.integers(1, 300))
        K = int(g.integers(1, V + 1))
        if trial % 3 == 0:
            vals = g.integers(-3, 4, size=V).astype(np.float32)   # many ties
        else:
            vals = g.normal(size=V).astype(np.float32)
        if dtype == "bf16":
            row = f32_to_bf16_bits(vals)
            ref_vals = bf16_bits_to_f32(row)
        else:
            row, ref_vals = vals, vals
        ids, got = oracle.topk_row(row, K)
        eids, evals = _lexsort_topk(ref_vals, K)
        np.testing.assert_array_equal(ids, eids)
        np.testing.assert_array_equal(got, evals)


def test_topk_signed_zero_and_inf():
    # -0 == +0 numerically, so they tie and order by id; -inf sorts last.
    row = np.array([-0.0, 0.0, -np.inf, -1.0, 0.0, -0.0, -np.inf, np.inf], np.float32)
    ids, vals = oracle.topk_row(row, 8)
    assert ids.tolist() == [7, 0, 1, 4, 5, 3, 2, 6]
    bits = f32_to_bf16_bits(row)
    ids2, _ = oracle.topk_row(bits, 8)
    assert ids2.tolist() == [7, 0, 1, 4, 5, 3, 2, 6]


def test_topk_k_equals_v_is_a_full_sort():
    g = np.random.default_rng(3)
    row = g.normal(size=50).astype(np.float32)
    ids, vals = oracle.topk_row(row, 50)
    assert sorted(ids.tolist()) == list(range(50))
    assert np.all(np.diff(vals) <= 0)


def test_topk_rejects_nan():
    row = np.array([1.0, np.nan, 0.0], np.float32)
    with pytest.raises(RuntimeError):
        oracle.topk_row(row, 2)


def test_topk_permutation_equivariance():
    g = np.random.default_rng(11)
    row = g.normal(size=500).astype(np.float32)   # distinct values: no ties
    perm = g.permutation(500)
    ids, vals = oracle.topk_row(row, 10)
    pid, pvals = oracle.topk_row(row[perm], 10)
    np.testing.assert_array_equal(perm[pid], ids)
    np.testing.assert_array_equal(vals, pvals)


def test_topk_skips_anchor_rows():
    cfg = config("tiny")
    x = gen_inputs(cfg)
    a = oracle.run(cfg, x)
    y = dict(x)
    y["logits"] = x["logits"].copy()
    y["logits"][:, 0, :] = -5.0
    y["hidden"] = x["hidden"].copy()
    y["hidden"][:, 0, :] = 0
    b = oracle.run(cfg, y)
    for k in ("ids", "scores", "tokens"):
        np.testing.assert_array_equal(a[k], b[k])


# ------------------------------------------------------ LayerNorm / GELU --

def test_layernorm_matches_torch_and_invariants():
    g = np.random.default_rng(5)
    for m in (4, 16, 128):
        x = g.normal(size=m) * 3 + 1
        eps = 1e-5
        y = oracle.layernorm(x, eps)
        ref = F.layer_norm(torch.from_numpy(x), (m,), eps=eps).numpy()
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
        v = x.var()
        assert abs(y.mean()) < 1e-12
        assert abs(y.var() - v / (v + eps)) < 1e-12
        np.testing.assert_allclose(oracle.layernorm(x + 7.5, eps), y, atol=1e-10)
        np.testing.assert_allclose(oracle.layernorm(1e4 * x, 0.0), oracle.layernorm(x, 0.0), atol=1e-10)
        gam = g.normal(size=m).astype(np.float32)
        bet = g.normal(size=m).astype(np.float32)
        ya = oracle.layernorm(x, eps, gam, bet)
        refa = F.layer_norm(torch.from_numpy(x), (m,), torch.from_numpy(gam.astype(np.float64)),
                            torch.from_numpy(bet.astype(np.float64)), eps=eps).numpy()
        np.testing.assert_allclose(ya, refa, rtol=1e-12, atol=1e-12)


def test_gelu_exact_erf_form():
    ts = np.linspace(-8, 8, 161)
    ref = F.gelu(torch.from_numpy(ts), approximate="none").numpy()
    got = np.array([oracle.gelu(t) for t in ts])
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-15)
    assert oracle.gelu(0.0) == 0.0
    for t in ts:
        assert abs(oracle.gelu(t) - oracle.gelu(-t) - t) < 1e-14


# ------------------------------------------- projections and the MLP head --

def _torch_reference(cfg, x, r_or):
    """Steps (2)-(4) with torch CPU library calls in float64, on the oracle's ids."""
    w = x["weights"]
    B, K, r = cfg["B"], cfg["K"], cfg["r"]
    ids = torch.from_numpy(r_or["ids"][0].astype(np.int64))            # [B][K]
    l = torch.from_numpy(r_or["vals"][0])                              # [B][K]
    h = _t(x["hidden"][0, 1:])                                         # [B][d]
    E = _t(x["embed"])
    b = F.layer_norm(F.linear(E[ids.reshape(-1)], _t(w["w_cand"])), (r,), eps=cfg["ln_eps"]).reshape(B, K, r)
    g = F.layer_norm(F.linear(h, _t(w["w_ctx"])), (r,), eps=cfg["ln_eps"])          # [B][r]
    bg = torch.cat([b, g[:, None, :].expand(B, K, r)], dim=-1)
    gam = torch.from_numpy(w["ln_gamma"].astype(np.float64))
    bet = torch.from_numpy(w["ln_beta"].astype(np.float64))
    z = F.layer_norm(F.linear(bg, _t(w["w_fuse"])), (r,), gam, bet, eps=cfg["ln_eps"])
    s = F.linear(torch.cat([h[:-1], h[1:]], dim=-1), _t(w["w_pair"]))                 # [B-1][r]
    return dict(b=b, g=g, z=z, s=s, l=l)


def test_represent_matches_torch_linear_layernorm():
    cfg = config("tiny")
    x = gen_inputs(cfg)
    r = oracle.run(cfg, x)
    ref = _torch_reference(cfg, x, r)
    for k in ("b", "g", "z", "s"):
        np.testing.assert_allclose(r[k][0], ref[k].numpy(), rtol=1e-10, atol=1e-10, err_msg=k)


@pytest.mark.parametrize("head", ["normal", "stress"])
def test_mlp_scores_match_torch(head):
    cfg = config("tiny")
    x = gen_inputs(cfg, head=head)
    r = oracle.run(cfg, x)
    ref = _torch_reference(cfg, x, r)
    w = x["weights"]
    B, K, r_ = cfg["B"], cfg["K"], cfg["r"]
    z, s, l = ref["z"], ref["s"], ref["l"]
    S = np.empty((B - 1, K, K))
    for p in range(B - 1):
        xin = torch.cat([
            s[p][None, None, :].expand(K, K, r_),
            z[p][:, None, :].expand(K, K, r_),
            z[p + 1][None, :, :].expand(K, K, r_),
            l[p][:, None, None].expand(K, K, 1),
            l[p + 1][None, :, None].expand(K, K, 1),
        ], dim=-1)
        hid = F.gelu(F.linear(xin, _t(w["w1"]), torch.from_numpy(w["b1"].astype(np.float64))))
        delta = F.linear(hid, torch.from_numpy(w["w2"].astype(np.float64))[None, :],
                         torch.from_numpy(w["b2"].astype(np.float64)))[..., 0]
        S[p] = (l[p + 1][None, :] + delta).numpy()
    np.testing.assert_allclose(r["scores"][0], S, rtol=1e-10, atol=1e-10)


def _only_block(w1, r, block):
    """Zero W1 outside one input block (s, z_a, z_b, l_a or l_b)."""
    cols = {"s": slice(0, r), "za": slice(r, 2 * r), "zb": slice(2 * r, 3 * r),
            "la": slice(3 * r, 3 * r + 1), "lb": slice(3 * r + 1, 3 * r + 2)}[block]
    out = np.zeros_like(w1)
    out[:, cols] = w1[:, cols]
    return out


@pytest.mark.parametrize("block", ["s", "za", "zb", "la", "lb"])
def test_mlp_concatenation_order(block):
    """With W1 restricted to one input block, delta depends on exactly the
    inputs the page puts in that block: s_p alone gives a constant per pair,
    z_p^a / l_p(a) vary only with a, z_{p+1}^b / l_{p+1}(b) only with b."""
    cfg = config("tiny")
    x = gen_inputs(cfg, head="stress")
    x["weights"]["w1"] = _only_block(x["weights"]["w1"], cfg["r"], block)
    r = oracle.run(cfg, x)
    d = r["delta"][0]                                   # [p][a][b]
    varies_a = np.ptp(d, axis=1).max() > 1e-9
    varies_b = np.ptp(d, axis=2).max() > 1e-9
    expect = {"s": (False, False), "za": (True, False), "la": (True, False),
              "zb": (False, True), "lb": (False, True)}[block]
    assert (varies_a, varies_b) == expect
    if block in ("la", "lb"):
        # closed form: delta = sum_j w2_j GELU(b1_j + W1[j][c] * l) + b2
        w = x["weights"]
        c = 3 * cfg["r"] + (0 if block == "la" else 1)
        col = bf16_bits_to_f32(x["weights"]["w1"][:, c]).astype(np.float64)
        for p in range(cfg["B"] - 1):
            for k in range(cfg["K"]):
                lv = r["vals"][0, p if block == "la" else p + 1, k]
                pre = torch.from_numpy(w["b1"].astype(np.float64) + col * lv)
                want = float((torch.from_numpy(w["w2"].astype(np.float64)) * F.gelu(pre)).sum()) + float(w["b2"][0])
                got = d[p, k, 0] if block == "la" else d[p, 0, k]
                assert abs(got - want) < 1e-10


def test_zero_initialised_output_layer_reproduces_drafter_argmax():
    """DCOCO: with the MLP output layer zero-initialised every S_p(a,b) equals the
    successor logit, so the walk returns the drafter's own per-slot argmax."""
    for name in ("tiny",):
        cfg = config(name)
        x = gen_inputs(cfg, head="zero")
        r = oracle.run(cfg, x)
        B, K = cfg["B"], cfg["K"]
        want = np.broadcast_to(r["vals"][:, 1:, None, :], r["scores"].shape)
        assert np.array_equal(r["scores"], want)
        assert (r["choice"] == 0).all()
        lg = x["logits"][0, 1:]
        np.testing.assert_array_equal(r["tokens"][0], np.argmax(lg, axis=1))
    # b2 = c shifts every score of a row equally: same walk
    x = gen_inputs(config("tiny"), head="zero")
    x["weights"]["b2"] = np.array([3.25], np.float32)
    r2 = oracle.run(config("tiny"), x)
    assert (r2["choice"] == 0).all()


# -------------------------------------------------------------- the walk --

def _brute_force_walk(S, K):
    """Among all K^(B-1) paths that start at rank 0, the prefix-first rule picks
    the one that is lexicographically best on (score of step 1, then step 2, ...),
    each tie going to the lower candidate index."""
    Bm1 = S.shape[0]
    best_key, best = None, None
    for tail in itertools.product(range(K), repeat=Bm1):
        path = (0,) + tail
        key = []
        for p in range(Bm1):
            key += [-S[p, path[p], path[p + 1]], path[p + 1]]
        key = tuple(key)
        if best_key is None or key < best_key:
            best_key, best = key, path
    return np.array(best)


def test_walk_matches_brute_force():
    g = np.random.default_rng(2)
    for trial in range(30):
        B, K = int(g.integers(2, 6)), int(g.integers(1, 4))
        S = g.integers(-2, 3, size=(1, B - 1, K, K)).astype(np.float64)  # many ties
        if trial % 2:
            S = g.normal(size=(1, B - 1, K, K))
        ids = g.integers(0, 100, size=(1, B, K)).astype(np.int32)
        desc = oracle.OracleDesc(V=100, B=B, K=K, d=32, de=32, r=16, h=16, dvec=16)
        tokens, choice = oracle.walk(desc, S, ids, 1)
        want = _brute_force_walk(S[0], K)
        np.testing.assert_array_equal(choice[0], want)
        np.testing.assert_array_equal(tokens[0], ids[0, np.arange(B), want])


# ------------------------------------------------- Global-Sum path rule --
# LiLiCorr, appendix E, Eq. 12: the path maximising the summed transition
# scores, by dynamic programming; slot 1 stays at rank 0 as in the walk.

def _paths(B, K):
    """Every path with slot 1 at rank 0: K^(B-1) tuples of choices."""
    for tail in itertools.product(range(K), repeat=B - 1):
        yield (0,) + tail


def _path_score(S, path):
    return sum(S[p, path[p], path[p + 1]] for p in range(len(path) - 1))


def _desc(B, K):
    return oracle.OracleDesc(V=100, B=B, K=K, d=32, de=32, r=16, h=16, dvec=16)


def test_viterbi_matches_brute_force():
    """Continuous random scores (a unique optimum): the same path and total as
    enumerating all K^(B-1) paths."""
    g = np.random.default_rng(11)
    for B, K in ((1, 3), (2, 3), (3, 4), (5, 4), (6, 3), (4, 6)):
        n = 3
        S = g.normal(size=(n, max(B - 1, 0), K, K))
        ids = g.integers(0, 100, size=(n, B, K)).astype(np.int32)
        tokens, choice, total = oracle.viterbi(_desc(B, K), S, ids, n)
        for i in range(n):
            best = max(_paths(B, K), key=lambda c: _path_score(S[i], c))
            np.testing.assert_array_equal(choice[i], best)
            np.testing.assert_array_equal(tokens[i], ids[i, np.arange(B), list(best)])
            assert total[i] == pytest.approx(_path_score(S[i], best), abs=1e-12)


def test_viterbi_ties_give_an_optimal_path():
    """Integer scores (many ties): the returned path attains the brute-force
    optimum and the reported total is its score."""
    g = np.random.default_rng(12)
    for trial in range(20):
        B, K = int(g.integers(2, 6)), int(g.integers(1, 5))
        S = g.integers(-2, 3, size=(1, B - 1, K, K)).astype(np.float64)
        ids = g.integers(0, 100, size=(1, B, K)).astype(np.int32)
        _, choice, total = oracle.viterbi(_desc(B, K), S, ids, 1)
        best = max(_path_score(S[0], c) for c in _paths(B, K))
        assert choice[0, 0] == 0
        assert _path_score(S[0], choice[0]) == best == total[0]


def test_viterbi_zero_head_takes_each_slot_argmax():
    """With the zero-initialised output layer S_p(a,b) = l_{p+1}(b) (DCOCO core
    method), so the best path takes every slot's largest logit: rank 0."""
    x = gen_inputs(config("tiny"), head="zero")
    ora = oracle.run(x["cfg"], x)
    desc = oracle.OracleDesc.from_config(x["cfg"])
    _, choice, total = oracle.viterbi(desc, ora["scores"], ora["ids"], x["cfg"]["n"])
    assert (choice == 0).all()
    assert total[0] == pytest.approx(ora["vals"][0, 1:, 0].sum(), abs=1e-12)


def test_viterbi_dominates_the_walk_and_ignores_pair_offsets():
    """The exact maximiser scores at least as high as the greedy walk's path
    (equal when there is one pair), and adding a constant to every score of a
    pair shifts the total by that constant without changing the path."""
    g = np.random.default_rng(13)
    for B, K in ((2, 5), (4, 4), (8, 3), (15, 4)):
        n = 4
        S = g.normal(size=(n, B - 1, K, K))
        ids = g.integers(0, 100, size=(n, B, K)).astype(np.int32)
        desc = _desc(B, K)
        _, choice, total = oracle.viterbi(desc, S, ids, n)
        _, wchoice = oracle.walk(desc, S, ids, n)
        for i in range(n):
            greedy = _path_score(S[i], wchoice[i])
            assert total[i] >= greedy - 1e-12
            if B == 2:
                assert total[i] == pytest.approx(greedy, abs=1e-12)
        c = g.normal(size=(n, B - 1, 1, 1)) * 5
        _, choice2, total2 = oracle.viterbi(desc, S + c, ids, n)
        np.testing.assert_array_equal(choice2, choice)
        np.testing.assert_allclose(total2, total + c.sum(axis=(1, 2, 3)), atol=1e-9)


# ---------------------------------------------- Geometric path rule --
# The DCOCO page names a Geometric rule (lambda = 0.75) without a formula; it
# is read as the path maximising sum_p lambda^p S_p(c_p, c_{p+1}).  These pins
# fix the oracle to that reading (which itself is unpinned by the pages).

def _discounted(S, path, lam):
    return sum(lam ** p * S[p, path[p], path[p + 1]] for p in range(len(path) - 1))


def test_geometric_matches_brute_force():
    g = np.random.default_rng(21)
    for lam in (0.75, 0.3, 1.0):
        for B, K in ((2, 3), (3, 4), (5, 4), (6, 3)):
            n = 3
            S = g.normal(size=(n, B - 1, K, K))
            ids = g.integers(0, 100, size=(n, B, K)).astype(np.int32)
            tokens, choice, total = oracle.viterbi(_desc(B, K), S, ids, n, lam=lam)
            for i in range(n):
                best = max(_paths(B, K), key=lambda c: _discounted(S[i], c, lam))
                np.testing.assert_array_equal(choice[i], best)
                assert total[i] == pytest.approx(_discounted(S[i], best, lam), abs=1e-12)


def test_geometric_small_lambda_is_the_walk():
    """For small lambda the discounted sum orders paths lexicographically by
    (step 1, step 2, ...), which is the prefix-first walk; weighting the
    steps the other way round would not give it.  Each pair's K x K tile is a
    permutation of 0..K^2-1 (gaps >= 1, range K^2-1, and rows with different
    maxima, so the continuation matters), and lambda = 1/(2K^2) makes every
    step outweigh all later ones together:
    sum_{q>p} lambda^(q-p) (K^2-1) < 1.  The shapes keep lambda^(B-2) well
    above float64 resolution next to the totals."""
    g = np.random.default_rng(22)
    for B, K in ((4, 4), (8, 3), (15, 2), (6, 6)):
        n = 6
        S = np.argsort(g.random(size=(n, B - 1, K * K)), axis=-1).reshape(n, B - 1, K, K).astype(np.float64)
        ids = g.integers(0, 100, size=(n, B, K)).astype(np.int32)
        _, choice, _ = oracle.viterbi(_desc(B, K), S, ids, n, lam=1.0 / (2 * K * K))
        _, wchoice = oracle.walk(_desc(B, K), S, ids, n)
        np.testing.assert_array_equal(choice, wchoice)


def test_geometric_rejects_non_positive_lambda():
    S = np.zeros((1, 2, 3, 3))
    ids = np.zeros((1, 3, 3), np.int32)
    for lam in (0.0, -0.5):
        with pytest.raises(RuntimeError):
            oracle.viterbi(_desc(3, 3), S, ids, 1, lam=lam)


# ------------------------------------------------------- beam search --
# The critique on the DCOCO page (weakness 2) proposes widening the walk into
# a beam of 2-4 paths; read as beam search on the summed transition score.

def test_beam_width_one_is_the_walk():
    """W = 1 keeps the single best extension at every step: the prefix-first
    walk, ties (integer scores) included."""
    g = np.random.default_rng(31)
    for trial in range(40):
        B, K = int(g.integers(2, 9)), int(g.integers(1, 7))
        S = g.integers(-3, 4, size=(3, B - 1, K, K)).astype(np.float32)
        ids = g.integers(0, 100, size=(3, B, K)).astype(np.int32)
        t1, c1, _ = oracle.beam(_desc(B, K), S, ids, 3, 1)
        t2, c2 = oracle.walk(_desc(B, K), S.astype(np.float64), ids, 3)
        np.testing.assert_array_equal(c1, c2)
        np.testing.assert_array_equal(t1, t2)


def test_beam_covering_every_path_is_the_optimum():
    """A width of K^(B-1) keeps every path, so the answer has the brute-force
    best summed score (integer scores: float32 sums are exact)."""
    g = np.random.default_rng(32)
    for B, K in ((2, 3), (3, 3), (4, 2), (4, 3)):
        S = g.integers(-5, 6, size=(2, B - 1, K, K)).astype(np.float32)
        ids = g.integers(0, 100, size=(2, B, K)).astype(np.int32)
        _, choice, total = oracle.beam(_desc(B, K), S, ids, 2, K ** (B - 1))
        for i in range(2):
            best = max(_path_score(S[i].astype(np.float64), c) for c in _paths(B, K))
            assert total[i] == best == _path_score(S[i].astype(np.float64), choice[i])


def test_beam_worked_example_beats_the_walk():
    """From rank 0 the walk takes successor 0 (5 > 4) and then can only add 0;
    a beam of two keeps the runner-up, whose next step is worth 10: 4 + 10."""
    S = np.zeros((1, 2, 2, 2), np.float32)
    S[0, 0, 0] = [5.0, 4.0]          # pair 0, from rank 0
    S[0, 1, 0] = [0.0, 0.0]          # pair 1, from candidate 0
    S[0, 1, 1] = [10.0, 0.0]         # pair 1, from candidate 1
    ids = np.arange(6, dtype=np.int32).reshape(1, 3, 2)
    _, c1, t1 = oracle.beam(_desc(3, 2), S, ids, 1, 1)
    _, c2, t2 = oracle.beam(_desc(3, 2), S, ids, 1, 2)
    np.testing.assert_array_equal(c1[0], [0, 0, 0])
    np.testing.assert_array_equal(c2[0], [0, 1, 0])
    assert (t1[0], t2[0]) == (5.0, 14.0)


def test_beam_tie_order_and_float32_sums():
    """Equal extension scores go to the lower beam index, then the lower
    successor; sums are single float32 additions (1 + 2^-24 rounds to 1)."""
    S = np.zeros((1, 2, 2, 2), np.float32)
    S[0, 0, 0] = [1.0, 1.0]                  # two equal first steps: beam 0 is b = 0
    S[0, 1, 0] = [0.0, 0.0]                  # from beam 0: 1 + 0
    S[0, 1, 1] = [2.0 ** -24, 0.0]           # from beam 1: 1 + 2^-24, which is 1 in float32
    ids = np.zeros((1, 3, 2), np.int32)
    _, c, t = oracle.beam(_desc(3, 2), S, ids, 1, 2)
    # every extension scores exactly 1.0 in float32, so beam 0 and successor 0
    # win (summed in float64, beam 1's 1 + 2^-24 would win instead)
    np.testing.assert_array_equal(c[0], [0, 0, 0])
    assert t[0] == np.float32(1.0)


# ---------------------------------------- top-m successor sparsification --
# The critique on the DCOCO page (weakness 3) proposes scoring only the top-m
# successors of each predecessor (O(BKm) instead of O(BK^2)); read as the
# first m of the next slot's top-K (the drafter's ranking).

@pytest.mark.parametrize("variant", ["mlp", "cosine"])
def test_top_m_keeps_the_first_m_successors(variant):
    x = gen_inputs(config("tiny", K=6, variant=variant), head="stress")
    dense = oracle.run(x["cfg"], x)
    for m in (0, 6, 9):   # 0 and m >= K: every successor
        got = oracle.run(dict(x["cfg"], succ_top_m=m), x)
        np.testing.assert_array_equal(got["scores"], dense["scores"])
    for m in (1, 2, 5):
        got = oracle.run(dict(x["cfg"], succ_top_m=m), x)
        S, D = got["scores"], got["delta"]
        np.testing.assert_array_equal(S[..., :m], dense["scores"][..., :m])
        np.testing.assert_array_equal(D[..., :m], dense["delta"][..., :m])
        assert np.isneginf(S[..., m:]).all() and np.isneginf(D[..., m:]).all()
        assert np.isfinite(S).sum() == S.shape[0] * S.shape[1] * 6 * m
        # no path rule can choose a dropped successor
        desc = oracle.OracleDesc.from_config(dict(x["cfg"], succ_top_m=m))
        n = x["cfg"]["n"]
        _, walk_c = oracle.walk(desc, S, got["ids"], n)
        _, vit_c, _ = oracle.viterbi(desc, S, got["ids"], n)
        _, beam_c, _ = oracle.beam(desc, S.astype(np.float32), got["ids"], n, 3)
        for c in (walk_c, vit_c, beam_c):
            assert (c[:, 1:] < m).all()


# ------------------------------------------- vocabulary normalisation --

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_log_normaliser_matches_scipy(dtype):
    from scipy.special import logsumexp
    rng = np.random.default_rng(5)
    for V in (1, 7, 1000, 151936):
        x = (rng.standard_normal(V) * 3 + rng.standard_normal() * 10).astype(np.float32)
        row = f32_to_bf16_bits(x) if dtype == "bf16" else x
        exact = bf16_bits_to_f32(row).astype(np.float64) if dtype == "bf16" else x.astype(np.float64)
        want = logsumexp(exact)
        assert abs(oracle.log_normaliser_row(row) - want) <= 1e-12 * max(1.0, abs(want))


def test_log_normaliser_closed_forms():
    # uniform row: log(V e^c) = c + log V
    for c, V in ((0.0, 151936), (-3.5, 1000), (17.25, 5)):
        got = oracle.log_normaliser_row(np.full(V, c, np.float32))
        assert abs(got - (c + np.log(V))) <= 1e-12 * max(1.0, abs(got))
    # two values, a copies of x1 and b copies of x2: log(a e^x1 + b e^x2)
    x1, x2, a, b = 2.0, -1.0, 3, 40
    row = np.array([x1] * a + [x2] * b, np.float32)
    want = np.log(a * np.exp(x1) + b * np.exp(x2))
    assert abs(oracle.log_normaliser_row(row) - want) <= 1e-13
    # one finite entry among -inf: that entry; all -inf: -inf
    row = np.full(64, -np.inf, np.float32)
    row[17] = 4.5
    assert oracle.log_normaliser_row(row) == 4.5
    assert oracle.log_normaliser_row(np.full(64, -np.inf, np.float32)) == -np.inf
    # near the float32 maximum the sum of exponentials would overflow; the
    # normaliser is still max + log(count of the maximum)
    big = np.float32(3.0e38)
    row = np.array([big, big, -big, 0.0], np.float32)
    assert abs(oracle.log_normaliser_row(row) - (float(big) + np.log(2.0))) <= 1e-12 * float(big)


def test_log_normaliser_rejects_nan_and_pos_inf():
    for bad in (np.nan, np.inf):
        row = np.zeros(8, np.float32)
        row[3] = bad
        with pytest.raises(RuntimeError):
            oracle.log_normaliser_row(row)


def test_log_normaliser_rows_skip_the_anchor():
    cfg = config("tiny")
    x = gen_inputs(cfg)
    d = oracle.OracleDesc.from_config(cfg)
    V, B, n = cfg["V"], cfg["B"], cfg["n"]
    logz = oracle.log_normaliser(d, x["logits"], n, (B + 1) * V, V, offset=V)
    rows = x["logits"].reshape(n, B + 1, V)
    for i in range(n):
        for s in range(B):
            assert logz[i, s] == oracle.log_normaliser_row(rows[i, s + 1])


def test_confidence_worked_example():
    # logits (2, 1, 0), K = 2: softmax of (2, 1, 0) and log Z = log(e^2 + e + 1)
    logz = oracle.log_normaliser_row(np.array([2.0, 1.0, 0.0], np.float32))
    assert abs(logz - 2.40760596444438) <= 1e-13
    ids, vals = oracle.topk_row(np.array([2.0, 1.0, 0.0], np.float32), 2)
    c = oracle.confidence(vals, np.float64(logz))
    want = np.array([[-0.40760596444438013, 0.6652409557748219, 0.0, 0.0, 1.0],
                     [-1.4076059644443801, 0.24472847105479764, 1.0, 1.0, 0.0]])
    np.testing.assert_allclose(c, want, rtol=0, atol=1e-13)
    assert list(oracle.CONF_FIELDS) == ["logprob", "prob", "gap", "rank", "top"]


def test_confidence_over_the_whole_vocabulary():
    """With K = V the candidates are the whole distribution: probabilities sum
    to one and descend, the gap ascends from zero, ranks span [0, 1] evenly and
    exactly one candidate is the top choice.  K = 1 has rank 0."""
    import math
    rng = np.random.default_rng(8)
    V = 300
    row = f32_to_bf16_bits((rng.standard_normal(V) * 2).astype(np.float32))
    ids, vals = oracle.topk_row(row, V)
    c = oracle.confidence(vals, oracle.log_normaliser_row(row))
    assert abs(math.fsum(c[:, 1]) - 1.0) <= 1e-12
    assert (np.diff(c[:, 1]) <= 0).all() and (np.diff(c[:, 2]) >= 0).all() and c[0, 2] == 0
    np.testing.assert_allclose(np.exp(c[:, 0]), c[:, 1], rtol=1e-15)
    np.testing.assert_array_equal(c[:, 3], np.arange(V) / (V - 1))
    assert c[:, 4].sum() == 1 and c[0, 4] == 1
    one = oracle.confidence(vals[:1], oracle.log_normaliser_row(row))
    assert one[0, 3] == 0 and one[0, 4] == 1


def test_confidence_shift_invariance():
    """Softmax ignores a constant added to every logit: log-probs, probabilities
    and gaps do not move, log Z moves by the constant."""
    rng = np.random.default_rng(9)
    x = rng.integers(-40, 40, 500).astype(np.float32) / 4   # exact in float32 after any shift below
    ids, vals = oracle.topk_row(x, 16)
    base = oracle.confidence(vals, oracle.log_normaliser_row(x))
    for c in (7.0, -13.5):
        ids2, vals2 = oracle.topk_row(x + np.float32(c), 16)
        lz = oracle.log_normaliser_row(x + np.float32(c))
        assert abs(lz - (oracle.log_normaliser_row(x) + c)) <= 1e-12
        np.testing.assert_array_equal(ids2, ids)
        np.testing.assert_allclose(oracle.confidence(vals2, lz), base, rtol=0, atol=1e-12)


# -------------------------------------------------------- cosine variant --

def test_cosine_scores_match_torch_and_bound():
    for sigma in (1.0, 8.0):
        cfg = config("tiny", variant="cosine", sigma=sigma)
        x = gen_inputs(cfg)
        r = oracle.run(cfg, x)
        ref = _torch_reference(cfg, x, r)
        w = x["weights"]
        z, l = ref["z"], ref["l"]
        o = F.normalize(F.linear(z, _t(w["w_out"])), dim=-1, eps=1e-12)
        i = F.normalize(F.linear(z, _t(w["w_in"])), dim=-1, eps=1e-12)
        S = l[1:, None, :] + sigma * torch.matmul(o[:-1], i[1:].transpose(1, 2))
        np.testing.assert_allclose(r["scores"][0], S.numpy(), rtol=1e-10, atol=1e-10)
        assert np.all(np.abs(r["scores"] - r["vals"][:, 1:, None, :]) <= sigma + 1e-12)


def test_cosine_identical_slots_reach_sigma():
    """With W_in = W_out and two identical slots (same hidden state, same
    candidates), the out and in vectors of a candidate coincide: cos = 1."""
    cfg = config("tiny", variant="cosine", sigma=8.0)
    x = gen_inputs(cfg)
    x["weights"]["w_in"] = x["weights"]["w_out"].copy()
    x["logits"] = x["logits"].copy()
    x["hidden"] = x["hidden"].copy()
    x["logits"][0, 2] = x["logits"][0, 1]
    x["hidden"][0, 2] = x["hidden"][0, 1]
    r = oracle.run(cfg, x)
    for a in range(cfg["K"]):
        assert abs(r["scores"][0, 0, a, a] - r["vals"][0, 1, a] - 8.0) < 1e-12


# ----------------------------------------------------------------- yield --

def test_yield_worked_example():
    g = _golden("yield_example.json")
    np.testing.assert_allclose(oracle.survival(g["conditional"]), g["survival"], rtol=1e-15)
    assert abs(oracle.expected_yield(g["conditional"]) - g["expected_yield"]) < 1e-12
    alpha = sum(g["conditional"]) / len(g["conditional"])
    assert abs(alpha - g["alpha"]) < 1e-15
    assert abs(oracle.iid_expected_yield(alpha, len(g["conditional"])) - g["iid_expected_yield"]) < 1e-12
    for a in (0.1, 0.5, 0.9):
        for gam in (1, 4, 15):
            assert abs(oracle.iid_expected_yield(a, gam) - (1 - a ** (gam + 1)) / (1 - a)) < 1e-12
    assert oracle.iid_expected_yield(1.0, 15) == 16.0


def test_accepted_prefix_hand_worked():
    """Greedy verification (Faster Decoding, "Verification can be parallel even
    when generation is sequential"): the verifier accepts draft positions in
    order until the first mismatch, so A is the length of the leading run of
    matches, not the number of matching positions.  Each expected value below
    is worked by hand from that definition."""
    T = lambda *rows: np.array(rows, dtype=np.int32)  # noqa: E731
    cases = [
        # (tokens, targets, A)
        ([5, 11, 7, 9], [5, 12, 7, 9], 1),      # a later run of matches after a miss does not count
        ([5, 11, 7, 9], [5, 11, 7, 9], 4),      # every position accepted: A = B
        ([4, 11, 7, 9], [5, 11, 7, 9], 0),      # the first position misses
        ([5, 11, 7, 9], [5, 11, 7, 8], 3),      # only the last misses
        ([5, 11, 7, 9], [5, 11, 3, 9], 2),      # a miss in the middle
        ([1, 2, 3, 4], [-1, 2, 3, 4], 0),       # an out-of-pool target (-1) never matches
    ]
    for tok, tgt, want in cases:
        got = oracle.accepted_lengths(T(tok), T(tgt))
        assert got.tolist() == [want], (tok, tgt, got, want)
    # all six as one batch: each block is judged on its own row
    got = oracle.accepted_lengths(T(*[c[0] for c in cases]), T(*[c[1] for c in cases]))
    assert got.tolist() == [c[2] for c in cases]
    # B = 1 and empty batches
    assert oracle.accepted_lengths(T([3]), T([3])).tolist() == [1]
    assert oracle.accepted_lengths(T([3]), T([2])).tolist() == [0]
    assert oracle.accepted_lengths(np.zeros((0, 4), np.int32), np.zeros((0, 4), np.int32)).size == 0


def test_accepted_prefix_brute_force():
    """Against a different formulation of the same definition: A is the
    largest k such that the first k positions all match, found by trying every
    k from B down to 0 on random token rows with planted mismatches."""
    rng = np.random.default_rng(7)
    n, B = 400, 15
    targets = rng.integers(0, 6, size=(n, B)).astype(np.int32)
    tokens = targets.copy()
    flip = rng.random((n, B)) < 0.15
    tokens[flip] += 1
    got = oracle.accepted_lengths(tokens, targets)
    for i in range(n):
        want = max(k for k in range(B + 1) if (tokens[i, :k] == targets[i, :k]).all())
        assert got[i] == want
    # a sample where matches after the first miss are common, so a count of
    # matching positions would disagree with the prefix length
    assert ((tokens == targets).sum(axis=1) != got).sum() > n // 4


def test_yield_tail_sum_identity_on_walks():
    """Sum over blocks of Y = A + 1 equals n + sum_k #{A >= k}: E[Y] = 1 + sum_k s_k
    holds exactly on any sample (mixed accepted-prefix lengths in one batch)."""
    cfg = config("tiny", n=64, B=15, K=4, V=300)
    x = gen_inputs(cfg, head="stress")
    r = oracle.run(cfg, x)
    codes = gen_targets(cfg)
    B = cfg["B"]
    targets = np.where(codes >= 0, np.take_along_axis(r["ids"], np.maximum(codes, 0)[..., None], 2)[..., 0], -1)
    A = oracle.accepted_lengths(r["tokens"], targets)
    assert len(set(A.tolist())) > 2
    n = A.size
    lhs = int((A + 1).sum())
    rhs = n + sum(int((A >= k).sum()) for k in range(1, B + 1))
    assert lhs == rhs
    s_k = [float((A >= k).mean()) for k in range(1, B + 1)]
    assert abs(float((A + 1).mean()) - (1 + sum(s_k))) < 1e-12
