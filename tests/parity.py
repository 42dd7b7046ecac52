"""Shared helpers of the GPU parity tests: cached inputs, one GPU pass through
the C-ABI, and the comparison gates.

Gates (the oracle is float64, the GPU computes with bf16 MFMA inputs and
float32 accumulation):
  * top-K ids and values: exact.
  * S:     |S_gpu - S_ora| <= TOL * max(|S_ora|, 1)
  * Delta: |D_gpu - D_ora| <= TOL * max(|D_ora|, rms of D_ora over the pair's
           K x K tile), with D = S - l_{p+1}(b) on each side; this gate sees
           errors of the size that decide the walk, which the S gate alone
           cannot (S is dominated by the successor logit).
  * walk:  teacher forced; at every step the GPU's successor, given the GPU's
           own predecessor, must be the oracle's argmax of that row unless the
           row's top-2 margin is below TOL * max(|S_max|, 1), in which case it
           must lie within that margin of the row maximum.
  TOL = 2e-2.
"""

from __future__ import annotations

import functools
import os

import numpy as np
import torch

import oracle
from draft_correction_amd import device
from workload import config, gen_inputs

TOL = 2e-2

oracle.set_threads(min(16, os.cpu_count() or 1))


@functools.lru_cache(maxsize=4)
def _inputs(name: str, head: str, ties: bool, overrides: tuple):
    cfg = config(name, **dict(overrides))
    return gen_inputs(cfg, head=head, ties=ties)


def inputs(name: str, head: str = "normal", ties: bool = False, **overrides):
    return _inputs(name, head, ties, tuple(sorted(overrides.items())))


_dev_cache = {}


def dev_inputs(x: dict) -> dict:
    key = id(x)
    if key not in _dev_cache:
        if len(_dev_cache) >= 2:
            _dev_cache.clear()
            torch.cuda.empty_cache()
        _dev_cache[key] = (x, device.inputs_to_device(x))
    return _dev_cache[key][1]


def gpu_run(x: dict, n: int | None = None, first: int = 0, reps: int = 1, fold: bool = False,
            corr=None, ws=None) -> dict:
    """One corrector_run over blocks [first, first+n) with every output captured.
    With fold=True the candidate projection reads the folded table E W_cand^T.
    `corr` and `ws` (optional) reuse a caller's handle and workspace."""
    cfg = x["cfg"]
    dev = dev_inputs(x)
    n = cfg["n"] - first if n is None else n
    own = corr is None
    if own:
        corr = device.make_corrector(cfg, dev, max_requests=max(n, 1))
    if fold:
        table = torch.empty(corr.table_bytes() // 4, dtype=torch.float32, device="cuda")
        corr.fold_table(table)
        corr.use_table(table)
    st = device.strides(cfg)
    B, K = cfg["B"], cfg["K"]
    tokens = torch.empty((n, B), dtype=torch.int32, device="cuda")
    choice = torch.empty((n, B), dtype=torch.int32, device="cuda")
    ids = torch.empty((n, B, K), dtype=torch.int32, device="cuda")
    vals = torch.empty((n, B, K), dtype=torch.float32, device="cuda")
    scores = torch.empty((n, max(B - 1, 0), K, K), dtype=torch.float32, device="cuda")
    if ws is None:
        ws = corr.new_workspace(n)
    for _ in range(reps):
        corr.run(n, dev["logits"], st["l_req"], st["l_slot"], dev["hidden"], st["h_req"], st["h_slot"],
                 tokens, ws, choice=choice, ids=ids, vals=vals, scores=scores,
                 l_offset=st["l_off"] + first * st["l_req"], h_offset=st["h_off"] + first * st["h_req"])
    r = cfg["r"]
    z = torch.empty((n, B, K, r), dtype=torch.float32, device="cuda")
    g = torch.empty((n, B, r), dtype=torch.float32, device="cuda")
    s = torch.empty((n, max(B - 1, 0), r), dtype=torch.float32, device="cuda")
    corr.intermediates(n, ws, z=z, g=g, s=s)
    torch.cuda.synchronize()
    out = dict(tokens=tokens, choice=choice, ids=ids, vals=vals, scores=scores, z=z, g=g, s=s)
    out = {k: v.cpu().numpy() for k, v in out.items()}
    if own:
        corr.close()
    return out


def gpu_chain(x: dict, n: int | None = None, first: int = 0, fold: bool = False) -> dict:
    """The pass as three C-ABI calls on one workspace: corrector_topk, then
    corrector_score on its ids and values, then corrector_walk on those
    scores; outputs as from gpu_run.  With fold=True a folded table is
    attached, so corrector_score gathers its rows."""
    cfg = x["cfg"]
    dev = dev_inputs(x)
    n = cfg["n"] - first if n is None else n
    corr = device.make_corrector(cfg, dev, max_requests=max(n, 1))
    if fold:
        table = torch.empty(corr.table_bytes() // 4, dtype=torch.float32, device="cuda")
        corr.fold_table(table)
        corr.use_table(table)
    st = device.strides(cfg)
    B, K, r = cfg["B"], cfg["K"], cfg["r"]
    ids = torch.empty((n, B, K), dtype=torch.int32, device="cuda")
    vals = torch.empty((n, B, K), dtype=torch.float32, device="cuda")
    scores = torch.empty((n, max(B - 1, 0), K, K), dtype=torch.float32, device="cuda")
    tokens = torch.empty((n, B), dtype=torch.int32, device="cuda")
    choice = torch.empty((n, B), dtype=torch.int32, device="cuda")
    ws = corr.new_workspace(n)
    corr.topk(n, dev["logits"], st["l_req"], st["l_slot"], ids, vals, ws, offset=st["l_off"] + first * st["l_req"])
    corr.score(n, ids, vals, dev["hidden"], st["h_req"], st["h_slot"], scores, ws,
               offset=st["h_off"] + first * st["h_req"])
    z = torch.empty((n, B, K, r), dtype=torch.float32, device="cuda")
    g = torch.empty((n, B, r), dtype=torch.float32, device="cuda")
    s = torch.empty((n, max(B - 1, 0), r), dtype=torch.float32, device="cuda")
    corr.intermediates(n, ws, z=z, g=g, s=s)
    corr.walk(n, scores, ids, tokens, choice)
    torch.cuda.synchronize()
    out = dict(tokens=tokens, choice=choice, ids=ids, vals=vals, scores=scores, z=z, g=g, s=s)
    out = {k: v.cpu().numpy() for k, v in out.items()}
    corr.close()
    return out


def oracle_run(x: dict, n: int | None = None, first: int = 0) -> dict:
    return oracle.run(x["cfg"], x, n=n, first=first)


# ------------------------------------------------------------------ gates --

def check_topk(gpu: dict, ora: dict, where: str = ""):
    np.testing.assert_array_equal(gpu["ids"], ora["ids"], err_msg="top-K ids " + where)
    np.testing.assert_array_equal(gpu["vals"].astype(np.float64), ora["vals"], err_msg="top-K values " + where)


def check_scores(gpu: dict, ora: dict, where: str = ""):
    S_g = gpu["scores"].astype(np.float64)
    S_o = ora["scores"]
    assert np.isfinite(S_g).all(), "non-finite GPU scores " + where
    bad = np.abs(S_g - S_o) > TOL * np.maximum(np.abs(S_o), 1.0)
    assert not bad.any(), "S gate %s: %d of %d, worst |diff| %.3g" % (
        where, bad.sum(), bad.size, np.abs(S_g - S_o).max())
    D_g = S_g - gpu["vals"][:, 1:, None, :].astype(np.float64)
    D_o = ora["delta"]
    rms = np.sqrt((D_o ** 2).mean(axis=(2, 3), keepdims=True))
    lim = TOL * np.maximum(np.abs(D_o), rms)
    bad = np.abs(D_g - D_o) > lim
    assert not bad.any(), "Delta gate %s: %d of %d, worst ratio %.3g" % (
        where, bad.sum(), bad.size, (np.abs(D_g - D_o) / np.maximum(lim, 1e-30)).max())


def check_walk(gpu: dict, ora: dict, where: str = "", exact: bool = False):
    """Teacher-forced walk check; returns (steps, exempt steps, departures from rank 0)."""
    S_o = ora["scores"]
    ch = gpu["choice"]
    n, B = ch.shape
    steps = exempt = moved = 0
    for i in range(n):
        assert ch[i, 0] == 0, where
        for p in range(B - 1):
            row = S_o[i, p, ch[i, p]]
            best = int(np.argmax(row))
            smax = row[best]
            tol = TOL * max(abs(smax), 1.0)
            second = np.max(np.delete(row, best)) if row.size > 1 else -np.inf
            steps += 1
            moved += int(ch[i, p + 1] != 0)
            if exact or smax - second >= tol:
                assert ch[i, p + 1] == best, "walk %s: request %d step %d: gpu %d oracle %d" % (
                    where, i, p, ch[i, p + 1], best)
            else:
                exempt += 1
                assert row[ch[i, p + 1]] >= smax - tol, "walk %s: request %d step %d" % (where, i, p)
        np.testing.assert_array_equal(
            gpu["tokens"][i], gpu["ids"][i, np.arange(B), ch[i]], err_msg="tokens " + where)
    return steps, exempt, moved


def check_intermediates(gpu: dict, ora: dict, where: str = "", variant: str = "mlp"):
    z_g, z_o = gpu["z"].astype(np.float64), ora["z"]
    assert np.all(np.abs(z_g - z_o) <= 1e-2 * np.maximum(np.abs(z_o), 1.0)), \
        "z %s worst %.3g" % (where, np.abs(z_g - z_o).max())
    g_g, g_o = gpu["g"].astype(np.float64), ora["g"]
    assert np.all(np.abs(g_g - g_o) <= 1e-3 * np.maximum(np.abs(g_o), 1.0)), \
        "g %s worst %.3g" % (where, np.abs(g_g - g_o).max())
    if variant == "mlp" and ora["s"].size and gpu["s"].size:
        s_g, s_o = gpu["s"].astype(np.float64), ora["s"]
        rms = np.sqrt((s_o ** 2).mean())
        assert np.all(np.abs(s_g - s_o) <= 1e-3 * np.maximum(np.abs(s_o), rms)), \
            "s %s worst %.3g" % (where, np.abs(s_g - s_o).max())


def check_all(gpu: dict, ora: dict, where: str = "", exact_walk: bool = False, variant: str = "mlp"):
    check_topk(gpu, ora, where)
    check_intermediates(gpu, ora, where, variant)
    check_scores(gpu, ora, where)
    return check_walk(gpu, ora, where, exact=exact_walk)


def select(gpu: dict, first: int, n: int) -> dict:
    return {k: v[first:first + n] for k, v in gpu.items()}


# ------------------------------------------------------- Global-Sum path --

def path_scores(S, choice, lam: float = 1.0):
    """Summed transition score of each request's path: S [n][B-1][K][K],
    choice [n][B]; pair p weighted by lam**p."""
    n, P = S.shape[0], S.shape[1]
    i = np.arange(n)[:, None]
    p = np.arange(P)[None, :]
    return (S[i, p, choice[:, :-1], choice[:, 1:]] * lam ** np.arange(P)[None, :]).sum(axis=1)


def check_beam(gpu: dict, cfg: dict, where: str = ""):
    """The beam-search path: the oracle's beam search run on the GPU's own
    float32 scores must give the same choices and tokens (both sides rank the
    same float32 sums)."""
    n, B = gpu["choice"].shape
    desc = oracle.OracleDesc.from_config(cfg)
    t, c, _ = oracle.beam(desc, gpu["scores"], gpu["ids"], n, cfg.get("beam_width", 4))
    np.testing.assert_array_equal(gpu["choice"], c, err_msg="beam path " + where)
    np.testing.assert_array_equal(gpu["tokens"], t, err_msg="beam tokens " + where)


def _beam_steps(S, width: int):
    """Beam search of one request over float32 scores S [B-1][K][K] (summed
    transition score, slot 1 at rank 0; extensions ranked by score
    descending, then beam index, then successor), returning the kept paths
    after every step (a list of tuples of candidate indices)."""
    beams = [(np.float32(0.0), (0,))]
    kept = []
    P, K = S.shape[0], S.shape[2]
    for p in range(P):
        ext = []
        for bi, (g, path) in enumerate(beams):
            row = S[p, path[-1]]
            for b in range(K):
                ext.append((np.float32(g + row[b]), bi, b, path + (b,)))
        ext.sort(key=lambda e: (-float(e[0]), e[1], e[2]))
        beams = [(e[0], e[3]) for e in ext[:width]]
        kept.append([e[3] for e in ext[:width]])
    return kept


def check_beam_bound(gpu: dict, ora: dict, cfg: dict, where: str = ""):
    """Ties the beam path back to the oracle's float64 scores.  Until the
    first step where the beams kept on the GPU's scores and on the oracle's
    (rounded to float32) differ, both hold the same paths, and each partial
    sum differs between the two by at most sum_{q<=p} eps_q (eps_q the largest
    |S_gpu - S_ora| of pair q).  A ranking can only flip between extensions
    whose oracle sums lie within twice that of each other, so at the first
    differing step every path kept only on the GPU side must lie within
    2 sum_{q<=p} eps_q (plus float32 rounding) of every path kept only on the
    oracle side.  Requests whose beams never differ end on the same path.
    Returns the number of requests whose beams differ somewhere."""
    width = cfg.get("beam_width", 4)
    n, B = gpu["choice"].shape
    if B < 2:
        return 0
    S_g = gpu["scores"]
    S_o = ora["scores"]
    diverged = 0
    for i in range(n):
        eps = np.cumsum(np.abs(S_g[i].astype(np.float64) - S_o[i]).max(axis=(1, 2)))
        kg = _beam_steps(S_g[i], width)
        ko = _beam_steps(S_o[i].astype(np.float32), width)
        assert tuple(gpu["choice"][i]) == kg[-1][0], "beam replay disagrees with the GPU path %s" % where
        def total(path, p):
            return sum(S_o[i, q, path[q], path[q + 1]] for q in range(p + 1))

        def slack(p):
            return 2 * eps[p] + 1e-5 * (p + 1) * max(1.0, float(np.abs(S_o[i, :p + 1]).max()))
        for p in range(B - 1):
            only_g = set(kg[p]) - set(ko[p])
            only_o = set(ko[p]) - set(kg[p])
            if not only_g and not only_o:
                continue
            diverged += 1
            worst = max(total(a, p) - total(b, p) for a in only_o for b in only_g)
            assert worst <= slack(p), "beam %s: request %d step %d: ranking flip of %.3g beyond the score error %.3g" % (
                where, i, p, worst, slack(p))
            break
        else:
            # the same paths were kept at every step; the best of the last
            # step can still differ where two final sums nearly tie
            mine, theirs = tuple(gpu["choice"][i]), ko[-1][0]
            if mine != theirs:
                diverged += 1
                assert total(theirs, B - 2) - total(mine, B - 2) <= slack(B - 2), "beam %s: request %d" % (where, i)
    return diverged


def check_global_sum(gpu: dict, ora: dict, cfg: dict, where: str = "", exact: bool = False, lam: float = 1.0):
    """Gates of the Global-Sum path (best summed score, slot 1 at rank 0), or
    with lam < 1 of the Geometric path (pair p weighted by lam**p; the sums
    below are then the weighted sums and eps_p is weighted the same way).

    1. The GPU's path is the oracle's dynamic program run on the GPU's own
       scores (in float64): identical, or (where the float32 sums of the GPU's
       sweep meet a near tie) a path whose summed score is within rounding of
       the optimum.
    2. Against the oracle's scores, the GPU's path loses at most what the score
       errors can explain: g*(S_ora) - g(S_ora, path_gpu) <= 2 sum_p eps_p,
       with eps_p the largest |S_gpu - S_ora| of pair p.
    With `exact` (identical scores on both sides) the paths must be equal.
    """
    n, B = gpu["choice"].shape
    desc = oracle.OracleDesc.from_config(cfg)
    assert (gpu["choice"][:, 0] == 0).all(), "slot 1 must stay at rank 0 " + where
    np.testing.assert_array_equal(gpu["tokens"], np.take_along_axis(gpu["ids"], gpu["choice"][:, :, None], 2)[:, :, 0],
                                  err_msg="tokens follow the choices " + where)
    if B < 2:
        return 0
    S_g = gpu["scores"].astype(np.float64)
    scale = max(1.0, float(np.abs(S_g).max()))
    slack = 1e-5 * (B - 1) * scale
    _, ch_ref, tot_ref = oracle.viterbi(desc, S_g, gpu["ids"], n, lam=lam)
    diff = (ch_ref != gpu["choice"]).any(axis=1)
    own = path_scores(S_g, gpu["choice"], lam)
    assert (np.abs(own[diff] - tot_ref[diff]) <= slack).all(), \
        "GPU path not optimal for its own scores %s: %s" % (where, np.abs(own - tot_ref).max())
    assert diff.mean() <= 0.05, "too many near-tie paths %s: %d of %d" % (where, diff.sum(), n)
    _, ch_o, tot_o = oracle.viterbi(desc, ora["scores"], ora["ids"], n, lam=lam)
    eps = (np.abs(S_g - ora["scores"]).max(axis=(2, 3)) * lam ** np.arange(B - 1)[None, :]).sum(axis=1)
    lost = tot_o - path_scores(ora["scores"], gpu["choice"], lam)
    assert (lost <= 2 * eps + slack).all(), "GPU path loses more than the score error %s" % where
    if exact:
        np.testing.assert_array_equal(gpu["choice"], ch_o, err_msg="exact path " + where)
    return int(diff.sum())
