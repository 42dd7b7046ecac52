"""GPU parity of the pass run as separate C-ABI calls: corrector_topk, then
corrector_score on the ids and values it wrote, then corrector_walk on those
scores.  corrector_score enqueues its own launches (the hidden-state
projection shares the candidate projection's launch, or runs alone when a
folded table is attached), so this covers a launch sequence corrector_run
does not use.  Every gate of tests/parity.py applies, against the oracle."""

import numpy as np
import pytest

import parity as P

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("fold", [False, True])
@pytest.mark.parametrize("name,head,n", [("tiny", "normal", None), ("tiny", "stress", None), ("b1", "stress", None),
                                         ("b1", "zero", None), ("b32", "stress", None), ("b32", "normal", None)])
def test_chain(name, head, n, fold):
    _log("chain %s head=%s fold=%s" % (name, head, fold))
    x = P.inputs(name, head=head)
    gpu = P.gpu_chain(x, n=n, fold=fold)
    ora = P.oracle_run(x, n=n)
    steps, exempt, moved = P.check_all(gpu, ora, "chain/%s/%s/fold=%s" % (name, head, fold),
                                       exact_walk=(head == "zero"))
    _log("  walk steps %d exempt %d moved %d" % (steps, exempt, moved))
    if head == "stress" and name != "tiny":
        assert moved > 0


@pytest.mark.parametrize("fold", [False, True])
def test_chain_matches_run(fold):
    """The split calls and corrector_run compute the same thing with the same
    kernels' arithmetic: identical outputs, bit for bit."""
    _log("chain vs run fold=%s" % fold)
    x = P.inputs("b32", head="stress")
    a = P.gpu_chain(x, fold=fold)
    b = P.gpu_run(x, fold=fold)
    for k in ("ids", "vals", "scores", "tokens", "choice", "z", "g", "s"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


@pytest.mark.parametrize("rule", ["global_sum", "geometric", "beam"])
@pytest.mark.parametrize("name", ["tiny", "b1", "b32"])
def test_chain_matches_run_rules(name, rule):
    """With the Global-Sum, Geometric and beam rules, corrector_run finishes
    the scores one wave per pair and takes each request's path in the wave of
    its last pair (K = 4 and 16 here); the split calls form the scores one
    workgroup per request and take the paths in corrector_walk.  Same scores
    and paths, bit for bit."""
    _log("chain vs run %s %s" % (rule, name))
    lam = 0.75 if rule == "geometric" else 1.0
    x = P.inputs(name, head="stress", path_rule=rule, path_lambda=lam, beam_width=3)
    a = P.gpu_chain(x)
    b = P.gpu_run(x)
    for k in ("ids", "vals", "scores", "tokens", "choice"):
        np.testing.assert_array_equal(a[k], b[k], err_msg="%s %s: %s" % (rule, name, k))


def test_chain_matches_run_long_runs():
    """80 requests at the batch-32 shape (V cut to 32768): 1200 pairs, so each
    workgroup of the MLP launch runs 18 or 19 pairs and its waves count
    several pairs each before the pairs' last block workgroups finish them and
    the requests' last pairs walk.  Same scores and paths as the split calls,
    bit for bit."""
    _log("chain vs run, 80 requests")
    x = P.inputs("b32", head="stress", n=80, V=32768)
    a = P.gpu_chain(x)
    b = P.gpu_run(x)
    for k in ("ids", "vals", "scores", "tokens", "choice"):
        np.testing.assert_array_equal(a[k], b[k], err_msg="80 requests: " + k)


@pytest.mark.parametrize("rule", ["global_sum", "geometric", "beam"])
def test_chain_matches_run_rules_top_m(rule):
    """The same comparison with only the first 8 successors of each pair
    scored (the rest -inf, written by the per-pair finishing waves): same
    scores and paths, and no path leaves the kept successors."""
    _log("chain vs run %s top-m 8" % rule)
    lam = 0.75 if rule == "geometric" else 1.0
    x = P.inputs("b32", head="stress", path_rule=rule, path_lambda=lam, beam_width=4, succ_top_m=8)
    a = P.gpu_chain(x)
    b = P.gpu_run(x)
    for k in ("scores", "tokens", "choice"):
        np.testing.assert_array_equal(a[k], b[k], err_msg="%s top-m: %s" % (rule, k))
    assert np.isneginf(b["scores"][..., 8:]).all()
    assert (b["choice"][:, 1:] < 8).all()


@pytest.mark.parametrize("rule", ["greedy", "global_sum", "beam"])
def test_chain_matches_run_cosine(rule):
    """The cosine variant: corrector_run forms the scores one wave per pair
    and takes each request's path in the wave of its last pair; the split
    calls form them one workgroup per request and take the paths in
    corrector_walk.  Same scores and paths, bit for bit."""
    _log("chain vs run cosine %s" % rule)
    x = P.inputs("cosine", sigma=8.0, path_rule=rule, beam_width=3)
    a = P.gpu_chain(x, n=6, first=5)
    b = P.gpu_run(x, n=6, first=5)
    for k in ("ids", "vals", "scores", "tokens", "choice"):
        np.testing.assert_array_equal(a[k], b[k], err_msg="cosine %s: %s" % (rule, k))


@pytest.mark.parametrize("fold", [False, True])
def test_chain_cosine(fold):
    _log("chain cosine fold=%s" % fold)
    x = P.inputs("cosine", sigma=8.0)
    gpu = P.gpu_chain(x, n=4, first=9, fold=fold)
    ora = P.oracle_run(x, n=4, first=9)
    P.check_all(gpu, ora, "chain/cosine", variant="cosine")


@pytest.mark.parametrize("variant,rule", [("b32", "greedy"), ("b32", "global_sum"), ("b32", "beam"),
                                          ("cosine", "greedy"), ("cosine", "global_sum")])
def test_chain_matches_run_k8(variant, rule):
    """K = 8 (score rows of two lanes in the per-pair finishing waves) over 8
    blocks, for both variants and the walk, Global-Sum and beam rules: the
    run's per-pair forms and the split calls' per-request forms give the same
    scores and paths, bit for bit."""
    _log("chain vs run K=8 %s %s" % (variant, rule))
    extra = dict(sigma=8.0) if variant == "cosine" else dict(head="stress")
    x = P.inputs(variant, K=8, path_rule=rule, beam_width=3, **extra)
    a = P.gpu_chain(x, n=8)
    b = P.gpu_run(x, n=8)
    for k in ("ids", "vals", "scores", "tokens", "choice"):
        np.testing.assert_array_equal(a[k], b[k], err_msg="K=8 %s %s: %s" % (variant, rule, k))
    assert (b["choice"] != 0).any()
