"""Workload shapes.

Every configuration describes one pass of the corrector over a batch of draft
blocks.  A block has ``B + 1`` positions: position 0 is the anchor (the last
committed token) and positions 1..B are the drafted slots.  The corrector reads
only the drafted slots; the anchor rows are present in the synthetic buffers so
that the strided addressing a real caller uses (skip the anchor row) is
exercised.

Shapes follow the DCOCO page ("Contextual Correction of Parallel Drafts for
Speculative Decoding", method details, steps (1)-(5)): 15 drafted slots plus an
anchor, K = 16 candidates, representation width r = 128 and a 386 -> 256 -> 1
GELU MLP on a Qwen3-8B-sized drafter (hidden width 4096, vocabulary 151936).
The cosine variant follows LiLiCorr section 3.2, Eq. 1.
"""

from __future__ import annotations

import copy

_BASE = dict(
    n=1,              # requests (= blocks) per pass
    B=15,             # drafted slots per block (anchor not counted)
    V=151936,         # vocabulary
    K=16,             # candidates per slot
    d=4096,           # drafter hidden width
    de=4096,          # embedding width
    r=128,            # representation width
    h=256,            # MLP hidden width
    dvec=128,         # cosine in/out vector width
    variant="mlp",    # "mlp" or "cosine"
    sigma=1.0,        # cosine scale
    logits_dtype="bf16",
    logits="zipf",    # "zipf" (Gumbel-perturbed Zipf) or "planted"
    tiers=(1.1,),     # Zipf exponents; request i gets tier floor(len*i/n)
    hidden_std=1.0,
    embed_std=0.02,
    weight_std=0.02,
    ln_eps=1e-5,
)


def _mk(index: int, **kw) -> dict:
    c = copy.deepcopy(_BASE)
    c.update(kw)
    c["index"] = index
    return c


CONFIGS = {
    # 1 request, 1 anchor + 3 drafted slots, V=1000, K=4, d=64, r=16,
    # MLP (3r+2=50) -> 32 -> 1; fp32 logits ~N(0,2) with 3 planted peaks.
    "tiny": _mk(0, n=1, B=3, V=1000, K=4, d=64, de=64, r=16, h=32, dvec=16,
                logits_dtype="f32", logits="planted", weight_std=0.1),
    # Qwen3-8B-shaped DCOCO corrector, one request.
    "b1": _mk(1, n=1),
    # Same shapes at concurrency 32, three entropy tiers in equal thirds.
    "b32": _mk(2, n=32, tiers=(0.8, 1.1, 1.6)),
    # Cosine in/out-vector variant at batch 32, on the batch-32 inputs.
    "cosine": _mk(3, n=32, tiers=(0.8, 1.1, 1.6), variant="cosine", seed_index=2),
    # Stress: 256 requests, K=32, hidden width 5120, hidden states ~N(0,3).
    "stress": _mk(4, n=256, K=32, d=5120, de=5120, hidden_std=3.0,
                  tiers=(0.8, 1.1, 1.6)),
}


def config(name: str, **overrides) -> dict:
    """Return a copy of configuration ``name`` with ``overrides`` applied."""
    c = copy.deepcopy(CONFIGS[name])
    c.update(overrides)
    c["name"] = name
    return c

