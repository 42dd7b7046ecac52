"""Expected token yield of one draft-verify cycle.

Faster Decoding, "Verification can be parallel even when generation is
sequential": with s_k the probability that the first k draft positions are
all accepted, a cycle that emits the accepted prefix plus one corrected or
bonus token yields E[Y] = 1 + sum_{k=1..gamma} s_k; with a constant
conditional acceptance probability alpha this is sum_{k=0..gamma} alpha^k.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

from __future__ import annotations

from typing import Sequence


def survival(conditional: Sequence[float]) -> list:
    """Prefix survival s_k = product of the first k conditional acceptances."""
    out, alive = [], 1.0
    for p in conditional:
        alive *= float(p)
        out.append(alive)
    return out


def expected_yield(conditional: Sequence[float]) -> float:
    """E[Y] = 1 + sum_k s_k."""
    return 1.0 + sum(survival(conditional))


def iid_expected_yield(alpha: float, gamma: int) -> float:
    """E[Y] under a constant conditional acceptance alpha: sum_{k=0..gamma} alpha^k."""
    return sum(float(alpha) ** k for k in range(gamma + 1))
