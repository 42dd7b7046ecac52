"""Expected token yield of one draft-verify cycle.

Faster Decoding, "Verification can be parallel even when generation is
sequential": s_k, the probability that the first k draft positions are all
accepted, is the product of the first k conditional acceptance probabilities;
a cycle emits the accepted prefix plus one corrected or bonus token, so its
expected yield is E[Y] = 1 + sum_{k=1..gamma} s_k.  With a constant
conditional acceptance alpha the sum is geometric:
E[Y] = (1 - alpha^(gamma+1)) / (1 - alpha), and gamma + 1 at alpha = 1.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

from __future__ import annotations

from typing import Sequence

import numpy as np


def survival(conditional: Sequence[float]) -> list:
    """Prefix survival s_1..s_gamma: cumulative products of the conditional
    acceptance probabilities."""
    return np.cumprod(np.asarray(conditional, dtype=np.float64)).tolist()


def expected_yield(conditional: Sequence[float]) -> float:
    """E[Y] = 1 + sum_k s_k."""
    return 1.0 + float(np.sum(survival(conditional)))


def iid_expected_yield(alpha: float, gamma: int) -> float:
    """E[Y] for a constant conditional acceptance alpha over gamma positions:
    the geometric series 1 + alpha + ... + alpha^gamma in closed form."""
    alpha = float(alpha)
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)
