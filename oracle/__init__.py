"""CPU oracle for the draft-correction pass.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path never imports this
package, and this package never imports the GPU library.
"""

from .oracle import (  # noqa: F401
    CONF_FIELDS,
    OracleDesc,
    confidence,
    accepted_lengths,
    beam,
    build,
    gelu,
    get_threads,
    layernorm,
    log_normaliser,
    log_normaliser_row,
    param_count,
    represent,
    run,
    score,
    set_threads,
    topk,
    topk_row,
    viterbi,
    walk,
)
from .yieldcalc import expected_yield, iid_expected_yield, survival  # noqa: F401
