"""fp64 CPU oracle for block-diffusion attention over a cached prefix.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run
anything here: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it. It shares no code with the HIP library.
"""

from .attention import (  # noqa: F401
    NEG_INF,
    widen,
    attention_rows,
    full,
    partial,
    merge,
    finalize,
    gather,
    online_state,
    state_from_partial,
)
from .retention import prefix_mass, select_retained  # noqa: F401
from .sequence import sequence_full, facache_step, split_rows  # noqa: F401
