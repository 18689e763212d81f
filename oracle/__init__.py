"""fp64 CPU oracle of softmax attention forward and backward (test infrastructure only).

Only the test-suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the GPU library.
"""

from .attention import (  # noqa: F401
    attention_bwd,
    attention_cols,
    attention_fwd,
    attention_rows,
    softmax_probs,
)
