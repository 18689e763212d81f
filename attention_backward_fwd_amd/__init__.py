"""MI355X-native fused exact-softmax attention forward and backward.

The computation lives in hand-written gfx950 HIP kernels behind the C ABI of
``libmi355_attn.so`` (declared in include/mi355_attn.h).  This package is the
thin Python binding of that ABI plus the seeded synthetic-input generator.
The library is loaded on first use; there is no CPU fallback.
"""

from .binding import (  # noqa: F401
    AttnError,
    BwdBuffers,
    attn_bwd,
    attn_bwd_postprocess,
    attn_bwd_preprocess,
    attn_bwd_workspace_bytes,
    attn_fwd,
    attn_shape,
    backward,
    forward,
    library,
    make_shape,
    shape_of,
)
