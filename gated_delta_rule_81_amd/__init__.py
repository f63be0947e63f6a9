"""MI355X-native Kimi Delta Attention (KDA) operator.

The computation lives in libkda.so (hand-written HIP kernels for gfx950,
C ABI in include/kda.h); this package is its thin Python binding.
"""
from .kda import (  # noqa: F401
    KdaError,
    decode_step,
    fwd_chunked,
    lib,
    status_string,
    workspace_bytes,
)
