"""MI355X (gfx950) hot path of the hybrid H/R/T masked-attention backbone.

The computation lives in libmtfm.so (HIP kernels behind the C ABI of
include/mtfm.h); `binding` marshals torch tensors into that ABI and
`tensors` moves host arrays to the device.  Build the library with
``python -m hybrid_masked_attention_amd.build``.
"""
from . import binding  # noqa: F401
