"""MI355X (gfx950) MXFP4 mixture-of-experts expert block.

The work runs in libmxfp4_moe.so (C ABI in include/mxfp4_moe.h); this
package only marshals torch tensors into it.
"""
from .native import (Dims, MoeLayer, Mxfp4Error, SavedState, Workspace, lib,  # noqa: F401
                     mxfp4_dequantize, mxfp4_moe_backward, mxfp4_moe_backward_dx, mxfp4_moe_forward,
                     mxfp4_moe_forward_noalloc, mxfp4_quantize, mxfp8_quantize,
                     workspace_bytes)
