"""w8a8_quantized_moe_amd -- a W8A8 MoE expert layer for AMD MI355X (gfx950).

The computation lives in libw8a8moe.so (hand-written HIP kernels behind the C
ABI of include/w8a8moe.h); this package is its thin Python binding.  Importing
it fails if the library has not been built: there is no CPU fallback.
"""
from ._lib import (CODE_FP8, CODE_FP8_FAST, CODE_INT8, LIB_PATH, PACK_GATE_UP, PACK_PLAIN, SCALE_CLIPPED,  # noqa: F401
                   SCALE_COL_RECIPROCAL, SCALE_DYNAMIC, SCALE_STATIC, W8A8Error, check, lib)
from .api import (MoEWeights, gemm, gemm_i32, moe_forward, moe_forward_fused, moe_forward_static, moe_gate_up_acc,
                  moe_workspace_layout,  # noqa: F401
                  pack_weights, quantize_rows, workspace_views)
