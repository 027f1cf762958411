"""little-lm training-step hot path on MI355X (gfx950): Python binding of libll.

The compute lives in libll.so (hand-written HIP kernels behind the C ABI of include/ll.h); this
package only marshals arguments (``_lib``) and allocates buffers through torch (``ops``).
"""
from . import _lib  # noqa: F401
from ._lib import (LL_BF16, LL_F32, LLError, LayerCfg, LayerGrads, LayerParams,  # noqa: F401
                   ll_fp8_quant_tensorwise, ll_fp8_quant_workspace_bytes, ll_fused_lce_fwd_bwd,
                   ll_fused_lce_workspace_bytes, ll_last_error, ll_layer_bwd, ll_layer_fwd,
                   ll_layer_saved_bytes, ll_layer_workspace_bytes, ll_status_string, ll_version,
                   llt_gemm, llt_gemm_nt, llt_gemm_splitk, llt_gemm_splitk_workspace_bytes)
