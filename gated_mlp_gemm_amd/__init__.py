"""MI355X (gfx950) fused SwiGLU GEMM: Y = SiLU(A.W1) (.) (A.W2).

The computation lives in the HIP library ``libswiglu.so`` (C ABI in
``include/swiglu.h``); ``gated_mlp_gemm_amd.swiglu`` is its ctypes binding.
Importing the package does not load the library; the first call does, and
fails loudly if it is not built (``python -m gated_mlp_gemm_amd.build``).
"""
from .swiglu import (  # noqa: F401
    SWIGLU_AUTO, SWIGLU_VARIANT_I, SWIGLU_VARIANT_S, SwigluError, load_library,
    make_workspace, swiglu_describe_launch, swiglu_down_proj, swiglu_fp8_scale_exp,
    swiglu_fused_gemm, swiglu_fused_gemm_fp8, swiglu_fused_gemm_noalloc,
    swiglu_fused_gemm_strided, swiglu_gated_mlp,
    swiglu_last_error, swiglu_m_switch, swiglu_pack_weights, swiglu_pack_weights_nk,
    swiglu_quantize_fp8, swiglu_select_variant, swiglu_silu_mul, swiglu_status_string,
    swiglu_unfused_ablation, swiglu_workspace_size,
)
