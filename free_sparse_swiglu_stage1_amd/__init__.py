"""Prox two-stage sparse SwiGLU FFN forward for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libprox.so`` (C ABI in include/prox.h);
this package is its thin Python binding.
"""
from .prox import (  # noqa: F401
    BF16, F32, MODES, STEP_NAMES, ProxError, Proxy, Weights, alloc_workspace, allocate_sparsity, chain_forward,
    chain_workspace_size, counts, effective_sparsity,
    ffn_forward, ffn_forward_timed, load_library, pack_weights, pack_weights_fp8, proxy_sizes, quantize_proxy, rmsnorm,
    stage1_select, stage2_exact, topk, version, workspace_init, workspace_size, W_FP8_E4M3, W_NATIVE,
)
