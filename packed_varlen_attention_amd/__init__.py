"""Packed 2D-RoPE variable-length attention for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libmf.so`` behind the C ABI in
``include/mf.h``; this package is its Python binding plus small allocation
helpers (PyTorch supplies device memory and the HIP stream).  Importing the
package loads the library and fails loudly if it has not been built.
"""
from ._binding import (  # noqa: F401
    EXPORTED, LIB_PATH, MF_TRACE_MAX, KernelTrace, Trace, MF_BF16, MF_F32, MF_ERR_HIP, MF_ERR_INVALID_ARG, MF_ERR_UNSUPPORTED,
    MF_ERR_WORKSPACE, MF_OK, MFError, abi_version, dtype_code, load_library, mf_mfma_probe, mf_pack, mf_pack_edit,
    mf_rope3d_apply, mf_rope3d_workspace_size,
    mf_rope2d_apply, mf_rope2d_workspace_size, mf_varlen_attn_bwd, mf_varlen_attn_fwd,
    mf_varlen_attn_workspace_size, status_string, mf_adaln_modulate, mf_block_workspace_size, mf_out_gated_residual,
    mf_qkv_rope, mf_adaln_modulate_bwd, mf_adaln_modulate_bwd_workspace_size, mf_out_gated_residual_bwd,
    mf_out_gated_residual_bwd_workspace_size, mf_qkv_rope_bwd, mf_qkv_rope_bwd_workspace_size,
)
from .api import (  # noqa: F401
    PROBE_VECTORS, PackResult, attn_bwd, attn_fwd, cfg_combine, mfma_probe, pack, pack_edit, rf_loss, rf_noise,
    rope2d_apply, rope3d_apply, adaln_modulate, block_workspace, out_gated_residual, qkv_rope, adaln_modulate_bwd,
    out_gated_residual_bwd, qkv_rope_bwd, rotated_buffer,
)

load_library()
