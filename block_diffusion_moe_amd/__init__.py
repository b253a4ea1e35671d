"""MI355X-native (gfx950) kernels for one block-diffusion MoE denoise step.

The computation lives in ``libbdmoe.so`` (hand-written HIP kernels behind a
C ABI declared in ``include/bdmoe.h``); this package is its ctypes binding.
Build the library with ``python -m block_diffusion_moe_amd.build``.
"""
import torch  # noqa: F401  (loads the HIP runtime the library binds to)

from .binding import (BDM_LAYOUT_MFMA_TILES, BDM_LAYOUT_MFMA_TILES_GU, BDM_LAYOUT_ROW_MAJOR,
                      BDM_MASK_ID_CLOVER, BDM_THRESHOLD_DEFAULT, BDM_VERIFY_EXACT, BDM_VERIFY_THRESHOLD, EXPORTS,
                      DEBUG_LIB_PATH, LIB_PATH, BdmError, MoeLayerC, MoeStack, Packed,
                      bdm_debug_bounds, bdm_denoise_block, bdm_denoise_workspace_bytes,
                      bdm_head_stat_parts, bdm_head_verify_workspace_bytes,
                      bdm_head_workspace_bytes, bdm_lm_head_stats, bdm_lm_head_unmask,
                      bdm_lm_head_verify, bdm_moe_block_forward, bdm_moe_block_forward_noalloc,
                      bdm_moe_workspace_bytes, BDM_STATIC_SCRATCH_BYTES,
                      bdm_unmask_from_stats, bdm_pack_gate_up, bdm_pack_weights,
                      bdm_packed_weight_elems,
                      bdm_rmsnorm, bdm_status_string, bdm_version, load, workspace)

__all__ = [
    "BDM_LAYOUT_MFMA_TILES", "BDM_LAYOUT_MFMA_TILES_GU", "BDM_LAYOUT_ROW_MAJOR",
    "BDM_MASK_ID_CLOVER", "BDM_THRESHOLD_DEFAULT", "BDM_VERIFY_EXACT", "BDM_VERIFY_THRESHOLD", "EXPORTS",
    "DEBUG_LIB_PATH", "LIB_PATH", "BdmError", "MoeLayerC", "MoeStack", "Packed",
    "bdm_debug_bounds", "bdm_denoise_block", "bdm_denoise_workspace_bytes",
    "bdm_head_stat_parts", "bdm_head_verify_workspace_bytes", "bdm_head_workspace_bytes",
    "bdm_lm_head_stats", "bdm_lm_head_verify",
    "bdm_unmask_from_stats", "bdm_lm_head_unmask", "bdm_moe_block_forward",
    "bdm_moe_block_forward_noalloc", "BDM_STATIC_SCRATCH_BYTES",
    "bdm_moe_workspace_bytes", "bdm_pack_gate_up", "bdm_pack_weights", "bdm_packed_weight_elems",
    "bdm_rmsnorm",
    "bdm_status_string", "bdm_version", "load", "workspace",
]
