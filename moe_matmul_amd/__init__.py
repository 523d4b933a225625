"""NVFP4 block-scaled grouped GEMM for AMD Instinct MI355X (gfx950).

The computation runs in the hand-written HIP library
(``libnvfp4_grouped_gemm.so``, C ABI in ``include/nvfp4_grouped_gemm.h``);
this package is its thin Python binding plus device-memory plumbing.
"""
from ._binding import (  # noqa: F401
    LIB_PATH, NVFP4_ERR_CONFIG, NVFP4_ERR_HIP, NVFP4_ERR_INVALID, NVFP4_ERR_MISALIGNED, NVFP4_ERR_WORKSPACE,
    NVFP4_MAX_DEVICE_GROUPS, NVFP4_MAX_GROUPS, NVFP4_OK, NVFP4_SCRATCH_BYTES, Nvfp4Error, load_library, nvfp4_device_group_tiles,
    nvfp4_error_string, nvfp4_grouped_gemm, nvfp4_grouped_gemm_config, nvfp4_grouped_gemm_device,
    nvfp4_grouped_gemm_ex, nvfp4_grouped_gemm_pow2, nvfp4_grouped_gemm_scratch, nvfp4_grouped_gemm_stages, nvfp4_grouped_gemm_validate, nvfp4_last_hip_error, nvfp4_launch_geometry,
    nvfp4_num_tile_configs, nvfp4_select_tile_config, nvfp4_sf_bytes, nvfp4_split_plan, nvfp4_splits_k_over_waves, nvfp4_tile_config_info, nvfp4_workspace_bytes,
    prepare,
)
