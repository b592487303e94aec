"""GALE 1-bit routed-expert matmul on AMD Instinct MI355X (gfx950).

The computation lives in libgale.so (HIP kernels behind the C ABI in
include/gale.h); this package is its ctypes binding.  torch provides device
memory and streams only.
"""
from .binding import (  # noqa: F401
    GALE_F16, GALE_F32, GALE_X_ROTATED, GALE_X_PREPARED, prepared_bytes, prepare_activations, GALE_PATH_DECODE, GALE_PATH_GROUPED,
    GALE_GROUPED_ITEMS, GALE_GROUPED_GEMM, GALE_DECODE_STAGED, GaleError, PackedMatrix,
    DescriptorTable, lib, exported_symbols, packed_sizes, check_canonical, pack_host, unpack_host, pack_device,
    pack_matrix, matrix_table, expert_table, debug_unpack_signs, debug_unpack_outliers, fwht1024,
    expert_gemv, expert_ffn, moe_layer_fwd, route_topk, gemv_workspace_bytes, ffn_workspace_bytes,
    moe_workspace_bytes, gale_tiles_flag, gale_layer_tiles_flag, GALE_OUTLIER_STAGE_SHIFT, gale_outlier_stage_flag,
    GALE_SYNC_NO_WAIT, GALE_SYNC_BYTES, GALE_ERR_SYNC, moe_workspace, sync_init, sync_status,
    decode_stack_workspace_bytes, layer_table, moe_decode_stack,
)
from .pack_files import Pack, PackWriter, LoadedStack, load_stack, read_manifest  # noqa: F401,E402
