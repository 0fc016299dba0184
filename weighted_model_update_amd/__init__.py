"""MI355X-native server-side FedAvg aggregation.

The aggregation runs in hand-written HIP kernels for gfx950 behind the C ABI
in include/fedavg.h (libfedavg.so); this package is its torch binding.
"""

from .fedavg import (  # noqa: F401
    FA_F32, FA_BF16, FA_WEIGHTS, FA_DELTAS, FA_DELTAS_ZERO_FILL, FA_COUNT_U8, FA_COUNT_U32, FA_MAX_CLIENTS, FA_MAX_N,
    FA_OPT_BLOCKS_PER_CU, FA_OPT_MASK_VECTORS_PER_BLOCK, FA_OPT_SPARSE_BLOCKS, FA_OPT_RESIDENT_PER_CU, FA_OPT_SPARSE_TILE,
    FA_OPT_TOPK_SAMPLED, FA_OPT_INDEX_TILES,
    EXPORTS, FedAvgError, StreamingAccumulator, load, library_path,
    fedavg_abi_version, fedavg_set_option, fedavg_aggregate, fedavg_workspace_size,
    arena_layout, client_arena,
    fedavg_begin, fedavg_accumulate, fedavg_finalize, fedavg_sync, fedavg_destroy,
    fedavg_accumulate_partial, fedavg_partial_info, fedavg_export_state, fedavg_resume,
    sparse_workspace_size, sparse_masked_accumulate, sparse_masked_accumulate_noalloc, fedavg_checksum,
    fedavg_sum_workspace_size,
    fedavg_checksum_sum,
    topk_workspace_size, topk_select, topk_count, SampleController, stream_windows,
)
