"""Seeded synthetic inputs for FedAvg aggregation.

This package only draws random numbers and lays them out; it performs none of
the aggregation arithmetic, so both the CPU oracle (``oracle/``) and the HIP
library (``weighted_model_update_amd``) can be fed from it without sharing any
of the method's code.

Every stream is keyed by ``SeedSequence([2026, cfg, role, client])`` with the
roles below, so a given (config, role, client) always yields the same numbers.
"""

from .configs import (  # noqa: F401
    ROLE_COUNTS, ROLE_BASE, ROLE_VALUES, ROLE_SUPPORT,
    CFG_DENSE_SMALL, CFG_ADAPTER, CFG_DENSE_2B, CFG_STREAM_8B, CFG_SPARSE_1B,
    dense_2b_tensor_shapes, stream_8b_tensor_shapes, adapter_segments,
    numel_of, CHUNK_BYTES_8B,
)
from .host import (  # noqa: F401
    rng, sample_counts, normal_f32, bf16_bits_from_f32, f32_from_bf16_bits,
    dense_clients_f32, dense_clients_bf16, adapter_presence, topk_sparse_deltas,
    uniform_sparse_support, laplace_tail_values,
)
