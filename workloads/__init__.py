"""Seeded synthetic inputs for paged-KV attention.

This package is shared by the tests, the bench and the smoke check. It holds
only random draws, lengths, page tables and pools: none of the attention
arithmetic lives here, so the oracle and the HIP path can both consume its
tensors without sharing any of the method's code.
"""

from .synth import (  # noqa: F401
    BASE_SEED,
    CONFIG_NAMES,
    Workload,
    make_config,
    make_decode,
    make_append,
    make_cascade,
    make_pod_mix,
    make_block_sparse,
    make_block_sparse_batch,
    to_ragged,
    make_sparse_video,
    SPARSE_VIDEO_NAME,
    POD_MIX_NAME,
    cascade_flat_tables,
    fp32_scale,
    to_fp8_cache,
    to_mxfp4_cache,
)
