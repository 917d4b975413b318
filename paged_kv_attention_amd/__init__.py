"""MI355X-native paged-KV attention: plan, paged decode (bf16 or FP8 KV),
append, cascade, variable block-sparse attention and state merge, backed by hand-written HIP kernels for gfx950 in libfi.so.

The shared library is required: importing works without it, but every call
raises until it is built (``python -m paged_kv_attention_amd.build``).
"""

from ._lib import FIError, LIB_PATH, SIGNATURES, load  # noqa: F401
from .api import (  # noqa: F401
    BlockSparsePlan,
    KernelTimer,
    Plan,
    Workspace,
    block_sparse_attention,
    cascade,
    check_page_tables,
    merge_states,
    paged_append,
    paged_decode,
    paged_decode_fp8,
    paged_decode_mxfp4,
    paged_decode_noalloc,
)
