"""Paged KV cache and PagedAttention hot path for AMD MI355X (gfx950).

The work is done by ``libpa.so`` (hand-written HIP kernels behind the C ABI
of ``include/pa.h``); this package marshals torch tensors into those calls
and wraps the host block manager.
"""

from ._lib import PAError, lib, status_string  # noqa: F401
from .api import (  # noqa: F401
    BlockManager,
    KVPool,
    OutOfBlocks,
    decode_shared_workspace,
    decode_workspace,
    pa_cache_append,
    pa_copy_blocks,
    pa_decode,
    pa_decode_append,
    pa_decode_noalloc,
    pa_decode_shared,
    pa_decode_shared_workspace_size,
    pa_decode_workspace_size,
    pa_mixed_batch,
    pa_set_tuning,
    pa_share_groups,
    pa_set_validate,
    pa_sha256,
    pa_gather_checksum,
    pa_gather_checksum_size,
    pa_plan_step,
    pa_prefill_chunk,
    pa_prefill_workspace_size,
    prefill_workspace,
    tuning,
)
