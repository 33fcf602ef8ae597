"""MI355X-native paged KV-cache attention.

HIP kernels for gfx950 behind a C ABI (include/pagedattn.h, built into
libpagedattn.so in this directory); `binding` marshals torch tensors into
that ABI and `runtime` keeps a device pool together with the host block
manager.  There is no CPU path: every computation runs in the library.
"""
from .binding import (  # noqa: F401
    PA_BF16, PA_DBG_BLOCK_ID, PA_DBG_CONTEXT_LEN, PA_DBG_COPY_PAIR, PA_DBG_KINDS, PA_DBG_SLOT, PA_FP8_E4M3, PA_EHIP, PA_EINVAL, PA_ENOMEM, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_F16, PA_F32, PA_OK,
    BlockManager, PagedAttnError, Scheduler, lib, make_cache, pa_cache, pa_copy_blocks, pa_decode,
    pa_decode_choose_partition, pa_decode_grouped, pa_decode_grouped_workspace_bytes, pa_decode_noalloc,
    pa_decode_workspace_bytes,
    pa_debug_counters, pa_kv_append, pa_prefill_choose_splits, pa_prefill_chunk, pa_prefill_chunk_split,
    pa_prefill_workspace_bytes, status_str,
)
