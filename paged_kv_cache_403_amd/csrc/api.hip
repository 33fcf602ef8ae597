// C ABI of the paged KV-cache attention library: argument validation, launch
// configuration, workspace sizing and error mapping.  Every check that needs
// only host-visible values runs before anything is enqueued.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "launch.h"
#include "pagedattn.h"

namespace {

constexpr int32_t kMaxGridYZ = 65535;

int elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : dtype == PA_FP8_E4M3 ? 1 : 2; }

bool is_fp8(const pa_cache* c) { return c->dtype == PA_FP8_E4M3; }

// Type of q / out / appended rows.
int32_t act_dtype(const pa_cache* c) { return is_fp8(c) ? c->act_dtype : c->dtype; }

// Validate the pool descriptor.
int check_cache(const pa_cache* c) {
  if (!c || !c->k_cache || !c->v_cache) return PA_EINVAL;
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0 || c->block_size <= 0 || c->head_dim <= 0) return PA_EINVAL;
  if (c->dtype != PA_F32 && c->dtype != PA_F16 && c->dtype != PA_BF16 && c->dtype != PA_FP8_E4M3) return PA_EINVAL;
  if (c->head_dim != 64 && c->head_dim != 128) return PA_EUNSUPPORTED;
  if (is_fp8(c)) {
    if (c->act_dtype != PA_F16 && c->act_dtype != PA_BF16) return PA_EINVAL;
    if (!(std::isfinite(c->k_scale) && c->k_scale > 0.f && std::isfinite(c->v_scale) && c->v_scale > 0.f))
      return PA_EINVAL;
    if (c->head_dim != 128 || c->block_size < 16) return PA_EUNSUPPORTED;
  }
  if (c->block_size != 8 && c->block_size != 16 && c->block_size != 32 && c->block_size != 64) return PA_EUNSUPPORTED;
  if (c->num_kv_heads > kMaxGridYZ) return PA_EUNSUPPORTED;
  return PA_OK;
}

int check_group(const pa_cache* c, int32_t num_q_heads, int32_t* group) {
  if (num_q_heads <= 0 || num_q_heads % c->num_kv_heads != 0) return PA_EINVAL;
  const int32_t g = num_q_heads / c->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return PA_EUNSUPPORTED;
  *group = g;
  return PA_OK;
}

int check_scale(float scale) { return (std::isfinite(scale) && scale > 0.f) ? PA_OK : PA_EINVAL; }

// Text of the calling thread's last HIP failure (or of pa_decode_noalloc's
// last refusal), for pa_last_error().
thread_local const char* g_last_hip_error = "";

int hip_status(hipError_t e) {
  if (e == hipSuccess) return PA_OK;
  g_last_hip_error = hipGetErrorString(e);
  return PA_EHIP;
}

// Tokens per partition actually used for a requested partition_size (one
// pass: the context rounded up to whole blocks, capped at INT32_MAX).
int32_t effective_partition(int32_t requested, int32_t block_size, int32_t max_context_len, int32_t chosen) {
  const int32_t p = requested == -1 ? chosen : requested;
  if (p != 0) return p;
  const int64_t c = max_context_len > 0 ? max_context_len : 1;
  return static_cast<int32_t>(std::min<int64_t>((c + block_size - 1) / block_size * block_size, INT32_MAX));
}

// Split-K workspace: partial softmax states [S][Hq][P][2] and outputs
// [S][Hq][P][D] (fp32), the work list [S * P][2] and its length (int32).
size_t workspace_for(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim, int64_t num_parts) {
  if (num_parts <= 1) return 0;
  return static_cast<size_t>(num_seqs * num_q_heads * num_parts * (head_dim + 2) * sizeof(float) +
                             num_seqs * num_parts * 2 * sizeof(int32_t) + 16);
}

// Prefix-grouped decode: partitions of `part` tokens, 2 * ceil(C / part)
// slots per row (prefix slots of the chunk, then the sequence's own).
constexpr int32_t kGroupedDefaultPartition = 1024;
constexpr int64_t kGroupedMergeLds = 56 * 1024;  // slot weights (dynamic); the merge kernel also holds 4 KiB of its own

struct GroupedLayout {
  int64_t parts, slots;
  size_t ml, o, suf_items, pre_items, seq_start, slot_base, nslots, counts, total;  // byte offsets
};

size_t align16(size_t x) { return (x + 15) / 16 * 16; }

GroupedLayout grouped_layout(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim, int64_t max_context_len,
                             int64_t part) {
  GroupedLayout g{};
  g.parts = std::max<int64_t>(1, (max_context_len + part - 1) / part);
  g.slots = 2 * g.parts;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align16(off + bytes);
    return at;
  };
  g.ml = take(num_seqs * num_q_heads * g.slots * 2 * sizeof(float));
  g.o = take(num_seqs * num_q_heads * g.slots * head_dim * sizeof(float));
  g.suf_items = take(num_seqs * g.parts * 2 * sizeof(int32_t));
  g.pre_items = take(num_seqs * g.parts * 4 * sizeof(int32_t));
  g.seq_start = take(num_seqs * sizeof(int32_t));
  g.slot_base = take(num_seqs * sizeof(int32_t));
  g.nslots = take(num_seqs * sizeof(int32_t));
  g.counts = take(2 * sizeof(int32_t));
  g.total = off;
  return g;
}

// The partition pa_decode_grouped uses: the default is 1024 tokens, but a
// prefix item keeps one block id per lane (at most 64 blocks), so 8-token
// blocks default to 512.  The workspace for the default is sized for 512,
// which covers both.
int32_t grouped_partition(int32_t requested, int32_t block_size) {
  if (requested != 0) return requested;
  return block_size < 16 ? 64 * block_size : kGroupedDefaultPartition;
}
constexpr int32_t kGroupedSmallestDefault = 512;

}  // namespace

extern "C" {

const char* pa_status_str(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_EINVAL: return "invalid argument";
    case PA_EUNSUPPORTED: return "unsupported shape or dtype";
    case PA_EWORKSPACE: return "workspace too small";
    case PA_ENOMEM: return "block pool exhausted";
    case PA_EHIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* pa_last_error(void) { return g_last_hip_error; }

int pa_debug_counters(uint64_t* counts, int32_t reset) {
#ifdef PA_DEBUG
  if (!counts) return PA_EINVAL;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_status(e);
  unsigned long long acc[PA_DBG_KINDS] = {};
  const bool r = reset != 0;
  if ((e = pa::debug_counts_decode(acc, r)) != hipSuccess || (e = pa::debug_counts_grouped(acc, r)) != hipSuccess ||
      (e = pa::debug_counts_prefill(acc, r)) != hipSuccess || (e = pa::debug_counts_kv_cache_ops(acc, r)) != hipSuccess)
    return hip_status(e);
  for (int k = 0; k < PA_DBG_KINDS; ++k) counts[k] = acc[k];
  return PA_OK;
#else
  (void)counts;
  (void)reset;
  return PA_EUNSUPPORTED;
#endif
}

int pa_kv_append(const pa_cache* cache, const void* k_new, const void* v_new, const int64_t* slot_mapping,
                 int32_t num_tokens, void* stream) {
  int rc = check_cache(cache);
  if (rc != PA_OK) return rc;
  if (num_tokens < 0) return PA_EINVAL;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping) return PA_EINVAL;
  if (is_fp8(cache))
    return hip_status(pa::launch_kv_append_fp8(k_new, v_new, slot_mapping, num_tokens, cache->k_cache, cache->v_cache,
                                               cache->num_blocks, cache->num_kv_heads, cache->block_size,
                                               cache->head_dim, cache->act_dtype, 1.0f / cache->k_scale,
                                               1.0f / cache->v_scale, static_cast<hipStream_t>(stream)));
  return hip_status(pa::launch_kv_append(k_new, v_new, slot_mapping, num_tokens, cache->k_cache, cache->v_cache,
                                         cache->num_blocks, cache->num_kv_heads, cache->block_size, cache->head_dim,
                                         elem_bytes(cache->dtype), static_cast<hipStream_t>(stream)));
}

int pa_copy_blocks(const pa_cache* cache, const int32_t* pairs, int32_t num_pairs, void* stream) {
  int rc = check_cache(cache);
  if (rc != PA_OK) return rc;
  if (num_pairs < 0) return PA_EINVAL;
  if (num_pairs == 0) return PA_OK;
  if (!pairs) return PA_EINVAL;
  const int64_t block_bytes = static_cast<int64_t>(cache->num_kv_heads) * cache->block_size * cache->head_dim *
                              elem_bytes(cache->dtype);
  return hip_status(pa::launch_copy_blocks(pairs, num_pairs, cache->k_cache, cache->v_cache, cache->num_blocks,
                                           block_bytes, static_cast<hipStream_t>(stream)));
}

int32_t pa_decode_choose_partition(const pa_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t max_context_len) {
  (void)num_q_heads;
  if (!cache || cache->num_kv_heads <= 0 || cache->block_size <= 0) return 0;
  const int64_t units = static_cast<int64_t>(num_seqs) * cache->num_kv_heads;
  // One pass when the batch gives the chip about two workgroups per compute
  // unit or more and no context is long: the one-pass grid starts the
  // longest sequences first, so uneven lengths balance out.  Otherwise split,
  // into the longest partitions that still give enough work items, since
  // every partition has a fixed start-up cost and a share of the merge:
  //  * a batch of fewer (sequence, KV head) units than two per compute unit
  //    is a few long contexts: partitions up to 16384 tokens, down to about
  //    two items per compute unit (measured on 4 x 131072 tokens, 8 KV heads:
  //    2048 / 4096 / 8192 / 16384-token partitions ran 346-360 / 335-341 /
  //    327-334 / 343 us);
  //  * otherwise long contexts sit beside short ones: partitions of up to
  //    2048 tokens, down to about a thousand items, so the short sequences
  //    fill in around the pieces of the long ones.
  if (max_context_len <= 512 || (units >= 512 && max_context_len <= 4096)) return 0;
  int32_t p = units < 512 ? 16384 : 2048;
  const int64_t want = units < 512 ? 512 : 1024;
  while (p > 512 && units * ((max_context_len + p - 1) / p) < want) p /= 2;
  return p < cache->block_size ? cache->block_size : p;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  // -1: the chooser never picks partitions shorter than 512 tokens (nor
  // shorter than a block)
  const int32_t p = partition_size == -1 ? 512 : partition_size;
  if (p <= 0) return 0;
  const int64_t parts = (static_cast<int64_t>(max_context_len) + p - 1) / p;
  return workspace_for(num_seqs, num_q_heads, head_dim, parts);
}

}  // extern "C"

namespace {

// Everything pa_decode checks and derives before it touches the GPU: the
// launch arguments (workspace pointers still unset) and the workspace bytes
// the launch needs (0 for one pass).  *nothing is set when the batch is
// empty: a valid no-op.
int decode_prepare(const pa_cache* cache, const void* q, void* out, int32_t num_seqs, int32_t num_q_heads,
                   const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                   int32_t max_context_len, float scale, int32_t partition_size, pa::DecodeArgs* a, size_t* need,
                   bool* nothing) {
  *nothing = false;
  int rc = check_cache(cache);
  if (rc != PA_OK) return rc;
  int32_t group = 0;
  if ((rc = check_group(cache, num_q_heads, &group)) != PA_OK) return rc;
  if ((rc = check_scale(scale)) != PA_OK) return rc;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len < 0) return PA_EINVAL;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * cache->block_size)
    return PA_EINVAL;
  if (num_seqs > kMaxGridYZ) return PA_EUNSUPPORTED;
  if (partition_size < -1) return PA_EINVAL;
  if (partition_size > 0 && partition_size % cache->block_size != 0) return PA_EINVAL;
  if (num_seqs == 0) {
    *nothing = true;
    return PA_OK;
  }
  if (!q || !out || !block_tables || !context_lens) return PA_EINVAL;
  const int32_t chosen = pa_decode_choose_partition(cache, num_seqs, num_q_heads, max_context_len);
  const int32_t part_tokens = effective_partition(partition_size, cache->block_size, max_context_len, chosen);
  const int32_t num_parts =
      max_context_len > 0 ? static_cast<int32_t>((static_cast<int64_t>(max_context_len) + part_tokens - 1) / part_tokens)
                          : 1;
  *need = workspace_for(num_seqs, num_q_heads, cache->head_dim, num_parts);
  *a = pa::DecodeArgs{};
  a->q = q;
  a->out = out;
  a->k_cache = cache->k_cache;
  a->v_cache = cache->v_cache;
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->scale = scale;
  if (is_fp8(cache)) {
    a->k_scale = cache->k_scale;
    a->v_scale = cache->v_scale;
  }
  a->dtype = cache->dtype;
  a->act_dtype = act_dtype(cache);
  a->head_dim = cache->head_dim;
  a->block_size = cache->block_size;
  a->group = group;
  a->num_seqs = num_seqs;
  a->num_kv_heads = cache->num_kv_heads;
  a->num_blocks = cache->num_blocks;
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->max_context_len = max_context_len;
  a->part_tokens = part_tokens;
  a->num_parts = num_parts;
  return PA_OK;
}

// Split-K partials [S][Hq][P][2] and [S][Hq][P][D] (fp32), then the work list
// and its length, carved out of `workspace` (need > 0 only).
void decode_carve(pa::DecodeArgs* a, void* workspace, int32_t num_q_heads) {
  const int64_t rows = static_cast<int64_t>(a->num_seqs) * num_q_heads * a->num_parts;
  a->ws_ml = static_cast<float*>(workspace);
  a->ws_o = a->ws_ml + rows * 2;
  a->ws_items = reinterpret_cast<int32_t*>(a->ws_o + rows * a->head_dim);
  a->ws_count = a->ws_items + static_cast<int64_t>(a->num_seqs) * a->num_parts * 2;
}

}  // namespace

extern "C" {

int pa_decode(const pa_cache* cache, const void* q, void* out, int32_t num_seqs, int32_t num_q_heads,
              const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
              int32_t max_context_len, float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
              void* stream) {
  pa::DecodeArgs a{};
  size_t need = 0;
  bool nothing = false;
  int rc = decode_prepare(cache, q, out, num_seqs, num_q_heads, block_tables, max_blocks_per_seq, context_lens,
                          max_context_len, scale, partition_size, &a, &need, &nothing);
  if (rc != PA_OK || nothing) return rc;
  if (need > 0 && (!workspace || workspace_bytes < need)) return PA_EWORKSPACE;
  if (need > 0) decode_carve(&a, workspace, num_q_heads);
  return hip_status(pa::launch_decode(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Everything pa_prefill_chunk and pa_prefill_chunk_split check and derive
// before they touch the GPU; *nothing is set when there is no row to run.
int prefill_prepare(const pa_cache* cache, const void* q, void* out, const int32_t* cu_q_lens,
                    const int32_t* context_lens, int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                    const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t max_q_len,
                    int32_t max_context_len, float scale, pa::PrefillArgs* out_args, bool* nothing) {
  *nothing = false;
  int rc = check_cache(cache);
  if (rc != PA_OK) return rc;
  if (cache->dtype == PA_F32) return PA_EUNSUPPORTED;
  int32_t group = 0;
  if ((rc = check_group(cache, num_q_heads, &group)) != PA_OK) return rc;
  if ((rc = check_scale(scale)) != PA_OK) return rc;
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || max_context_len < 0 || max_blocks_per_seq <= 0)
    return PA_EINVAL;
  if (max_q_len > max_context_len) return PA_EINVAL;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * cache->block_size)
    return PA_EINVAL;
  if (num_seqs > kMaxGridYZ) return PA_EUNSUPPORTED;
  // the block-table entries of the longest context are staged in LDS
  if (pa::prefill_lds_bytes(cache->dtype, cache->head_dim, cache->block_size, max_context_len) > pa::kPrefillMaxLds)
    return PA_EUNSUPPORTED;
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0) {
    *nothing = true;
    return PA_OK;
  }
  if (!q || !out || !cu_q_lens || !context_lens || !block_tables) return PA_EINVAL;
  pa::PrefillArgs& a = *out_args;
  a = pa::PrefillArgs{};
  a.q = q;
  a.out = out;
  a.k_cache = cache->k_cache;
  a.v_cache = cache->v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.cu_q_lens = cu_q_lens;
  a.scale = scale;
  a.dtype = act_dtype(cache);  // the matrix type; FP8 codes are widened to it exactly
  if (is_fp8(cache)) {
    a.kv_fp8 = 1;
    a.k_scale = cache->k_scale;
    a.v_scale = cache->v_scale;
  }
  a.head_dim = cache->head_dim;
  a.block_size = cache->block_size;
  a.group = group;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.num_kv_heads = cache->num_kv_heads;
  a.num_blocks = cache->num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_q_len = max_q_len;
  a.max_context_len = max_context_len;
  return PA_OK;
}

size_t prefill_workspace(int32_t total_q, int32_t num_q_heads, int32_t head_dim, int32_t key_splits) {
  if (total_q <= 0 || num_q_heads <= 0 || head_dim <= 0 || key_splits <= 1) return 0;
  return static_cast<size_t>(total_q) * num_q_heads * key_splits * (head_dim + 2) * sizeof(float);
}

}  // namespace

extern "C" {

int pa_prefill_chunk(const pa_cache* cache, const void* q, void* out, const int32_t* cu_q_lens,
                     const int32_t* context_lens, int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                     const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t max_q_len,
                     int32_t max_context_len, float scale, void* stream) {
  pa::PrefillArgs a{};
  bool nothing = false;
  const int rc = prefill_prepare(cache, q, out, cu_q_lens, context_lens, num_seqs, total_q, num_q_heads,
                                 block_tables, max_blocks_per_seq, max_q_len, max_context_len, scale, &a, &nothing);
  if (rc != PA_OK || nothing) return rc;
  return hip_status(pa::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

int32_t pa_prefill_choose_splits(const pa_cache* cache, int32_t num_seqs, int32_t num_q_heads, int32_t max_q_len,
                                 int32_t max_context_len) {
  if (!cache || cache->num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0) return 1;
  return pa::prefill_choose_splits(num_seqs, cache->num_kv_heads, num_q_heads / cache->num_kv_heads, max_q_len,
                                   max_context_len);
}

size_t pa_prefill_workspace_bytes(int32_t total_q, int32_t num_q_heads, int32_t head_dim, int32_t key_splits) {
  return prefill_workspace(total_q, num_q_heads, head_dim, key_splits);
}

int pa_prefill_chunk_split(const pa_cache* cache, const void* q, void* out, const int32_t* cu_q_lens,
                           const int32_t* context_lens, int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                           const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t max_q_len,
                           int32_t max_context_len, float scale, int32_t key_splits, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (key_splits < 0) return PA_EINVAL;
  if (key_splits > pa::kPrefillMaxSplits) return PA_EUNSUPPORTED;
  pa::PrefillArgs a{};
  bool nothing = false;
  const int rc = prefill_prepare(cache, q, out, cu_q_lens, context_lens, num_seqs, total_q, num_q_heads,
                                 block_tables, max_blocks_per_seq, max_q_len, max_context_len, scale, &a, &nothing);
  if (rc != PA_OK || nothing) return rc;
  const int32_t k = key_splits == 0 ? pa::prefill_choose_splits(num_seqs, cache->num_kv_heads, a.group, max_q_len,
                                                                max_context_len)
                                    : key_splits;
  if (k > 1) {
    const size_t need = prefill_workspace(total_q, num_q_heads, cache->head_dim, k);
    if (!workspace || workspace_bytes < need) return PA_EWORKSPACE;
    a.key_splits = k;
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = a.ws_o + static_cast<size_t>(total_q) * num_q_heads * k * cache->head_dim;
  }
  return hip_status(pa::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

extern "C" {

size_t pa_decode_grouped_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                         int32_t max_context_len, int32_t partition_size) {
  const int32_t part = partition_size == 0 ? kGroupedSmallestDefault : partition_size;
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0 || part <= 0) return 0;
  return grouped_layout(num_seqs, num_q_heads, head_dim, max_context_len, part).total;
}

int pa_decode_grouped(const pa_cache* cache, const void* q, void* out, int32_t num_seqs, int32_t num_q_heads,
                      const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                      int32_t max_context_len, float scale, const int32_t* group_start, int32_t num_groups,
                      int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_cache(cache);
  if (rc != PA_OK) return rc;
  if (cache->dtype == PA_F32) return PA_EUNSUPPORTED;
  int32_t group = 0;
  if ((rc = check_group(cache, num_q_heads, &group)) != PA_OK) return rc;
  if ((rc = check_scale(scale)) != PA_OK) return rc;
  if (num_seqs < 0 || num_groups < 0 || max_blocks_per_seq <= 0 || max_context_len < 0) return PA_EINVAL;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * cache->block_size)
    return PA_EINVAL;
  const int32_t part = grouped_partition(partition_size, cache->block_size);
  if (part <= 0 || part % 32 != 0 || part % cache->block_size != 0 || part / cache->block_size > 64) return PA_EINVAL;
  if (num_seqs > pa::kGroupedMaxSeqs) return PA_EUNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!q || !out || !block_tables || !context_lens || (num_groups > 0 && !group_start)) return PA_EINVAL;
  const GroupedLayout L = grouped_layout(num_seqs, num_q_heads, cache->head_dim, max_context_len, part);
  // the merge keeps the slot weights of one KV head's q heads in LDS
  if (static_cast<int64_t>(group) * L.slots * sizeof(float) > kGroupedMergeLds) return PA_EUNSUPPORTED;
  if (!workspace || workspace_bytes < L.total) return PA_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);

  pa::GroupedArgs g{};
  pa::DecodeArgs& a = g.d;
  a.q = q;
  a.out = out;
  a.k_cache = cache->k_cache;
  a.v_cache = cache->v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.ws_ml = reinterpret_cast<float*>(ws + L.ml);
  a.ws_o = reinterpret_cast<float*>(ws + L.o);
  a.ws_items = reinterpret_cast<int32_t*>(ws + L.suf_items);
  a.ws_count = reinterpret_cast<int32_t*>(ws + L.counts);
  a.scale = scale;
  if (is_fp8(cache)) {
    a.k_scale = cache->k_scale;
    a.v_scale = cache->v_scale;
  }
  a.dtype = cache->dtype;
  a.act_dtype = act_dtype(cache);
  a.head_dim = cache->head_dim;
  a.block_size = cache->block_size;
  a.group = group;
  a.num_seqs = num_seqs;
  a.num_kv_heads = cache->num_kv_heads;
  a.num_blocks = cache->num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.part_tokens = part;
  a.num_parts = static_cast<int32_t>(L.slots);
  g.group_start = num_groups > 0 ? group_start : nullptr;
  g.num_groups = num_groups;
  g.seq_start = reinterpret_cast<int32_t*>(ws + L.seq_start);
  g.slot_base = reinterpret_cast<int32_t*>(ws + L.slot_base);
  g.nslots = reinterpret_cast<int32_t*>(ws + L.nslots);
  g.pre_items = reinterpret_cast<int32_t*>(ws + L.pre_items);
  g.pre_count = a.ws_count + 1;
  return hip_status(pa::launch_decode_grouped(g, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- split decode without a caller workspace ----------------------------------------
//
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid allocation): pa_decode with its
// split-K partials and work list in a fixed device array of kScratchBytes
// instead of a caller workspace.  Each device the library runs on holds its
// own copy of the array from the first such call until the process ends; its
// address on a device is looked up once, with that device current, and kept.
// Calls that overlap on one device share the array and race.  Nothing in it
// has to start at zero: the planner writes the work list and its length before
// the walk reads them, and every partial is written before the merge reads it.
namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kScratchMaxDev = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchMaxDev];  // address of `scratch` on each device (null until looked up)
thread_local char g_refusal[192];

int refuse(int status, const char* fmt, long long a, long long b) {
  std::snprintf(g_refusal, sizeof(g_refusal), fmt, a, b);
  g_last_hip_error = g_refusal;
  return status;
}

// Device address of the array on the current device, which must be the
// stream's.
int scratch_of_current_device(void* stream, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kScratchMaxDev)
    return refuse(PA_EUNSUPPORTED, "pa_decode_noalloc: device %lld is beyond the %lld devices it keeps", dev,
                  kScratchMaxDev);
  if (stream) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return hip_status(e);
    if (sdev != dev)
      return refuse(PA_EINVAL, "pa_decode_noalloc: the stream is on device %lld, the current device is %lld",
                    sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return refuse(PA_EHIP, "pa_decode_noalloc: no address for the scratch array on device %lld%lld", dev, 0);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_decode_noalloc(const pa_cache* cache, const void* q, void* out, int32_t num_seqs, int32_t num_q_heads,
                      const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                      int32_t max_context_len, float scale, int32_t partition_size, void* stream) {
  pa::DecodeArgs a{};
  size_t need = 0;
  bool nothing = false;
  int rc = decode_prepare(cache, q, out, num_seqs, num_q_heads, block_tables, max_blocks_per_seq, context_lens,
                          max_context_len, scale, partition_size, &a, &need, &nothing);
  if (rc != PA_OK || nothing) return rc;
  if (need > kScratchBytes)
    return refuse(PA_EWORKSPACE, "pa_decode_noalloc: the split needs %lld bytes of scratch, the fixed array holds %lld",
                  static_cast<long long>(need), static_cast<long long>(kScratchBytes));
  if (need > 0) {
    void* ws = nullptr;
    if ((rc = scratch_of_current_device(stream, &ws)) != PA_OK) return rc;
    decode_carve(&a, ws, num_q_heads);
  }
  return hip_status(pa::launch_decode(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
