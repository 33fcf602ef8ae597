// Internal launch interface between the C ABI layer (api.hip) and the
// kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct DecodeArgs {
  const void* q;
  void* out;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_ml;  // [S][Hq][num_parts][2]  (max in log2 units, sum of weights)
  float* ws_o;   // [S][Hq][num_parts][D]  normalised partial outputs
  int32_t* ws_items;  // [S * num_parts][2]  (sequence, partition) work list
  int32_t* ws_count;  // [1]  entries in ws_items
  float scale;
  float k_scale = 1.f, v_scale = 1.f;  // FP8 pool scales (1 otherwise)
  int32_t dtype, head_dim, block_size, group;
  int32_t act_dtype;  // q / out type: dtype, or F16 / BF16 for an FP8 pool
  int32_t num_seqs, num_kv_heads, num_blocks, max_blocks_per_seq;
  int32_t max_context_len;  // host bound; device lengths are clamped to it
  int32_t part_tokens;  // tokens per partition (multiple of block_size)
  int32_t num_parts;    // ceil(max_context_len / part_tokens); grouped: workspace slots per row
};

// Prefix-grouped decode (grouped.hip): a planner, one persistent kernel for
// the shared-prefix and suffix items, and a merge kernel.
struct GroupedArgs {
  DecodeArgs d;                // num_parts = slots per row; ws_items / ws_count = suffix list
  const int32_t* group_start;  // [num_groups + 1] hint: runs of sequences that may share a prefix
  int32_t num_groups;
  int32_t* seq_start;   // [S]  shared tokens of each sequence (its own part starts there)
  int32_t* slot_base;   // [S]  prefix slots of its chunk
  int32_t* nslots;      // [S]
  int32_t* pre_items;   // [S * ceil(max_context / part) / 2][8]  (first member, members, partition, reference, shared length)
  int32_t* pre_count;   // [1]
};

// Sequences one grouped-decode planner workgroup can hold in LDS.
constexpr int32_t kGroupedMaxSeqs = 4096;

hipError_t launch_decode_grouped(const GroupedArgs& a, hipStream_t st);

struct PrefillArgs {
  const void* q;
  void* out;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_q_lens;
  float scale;
  int32_t dtype, head_dim, block_size, group;
  int32_t num_seqs, total_q, num_kv_heads, num_blocks, max_blocks_per_seq;
  int32_t max_q_len, max_context_len;
  // FP8 pool: dtype above is the activation type; the pool holds E4M3 codes
  // that mean code * k_scale (K) and code * v_scale (V)
  int32_t kv_fp8 = 0;
  float k_scale = 1.f, v_scale = 1.f;
  // key split: each row tile's key tiles in key_splits ranges, whose
  // partials (ws_o: [total_q * Hq][key_splits][head_dim] unnormalised,
  // ws_ml: [.][key_splits][2] running max in log2 units and sum) a second
  // kernel merges by log-sum-exp; 1 = no split, no workspace
  int32_t key_splits = 1;
  float* ws_o = nullptr;
  float* ws_ml = nullptr;
};

hipError_t launch_kv_append(const void* k_new, const void* v_new, const int64_t* slots, int32_t num_tokens,
                            void* k_cache, void* v_cache, int32_t num_blocks, int32_t num_kv_heads,
                            int32_t block_size, int32_t head_dim, int32_t elem_bytes, hipStream_t st);

// Append into an FP8 pool: rows of act_dtype (F16 / BF16) quantised with the
// fp32 reciprocals of the scales.
hipError_t launch_kv_append_fp8(const void* k_new, const void* v_new, const int64_t* slots, int32_t num_tokens,
                                void* k_cache, void* v_cache, int32_t num_blocks, int32_t num_kv_heads,
                                int32_t block_size, int32_t head_dim, int32_t act_dtype, float k_inv, float v_inv,
                                hipStream_t st);

hipError_t launch_copy_blocks(const int32_t* pairs, int32_t num_pairs, void* k_cache, void* v_cache,
                              int32_t num_blocks, int64_t block_bytes, hipStream_t st);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st);

// Key splits of chunked prefill: at most kPrefillMaxSplits; the library's
// choice spreads a batch of few row tiles over about kPrefillTargetItems
// workgroups (one per compute unit), each range keeping >= 4 key tiles.
constexpr int32_t kPrefillMaxSplits = 8;
constexpr int64_t kPrefillTargetItems = 256;
int32_t prefill_choose_splits(int32_t num_seqs, int32_t num_kv_heads, int32_t group, int32_t max_q_len,
                              int32_t max_context_len);

// Dynamic LDS one chunked-prefill workgroup needs: two K/V tile stages plus
// the block-table entries of every key tile (bound by max_context_len).  The
// bound leaves 1 KiB of the 160 KiB for the kernel's static LDS.
constexpr size_t kPrefillMaxLds = 159 * 1024;
size_t prefill_lds_bytes(int32_t dtype, int32_t head_dim, int32_t block_size, int32_t max_context_len);

#ifdef PA_DEBUG
// Checking build: each kernel unit's counters (common.h, PA_DEBUG_UNIT),
// added into acc[PA_DBG_KINDS] on the current device, then cleared if reset.
hipError_t debug_counts_decode(unsigned long long* acc, bool reset);
hipError_t debug_counts_grouped(unsigned long long* acc, bool reset);
hipError_t debug_counts_prefill(unsigned long long* acc, bool reset);
hipError_t debug_counts_kv_cache_ops(unsigned long long* acc, bool reset);
#endif

}  // namespace pa
