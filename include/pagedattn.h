/*
 * pagedattn.h — C ABI of the paged KV-cache attention library (gfx950).
 *
 * The operation (PagedAttention, as the pages describe it): the KV cache is
 * cut into fixed-size physical blocks of `block_size` token slots drawn from
 * one global pool; each sequence keeps a block table mapping its logical
 * blocks to physical ones; decode appends the current token's K/V to the
 * cache and then attends over the whole context read block by block through
 * the table; chunked prefill attends a chunk of new tokens causally over the
 * cached context plus itself; identical prefixes share read-only blocks and
 * are copied on write.  Sources: lshu.cn/news/11644, "方案：页式内存管理",
 * "收益分析" and "性能关键路径与瓶颈"; zzmblog.top vLLM guide,
 * "Transformer推理与KV缓存" and "PagedAttention核心设计"; 5x10.cn/post/462,
 * "分块预填充".
 *
 * Conventions for every call
 *  - Pointers marked "device" are HIP device (or managed) memory; "host"
 *    pointers are ordinary CPU memory.  The caller owns every buffer; the
 *    library keeps no caller pointer after a call returns and allocates
 *    nothing (pa_decode_noalloc's fixed scratch array, below, is part of the
 *    library's code object).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Device calls are asynchronous on that stream; a call returns once its
 *    kernels are enqueued.  Calls hold no global state and may be issued
 *    from several host threads.
 *  - Arguments the host can see are validated before anything is launched:
 *    PA_EINVAL (bad pointer/size/range), PA_EUNSUPPORTED (a shape outside
 *    the compiled instances), PA_EWORKSPACE (workspace too small).  Then
 *    nothing is enqueued.  PA_EHIP reports a failed launch.
 *  - Device-resident metadata (slot ids, block tables, context lengths,
 *    copy pairs) is trusted, but never used as an address when out of range:
 *    such slots and copy pairs are skipped, such block ids replaced by block
 *    0 and lengths clamped to the host bounds; the result for that
 *    token/sequence is then undefined, and nothing faults.
 *  - Compiled instances: dtype {f32, f16, bf16} x head_dim {64, 128} x
 *    block_size {8, 16, 32, 64} (zzmblog.top vLLM guide, "核心参数调优":
 *    larger blocks for long contexts, 8 for many short sequences);
 *    num_q_heads a multiple of num_kv_heads with group size
 *    num_q_heads/num_kv_heads in {1, 2, 4, 8}.  pa_prefill_chunk needs f16
 *    or bf16 (its contractions run on the matrix cores); pa_decode_grouped
 *    needs f16 or bf16 (any of the block sizes).  An FP8 pool (see pa_cache)
 *    has head_dim 128, block_size 16..64 and f16 or bf16 activations, and is
 *    supported by pa_kv_append, pa_copy_blocks, pa_decode,
 *    pa_prefill_chunk and pa_decode_grouped.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 } pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_EINVAL = 1,
  PA_EUNSUPPORTED = 2,
  PA_EWORKSPACE = 3,
  PA_ENOMEM = 4, /* block manager: the free pool cannot cover the request */
  PA_EHIP = 5
} pa_status;

/* The paged pool (the pages leave the layout open).  Two device arrays in
 * `dtype`, each made of one contiguous tile per (block, KV head):
 *   k_cache  [num_blocks][num_kv_heads][block_size][head_dim]  (token rows)
 *   v_cache  [num_blocks][num_kv_heads][head_dim][block_size]  (V transposed
 *            inside the tile, so the PV contraction reads keys contiguously)
 * Token slot s lives in block s / block_size at position s % block_size.
 *
 * FP8 pool (dtype PA_FP8_E4M3; lshu.cn/news/11644, "性能关键路径与瓶颈":
 * quantising the KV cache halves what decode reads): elements are one-byte
 * codes of the OCP E4M3 format without infinities (bias 7, 3 mantissa bits,
 * largest finite 448, S.1111.111 = NaN).  q, out and the K/V rows given to
 * pa_kv_append are in `act_dtype` (PA_F16 or PA_BF16); a stored code is the
 * nearest E4M3 value to x * (1 / scale) -- the reciprocal and the product in
 * fp32 -- ties to the even code, magnitudes past 448 saturating, and its
 * value is code * scale, with `k_scale` for K and `v_scale` for V (positive
 * and finite).  For the other dtypes act_dtype, k_scale and v_scale are
 * ignored (a zero-initialised descriptor stays valid). */
typedef struct {
  void* k_cache;
  void* v_cache;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t head_dim;
  int32_t dtype;     /* pa_dtype of the pool's elements */
  int32_t act_dtype; /* FP8 pool: pa_dtype of q, out and appended rows */
  float k_scale;     /* FP8 pool: value = code * scale */
  float v_scale;
} pa_cache;

/* Write new tokens' K/V into their cache slots (decode appends the current
 * token before attending: zzmblog.top vLLM guide, "Transformer推理与KV缓存";
 * lshu.cn/news/11644, "方案：页式内存管理", the append rule).
 *   k_new, v_new  device [num_tokens][num_kv_heads][head_dim] in the
 *                 activation type (the pool's dtype; act_dtype for an FP8
 *                 pool, whose rows are quantised as pa_cache describes)
 *   slot_mapping  device int64 [num_tokens]; slot < 0 skips the token
 * Slots of one call must be distinct. */
int pa_kv_append(const pa_cache* cache, const void* k_new, const void* v_new,
                 const int64_t* slot_mapping, int32_t num_tokens, void* stream);

/* Copy-on-write of shared prefix blocks (lshu.cn/news/11644, "收益分析":
 * identical prompts share read-only physical blocks; a later divergence is
 * handled by copy-on-write).  For each pair (src, dst), in order, the whole
 * K and V tiles of block src (all heads, all slots) are copied to block dst.
 *   pairs  device int32 [num_pairs][2] = (src, dst)
 * A dst must not appear as a src or dst of another pair of the same call. */
int pa_copy_blocks(const pa_cache* cache, const int32_t* pairs, int32_t num_pairs, void* stream);

/* Bytes of device workspace pa_decode needs for split-K partitions
 * (0 when partition_size == 0). */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size);

/* Paged decode attention: one query token per sequence attends over its
 * whole context read through its block table (lshu.cn/news/11644,
 * "方案：页式内存管理": the kernel reads the scattered blocks of a request
 * through its block table as one logical K/V sequence; "性能关键路径与瓶颈":
 * decode is bound by reading the KV cache).
 *   q, out          device [num_seqs][num_q_heads][head_dim] in the
 *                   activation type (act_dtype for an FP8 pool);
 *                   q head h reads KV head h / (num_q_heads / num_kv_heads)
 *   block_tables    device int32 [num_seqs][max_blocks_per_seq]
 *   context_lens    device int32 [num_seqs]; counts the token appended this
 *                   step; 0 gives a zero output row
 *   max_context_len host bound on every context_lens entry
 *                   (<= max_blocks_per_seq * block_size)
 *   scale           softmax scale (usually 1/sqrt(head_dim))
 *   partition_size  0 = one pass per (sequence, KV head); otherwise a
 *                   multiple of block_size: the context is split into
 *                   partitions of that many tokens whose softmax states are
 *                   merged by log-sum-exp; -1 lets the library choose from
 *                   the shape (pa_decode_choose_partition).  Split decode runs
 *                   three kernels on `stream`: a one-workgroup planner lists
 *                   the (sequence, partition) pairs that hold tokens, a
 *                   device-sized grid walks that list, and a merge kernel
 *                   combines each row's partitions
 *   workspace       device scratch of at least pa_decode_workspace_bytes()
 *                   for the partition size actually used (may be NULL when
 *                   that is 0; for -1, pa_decode_workspace_bytes(..., -1)
 *                   covers every choice): partial states, the work list and
 *                   its length, all rewritten by each call, so calls that
 *                   share a workspace must be ordered on one stream
 * Output is rounded to the activation type (round to nearest even).  With
 * an FP8 pool the codes are widened exactly and the scales applied in fp32
 * (k_scale folded into the softmax scale, v_scale into the normalisation). */
int pa_decode(const pa_cache* cache, const void* q, void* out, int32_t num_seqs, int32_t num_q_heads,
              const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
              int32_t max_context_len, float scale, int32_t partition_size, void* workspace,
              size_t workspace_bytes, void* stream);

/* The partition size pa_decode uses for partition_size == -1 (host only):
 * 0 (one pass) for short contexts, or for contexts up to 4096 tokens when
 * the batch has at least 512 (sequence, KV head) units; otherwise a power of
 * two from 512 up to 2048 tokens (up to 16384 when there are fewer than 512
 * units, i.e. a few long contexts), the largest that still yields about
 * 1024 (512) work items. */
int32_t pa_decode_choose_partition(const pa_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t max_context_len);

/* pa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments, kernels and result as pa_decode, but no workspace
 * argument -- a split keeps its partial states and work list in a fixed
 * device array of 32 MiB (33554432 bytes) inside the library.  Each device
 * the library runs on holds its own copy of that array from the first call
 * on it until the process ends; the call itself allocates nothing.
 *   stream  must belong to the current device (else PA_EINVAL)
 * A split whose pa_decode workspace would exceed the array returns
 * PA_EWORKSPACE before anything is enqueued (pa_last_error() then states
 * the bytes needed and the limit); one-pass decodes need no scratch.  Every
 * call on a device shares that device's array and leaves its contents
 * behind: calls that overlap on one device (several streams, or several
 * host threads) race and must be ordered by the caller.  Nothing in the
 * array has to start at zero. */
int pa_decode_noalloc(const pa_cache* cache, const void* q, void* out, int32_t num_seqs, int32_t num_q_heads,
                      const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                      int32_t max_context_len, float scale, int32_t partition_size, void* stream);

/* Bytes of device workspace pa_decode_grouped needs (partition_size as
 * passed to it; 0 = the default, sized for the smaller default of 8-token
 * blocks, so it covers every block size). */
size_t pa_decode_grouped_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                         int32_t max_context_len, int32_t partition_size);

/* Prefix-grouped decode: the same result as pa_decode, but blocks that
 * several sequences of the batch share (forks of one prompt keep its blocks
 * read-only until copy-on-write: lshu.cn/news/11644, "收益分析") are read
 * once for all of them -- prefix caching within the batch, which the same
 * page counts among the decode-side savings ("性能关键路径与瓶颈").
 * Arguments as for pa_decode, f16 or bf16 caches, plus:
 *   group_start     device int32 [num_groups + 1]: sequences
 *                   group_start[g] .. group_start[g+1]-1 are likely to share
 *                   a prefix (e.g. forks of one prompt).  A hint only: the
 *                   library cuts the batch into runs at these starts, splits
 *                   runs into chunks of at most 32 / (num_q_heads /
 *                   num_kv_heads) sequences, and measures on the block
 *                   tables how many leading full blocks each sequence has in
 *                   common with its chunk's longest sequence; any grouping
 *                   (NULL with num_groups 0 included) gives the same result
 *   partition_size  0 = 1024 (512 for 8-token blocks); else a multiple of
 *                   32 and of block_size, at most 64 blocks: tokens per
 *                   partition of both the shared prefix and each sequence's
 *                   own suffix
 *   workspace       device scratch of at least
 *                   pa_decode_grouped_workspace_bytes(); rewritten by each
 *                   call, so calls sharing it must be ordered on one stream
 * PA_EUNSUPPORTED above 4096 sequences, or when (num_q_heads /
 * num_kv_heads) * 2 * ceil(max_context_len / partition) exceeds 14336 (the
 * merge's per-head slot weights live in 56 KiB of LDS; with 1024-token
 * partitions that is 917504 tokens of context at 8 q heads per KV head).  Runs four kernels
 * on `stream`: a one-workgroup planner, the shared-prefix kernel (matrix
 * cores, one chunk's rows per workgroup), the suffix partitions of the split
 * decode kernel, and the log-sum-exp merge. */
int pa_decode_grouped(const pa_cache* cache, const void* q, void* out, int32_t num_seqs, int32_t num_q_heads,
                      const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                      int32_t max_context_len, float scale, const int32_t* group_start, int32_t num_groups,
                      int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream);

/* Chunked-prefill attention (5x10.cn/post/462, "分块预填充"; lshu.cn/news/11644,
 * "整体架构": long prompts are split into chunks over several iterations and
 * batched with decode tokens).  Sequence s has n_s = cu_q_lens[s+1] -
 * cu_q_lens[s] query rows, already appended to its cache, so its context has
 * context_lens[s] >= n_s tokens; row i sits at position
 * context_lens[s] - n_s + i and attends keys 0..that position (causal).
 *   q, out        device [total_q][num_q_heads][head_dim], f16 or bf16
 *   cu_q_lens     device int32 [num_seqs + 1], cu_q_lens[0] = 0,
 *                 cu_q_lens[num_seqs] = total_q
 *   context_lens  device int32 [num_seqs]
 *   max_q_len, max_context_len  host bounds of n_s and context_lens
 * A workgroup stages its sequence's block-table entries in LDS beside its
 * K/V tile buffers (159 KiB in all), so contexts whose table does not fit
 * return PA_EUNSUPPORTED: the longest accepted is 364,544 tokens at
 * block_size 16 and head_dim 128.  With an FP8 pool the codes are widened
 * exactly to the activation type as the K/V tiles are staged, and the
 * scales enter in fp32 (k_scale folded into the softmax scale, v_scale into
 * the normalisation); the output is rounded to the activation type. */
int pa_prefill_chunk(const pa_cache* cache, const void* q, void* out, const int32_t* cu_q_lens,
                     const int32_t* context_lens, int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                     const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t max_q_len,
                     int32_t max_context_len, float scale, void* stream);

/* Chunked prefill as pa_prefill_chunk, with each workgroup's keys split into
 * key_splits ranges run by workgroups of their own, whose partial results
 * (per row: output unnormalised, running max, sum) are combined by
 * log-sum-exp -- the merge of split-K decode (partial results over disjoint
 * key sets combine exactly) -- in a second kernel.  A batch of few chunks
 * otherwise occupies few compute units (a workgroup takes 256 rows of one KV
 * head: one 512-token chunk at 4 q heads per KV head and 8 KV heads is 64
 * workgroups); the split spreads it over the chip.
 *   key_splits    1..8; 1 runs pa_prefill_chunk (no workspace needed); 0
 *                 takes pa_prefill_choose_splits()
 *   workspace     device, 16-byte aligned, at least
 *                 pa_prefill_workspace_bytes(total_q, num_q_heads, head_dim,
 *                 key_splits) bytes (fp32 partials); rewritten by each call,
 *                 so calls sharing it must be ordered on one stream
 * Errors as pa_prefill_chunk, plus PA_EINVAL for key_splits < 0,
 * PA_EUNSUPPORTED above 8 and PA_EWORKSPACE for a missing or short
 * workspace, all before anything is enqueued.  Outputs equal
 * pa_prefill_chunk's up to the rounding of the merge. */
int pa_prefill_chunk_split(const pa_cache* cache, const void* q, void* out, const int32_t* cu_q_lens,
                           const int32_t* context_lens, int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                           const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t max_q_len,
                           int32_t max_context_len, float scale, int32_t key_splits, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Key splits the library takes for a prefill batch (host arithmetic only):
 * 1 when the batch gives 256 workgroups (one per compute unit) or more,
 * otherwise enough to reach that, at most 8 and keeping at least 4 key tiles
 * of 64 keys per range of the longest context. */
int32_t pa_prefill_choose_splits(const pa_cache* cache, int32_t num_seqs, int32_t num_q_heads, int32_t max_q_len,
                                 int32_t max_context_len);

/* Workspace bytes of pa_prefill_chunk_split: total_q * num_q_heads *
 * key_splits * (head_dim + 2) floats; 0 for key_splits <= 1. */
size_t pa_prefill_workspace_bytes(int32_t total_q, int32_t num_q_heads, int32_t head_dim, int32_t key_splits);

const char* pa_status_str(int status);

/* HIP's text for the calling thread's most recent PA_EHIP, or the reason of
 * pa_decode_noalloc's most recent refusal ("" if none); valid until the
 * thread's next call into the library. */
const char* pa_last_error(void);

/* ---- checking build ------------------------------------------------------
 * libpagedattn_debug.so is this library compiled with PA_DEBUG.  Its kernels
 * behave as the product's and also count, in counters each device holds,
 * the device metadata that the trust rule above has them clamp or skip:
 *   PA_DBG_BLOCK_ID     a block-table entry inside a sequence's length that
 *                       is outside [0, num_blocks) (read as block 0)
 *   PA_DBG_CONTEXT_LEN  a context length outside [0, max_context_len), or,
 *                       in pa_prefill_chunk, shorter than its query rows
 *   PA_DBG_SLOT         pa_kv_append: a slot >= num_blocks * block_size
 *                       (skipped; a negative slot is the documented skip
 *                       and is not counted)
 *   PA_DBG_COPY_PAIR    pa_copy_blocks: a pair whose src or dst is outside
 *                       [0, num_blocks) (skipped)
 * Slots and pairs are counted once each; the attention kinds count the
 * lanes that met the case, a figure that depends on the launch shape, so
 * zero versus nonzero is what they tell.
 * pa_debug_counters waits for the current device to go idle, writes the
 * counters of that device into counts (host uint64 [PA_DBG_KINDS]) and, when
 * reset is nonzero, clears them.  PA_EINVAL for a NULL counts; the product
 * library returns PA_EUNSUPPORTED and writes nothing. */
typedef enum {
  PA_DBG_BLOCK_ID = 0,
  PA_DBG_CONTEXT_LEN = 1,
  PA_DBG_SLOT = 2,
  PA_DBG_COPY_PAIR = 3,
  PA_DBG_KINDS = 4
} pa_debug_kind;
int pa_debug_counters(uint64_t* counts, int32_t reset);

/* ---- host block manager (CPU only, no HIP calls) -------------------------
 * Bookkeeping of the paged cache (lshu.cn/news/11644, "方案：页式内存管理" and
 * "收益分析"): one global pool; a FIFO free pool (blocks handed out from the
 * front, returned to the back); a per-sequence block table; a new block only
 * when the last one is full; all blocks returned when a sequence is freed;
 * forks share the parent's blocks read-only with reference counts, and the
 * first write into a block held by more than one sequence first moves the
 * writer to a fresh block and emits a (shared, fresh) copy pair.
 * Sequence ids are caller-chosen int32 values.  Not thread-safe per handle. */
typedef struct pa_bm pa_bm;

/* free_order: host int32 [free_len], the pool's initial free list, front
 * first; blocks not listed are never handed out (e.g. a poison block that
 * table padding points at).  NULL = 0..num_blocks-1.  Returns NULL on bad
 * arguments. */
pa_bm* pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order, int32_t free_len);
void pa_bm_destroy(pa_bm* bm);
int pa_bm_add_seq(pa_bm* bm, int32_t seq);
/* child shares parent's first ceil(keep/block_size) blocks; keep <= parent length */
int pa_bm_fork(pa_bm* bm, int32_t parent, int32_t child, int32_t keep);
/* Grow `seq` by n_tokens: slots_out host int64 [n_tokens]; cow_pairs_out
 * host int32 [cow_cap][2]; *n_cow_out pairs written.  All-or-nothing:
 * PA_ENOMEM leaves the state unchanged. */
int pa_bm_append(pa_bm* bm, int32_t seq, int32_t n_tokens, int64_t* slots_out, int32_t* cow_pairs_out,
                 int32_t cow_cap, int32_t* n_cow_out);
/* pa_bm_append for num_seqs sequences in order, slots concatenated in that
 * order (the step's slot mapping) and copy pairs concatenated.  Stops at the
 * first failure; *n_done_out tells how many sequences were appended. */
int pa_bm_append_batch(pa_bm* bm, const int32_t* seqs, const int32_t* n_tokens, int32_t num_seqs,
                       int64_t* slots_out, int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow_out,
                       int32_t* n_done_out);
int pa_bm_free_seq(pa_bm* bm, int32_t seq);
/* Table of one sequence: out host int32 [cap]; *len_out = blocks held. */
int pa_bm_table(const pa_bm* bm, int32_t seq, int32_t* out, int32_t cap, int32_t* len_out);
/* Padded tables of several sequences: out host int32 [num_seqs][max_blocks],
 * entries past a table's end set to pad_block; lens_out host int32
 * [num_seqs] (may be NULL) receives the sequences' token counts. */
int pa_bm_tables(const pa_bm* bm, const int32_t* seqs, int32_t num_seqs, int32_t* out, int32_t max_blocks,
                 int32_t pad_block, int32_t* lens_out);
int pa_bm_seq_len(const pa_bm* bm, int32_t seq, int32_t* len_out);
int32_t pa_bm_num_free(const pa_bm* bm);
/* The free list front first: out host int32 [cap]; returns entries written. */
int32_t pa_bm_free_list(const pa_bm* bm, int32_t* out, int32_t cap);
/* Reference count of a block (0 when free or never handed out). */
int32_t pa_bm_refcount(const pa_bm* bm, int32_t block);

/* Pool occupancy, for the memory-waste figure the pages compare against
 * static reservation (lshu.cn/news/11644, "问题：KV Cache 的内存困境" and
 * "收益分析"; m.ypxx.net, "2.1 PagedAttention分页注意力核心机制": paged
 * blocks leave at most a partly filled last block per sequence).
 * blocks_in_use: blocks with a nonzero reference count; slots_filled: over
 * those blocks, the slots holding tokens (a block shared by several
 * sequences counts the most any of them has written into it).  Internal
 * waste = 1 - slots_filled / (blocks_in_use * block_size). */
int pa_bm_usage(const pa_bm* bm, int64_t* blocks_in_use, int64_t* slots_filled);

/* ---- host scheduler loop (CPU only, no HIP calls) --------------------------
 * One call of pa_sched_step is one iteration of the centralized scheduler
 * (lshu.cn/news/11644, "整体架构": check the free pool, pull waiting requests,
 * allocate blocks, prefill long prompts in chunks over several iterations,
 * batch every running request's current token, and free a finished
 * request's blocks at once), over a block manager the caller owns.  Request
 * ids are sequence ids of that manager (>= 0, unused there).  Conventions:
 * a token budget per iteration; decode tokens first (oldest admission
 * first), then the next chunk of prompts being prefilled, then new requests
 * in arrival order; a chunk is bounded by the prompt's remainder, the budget
 * left and the pool's room; a decode token that finds the pool empty
 * preempts the newest running request not yet scheduled in the iteration
 * (freed, put back at the front of the queue, prefilled again from its
 * first token); the iteration that caches a prompt's last token yields the
 * first new token, each decode one more; a request that has produced
 * max_new_tokens finishes and its blocks are freed by the next call.  The
 * caller runs each batch's kernels (append, then prefill / decode) before
 * the next call, on one stream. */
typedef struct pa_sched pa_sched;

typedef struct {
  int32_t num_decode;    /* reqs[0 .. num_decode-1]: one token each */
  int32_t num_prefill;   /* reqs[num_decode ..]: prompt chunks of n_new tokens */
  int64_t num_slots;     /* slots[]: the batch's tokens in batch order */
  int32_t num_pairs;     /* copy pairs (none without forks) */
  int32_t num_finished;  /* requests whose last token this batch yields */
  int32_t num_preempted; /* requests sent back to the queue */
} pa_sched_batch;

/* NULL on bad arguments.  `bm` must outlive the scheduler. */
pa_sched* pa_sched_create(pa_bm* bm, int32_t max_batched_tokens, int32_t max_running);
void pa_sched_destroy(pa_sched* s);
/* Queue a request (arrival order = call order). */
int pa_sched_add(pa_sched* s, int32_t req, int32_t prompt_len, int32_t max_new_tokens);
/* Requests not yet finished (queued or running). */
int32_t pa_sched_unfinished(const pa_sched* s);
/* One iteration.  Host outputs: reqs / n_new [cap >= min(requests,
 * max_running)], slots [slot_cap >= max_batched_tokens], pairs [pair_cap]
 * (may be NULL with pair_cap 0), finished / preempted [list_cap >= requests
 * added].  PA_EINVAL (too small) before any state changes. */
int pa_sched_step(pa_sched* s, int32_t* reqs, int32_t* n_new, int32_t cap, int64_t* slots, int64_t slot_cap,
                  int32_t* pairs, int32_t pair_cap, int32_t* finished, int32_t* preempted, int32_t list_cap,
                  pa_sched_batch* out);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
