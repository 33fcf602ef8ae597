// Data movement into the paged pool: token append through a slot mapping
// (quantising to E4M3 codes for an FP8 pool), and whole-block copies for
// copy-on-write.
//
// Append (zzmblog.top vLLM guide, "Transformer推理与KV缓存"; lshu.cn/news/11644,
// "方案：页式内存管理"): token t's K and V rows ([num_kv_heads][head_dim]) go
// to block slot_mapping[t] / block_size, row slot_mapping[t] % block_size of
// every head's tile.  Copy (lshu.cn/news/11644, "收益分析"): a shared block
// about to be written is duplicated whole into a fresh block first.
//
// Pool layout: K tiles are [block_size][head_dim] (token rows), V tiles are
// [head_dim][block_size] (V kept transposed inside each block, so the PV
// contraction reads keys contiguously).  Both are HBM streams: source rows
// are read in 16-byte chunks, a wavefront covering 1 KiB of consecutive
// source bytes per instruction.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

// One workgroup per (run of kAppendTok consecutive tokens, KV head).  K
// rows are token rows of the tile, so each 16-byte chunk of a source row is
// stored whole.  V goes to the transposed tile, where a token is one element
// of each of head_dim rows: the run's V rows are staged in LDS and written
// back column by column, consecutive lanes taking consecutive tokens of one
// head_dim row.  Tokens with consecutive slots in a block (a prompt chunk, a
// long context being filled) then land in one contiguous span of each row
// per store instruction instead of one element per cache line; scattered
// slots (one decode token per sequence) are no worse than element stores.
constexpr int kAppendTok = 16;
constexpr int kAppendMaxDim = 128;

template <typename E>
__global__ __launch_bounds__(256) void kv_append_kernel(const E* __restrict__ k_new, const E* __restrict__ v_new,
                                                        const int64_t* __restrict__ slots, int num_tokens,
                                                        int head_dim, int num_kv_heads, int block_size,
                                                        int64_t num_slots, E* __restrict__ kc, E* __restrict__ vc) {
  constexpr int VEC = 16 / sizeof(E);
  constexpr int PITCH = kAppendMaxDim + VEC;  // LDS row pitch (elements): 16-byte aligned rows
  __shared__ __attribute__((aligned(16))) E vs[kAppendTok][PITCH];
  __shared__ int64_t sl[kAppendTok];
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * kAppendTok;
  const int tid = threadIdx.x;
  const int cpr = head_dim / VEC;  // 16-byte chunks per row
  if (tid < kAppendTok) {
    const int t = t0 + tid;
    const int64_t slot = t < num_tokens ? slots[t] : -1;
    PA_DEBUG_COUNT(PA_DBG_SLOT, h == 0 && slot >= num_slots);
    sl[tid] = (slot >= 0 && slot < num_slots) ? slot : -1;
  }
  // K needs no exchange: each thread reads its token's slot itself, so the
  // slot, K and V loads are in flight together (sl[] serves the V phase)
  for (int c = tid; c < kAppendTok * cpr; c += blockDim.x) {
    const int r = c / cpr, cc = c - r * cpr;
    const int t = t0 + r;
    if (t >= num_tokens) continue;
    const int64_t src = (static_cast<int64_t>(t) * num_kv_heads + h) * head_dim + cc * VEC;
    const int64_t slot = slots[t];
    const u32x4 kv = load16(k_new + src);
    store16(&vs[r][cc * VEC], load16(v_new + src));
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t tile = (slot / block_size) * num_kv_heads + h;  // (block, head) tile index
    store16(kc + (tile * block_size + slot % block_size) * head_dim + cc * VEC, kv);
  }
  __syncthreads();
  for (int e = tid; e < kAppendTok * head_dim; e += blockDim.x) {
    const int j = e % kAppendTok, d = e / kAppendTok;
    const int64_t slot = sl[j];
    if (slot < 0) continue;
    const int64_t tile = (slot / block_size) * num_kv_heads + h;
    vc[(tile * head_dim + d) * block_size + slot % block_size] = vs[j][d];
  }
}

// Append into an FP8 pool, laid out like kv_append_kernel: one workgroup
// per (run of kAppendTok tokens, KV head).  Each thread takes 16 elements of
// a (token, head) row (two 16-byte chunks of 16-bit activations), multiplies
// them by the fp32 reciprocal of the scale and rounds them to E4M3 codes;
// the K codes are stored as one 16-byte chunk, the V codes are staged in LDS
// and written back by head_dim row, consecutive lanes taking consecutive
// tokens.
template <typename AT>
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(const typename AT::elem* __restrict__ k_new,
                                                            const typename AT::elem* __restrict__ v_new,
                                                            const int64_t* __restrict__ slots, int num_tokens,
                                                            int head_dim, int num_kv_heads, int block_size,
                                                            int64_t num_slots, float k_inv, float v_inv,
                                                            uint8_t* __restrict__ kc, uint8_t* __restrict__ vc) {
  __shared__ __attribute__((aligned(16))) uint8_t vs[kAppendTok][kAppendMaxDim + 16];
  __shared__ int64_t sl[kAppendTok];
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * kAppendTok;
  const int tid = threadIdx.x;
  const int gpr = head_dim / 16;  // 16-code groups per row
  if (tid < kAppendTok) {
    const int t = t0 + tid;
    const int64_t slot = t < num_tokens ? slots[t] : -1;
    PA_DEBUG_COUNT(PA_DBG_SLOT, h == 0 && slot >= num_slots);
    sl[tid] = (slot >= 0 && slot < num_slots) ? slot : -1;
  }
  auto codes = [](const typename AT::elem* src, float inv) {
    float x[16];
    widen16<AT>(load16(src), x);
    widen16<AT>(load16(src + 8), x + 8);
    u32x4 q;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      q[w] = to_e4m3(x[4 * w] * inv) | (to_e4m3(x[4 * w + 1] * inv) << 8) | (to_e4m3(x[4 * w + 2] * inv) << 16) |
             (to_e4m3(x[4 * w + 3] * inv) << 24);
    return q;
  };
  for (int c = tid; c < kAppendTok * gpr; c += blockDim.x) {
    const int r = c / gpr, cc = c - r * gpr;
    const int t = t0 + r;
    if (t >= num_tokens) continue;
    const int64_t src = (static_cast<int64_t>(t) * num_kv_heads + h) * head_dim + cc * 16;
    const int64_t slot = slots[t];
    const u32x4 kq = codes(k_new + src, k_inv);
    store16(&vs[r][cc * 16], codes(v_new + src, v_inv));
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t tile = (slot / block_size) * num_kv_heads + h;
    store16(kc + (tile * block_size + slot % block_size) * head_dim + cc * 16, kq);
  }
  __syncthreads();
  for (int e = tid; e < kAppendTok * head_dim; e += blockDim.x) {
    const int j = e % kAppendTok, d = e / kAppendTok;
    const int64_t slot = sl[j];
    if (slot < 0) continue;
    const int64_t tile = (slot / block_size) * num_kv_heads + h;
    vc[(tile * head_dim + d) * block_size + slot % block_size] = vs[j][d];
  }
}

// blockIdx.y = pair; the block's tiles are copied as 16-byte chunks.
__global__ __launch_bounds__(256) void copy_blocks_kernel(const int32_t* __restrict__ pairs, int num_blocks,
                                                          int64_t chunks_per_block, u32x4* __restrict__ kc,
                                                          u32x4* __restrict__ vc) {
  const int p = blockIdx.y;
  const int src = pairs[2 * p], dst = pairs[2 * p + 1];
  PA_DEBUG_COUNT(PA_DBG_COPY_PAIR, (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) && blockIdx.x == 0 &&
                                     threadIdx.x == 0);
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const u32x4* ks = kc + src * chunks_per_block;
  const u32x4* vs = vc + src * chunks_per_block;
  u32x4* kd = kc + dst * chunks_per_block;
  u32x4* vd = vc + dst * chunks_per_block;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < chunks_per_block;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

}  // namespace

hipError_t launch_kv_append(const void* k_new, const void* v_new, const int64_t* slots, int32_t num_tokens,
                            void* k_cache, void* v_cache, int32_t num_blocks, int32_t num_kv_heads,
                            int32_t block_size, int32_t head_dim, int32_t elem_bytes, hipStream_t st) {
  if (num_tokens <= 0 || num_kv_heads <= 0) return hipSuccess;
  if (head_dim > kAppendMaxDim || head_dim * elem_bytes % 16 != 0 || num_kv_heads > 65535)
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((static_cast<int64_t>(num_tokens) + kAppendTok - 1) / kAppendTok),
                  static_cast<unsigned>(num_kv_heads));
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
  if (elem_bytes == 4) {
    hipLaunchKernelGGL(kv_append_kernel<uint32_t>, grid, dim3(256), 0, st, static_cast<const uint32_t*>(k_new),
                       static_cast<const uint32_t*>(v_new), slots, num_tokens, head_dim, num_kv_heads, block_size,
                       num_slots, static_cast<uint32_t*>(k_cache), static_cast<uint32_t*>(v_cache));
  } else {
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(k_new),
                       static_cast<const uint16_t*>(v_new), slots, num_tokens, head_dim, num_kv_heads, block_size,
                       num_slots, static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache));
  }
  return hipGetLastError();
}

hipError_t launch_kv_append_fp8(const void* k_new, const void* v_new, const int64_t* slots, int32_t num_tokens,
                                void* k_cache, void* v_cache, int32_t num_blocks, int32_t num_kv_heads,
                                int32_t block_size, int32_t head_dim, int32_t act_dtype, float k_inv, float v_inv,
                                hipStream_t st) {
  if (num_tokens <= 0 || num_kv_heads <= 0) return hipSuccess;
  if (head_dim > kAppendMaxDim || head_dim % 16 != 0 || num_kv_heads > 65535) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((static_cast<int64_t>(num_tokens) + kAppendTok - 1) / kAppendTok),
                  static_cast<unsigned>(num_kv_heads));
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
  if (act_dtype == 1)
    hipLaunchKernelGGL(kv_append_fp8_kernel<F16>, grid, dim3(256), 0, st, static_cast<const F16::elem*>(k_new),
                       static_cast<const F16::elem*>(v_new), slots, num_tokens, head_dim, num_kv_heads, block_size,
                       num_slots, k_inv, v_inv, static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache));
  else
    hipLaunchKernelGGL(kv_append_fp8_kernel<BF16>, grid, dim3(256), 0, st, static_cast<const BF16::elem*>(k_new),
                       static_cast<const BF16::elem*>(v_new), slots, num_tokens, head_dim, num_kv_heads, block_size,
                       num_slots, k_inv, v_inv, static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache));
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const int32_t* pairs, int32_t num_pairs, void* k_cache, void* v_cache,
                              int32_t num_blocks, int64_t block_bytes, hipStream_t st) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t chunks = block_bytes / 16;
  const int64_t want = (chunks + 255) / 256;
  const int gx = static_cast<int>(want < 16 ? want : 16);
  for (int32_t p0 = 0; p0 < num_pairs; p0 += 65535) {
    const int32_t np = num_pairs - p0 < 65535 ? num_pairs - p0 : 65535;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, np), dim3(256), 0, st, pairs + 2 * static_cast<int64_t>(p0),
                       num_blocks, chunks, static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

PA_DEBUG_UNIT(kv_cache_ops)

}  // namespace pa
