// Paged decode attention for gfx950.
//
// One query token per sequence attends over its context, which is read block
// by block through the sequence's block table (lshu.cn/news/11644,
// "方案：页式内存管理": the kernel reads a request's scattered blocks through
// its block table as one logical K/V sequence).  Decode is bound by reading
// the KV cache from HBM ("性能关键路径与瓶颈": decode latency is about the
// KV-cache bytes over memory bandwidth), so the kernel is built around the
// K/V stream:
//
//  * one workgroup = (sequence, KV head, partition of the context); its four
//    wavefronts take the partition's blocks round robin, so the G q heads
//    that share a KV head read each K/V tile once (grouped-query attention);
//  * a (block, KV head) tile is one contiguous slab (K: block_size rows of
//    head_dim; V: head_dim rows of block_size); a wavefront reads it with
//    16-byte loads, 64 lanes covering 1 KiB contiguous per instruction;
//  * QK: each lane holds one 16-byte chunk of NI token rows of K; the
//    per-chunk dot products (v_dot2 for 16-bit types) are summed across the
//    lanes of a row with a transposing butterfly (DPP / ds_swizzle), so the
//    G*NI partial sums of a row take G*NI-1 exchanges and each lane ends with
//    whole scores of one head;
//  * online softmax in the exp2 domain (scores times scale*log2(e)), one exp
//    per (head, token); fp32 state per head;
//  * PV: a lane holds VEC consecutive tokens of one V row (one head_dim
//    index); the tokens' probabilities come through a small per-wave LDS
//    buffer; partial sums over the token groups are combined at the end;
//  * block-table entries are fetched 64 at a time into a VGPR and read with
//    v_readlane;
//  * the four wavefronts' states are merged in LDS; with one partition the
//    normalised row is written in the storage type, otherwise (m, l, o) go to
//    the workspace and a second kernel merges partitions by log-sum-exp.
#include <algorithm>
#include <atomic>

#include "common.h"
#include "decode_item.h"
#include "launch.h"

namespace pa {

namespace {

// Grid (partition, KV head, sequence): used when every sequence has a single
// partition, so no workgroup is launched without work.  Workgroups are
// dispatched in blockIdx order, so with up to kRankMax sequences the one at
// grid position z takes the z-th longest sequence (ties by index): the
// longest contexts start first and the short ones fill the tail, instead of
// a long one starting last and running alone (greedy longest-first list
// scheduling).  Each workgroup ranks the lengths itself from LDS.
constexpr int kRankMax = 256;
template <typename ST, int D, int BS, int G, typename AT = ST>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(decode_waves_per_eu<ST, D, BS, G, false>(), 8)))
void decode_kernel(DecodeParams P) {
  __shared__ DecodeLds<G, D, BS> sh;
  __shared__ int lens_sh[kRankMax];
  __shared__ int pick;
  const int S = gridDim.z;
  int s = blockIdx.z;
  if (S <= kRankMax) {
    for (int t = threadIdx.x; t < S; t += kThreads) lens_sh[t] = clamp_len(P.ctx_lens[t], P.max_context);
    __syncthreads();
    for (int t = threadIdx.x; t < S; t += kThreads) {
      const int Lt = lens_sh[t];
      int r = 0;
      for (int j = 0; j < S; ++j) {
        const int Lj = lens_sh[j];
        r += (Lj > Lt) || (Lj == Lt && j < t);
      }
      if (r == static_cast<int>(blockIdx.z)) pick = t;
    }
    __syncthreads();
    s = __builtin_amdgcn_readfirstlane(pick);
  }
  decode_item<ST, D, BS, G, AT>(sh, P, s, blockIdx.y, blockIdx.x, clamp_len(P.ctx_lens[s], P.max_context));
}

// Persistent variant for split contexts.  A grid the size of the chip walks
// the compact list of (sequence, partition) pairs written by
// decode_plan_kernel, times the KV heads: sequences shorter than the longest
// one cost nothing for the partitions they do not have.  Consecutive items
// are the KV heads of one (sequence, partition), which read neighbouring
// tiles of the same blocks.
template <typename ST, int D, int BS, int G, typename AT = ST>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(decode_waves_per_eu<ST, D, BS, G, true>(), 8)))
void decode_persistent_kernel(DecodeParams P) {
  __shared__ DecodeLds<G, D, BS> sh;
  const int hk = P.num_kv_heads;
  const int n = __builtin_amdgcn_readfirstlane(*P.n_items) * hk;
  for (int it = blockIdx.x; it < n; it += gridDim.x) {
    const int item = it / hk;
    const int kvh = it - item * hk;
    const int s = __builtin_amdgcn_readfirstlane(P.items[2 * item]);
    const int part = __builtin_amdgcn_readfirstlane(P.items[2 * item + 1]);
    const int L = clamp_len(P.ctx_lens[s], P.max_context);
    __syncthreads();  // the previous item's LDS merge is complete
    decode_item<ST, D, BS, G, AT, split_tile_buffers<ST, D, BS, G>()>(sh, P, s, kvh, part, L);
  }
}

// Work list of the persistent kernel: every (sequence, partition) pair with
// tokens in it (a sequence of length 0 gets one pair, whose item writes its
// zero output), largest first.  The persistent grid deals the list out round
// robin, so putting the full partitions first and the short last ones after
// them in falling size leaves short items for the end -- the same
// longest-first rule as the one-pass grid.  The full partitions come first in
// sequence order; each sequence's last partition then goes into one of
// kPlanBuckets size classes of part_tokens / kPlanBuckets tokens (a counting
// sort; order inside a class is whatever the atomics give -- each pair is
// computed the same way wherever it lands).  Every thread works: the full
// partitions of kPlanThreads sequences at a time are laid out by a workgroup
// prefix sum and written one pair per thread, so a few very long contexts
// (hundreds of partitions each) do not leave a few threads writing them in
// turn.
constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kPlanBuckets = 32;

// Inclusive prefix sum of x over the workgroup's kPlanThreads threads
// (wsum: kPlanWaves ints of LDS, free again when this returns).
__device__ __forceinline__ int plan_inclusive_scan(int x, int* wsum) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int add = 0;
  for (int i = 0; i < w; ++i) add += wsum[i];
  __syncthreads();
  return x + add;
}

__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(const int32_t* __restrict__ ctx_lens, int num_seqs,
                                                                   int max_context, int part_tokens,
                                                                   int32_t* __restrict__ items,
                                                                   int32_t* __restrict__ n_items) {
  __shared__ int count[kPlanBuckets];  // last partitions per size class
  __shared__ int start[kPlanBuckets];
  __shared__ int wsum[kPlanWaves];
  __shared__ int incl[kPlanThreads];
  __shared__ int nfull;
  const int tid = threadIdx.x;
  // size class of a partition of t tokens (t = 0 only for an empty sequence)
  auto bucket = [&](int t) { return t <= 0 ? 0 : static_cast<int>((static_cast<int64_t>(t - 1) * kPlanBuckets) / part_tokens); };
  auto parts_of = [&](int L) { return L == 0 ? 1 : (L + part_tokens - 1) / part_tokens; };
  if (tid < kPlanBuckets) count[tid] = 0;
  if (tid == 0) nfull = 0;
  __syncthreads();
  int my_full = 0;
  for (int s = tid; s < num_seqs; s += kPlanThreads) {
    const int L = clamp_len(ctx_lens[s], max_context);
    const int np = parts_of(L);
    my_full += np - 1;
    atomicAdd(&count[bucket(L - (np - 1) * part_tokens)], 1);
  }
  if (my_full) atomicAdd(&nfull, my_full);
  __syncthreads();
  if (tid == 0) {
    int acc = nfull;  // the full partitions take [0, nfull)
    for (int k = kPlanBuckets - 1; k >= 0; --k) {
      start[k] = acc;
      acc += count[k];
    }
    *n_items = acc;
  }
  __syncthreads();
  // full partitions: sequence order, each sequence's partitions in order
  int base = 0;
  for (int c0 = 0; c0 < num_seqs; c0 += kPlanThreads) {
    const int s = c0 + tid;
    const int f = s < num_seqs ? parts_of(clamp_len(ctx_lens[s], max_context)) - 1 : 0;
    incl[tid] = plan_inclusive_scan(f, wsum);
    __syncthreads();
    const int total = incl[kPlanThreads - 1];
    for (int i = tid; i < total; i += kPlanThreads) {
      int lo = 0, hi = kPlanThreads - 1;  // the first thread whose inclusive sum passes i
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (incl[mid] > i) hi = mid;
        else lo = mid + 1;
      }
      const int first = lo == 0 ? 0 : incl[lo - 1];
      items[2 * (base + i)] = c0 + lo;
      items[2 * (base + i) + 1] = i - first;
    }
    base += total;
    __syncthreads();  // incl is rewritten by the next chunk
  }
  // last partitions, by size class
  for (int s = tid; s < num_seqs; s += kPlanThreads) {
    const int L = clamp_len(ctx_lens[s], max_context);
    const int np = parts_of(L);
    const int at = atomicAdd(&start[bucket(L - (np - 1) * part_tokens)], 1);
    items[2 * at] = s;
    items[2 * at + 1] = np - 1;
  }
}

// Log-sum-exp merge of the partitions of one (sequence, q head); ST is the
// output type.  M = max_p m_p, w_p = l_p 2^(m_p - M), out = sum_p w_p o_p /
// sum_p w_p (partials hold normalised o_p and m in log2 units).  Each thread
// takes 4 consecutive elements of the row (one 16-byte load per partition),
// and the workgroup's kRedThreads / (D / 4) partition slots take the
// partitions round robin, so many loads are in flight even for a few rows
// with hundreds of partitions; the slots' sums are added in slot order at the
// end (the same order on every run).  No LDS grows with the partition count.
constexpr int kRedThreads = 256;
template <typename ST, int D>
__global__ __launch_bounds__(kRedThreads) void decode_reduce_kernel(const float* __restrict__ ws_ml,
                                                                    const float* __restrict__ ws_o,
                                                                    const int32_t* __restrict__ ctx_lens,
                                                                    int max_context, int part_tokens, int max_parts,
                                                                    int num_q_heads,
                                                                    typename ST::elem* __restrict__ out) {
  constexpr int LPP = D / 4;                // threads per partition row
  constexpr int SLOTS = kRedThreads / LPP;  // partitions taken at once
  __shared__ float wmax[kRedThreads / 64];
  __shared__ float4 slot_num[SLOTS][LPP];
  __shared__ float slot_den[SLOTS];
  const int h = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int L = clamp_len(ctx_lens[s], max_context);
  const int np = (L + part_tokens - 1) / part_tokens;
  if (np <= 1) return;  // written directly by the decode kernel
  const int64_t qh = static_cast<int64_t>(s) * num_q_heads + h;
  const float* ml = ws_ml + 2 * qh * max_parts;
  float M = -INFINITY;
  for (int p = tid; p < np; p += kRedThreads) M = fmaxf(M, ml[2 * p]);
  M = fmaxf(M, xor_lane<1>(M));
  M = fmaxf(M, xor_lane<2>(M));
  M = fmaxf(M, xor_lane<4>(M));
  M = fmaxf(M, xor_lane<8>(M));
  M = fmaxf(M, xor_lane<16>(M));
  M = fmaxf(M, xor_lane<32>(M));
  if (lane_id() == 0) wmax[tid >> 6] = M;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kRedThreads / 64; ++w) M = fmaxf(M, wmax[w]);
  const int slot = tid / LPP, c = tid % LPP;
  const float* o = ws_o + qh * max_parts * D + c * 4;
  float4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  auto add = [&](float w, const float4& v) __attribute__((always_inline)) {
    num.x = __builtin_fmaf(w, v.x, num.x);
    num.y = __builtin_fmaf(w, v.y, num.y);
    num.z = __builtin_fmaf(w, v.z, num.z);
    num.w = __builtin_fmaf(w, v.w, num.w);
    den += w;
  };
  // eight of the slot's partitions per step: their loads are all issued
  // before the first is used (the sums still run in partition order)
  constexpr int U = 8;
  int p = slot;
  for (; p + (U - 1) * SLOTS < np; p += U * SLOTS) {
    float w[U];
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pu = p + u * SLOTS;
      w[u] = ml[2 * pu + 1] * __builtin_amdgcn_exp2f(ml[2 * pu] - M);
      v[u] = *reinterpret_cast<const float4*>(o + static_cast<int64_t>(pu) * D);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) add(w[u], v[u]);
  }
  for (; p < np; p += SLOTS) {
    const float w = ml[2 * p + 1] * __builtin_amdgcn_exp2f(ml[2 * p] - M);
    add(w, *reinterpret_cast<const float4*>(o + static_cast<int64_t>(p) * D));
  }
  slot_num[slot][c] = num;
  if (c == 0) slot_den[slot] = den;
  __syncthreads();
  if (tid < LPP) {
    float4 n = slot_num[0][tid];
    float d = slot_den[0];
#pragma unroll
    for (int k = 1; k < SLOTS; ++k) {
      const float4 x = slot_num[k][tid];
      n.x += x.x;
      n.y += x.y;
      n.z += x.z;
      n.w += x.w;
      d += slot_den[k];
    }
    typename ST::elem* dst = out + qh * D + tid * 4;
    dst[0] = narrow<ST>(n.x / d);
    dst[1] = narrow<ST>(n.y / d);
    dst[2] = narrow<ST>(n.z / d);
    dst[3] = narrow<ST>(n.w / d);
  }
}

// Workgroups of a persistent kernel: as many as fit on the device at once
// (queried once per kernel and device).
template <typename KernelTag>
int resident_grid(const void* kernel) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cached[kMaxDev];  // 0 = not yet queried; racing writers store the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) dev = 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess || per_cu <= 0)
      per_cu = 2;
    n = cus * per_cu;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <typename ST, int D, int BS, int G, typename AT>
struct PersistentTag {};

template <typename ST, int D, int BS, int G, typename AT = ST>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  DecodeParams P{};
  P.q = a.q;
  P.kc = a.k_cache;
  P.vc = a.v_cache;
  P.tables = a.block_tables;
  P.ctx_lens = a.context_lens;
  P.items = a.ws_items;
  P.n_items = a.ws_count;
  P.out = a.out;
  P.ws_ml = a.ws_ml;
  P.ws_o = a.ws_o;
  P.scale_log2 = a.scale * kLog2e * a.k_scale;
  P.v_scale = a.v_scale;
  P.max_blocks = a.max_blocks_per_seq;
  P.max_context = a.max_context_len;
  P.num_blocks = a.num_blocks;
  P.num_kv_heads = a.num_kv_heads;
  P.part_tokens = a.part_tokens;
  P.max_parts = a.num_parts;
  if (a.num_parts <= 1) {
    hipLaunchKernelGGL((decode_kernel<ST, D, BS, G, AT>), dim3(1, a.num_kv_heads, a.num_seqs), dim3(kThreads), 0, st, P);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, a.context_lens, a.num_seqs,
                     a.max_context_len, a.part_tokens, a.ws_items, a.ws_count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t upper = static_cast<int64_t>(a.num_seqs) * a.num_parts * a.num_kv_heads;
  const int grid = static_cast<int>(std::min<int64_t>(
      upper, resident_grid<PersistentTag<ST, D, BS, G, AT>>(
                 reinterpret_cast<const void*>(&decode_persistent_kernel<ST, D, BS, G, AT>))));
  hipLaunchKernelGGL((decode_persistent_kernel<ST, D, BS, G, AT>), dim3(grid), dim3(kThreads), 0, st, P);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int num_q_heads = a.num_kv_heads * G;
  hipLaunchKernelGGL((decode_reduce_kernel<AT, D>), dim3(num_q_heads, a.num_seqs), dim3(kRedThreads), 0, st,
                     a.ws_ml, a.ws_o, a.context_lens,
                     a.max_context_len, a.part_tokens, a.num_parts, num_q_heads,
                     static_cast<typename AT::elem*>(a.out));
  return hipGetLastError();
}

template <typename ST, int D, int BS, typename AT = ST>
hipError_t by_group(const DecodeArgs& a, hipStream_t st) {
  switch (a.group) {
    case 1: return launch_decode_t<ST, D, BS, 1, AT>(a, st);
    case 2: return launch_decode_t<ST, D, BS, 2, AT>(a, st);
    case 4: return launch_decode_t<ST, D, BS, 4, AT>(a, st);
    case 8: return launch_decode_t<ST, D, BS, 8, AT>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename ST, int D, typename AT = ST>
hipError_t by_block(const DecodeArgs& a, hipStream_t st) {
  switch (a.block_size) {
    case 8:
      if constexpr (ST::bytes == 1) return hipErrorInvalidValue;  // a 16-byte chunk of codes spans 16 keys
      else return by_group<ST, D, 8, AT>(a, st);
    case 16: return by_group<ST, D, 16, AT>(a, st);
    case 32: return by_group<ST, D, 32, AT>(a, st);
    case 64: return by_group<ST, D, 64, AT>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename ST>
hipError_t by_dim(const DecodeArgs& a, hipStream_t st) {
  switch (a.head_dim) {
    case 64: return by_block<ST, 64>(a, st);
    case 128: return by_block<ST, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

// FP8 pool: head_dim 128, 16-bit activations.
hipError_t by_act_fp8(const DecodeArgs& a, hipStream_t st) {
  if (a.head_dim != 128) return hipErrorInvalidValue;
  switch (a.act_dtype) {
    case 1: return by_block<FP8, 128, F16>(a, st);
    case 2: return by_block<FP8, 128, BF16>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case 0: return by_dim<F32>(a, st);
    case 1: return by_dim<F16>(a, st);
    case 2: return by_dim<BF16>(a, st);
    case 3: return by_act_fp8(a, st);
  }
  return hipErrorInvalidValue;
}

PA_DEBUG_UNIT(decode)

}  // namespace pa
