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
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

template <typename ST, int D, int BS, int G>
struct DecodeShape {
  static constexpr int VEC = 16 / ST::bytes;  // elements per 16-byte chunk
  static constexpr int LPR = D / VEC;         // lanes covering one K row
  static constexpr int RPI = 64 / LPR;        // K rows per load instruction
  static constexpr int NI = BS / RPI;         // load instructions per tile (K and V alike)
  static constexpr int NV = G * NI;           // partial dot products per lane per tile
  static constexpr int NRED = NV > LPR ? NV / LPR : 1;  // scores per lane after the transpose
  static constexpr int HALV = ilog2(NV / NRED);         // halving steps of the transpose
  static constexpr int LOG_G = ilog2(G);
  static constexpr int CPD = BS / VEC;  // V chunks per head_dim row
  static constexpr bool PREFETCH = NI <= 4;
  static_assert(LPR >= 8 && LPR <= 32 && (LPR & (LPR - 1)) == 0, "row lanes");
  static_assert(NI >= 1 && RPI * NI == BS, "tile rows");
  static_assert(NRED <= NI, "a lane's scores share one head");
  static_assert(HALV >= LOG_G, "head bits");
  static_assert(CPD >= 2 && CPD <= 8, "token groups");
};

// ---- transposing butterfly over the lanes of one K row -----------------------
// Step T exchanges with lane ^ (LPR >> (T+1)).  While a lane holds more than
// one value it keeps half (the lower half if its mask bit is clear) and adds
// the partner's copy of that half; after that it adds the partner's value.
template <int NV, int LPR, int T>
struct RowReduce {
  static constexpr int M = LPR >> (T + 1);
  static constexpr int N = (NV >> T) > 0 ? (NV >> T) : 1;
  static __device__ __forceinline__ void run(float* v, int seg) {
    if constexpr (M >= 1) {
      if constexpr (N > 1) {
        const bool upper = (seg & M) != 0;
#pragma unroll
        for (int j = 0; j < N / 2; ++j) {
          const float keep = upper ? v[N / 2 + j] : v[j];
          const float send = upper ? v[j] : v[N / 2 + j];
          v[j] = keep + xor_lane<M>(send);
        }
      } else {
        v[0] += xor_lane<M>(v[0]);
      }
      RowReduce<NV, LPR, T + 1>::run(v, seg);
    }
  }
};

// Inverse of halving steps T..0: each lane's N values become 2^(T+1) N values
// in index order, gathered from its partners.
template <int NV, int LPR, int T>
struct RowBroadcast {
  static constexpr int M = LPR >> (T + 1);
  static constexpr int N = NV >> (T + 1);
  static __device__ __forceinline__ void run(float* v, int seg) {
    const bool upper = (seg & M) != 0;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const float other = xor_lane<M>(v[j]);
      const float mine = v[j];
      v[j] = upper ? other : mine;
      v[N + j] = upper ? mine : other;
    }
    if constexpr (T > 0) RowBroadcast<NV, LPR, T - 1>::run(v, seg);
  }
};

// max over the lanes that hold other tokens of the same head: the halving
// steps LOG_G..HALV-1 (token bits inside a row) ...
template <int LPR, int T, int END>
__device__ __forceinline__ float max_steps(float x) {
  if constexpr (T < END) {
    x = fmaxf(x, xor_lane<(LPR >> (T + 1))>(x));
    return max_steps<LPR, T + 1, END>(x);
  }
  return x;
}
template <int LPR, int T, int END>
__device__ __forceinline__ float sum_steps(float x) {
  if constexpr (T < END) {
    x += xor_lane<(LPR >> (T + 1))>(x);
    return sum_steps<LPR, T + 1, END>(x);
  }
  return x;
}
// ... and the rows of the wavefront (masks LPR .. 32)
template <int M>
__device__ __forceinline__ float rows_max(float x) {
  if constexpr (M <= 32) {
    x = fmaxf(x, xor_lane<(M <= 32 ? M : 32)>(x));
    return rows_max<M * 2>(x);
  }
  return x;
}
template <int M>
__device__ __forceinline__ float rows_sum(float x) {
  if constexpr (M <= 32) {
    x += xor_lane<(M <= 32 ? M : 32)>(x);
    return rows_sum<M * 2>(x);
  }
  return x;
}
// sum over the lanes of one V row's token groups (masks 1 .. CPD/2)
template <int M, int CPD>
__device__ __forceinline__ float groups_sum(float x) {
  if constexpr (M < CPD) {
    x += xor_lane<M>(x);
    return groups_sum<M * 2, CPD>(x);
  }
  return x;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename ST, int D, int BS, int G>
__global__ __launch_bounds__(kThreads) void decode_kernel(const typename ST::elem* __restrict__ q,
                                                          const typename ST::elem* __restrict__ kc,
                                                          const typename ST::elem* __restrict__ vc,
                                                          const int32_t* __restrict__ tables, int max_blocks,
                                                          const int32_t* __restrict__ ctx_lens, int max_context,
                                                          int num_blocks, int num_kv_heads, float scale_log2,
                                                          int part_tokens,
                                                          int max_parts, typename ST::elem* __restrict__ out,
                                                          float* __restrict__ ws_ml, float* __restrict__ ws_o) {
  using S = DecodeShape<ST, D, BS, G>;
  constexpr int VEC = S::VEC, LPR = S::LPR, RPI = S::RPI, NI = S::NI, NV = S::NV, NRED = S::NRED,
                CPD = S::CPD;
  using elem = typename ST::elem;

  __shared__ float red_acc[kWaves][G][D];
  __shared__ float red_m[kWaves][G];
  __shared__ float red_l[kWaves][G];
  __shared__ __attribute__((aligned(16))) float p_lds[kWaves][G][BS];

  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int s = blockIdx.z;
  const int num_q_heads = num_kv_heads * G;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int seg = lane % LPR;  // 16-byte chunk of a K row
  const int row = lane / LPR;  // K row within a load instruction
  const int tg = lane % CPD;   // V token group: tokens tg*VEC .. tg*VEC+VEC-1

  // device lengths are clamped to the host bound (which the table also holds)
  int L = ctx_lens[s];
  L = L < 0 ? 0 : (L > max_context ? max_context : L);
  const int nparts = (L + part_tokens - 1) / part_tokens;
  if (L == 0) {
    if (part == 0) {
      for (int e = tid; e < G * D; e += kThreads)
        out[(static_cast<int64_t>(s) * num_q_heads + kvh * G) * D + e] = narrow<ST>(0.f);
    }
    return;
  }
  if (part >= nparts) return;

  const int tok_end = min(L, (part + 1) * part_tokens);
  const int blk_begin = part * (part_tokens / BS);
  const int nb = (tok_end + BS - 1) / BS - blk_begin;  // blocks in this partition

  // where this lane's reduced scores sit: head h_own, tokens i*RPI + row
  int off = 0;
#pragma unroll
  for (int t = 0; t < S::HALV; ++t) off += (seg & (LPR >> (t + 1))) ? (NV >> (t + 1)) : 0;
  const int h_own = off / NI;
  const int i_own = off % NI;
  bool owner = true;  // one lane per distinct reduced value counts it in l
#pragma unroll
  for (int t = S::HALV; t < ilog2(LPR); ++t) owner = owner && !(seg & (LPR >> (t + 1)));

  u32x4 qv[G];
  const elem* qrow = q + (static_cast<int64_t>(s) * num_q_heads + kvh * G) * D + seg * VEC;
#pragma unroll
  for (int h = 0; h < G; ++h) qv[h] = load16(qrow + h * D);

  float m[G], acc[G][NI];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
#pragma unroll
    for (int i = 0; i < NI; ++i) acc[h][i] = 0.f;
  }
  float l_own = 0.f;

  const int32_t* trow = tables + static_cast<int64_t>(s) * max_blocks + blk_begin;
  const int64_t head_off = static_cast<int64_t>(kvh) * BS * D;
  const int64_t blk_stride = static_cast<int64_t>(num_kv_heads) * BS * D;
  const int lane_off = lane * VEC;

  const int my_blocks = nb > wave ? (nb - wave + kWaves - 1) / kWaves : 0;
  int tbl_base = -64;
  int tbl_v = 0;
  auto block_id = [&](int j) -> int {
    if (j - tbl_base >= 64) {
      tbl_base = j;
      const int jj = j + lane;
      tbl_v = jj < my_blocks ? trow[wave + jj * kWaves] : 0;
    }
    const int b = __builtin_amdgcn_readlane(tbl_v, j - tbl_base);
    return (b >= 0 && b < num_blocks) ? b : 0;  // never dereference out of range
  };

  auto load_tile = [&](int j, u32x4* kr, u32x4* vr) {
    const int64_t base = static_cast<int64_t>(block_id(j)) * blk_stride + head_off + lane_off;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      kr[i] = load16_nt(kc + base + i * 64 * VEC);
      vr[i] = load16_nt(vc + base + i * 64 * VEC);
    }
  };

  float* pw = &p_lds[wave][0][0];

  auto process = [&](int j, const u32x4* kr, const u32x4* vr) {
    const int blk = blk_begin + wave + j * kWaves;
    const bool partial = blk * BS + BS > tok_end;
    // QK partial dot products, index h*NI + i
    float v[NV];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < NI; ++i) v[h * NI + i] = dot16<ST>(qv[h], kr[i], 0.f);
    RowReduce<NV, LPR, 0>::run(v, seg);
    float bm = -INFINITY;
#pragma unroll
    for (int j2 = 0; j2 < NRED; ++j2) {
      float x = v[j2] * scale_log2;
      if (partial) x = (blk * BS + (i_own + j2) * RPI + row < tok_end) ? x : -INFINITY;
      v[j2] = x;
      bm = fmaxf(bm, x);
    }
    // block max of each head, known to every lane
    bm = max_steps<LPR, S::LOG_G, S::HALV>(bm);
    bm = rows_max<LPR>(bm);
    float bmh[G];
    bmh[0] = bm;
    if constexpr (S::LOG_G > 0) RowBroadcast<G, LPR, S::LOG_G - 1>::run(bmh, seg);
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mn = fmaxf(m[h], bmh[h]);
      alpha[h] = __builtin_amdgcn_exp2f(m[h] - mn);
      m[h] = mn;
    }
    // probabilities of this lane's scores, shared through LDS
    float ps = 0.f;
#pragma unroll
    for (int j2 = 0; j2 < NRED; ++j2) {
      const float p = __builtin_amdgcn_exp2f(v[j2] - m[h_own]);
      ps += p;
      pw[h_own * BS + (i_own + j2) * RPI + row] = p;
    }
    l_own = l_own * alpha[h_own] + (owner ? ps : 0.f);
    wave_lds_sync();

    float vt[NI][VEC];
#pragma unroll
    for (int i = 0; i < NI; ++i) widen16<ST>(vr[i], vt[i]);
    if (partial) {
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        const bool ok = blk * BS + tg * VEC + c < tok_end;
#pragma unroll
        for (int i = 0; i < NI; ++i) vt[i][c] = ok ? vt[i][c] : 0.f;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float p[VEC];
#pragma unroll
      for (int c = 0; c < VEC; c += 4) {
        const float4 x = *reinterpret_cast<const float4*>(pw + h * BS + tg * VEC + c);
        p[c] = x.x;
        p[c + 1] = x.y;
        p[c + 2] = x.z;
        p[c + 3] = x.w;
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float a = acc[h][i] * alpha[h];
#pragma unroll
        for (int c = 0; c < VEC; ++c) a = __builtin_fmaf(p[c], vt[i][c], a);
        acc[h][i] = a;
      }
    }
    wave_lds_sync();  // the next tile's probabilities overwrite pw
  };

  if (my_blocks > 0) {
    if constexpr (S::PREFETCH) {
      u32x4 ka[NI], va[NI], kb[NI], vb[NI];
      load_tile(0, ka, va);
      int j = 0;
      while (true) {
        if (j + 1 < my_blocks) load_tile(j + 1, kb, vb);
        process(j, ka, va);
        if (++j >= my_blocks) break;
        if (j + 1 < my_blocks) load_tile(j + 1, ka, va);
        process(j, kb, vb);
        if (++j >= my_blocks) break;
      }
    } else {
      for (int j = 0; j < my_blocks; ++j) {
        u32x4 ka[NI], va[NI];
        load_tile(j, ka, va);
        process(j, ka, va);
      }
    }
  }

  // l of every head: sum over the lanes holding that head's tokens, then
  // gather the G heads
  float lh[G];
  {
    float x = sum_steps<LPR, S::LOG_G, ilog2(LPR)>(l_own);
    x = rows_sum<LPR>(x);
    lh[0] = x;
    if constexpr (S::LOG_G > 0) RowBroadcast<G, LPR, S::LOG_G - 1>::run(lh, seg);
  }
  // PV partial sums: combine the token groups of each V row
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < NI; ++i) acc[h][i] = groups_sum<1, CPD>(acc[h][i]);
  if (tg == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < NI; ++i) red_acc[wave][h][(i * 64 + lane) / CPD] = acc[h][i];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      red_m[wave][h] = m[h];
      red_l[wave][h] = lh[h];
    }
  }
  __syncthreads();

  // combine the four wavefronts
  for (int e = tid; e < G * D; e += kThreads) {
    const int h = e / D, d = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (red_l[w][h] > 0.f) M = fmaxf(M, red_m[w][h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (red_l[w][h] > 0.f) {
        const float sc = __builtin_amdgcn_exp2f(red_m[w][h] - M);
        num = __builtin_fmaf(red_acc[w][h][d], sc, num);
        den = __builtin_fmaf(red_l[w][h], sc, den);
      }
    }
    const int64_t qh = static_cast<int64_t>(s) * num_q_heads + kvh * G + h;
    if (nparts == 1) {
      out[qh * D + d] = narrow<ST>(num / den);
    } else {
      const int64_t pidx = qh * max_parts + part;
      ws_o[pidx * D + d] = num / den;
      if (d == 0) {
        ws_ml[2 * pidx] = M;
        ws_ml[2 * pidx + 1] = den;
      }
    }
  }
}

// Log-sum-exp merge of the partitions of one (sequence, q head).
template <typename ST, int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(const float* __restrict__ ws_ml,
                                                          const float* __restrict__ ws_o,
                                                          const int32_t* __restrict__ ctx_lens, int max_context,
                                                          int part_tokens, int max_parts, int num_q_heads,
                                                          typename ST::elem* __restrict__ out) {
  extern __shared__ float w_sh[];  // [max_parts]
  __shared__ float M_sh;
  const int h = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
  int L = ctx_lens[s];
  L = L < 0 ? 0 : (L > max_context ? max_context : L);
  const int np = (L + part_tokens - 1) / part_tokens;
  if (np <= 1) return;  // written directly by the decode kernel
  const int64_t qh = static_cast<int64_t>(s) * num_q_heads + h;
  const float* ml = ws_ml + 2 * qh * max_parts;
  if (d == 0) {
    float M = -INFINITY;
    for (int p = 0; p < np; ++p) M = fmaxf(M, ml[2 * p]);
    M_sh = M;
  }
  __syncthreads();
  const float M = M_sh;
  for (int p = d; p < np; p += D) w_sh[p] = ml[2 * p + 1] * __builtin_amdgcn_exp2f(ml[2 * p] - M);
  __syncthreads();
  const float* o = ws_o + qh * max_parts * D + d;
  float num = 0.f, den = 0.f;
  for (int p = 0; p < np; ++p) {
    const float w = w_sh[p];
    num = __builtin_fmaf(w, o[static_cast<int64_t>(p) * D], num);
    den += w;
  }
  out[qh * D + d] = narrow<ST>(num / den);
}

template <typename ST, int D, int BS, int G>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.num_parts, a.num_kv_heads, a.num_seqs);
  using elem = typename ST::elem;
  hipLaunchKernelGGL((decode_kernel<ST, D, BS, G>), grid, dim3(kThreads), 0, st,
                     static_cast<const elem*>(a.q), static_cast<const elem*>(a.k_cache),
                     static_cast<const elem*>(a.v_cache), a.block_tables, a.max_blocks_per_seq, a.context_lens,
                     a.max_context_len, a.num_blocks, a.num_kv_heads, a.scale * kLog2e, a.part_tokens, a.num_parts,
                     static_cast<elem*>(a.out), a.ws_ml, a.ws_o);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_parts <= 1) return e;
  const int num_q_heads = a.num_kv_heads * G;
  hipLaunchKernelGGL((decode_reduce_kernel<ST, D>), dim3(num_q_heads, a.num_seqs), dim3(D),
                     a.num_parts * sizeof(float), st, a.ws_ml, a.ws_o, a.context_lens,
                     a.max_context_len, a.part_tokens, a.num_parts, num_q_heads, static_cast<elem*>(a.out));
  return hipGetLastError();
}

template <typename ST, int D, int BS>
hipError_t by_group(const DecodeArgs& a, hipStream_t st) {
  switch (a.group) {
    case 1: return launch_decode_t<ST, D, BS, 1>(a, st);
    case 2: return launch_decode_t<ST, D, BS, 2>(a, st);
    case 4: return launch_decode_t<ST, D, BS, 4>(a, st);
    case 8: return launch_decode_t<ST, D, BS, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename ST, int D>
hipError_t by_block(const DecodeArgs& a, hipStream_t st) {
  switch (a.block_size) {
    case 16: return by_group<ST, D, 16>(a, st);
    case 32: return by_group<ST, D, 32>(a, st);
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

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case 0: return by_dim<F32>(a, st);
    case 1: return by_dim<F16>(a, st);
    case 2: return by_dim<BF16>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
