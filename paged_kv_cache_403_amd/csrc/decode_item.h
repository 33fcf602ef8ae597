// The decode work item shared by the split decode kernels and prefix-grouped
// decode: the G q heads of one KV head of one sequence over one partition of
// its tokens, read from the paged pool with four wavefronts (design notes in
// decode.hip).
#pragma once

#include <type_traits>

#include "common.h"
#include "mfma.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
#ifndef PA_DECODE_NBUF16
#define PA_DECODE_NBUF16 2
#endif
#ifndef PA_DECODE_NBUF32
#define PA_DECODE_NBUF32 1
#endif



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
  // register buffers of the tile pipeline (each NI 16-byte chunks of K and V)
  static constexpr int NBUF = NI <= 4 ? PA_DECODE_NBUF16 : PA_DECODE_NBUF32;
  static_assert(LPR >= 8 && LPR <= 32 && (LPR & (LPR - 1)) == 0, "row lanes");
  static_assert(NI >= 1 && RPI * NI == BS, "tile rows");
  static_assert(NRED <= NI, "a lane's scores share one head");
  static_assert(HALV >= LOG_G, "head bits");
  static_assert(CPD >= 1 && CPD <= 8, "token groups");
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

// Arguments shared by the decode kernels.
struct DecodeParams {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* tables;
  const int32_t* ctx_lens;
  const int32_t* items;    // persistent kernel: (sequence, partition) pairs
  const int32_t* n_items;  // persistent kernel: number of pairs
  void* out;
  float* ws_ml;
  float* ws_o;
  float scale_log2;  // softmax scale * log2(e) (* k_scale for an FP8 pool)
  float v_scale;     // FP8 pool: V value = code * v_scale
  int32_t max_blocks, max_context, num_blocks, num_kv_heads, part_tokens, max_parts;
};

// Key tile of the decode loop: a whole block, except that 64-token blocks
// are walked in 32-token parts where a whole block's registers (K and V
// chunks, G heads of accumulators) would leave one wavefront per SIMD or
// spill: fp32 pools, and 16-bit pools of head_dim 128 with more than 2 q
// heads per KV head (more than 4 at head_dim 64 or with 1-byte codes).
template <typename ST, int D, int G>
constexpr int decode_tile(int BS) {
  return BS <= 32 ? BS
                  : ((ST::bytes == 1 && G <= 4) || (ST::bytes == 2 && (G <= 2 || (D == 64 && G <= 4))) ? 64 : 32);
}

// Register tile buffers of the split decode items' walk (the persistent
// split kernel and the prefix-grouped suffix kernel): one -- no prefetch
// inside a wavefront -- for head_dim 128 with 16-token tiles and 4 q heads
// per KV head, where a second buffer costs the registers of two more
// resident wavefronts per SIMD (~120 registers instead of ~245) and those
// wavefronts hide the items' loads better than the prefetch does;
// otherwise the shape's choice.  (The one-pass grid runs faster with the
// prefetch.)
template <typename ST, int D, int BS, int G>
constexpr int split_tile_buffers() {
  return (D == 128 && G == 4 && decode_tile<ST, D, G>(BS) == 16) ? 1 : 0;
}

// Shapes whose walk state would otherwise leave one wavefront per SIMD: 8 q
// heads per KV head on 16-bit and FP8 pools (G sets of q chunks,
// accumulators and probability reads per lane), and FP8 pools with tiles of
// 32 or more tokens at 2 or more q heads (each 16-byte V chunk widens to
// sixteen fp32 values) -- as long as a lane holds at most 32 accumulators.
// Unconstrained, the compiler gave them 177-503 registers; with one register
// tile buffer and a bound of two wavefronts per SIMD they take 97-232, with
// no spills, and run up to 1.55x faster (bit-identical output).  fp32 pools
// at 8 q heads ran 10-13% slower that way and keep the shape's choice.
template <typename ST, int D, int BS, int G>
constexpr bool decode_lean() {
  constexpr int TS = decode_tile<ST, D, G>(BS);
  return ST::bytes <= 2 && G * DecodeShape<ST, D, TS, G>::NI <= 32 &&
         (G == 8 || (ST::bytes == 1 && G >= 2 && TS >= 32));
}

// Wavefronts per SIMD a decode kernel is held to (amdgpu_waves_per_eu):
// two for the lean shapes above; for the split items (persistent split
// kernel, grouped suffix kernel) three for 16-bit pools of head_dim 128
// with 32-token tiles and 4 q heads per KV head (168 registers fit without
// spills, against 186 unconstrained: one more resident workgroup per compute
// unit keeps more loads in flight); otherwise what the compiler gives.
template <typename ST, int D, int BS, int G, bool SPLIT>
constexpr int decode_waves_per_eu() {
  return (SPLIT && ST::bytes == 2 && D == 128 && decode_tile<ST, D, G>(BS) == 32 && G == 4) ? 3
         : decode_lean<ST, D, BS, G>()                                                          ? 2
                                                                                                 : 1;
}

template <int G, int D, int BS>
struct DecodeLds {
  float red_acc[kWaves][G][D];
  float red_m[kWaves][G];
  float red_l[kWaves][G];
  __attribute__((aligned(16))) float p_lds[kWaves][G][BS];
};

__device__ __forceinline__ int clamp_len(int L, int max_context) {
  PA_DEBUG_COUNT(PA_DBG_CONTEXT_LEN, L < 0 || L > max_context);
  return L < 0 ? 0 : (L > max_context ? max_context : L);
}

// One wavefront's part of a decode work item: the G q heads of one KV head
// against the key tiles first, first + kWaves, first + 2 kWaves, ... of one
// sequence.  The lane geometry of the QK butterfly and of the PV token
// groups, the q registers, the online softmax state and the tile walk.  (The
// state is kept free of lane-dependent indexing -- a lane's own head is
// picked by selects -- so the compiler keeps it in registers.)
// NBO > 0 overrides the number of register tile buffers (otherwise one for
// the lean shapes, else the shape's choice).
template <typename ST, int D, int BS, int G, typename AT = ST, int NBO = 0>
struct DecodeWave {
  static constexpr int TS = decode_tile<ST, D, G>(BS);  // tokens per key tile
  static constexpr int SUB = BS / TS;                   // tiles per block
  using S = DecodeShape<ST, D, TS, G>;
  static constexpr int NBUF = NBO > 0 ? NBO : (decode_lean<ST, D, BS, G>() ? 1 : S::NBUF);
  static constexpr int VEC = S::VEC, LPR = S::LPR, RPI = S::RPI, NI = S::NI, NV = S::NV, NRED = S::NRED,
                       CPD = S::CPD;
  static constexpr int QCH = VEC * AT::bytes / 16;  // 16-byte q chunks per K chunk
  static_assert(ST::bytes == AT::bytes || (ST::bytes == 1 && AT::bytes == 2), "pool / activation types");
  using elem = typename ST::elem;
  using aelem = typename AT::elem;

  int lane, seg, row, tg, h_own, i_own;
  bool owner;
  u32x4 qv[G][QCH];
  float m[G], acc[G][NI];
  float l_own;

  __device__ __forceinline__ DecodeWave() {
    lane = lane_id();
    seg = lane % LPR;  // 16-byte chunk of a K row
    row = lane / LPR;  // K row within a load instruction
    tg = lane % CPD;   // V token group: tokens tg*VEC .. tg*VEC+VEC-1
    // where this lane's reduced scores sit: head h_own, tokens i*RPI + row
    int off = 0;
#pragma unroll
    for (int t = 0; t < S::HALV; ++t) off += (seg & (LPR >> (t + 1))) ? (NV >> (t + 1)) : 0;
    h_own = off / NI;
    i_own = off % NI;
    owner = true;  // one lane per distinct reduced value counts it in l
#pragma unroll
    for (int t = S::HALV; t < ilog2(LPR); ++t) owner = owner && !(seg & (LPR >> (t + 1)));
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
#pragma unroll
      for (int i = 0; i < NI; ++i) acc[h][i] = 0.f;
    }
    l_own = 0.f;
  }

  __device__ __forceinline__ void load_q(const DecodeParams& P, int s, int kvh) {
    const aelem* __restrict__ q = static_cast<const aelem*>(P.q);
    const aelem* qrow = q + (static_cast<int64_t>(s) * P.num_kv_heads * G + kvh * G) * D + seg * VEC;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < QCH; ++c) qv[h][c] = load16(qrow + h * D + c * (16 / AT::bytes));
  }

  // Tiles first, first + stride, ... (count of them; absolute tile indices
  // of the sequence, TS tokens each) of KV head kvh of sequence s; keys at
  // or past tok_end are masked out.  pw: this wavefront's G * TS floats of
  // LDS for the probabilities.
  __device__ __forceinline__ void walk(const DecodeParams& P, float* pw, int s, int kvh, int first, int stride,
                                       int count, int tok_end) {
    const elem* __restrict__ kc = static_cast<const elem*>(P.kc);
    const elem* __restrict__ vc = static_cast<const elem*>(P.vc);
    const float scale_log2 = P.scale_log2;
    const int32_t* trow = P.tables + static_cast<int64_t>(s) * P.max_blocks;
    const int64_t head_off = static_cast<int64_t>(kvh) * BS * D;
    const int64_t blk_stride = static_cast<int64_t>(P.num_kv_heads) * BS * D;
    const int lane_off = lane * VEC;
    // a V^T tile part is TS keys of each of D rows (rows BS apart)
    const int v_lane_off = SUB == 1 ? lane_off : (lane / CPD) * BS + (lane % CPD) * VEC;
    const int num_blocks = P.num_blocks;

    // address of a tile from its physical block id (never dereferenced out
    // of range); the K chunks are issued before the V chunks so the scores
    // can start while V is still arriving
    auto tile_base = [&](int b) __attribute__((always_inline)) -> int64_t {
      b = (b >= 0 && b < num_blocks) ? b : 0;
      return static_cast<int64_t>(b) * blk_stride + head_off;
    };
    auto load_k = [&](int b, int sub, u32x4* kr) __attribute__((always_inline)) {
      const int64_t kbase = tile_base(b) + sub * TS * D + lane_off;
#pragma unroll
      for (int i = 0; i < NI; ++i) kr[i] = load16_nt(kc + kbase + i * 64 * VEC);
    };
    auto load_v = [&](int b, int sub, u32x4* vr) __attribute__((always_inline)) {
      const int64_t vbase = tile_base(b) + sub * TS + v_lane_off;
#pragma unroll
      for (int i = 0; i < NI; ++i) vr[i] = load16_nt(vc + vbase + i * (64 / CPD) * BS);
    };
    auto load_tile = [&](int b, int sub, u32x4* kr, u32x4* vr) __attribute__((always_inline)) {
      load_k(b, sub, kr);
      load_v(b, sub, vr);
    };

    // QK, the online-softmax update and the tile's probabilities in LDS;
    // each head's rescale factor is left in alpha
    auto scores = [&](int t, const u32x4* kr, float* alpha) __attribute__((always_inline)) {
      const int t0 = t * TS;  // first token of the tile
      const bool partial = t0 + TS > tok_end;
      // QK partial dot products, index h*NI + i
      float v[NV];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          if constexpr (ST::bytes == 1)
            v[h * NI + i] = dot_fp8<AT>(qv[h], kr[i], 0.f);
          else
            v[h * NI + i] = dot16<ST>(qv[h][0], kr[i], 0.f);
        }
      RowReduce<NV, LPR, 0>::run(v, seg);
      float bm = -INFINITY;
#pragma unroll
      for (int j2 = 0; j2 < NRED; ++j2) {
        float x = v[j2] * scale_log2;
        if (partial) x = (t0 + (i_own + j2) * RPI + row < tok_end) ? x : -INFINITY;
        v[j2] = x;
        bm = fmaxf(bm, x);
      }
      // block max of each head, known to every lane
      bm = max_steps<LPR, S::LOG_G, S::HALV>(bm);
      bm = rows_max<LPR>(bm);
      float bmh[G];
      bmh[0] = bm;
      if constexpr (S::LOG_G > 0) RowBroadcast<G, LPR, S::LOG_G - 1>::run(bmh, seg);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], bmh[h]);
        alpha[h] = __builtin_amdgcn_exp2f(m[h] - mn);
        m[h] = mn;
      }
      // this lane's head's max and rescale factor, by selects (a lane-dependent
      // index into the state would keep it out of registers)
      float m_own = m[0], alpha_own = alpha[0];
#pragma unroll
      for (int h = 1; h < G; ++h) {
        m_own = h_own == h ? m[h] : m_own;
        alpha_own = h_own == h ? alpha[h] : alpha_own;
      }
      // probabilities of this lane's scores, shared through LDS
      float ps = 0.f;
#pragma unroll
      for (int j2 = 0; j2 < NRED; ++j2) {
        const float p = __builtin_amdgcn_exp2f(v[j2] - m_own);
        ps += p;
        pw[h_own * TS + (i_own + j2) * RPI + row] = p;
      }
      l_own = l_own * alpha_own + (owner ? ps : 0.f);
      wave_lds_sync();
    };

    // PV of the tile's probabilities (V rows past tok_end zeroed: a zero
    // probability would not cancel a NaN)
    auto accumulate = [&](int t, const u32x4* vr, const float* alpha) __attribute__((always_inline)) {
      const int t0 = t * TS;
      const bool partial = t0 + TS > tok_end;
      float vt[NI][VEC];
#pragma unroll
      for (int i = 0; i < NI; ++i) widen16<ST>(vr[i], vt[i]);
      if (partial) {
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
          const bool ok = t0 + tg * VEC + c < tok_end;
#pragma unroll
          for (int i = 0; i < NI; ++i) vt[i][c] = ok ? vt[i][c] : 0.f;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float p[VEC];
#pragma unroll
        for (int c = 0; c < VEC; c += 4) {
          const float4 x = *reinterpret_cast<const float4*>(pw + h * TS + tg * VEC + c);
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

    auto process = [&](int t, const u32x4* kr, const u32x4* vr) __attribute__((always_inline)) {
      float alpha[G];
      scores(t, kr, alpha);
      accumulate(t, vr, alpha);
    };

    // The tiles in chunks of 64: one vector load brings the chunk's
    // block-table entries into a VGPR (read back with v_readlane), then a
    // software pipeline over NBUF register buffers keeps the loads of tile
    // j + NBUF - 1 in flight while tile j is processed.  In the steady state
    // every prefetched tile exists, so no load is conditional and each wait
    // covers only the tile about to be used; the last tiles of a chunk run in
    // an unrolled tail.  (Reloading K of tile j + 1 as soon as tile j's
    // scores are done, before its PV, keeps both halves of a tile live at
    // once: 256 registers and one wavefront per SIMD at 4 q heads per KV
    // head, against 168 and three.)
    for (int c0 = 0; c0 < count; c0 += 64) {
      const int cn = min(64, count - c0);
      const int tv = lane < cn ? trow[(first + (c0 + lane) * stride) / SUB] : 0;
      PA_DEBUG_COUNT(PA_DBG_BLOCK_ID, tv < 0 || tv >= P.num_blocks);
      auto block_id = [&](int j) __attribute__((always_inline)) -> int { return __builtin_amdgcn_readlane(tv, j); };
      auto sub_of = [&](int j) __attribute__((always_inline)) -> int { return SUB == 1 ? 0 : (first + (c0 + j) * stride) % SUB; };
      auto tile_of = [&](int j) __attribute__((always_inline)) -> int { return first + (c0 + j) * stride; };
      constexpr int NB = NBUF;
      u32x4 kb[NB][NI], vb[NB][NI];
#pragma unroll
      for (int b = 0; b < NB - 1; ++b)
        if (b < cn) load_tile(block_id(b), sub_of(b), kb[b], vb[b]);
      int j0 = 0;
      for (; j0 + 2 * NB - 2 < cn; j0 += NB) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          load_tile(block_id(j0 + b + NB - 1), sub_of(j0 + b + NB - 1), kb[(b + NB - 1) % NB],
                    vb[(b + NB - 1) % NB]);
          process(tile_of(j0 + b), kb[b], vb[b]);
        }
      }
#pragma unroll
      for (int b = 0; b < 2 * NB - 1; ++b) {
        const int j = j0 + b;
        if (j < cn) {
          if (j + NB - 1 < cn)
            load_tile(block_id(j + NB - 1), sub_of(j + NB - 1), kb[(b + NB - 1) % NB], vb[(b + NB - 1) % NB]);
          process(tile_of(j), kb[b % NB], vb[b % NB]);
        }
      }
    }
  }

  // Row sums of every head (sum over the lanes holding that head's tokens,
  // then the G heads gathered), and the PV partial sums of each V row
  // combined over its token groups (valid in lanes with tg == 0).
  __device__ __forceinline__ void finish(float* lh) {
    float x = sum_steps<LPR, S::LOG_G, ilog2(LPR)>(l_own);
    x = rows_sum<LPR>(x);
    lh[0] = x;
    if constexpr (S::LOG_G > 0) RowBroadcast<G, LPR, S::LOG_G - 1>::run(lh, seg);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < NI; ++i) acc[h][i] = groups_sum<1, CPD>(acc[h][i]);
  }

  // head_dim index of acc[h][i] in a lane with tg == 0
  __device__ __forceinline__ int dim_of(int i) const { return (i * 64 + lane) / CPD; }
};

// Decode shapes walked on the matrix cores, where the vector walk's per-byte
// work (G heads of dot products and multiply-adds per K/V element, and the
// widening of FP8 codes) leaves it bound by the vector ALUs: head_dim 128
// at 8 q heads per KV head with FP8 pools of 16- to 64-token blocks or
// 16-bit pools of 16- or 32-token blocks, and FP8 pools of 16-token blocks
// at 4 q heads.  Measured against the vector walk (flushed medians): 1.43-
// 1.84x with FP8 and 1.09-1.32x with 16-bit pools at 8 q heads, 1.08x for
// FP8 at 4 q heads in one pass; 16-bit pools with 64-token blocks at 8 q
// heads ran 0.93x, and at 4 q heads 16-bit pools gained nothing (they are
// bound by HBM already) and FP8 with 32- or 64-token blocks lost 2-10%.
template <typename ST, int D, int BS, int G>
constexpr bool decode_mfma() {
  return D == 128 && ST::bytes <= 2 && BS >= 16 &&
         ((G == 8 && (ST::bytes == 1 || BS <= 32)) || (ST::bytes == 1 && G == 4 && BS == 16));
}

// Register tile buffers of the matrix-core walk: two (the next tile's loads
// in flight while a tile is processed) for the split items of FP8 pools at 4
// q heads per KV head, which hold two wavefronts per SIMD either way (184 or
// 216 registers) and ran 5% faster so (97.5 -> 92.3 us on the shared-prefix
// batch); one otherwise -- the second buffer cost one-pass and 8-head
// shapes a resident wavefront, or spilled (16-bit pools), for no gain.  The
// split kernels are the callers that pass NBO = split_tile_buffers() (1 for
// that shape); the one-pass kernel passes 0.
template <typename ST, int D, int BS, int G, int NBO>
constexpr int mx_tile_buffers() {
  return (NBO == 1 && ST::bytes == 1 && G == 4) ? 2 : 1;
}

// One wavefront's part of a decode work item on the matrix cores
// (v_mfma_f32_16x16x32).  A key tile is 32 tokens.  The G q heads are the
// columns of the products (16 columns, the ones past G zero):
//  * S^T = K Q^T in two 16-token groups: lane (m, g) = (l % 16, l / 16)
//    feeds K row tau_X(m) = 8 (m / 4) + 4 X + m % 4 of the tile (group X)
//    and 8 dimensions of it per product, so the accumulator of lane (n, g)
//    holds head n's scores of tokens 8 g + 4 X + i -- over both groups the 8
//    tokens 8 g .. 8 g + 7, which is the B-operand layout of
//  * O^T = V^T P^T (k = the tile's 32 tokens): lane (m, g) reads 8
//    consecutive tokens of V^T row 16 ds + m straight from the pool's
//    transposed V tile; P enters as a 16-bit value and its remainder (two
//    products), so the probabilities keep about 16 significant bits;
//  * online softmax per head in the exp2 domain on the accumulators (the
//    four lanes of a head's column combine by two exchanges);
//  * K and V come from the pool with 16-byte loads (8 bytes for FP8 V),
//    FP8 codes widened exactly to the activation type.  The dimensions a
//    lane feeds per K product are 32 kk + 8 g (16-bit) or, so that one
//    16-byte load of codes feeds two products, 64 (kk / 2) + 16 g +
//    8 (kk % 2); q is laid out the same way.
// A tile may start before the partition (32-token tiles over 16-token
// blocks): tokens outside [tok_lo, tok_end) are masked out of the scores,
// and V rows at or past tok_end are zeroed (a zero probability would not
// cancel a NaN in an unused slot).
template <typename ST, int D, int BS, int G, typename AT, int NB = 1>
struct DecodeWaveMx {
  static constexpr int TS = 32;                     // tokens per key tile
  static constexpr int SUB = BS > TS ? BS / TS : 1;  // tiles per block
  static constexpr int NBT = BS < TS ? TS / BS : 1;  // blocks per tile
  static constexpr bool FP8P = ST::bytes == 1;
  static constexpr int KLD = FP8P ? 4 : 8;  // 16-byte K loads per lane per tile
  static_assert(D == 128 && G <= 16 && NBT <= 2, "matrix-core decode shape");
  using elem = typename ST::elem;
  using aelem = typename AT::elem;

  int lane, m, g;
  u32x4 qb[4];   // q as the B operand of the 4 K products
  f32x4 o[8];    // O^T: lane (n, g) holds dims 16 ds + 4 g + i of head n
  float m_run;   // running max of head n (lane % 16), in log2 units
  float l_run;   // this lane's share of head n's sum

  __device__ __forceinline__ DecodeWaveMx() {
    lane = lane_id();
    m = lane & 15;
    g = lane >> 4;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) o[ds] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
  }

  // first dimension of the 8 a lane of group gg feeds to K product kk
  static __device__ __forceinline__ int dmap(int kk, int gg) {
    return FP8P ? 64 * (kk >> 1) + 16 * gg + 8 * (kk & 1) : 32 * kk + 8 * gg;
  }

  __device__ __forceinline__ void load_q(const DecodeParams& P, int s, int kvh) {
    const aelem* __restrict__ q = static_cast<const aelem*>(P.q);
    const int n = m;  // this lane's column
    const aelem* qrow = q + (static_cast<int64_t>(s) * P.num_kv_heads * G + kvh * G + (n < G ? n : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qb[kk] = n < G ? load16(qrow + dmap(kk, g)) : u32x4{0, 0, 0, 0};
  }

  __device__ __forceinline__ void walk(const DecodeParams& P, int s, int kvh, int first, int stride, int count,
                                       int tok_lo, int tok_end) {
    const elem* __restrict__ kc = static_cast<const elem*>(P.kc);
    const elem* __restrict__ vc = static_cast<const elem*>(P.vc);
    const float scale_log2 = P.scale_log2;
    const int32_t* trow = P.tables + static_cast<int64_t>(s) * P.max_blocks;
    const int64_t head_off = static_cast<int64_t>(kvh) * BS * D;
    const int64_t blk_stride = static_cast<int64_t>(P.num_kv_heads) * BS * D;
    const int num_blocks = P.num_blocks;
    // this lane's K rows (tile tokens) of the two groups and its V tokens
    const int tk0 = 8 * (m >> 2) + (m & 3), tk1 = tk0 + 4;
    const int tv = 8 * g;

    auto base_of = [&](int b) __attribute__((always_inline)) -> int64_t {
      b = (b >= 0 && b < num_blocks) ? b : 0;
      return static_cast<int64_t>(b) * blk_stride + head_off;
    };
    // element offset, within the tile's block(s), of tile token tk's K row
    // and of V^T row 0 at tile token tk; the block is bA or bB (NBT == 2)
    auto k_off = [&](int sub, int tk) __attribute__((always_inline)) -> int {
      return ((sub * TS + tk) % BS) * D;
    };
    auto v_off = [&](int sub, int tk) __attribute__((always_inline)) -> int { return (sub * TS + tk) % BS; };

    auto load_tile = [&](int bA, int bB, int sub, u32x4* kr, u32x4* vr) __attribute__((always_inline)) {
      const int64_t b0 = base_of(NBT == 2 && tk0 >= BS ? bB : bA);
      const int64_t b1 = base_of(NBT == 2 && tk1 >= BS ? bB : bA);
      const int64_t bv = base_of(NBT == 2 && tv >= BS ? bB : bA);
      const elem* k0 = kc + b0 + k_off(sub, tk0);
      const elem* k1 = kc + b1 + k_off(sub, tk1);
      if constexpr (FP8P) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          kr[p] = load16_nt(k0 + 64 * p + 16 * g);
          kr[2 + p] = load16_nt(k1 + 64 * p + 16 * g);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          kr[kk] = load16_nt(k0 + dmap(kk, g));
          kr[4 + kk] = load16_nt(k1 + dmap(kk, g));
        }
      }
      const elem* v0 = vc + bv + v_off(sub, tv) + static_cast<int64_t>(m) * BS;
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) {
        if constexpr (FP8P) {
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
          const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(v0 + 16 * ds * BS));
          vr[ds] = u32x4{w[0], w[1], 0u, 0u};
        } else {
          vr[ds] = load16_nt(v0 + 16 * ds * BS);
        }
      }
    };

    // the K operand of product kk of group X
    auto k_operand = [&](const u32x4* kr, int X, int kk) __attribute__((always_inline)) -> u32x4 {
      if constexpr (FP8P) {
        const u32x4& w = kr[2 * X + (kk >> 1)];
        const uint32_t a = (kk & 1) ? w[2] : w[0];
        const uint32_t b = (kk & 1) ? w[3] : w[1];
        return u32x4{widen_fp8_pair<AT, false>(a), widen_fp8_pair<AT, true>(a), widen_fp8_pair<AT, false>(b),
                     widen_fp8_pair<AT, true>(b)};
      } else {
        return kr[4 * X + kk];
      }
    };

    auto process = [&](int t, const u32x4* kr, const u32x4* vr) __attribute__((always_inline)) {
      const int t0 = t * TS;
      const bool edge = t0 < tok_lo || t0 + TS > tok_end;
      // scores of tokens 8 g + 4 X + i for head (lane % 16)
      f32x4 sc[2];
#pragma unroll
      for (int X = 0; X < 2; ++X) {
        sc[X] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) sc[X] = mfma16<AT>(k_operand(kr, X, kk), qb[kk], sc[X]);
      }
      float x[8];
      float mx = -INFINITY;
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sc[X][i] * scale_log2;
          if (edge) {
            const int tok = t0 + 8 * g + 4 * X + i;
            v = (tok >= tok_lo && tok < tok_end) ? v : -INFINITY;
          }
          x[4 * X + i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, xor_lane<16>(mx));
      mx = fmaxf(mx, xor_lane<32>(mx));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float p[8];
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(x[e] - m_new);
        ps += p[e];
      }
      l_run = l_run * alpha + ps;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
        for (int ds = 0; ds < 8; ++ds) o[ds] *= alpha;
      }
      // P^T as a 16-bit value and its remainder
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        hi[k] = pack2<AT>(p[2 * k], p[2 * k + 1]);
        float h0, h1;
        widen2<AT>(hi[k], h0, h1);
        lo[k] = pack2<AT>(p[2 * k] - h0, p[2 * k + 1] - h1);
      }
      const u32x4 phi{hi[0], hi[1], hi[2], hi[3]};
      const u32x4 plo{lo[0], lo[1], lo[2], lo[3]};
      // V^T rows: tokens 8 g .. 8 g + 7 of the tile; those at or past
      // tok_end are zeroed
      const int vend = tok_end - (t0 + tv);  // tokens of this lane's 8 that are kept (may be <= 0 or >= 8)
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) {
        u32x4 a;
        if constexpr (FP8P) {
          a = u32x4{widen_fp8_pair<AT, false>(vr[ds][0]), widen_fp8_pair<AT, true>(vr[ds][0]),
                    widen_fp8_pair<AT, false>(vr[ds][1]), widen_fp8_pair<AT, true>(vr[ds][1])};
        } else {
          a = vr[ds];
        }
        if (vend < 8) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t keep_lo = 2 * k < vend ? 0x0000ffffu : 0u;
            const uint32_t keep_hi = 2 * k + 1 < vend ? 0xffff0000u : 0u;
            a[k] &= (keep_lo | keep_hi);
          }
        }
        o[ds] = mfma16<AT>(a, phi, o[ds]);
        o[ds] = mfma16<AT>(a, plo, o[ds]);
      }
    };

    // tiles in chunks of 64: their block-table entries come in one vector
    // load per block of a tile (read back with v_readlane); entries at or past
    // tok_end are never read
    for (int c0 = 0; c0 < count; c0 += 64) {
      const int cn = min(64, count - c0);
      const int tl = first + (c0 + lane) * stride;  // this lane's tile of the chunk
      const int eA = NBT == 2 ? 2 * tl : tl / SUB;
      const int tvA = (lane < cn && eA * BS < tok_end) ? trow[eA] : 0;
      const int tvB = (NBT == 2 && lane < cn && (eA + 1) * BS < tok_end) ? trow[eA + 1] : 0;
      PA_DEBUG_COUNT(PA_DBG_BLOCK_ID, lane < cn && eA * BS < tok_end && (tvA < 0 || tvA >= num_blocks));
      PA_DEBUG_COUNT(PA_DBG_BLOCK_ID,
                     NBT == 2 && lane < cn && (eA + 1) * BS < tok_end && (tvB < 0 || tvB >= num_blocks));
      auto tile_of = [&](int j) __attribute__((always_inline)) -> int { return first + (c0 + j) * stride; };
      auto load_j = [&](int j, u32x4* kr, u32x4* vr) __attribute__((always_inline)) {
        load_tile(__builtin_amdgcn_readlane(tvA, j), NBT == 2 ? __builtin_amdgcn_readlane(tvB, j) : 0,
                  SUB == 1 ? 0 : tile_of(j) % SUB, kr, vr);
      };
      if constexpr (NB == 1) {
        u32x4 kb[KLD], vb[8];
        for (int j = 0; j < cn; ++j) {
          load_j(j, kb, vb);
          process(tile_of(j), kb, vb);
        }
      } else {
        static_assert(NB == 2, "tile buffers");
        u32x4 kb0[KLD], vb0[8], kb1[KLD], vb1[8];
        load_j(0, kb0, vb0);
        int j = 0;
        for (; j + 2 <= cn; j += 2) {
          load_j(j + 1, kb1, vb1);
          process(tile_of(j), kb0, vb0);
          if (j + 2 < cn) load_j(j + 2, kb0, vb0);
          process(tile_of(j + 1), kb1, vb1);
        }
        if (j < cn) process(tile_of(j), kb0, vb0);
      }
    }
  }

  // the head sums over the four lanes of each column, and the wavefront's
  // state into LDS: O^T of head n < G at red_acc[wave][n], (m, l) by the
  // lanes of group 0
  __device__ __forceinline__ void store(DecodeLds<G, D, BS>& sh, int wave) {
    float l = l_run;
    l += xor_lane<16>(l);
    l += xor_lane<32>(l);
    const int n = m;
    if (n < G) {
#pragma unroll
      for (int ds = 0; ds < 8; ++ds)
        *reinterpret_cast<float4*>(&sh.red_acc[wave][n][16 * ds + 4 * g]) =
            float4{o[ds][0], o[ds][1], o[ds][2], o[ds][3]};
      if (g == 0) {
        sh.red_m[wave][n] = m_run;
        sh.red_l[wave][n] = l;
      }
    }
  }
};

// One work item: the G q heads of KV head `kvh` of sequence `s` over the
// tokens of partition `part` (the whole context when it is the only one),
// read by the workgroup's four wavefronts taking the partition's tiles round
// robin.  L is the sequence's clamped context length.  With one partition the
// normalised rows are written to `out`, otherwise (m, l, o) partials go to
// the workspace.  Prefix-grouped decode passes the first token of the
// sequence's own part as `start` (the partitions then cover start..L-1) and
// `partial` to leave partials, at slot slot0 + part, even for a single
// partition.
// ST is the pool's element type, AT the type of q and out (the same except
// for FP8 pools, whose codes meet 16-bit q values).  NBO: register tile
// buffers of the walk (0: the shape's choice).
template <typename ST, int D, int BS, int G, typename AT = ST, int NBO = 0>
__device__ __forceinline__ void decode_item(DecodeLds<G, D, BS>& sh, const DecodeParams& P, int s, int kvh,
                                            int part, int L, int start = 0, int slot0 = 0, bool partial = false) {
  constexpr bool MX = decode_mfma<ST, D, BS, G>();
  using W = std::conditional_t<MX, DecodeWaveMx<ST, D, BS, G, AT, mx_tile_buffers<ST, D, BS, G, NBO>()>,
                               DecodeWave<ST, D, BS, G, AT, NBO>>;
  constexpr int TS = W::TS;
  using aelem = typename AT::elem;
  aelem* __restrict__ out = static_cast<aelem*>(P.out);
  const int num_q_heads = P.num_kv_heads * G;
  const int part_tokens = P.part_tokens;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int nparts = L > start ? (L - start + part_tokens - 1) / part_tokens : 0;
  if (L == 0 && !partial) {
    if (part == 0) {
      for (int e = tid; e < G * D; e += kThreads)
        out[(static_cast<int64_t>(s) * num_q_heads + kvh * G) * D + e] = narrow<AT>(0.f);
    }
    return;
  }
  if (part >= nparts) return;

  const int tok_begin = start + part * part_tokens;  // a multiple of BS
  const int tok_end = min(L, tok_begin + part_tokens);
  const int tile_begin = tok_begin / TS;  // a multiple of SUB (matrix-core walk: may start before tok_begin)
  const int nb = (tok_end + TS - 1) / TS - tile_begin;  // key tiles in this partition
  const int my_tiles = nb > wave ? (nb - wave + kWaves - 1) / kWaves : 0;

  W w;
  w.load_q(P, s, kvh);
  if constexpr (MX) {
    w.walk(P, s, kvh, tile_begin + wave, kWaves, my_tiles, tok_begin, tok_end);
    w.store(sh, wave);
  } else {
    w.walk(P, &sh.p_lds[wave][0][0], s, kvh, tile_begin + wave, kWaves, my_tiles, tok_end);
    float lh[G];
    w.finish(lh);
    if (w.tg == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < W::NI; ++i) sh.red_acc[wave][h][w.dim_of(i)] = w.acc[h][i];
    }
    if (w.lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        sh.red_m[wave][h] = w.m[h];
        sh.red_l[wave][h] = lh[h];
      }
    }
  }
  __syncthreads();

  // combine the four wavefronts
  for (int e = tid; e < G * D; e += kThreads) {
    const int h = e / D, d = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv)
      if (sh.red_l[wv][h] > 0.f) M = fmaxf(M, sh.red_m[wv][h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) {
      if (sh.red_l[wv][h] > 0.f) {
        const float sc = __builtin_amdgcn_exp2f(sh.red_m[wv][h] - M);
        num = __builtin_fmaf(sh.red_acc[wv][h][d], sc, num);
        den = __builtin_fmaf(sh.red_l[wv][h], sc, den);
      }
    }
    const int64_t qh = static_cast<int64_t>(s) * num_q_heads + kvh * G + h;
    float o = num / den;
    if constexpr (ST::bytes == 1) o *= P.v_scale;
    if (nparts == 1 && !partial) {
      out[qh * D + d] = narrow<AT>(o);
    } else {
      const int64_t pidx = qh * P.max_parts + slot0 + part;
      P.ws_o[pidx * D + d] = o;
      if (d == 0) {
        P.ws_ml[2 * pidx] = M;
        P.ws_ml[2 * pidx + 1] = den;
      }
    }
  }
}

}  // namespace

}  // namespace pa
