// The decode work item shared by the split decode kernels and prefix-grouped
// decode: the G q heads of one KV head of one sequence over one partition of
// its tokens, read from the paged pool with four wavefronts (design notes in
// decode.hip).
#pragma once

#include "common.h"

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
  using W = DecodeWave<ST, D, BS, G, AT, NBO>;
  constexpr int TS = W::TS, NI = W::NI;
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
  const int tile_begin = tok_begin / TS;                 // a multiple of SUB
  const int nb = (tok_end + TS - 1) / TS - tile_begin;  // key tiles in this partition
  const int my_tiles = nb > wave ? (nb - wave + kWaves - 1) / kWaves : 0;

  W w;
  w.load_q(P, s, kvh);
  w.walk(P, &sh.p_lds[wave][0][0], s, kvh, tile_begin + wave, kWaves, my_tiles, tok_end);
  float lh[G];
  w.finish(lh);
  if (w.tg == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < NI; ++i) sh.red_acc[wave][h][w.dim_of(i)] = w.acc[h][i];
  }
  if (w.lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sh.red_m[wave][h] = w.m[h];
      sh.red_l[wave][h] = lh[h];
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
