// Chunked-prefill attention over the paged cache, on the gfx950 matrix cores.
//
// A chunk of n new tokens of a sequence (already appended, so the context
// holds L >= n tokens) attends causally: row i sits at position L - n + i and
// sees keys 0..L - n + i (5x10.cn/post/462, "分块预填充"; lshu.cn/news/11644,
// "整体架构": long prompts are split into chunks over several iterations).
// Prefill is bound by the matrix units ("性能关键路径与瓶颈"), so both
// contractions run as v_mfma_f32_32x32x16_{bf16,f16}:
//
//  * one workgroup = (sequence, KV head, tile of 128 rows); a row is a (token,
//    q head of the group) pair, so the G q heads sharing a KV head share every
//    K/V tile; four wavefronts own 32 rows each;
//  * keys come in tiles of 64 gathered through the block table (64/BS
//    blocks), staged in LDS with double buffering: K as [key][dim], V as
//    [dim][key] -- the pool keeps V transposed inside each block, so the PV
//    operand is read with 16-byte LDS loads and no transposition;
//  * S^T = K Q^T with Q held in registers as the B operand; K rows are fed to
//    the A operand in the order that makes each lane's accumulator hold 8
//    consecutive keys of its own row per 16-key step, which is exactly the
//    B-operand layout of O^T = V^T P^T -- probabilities never leave the lane;
//  * online softmax per row in the exp2 domain (fp32 state), causal masking
//    only on tiles that cross a row's diagonal, fully masked tiles skipped;
//  * P enters the PV contraction as two 16-bit parts (nearest value and
//    remainder), two MFMAs per step, so the probabilities carry ~16
//    significant bits: with bf16 outputs the output rounding then dominates
//    the error budget.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // rows per workgroup
constexpr int kKeys = 64;           // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <typename ST>
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c);
template <>
__device__ __forceinline__ f32x16 mfma32<BF16>(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<F16>(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}

// two fp32 -> one dword of two 16-bit values (round to nearest even)
template <typename ST>
__device__ __forceinline__ uint32_t pack2(float a, float b);
template <>
__device__ __forceinline__ uint32_t pack2<BF16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, bf16x2{static_cast<__bf16>(a), static_cast<__bf16>(b)});
}
template <>
__device__ __forceinline__ uint32_t pack2<F16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, f16x2{static_cast<_Float16>(a), static_cast<_Float16>(b)});
}

// A-operand row m of a 32-key subtile holds key perm(m): bits 2 and 3 swapped.
__device__ __forceinline__ int key_perm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <typename ST, int D, int BS, int G>
struct PrefillShape {
  static constexpr int KPAD = D + 8;       // K tile row stride (elements)
  static constexpr int VPAD = kKeys + 8;   // V^T tile row stride (elements)
  static constexpr int K_ELEMS = kKeys * KPAD;
  static constexpr int V_ELEMS = D * VPAD;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int CHUNKS = kKeys * D / 8;       // 16-byte chunks per K (and per V) tile
  static constexpr int PER_THREAD = CHUNKS / kThreads;
  static constexpr int BLOCKS = kKeys / BS;          // cache blocks per tile
  static constexpr int CPB = BS * D / 8;             // chunks per block tile
  static constexpr int TOK = kRows / G;              // tokens per workgroup tile
  static constexpr int KSTEPS = D / 16;
  static constexpr int DSUB = D / 32;
  static_assert(PER_THREAD * kThreads == CHUNKS, "tile chunks");
  static_assert(BLOCKS * BS == kKeys, "blocks per tile");
};

template <typename ST, int D, int BS, int G>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(
    const typename ST::elem* __restrict__ q, const typename ST::elem* __restrict__ kc,
    const typename ST::elem* __restrict__ vc, const int32_t* __restrict__ tables, int max_blocks,
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ cu_q, int num_blocks, int num_kv_heads,
    float scale_log2, typename ST::elem* __restrict__ out) {
  using S = PrefillShape<ST, D, BS, G>;
  using elem = typename ST::elem;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  elem* smem = reinterpret_cast<elem*>(smem_raw);

  const int g = blockIdx.y;
  const int s = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;  // which 8 of 16 along the contraction
  const int nl = lane & 31;    // this lane's row within the wave

  const int q0 = cu_q[s];
  const int n = cu_q[s + 1] - q0;
  int L = ctx_lens[s];
  L = L > max_blocks * BS ? max_blocks * BS : L;
  // heavier tiles (later tokens see more keys) are dispatched first
  const int tile = gridDim.x - 1 - blockIdx.x;
  const int tok0 = tile * S::TOK;
  if (n <= 0 || tok0 >= n || L < n) return;
  const int num_q_heads = num_kv_heads * G;

  // this lane's row
  const int r = wave * 32 + nl;
  const int tok = tok0 + r / G;
  const int hq = g * G + r % G;
  const bool row_ok = tok < n;
  const int pos = L - n + (row_ok ? tok : n - 1);  // last key this row sees

  // Q as the B operand of S^T = K Q^T: lane holds q[row][16 kk + 8 half .. +8]
  u32x4 qb[S::KSTEPS];
  {
    const elem* qp = q + (static_cast<int64_t>(q0 + (row_ok ? tok : 0)) * num_q_heads + hq) * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < S::KSTEPS; ++kk) qb[kk] = row_ok ? load16(qp + kk * 16) : u32x4{0, 0, 0, 0};
  }

  const int tok_last = min(n, tok0 + S::TOK) - 1;
  const int kmax = L - n + tok_last;  // last key any row of the tile sees
  const int ntiles = kmax / kKeys + 1;
  const int diag0 = L - n + tok0;  // keys above this may be masked for some row
  const int nblk_valid = (L + BS - 1) / BS;

  const int32_t* trow = tables + static_cast<int64_t>(s) * max_blocks;
  const int64_t head_k = static_cast<int64_t>(g) * BS * D;
  const int64_t blk_stride = static_cast<int64_t>(num_kv_heads) * BS * D;

  u32x4 kst[S::PER_THREAD], vst[S::PER_THREAD];

  // global -> registers for tile t
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < S::PER_THREAD; ++i) {
      const int c = tid + i * kThreads;
      const int b = c / S::CPB;  // block within the tile
      const int cc = c % S::CPB;
      const int kb = t * S::BLOCKS + b;
      if (kb < nblk_valid) {
        int blk = trow[kb];
        blk = (blk >= 0 && blk < num_blocks) ? blk : 0;
        const int64_t base = static_cast<int64_t>(blk) * blk_stride + head_k + static_cast<int64_t>(cc) * 8;
        kst[i] = load16(kc + base);
        vst[i] = load16(vc + base);
      } else {
        kst[i] = u32x4{0, 0, 0, 0};
        vst[i] = u32x4{0, 0, 0, 0};
      }
    }
  };
  // registers -> LDS stage; keys at or past L are zeroed in V (and K)
  auto stage = [&](int t, int buf) {
    elem* kl = smem + buf * S::STAGE;
    elem* vl = kl + S::K_ELEMS;
    const bool tail = (t + 1) * kKeys > L;
#pragma unroll
    for (int i = 0; i < S::PER_THREAD; ++i) {
      const int c = tid + i * kThreads;
      const int b = c / S::CPB;
      const int cc = c % S::CPB;
      // K chunk: key row within block, 8 dims
      const int krow = cc / (D / 8);
      const int kdc = cc % (D / 8);
      u32x4 kv = kst[i];
      // V^T chunk: one dim, 8 consecutive keys of the block
      const int vdim = cc / (BS / 8);
      const int vkc = cc % (BS / 8);
      u32x4 vv = vst[i];
      if (tail) {
        const int key_k = t * kKeys + b * BS + krow;
        if (key_k >= L) kv = u32x4{0, 0, 0, 0};
        const int key_v = t * kKeys + b * BS + vkc * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = key_v + 2 * e < L ? 0x0000ffffu : 0u;
          const uint32_t hi = key_v + 2 * e + 1 < L ? 0xffff0000u : 0u;
          vv[e] &= (lo | hi);
        }
      }
      store16(kl + (b * BS + krow) * S::KPAD + kdc * 8, kv);
      store16(vl + vdim * S::VPAD + b * BS + vkc * 8, vv);
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o_acc[S::DSUB];
#pragma unroll
  for (int ds = 0; ds < S::DSUB; ++ds) o_acc[ds] = f32x16{};

  fetch(0);
  stage(0, 0);
  __syncthreads();

  const int arow = key_perm(nl);
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) fetch(t + 1);
    const elem* kl = smem + buf * S::STAGE;
    const elem* vl = kl + S::K_ELEMS;

    // S^T for the two 32-key subtiles
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < S::KSTEPS; ++kk) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kl + (ks * 32 + arow) * S::KPAD + kk * 16 + half * 8);
        sacc[ks] = mfma32<ST>(a, qb[kk], sacc[ks]);
      }
    }
    // lane value j of subtile ks is key t*64 + 32 ks + 16 (j/8) + 8 half + j%8
    const int kbase = t * kKeys + half * 8;
    if (t * kKeys + kKeys - 1 > diag0) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kbase + ks * 32 + (j >> 3) * 16 + (j & 7);
          sacc[ks][j] = key <= pos ? sacc[ks][j] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[ks][j]);
    mx = fmaxf(mx, xor_lane<32>(mx));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    // P^T as B operand, one per 16-key step: the 16-bit value nearest p and
    // the 16-bit value nearest the remainder, so P V keeps fp32-like accuracy
    // and the output's own rounding is the only visible error
    u32x4 pb[4], pl[4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int a8 = 0; a8 < 2; ++a8) {
        float p[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          p[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[ks][a8 * 8 + u], scale_log2, -m_new));
          psum += p[u];
        }
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          hi[w] = pack2<ST>(p[2 * w], p[2 * w + 1]);
          float h0, h1;
          widen2<ST>(hi[w], h0, h1);
          lo[w] = pack2<ST>(p[2 * w] - h0, p[2 * w + 1] - h1);
        }
        pb[ks * 2 + a8] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        pl[ks * 2 + a8] = u32x4{lo[0], lo[1], lo[2], lo[3]};
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int ds = 0; ds < S::DSUB; ++ds) o_acc[ds] *= alpha;
    // O^T += V^T P^T
#pragma unroll
    for (int kk2 = 0; kk2 < 4; ++kk2) {
#pragma unroll
      for (int ds = 0; ds < S::DSUB; ++ds) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(vl + (ds * 32 + nl) * S::VPAD + kk2 * 16 + half * 8);
        o_acc[ds] = mfma32<ST>(a, pb[kk2], o_acc[ds]);
        o_acc[ds] = mfma32<ST>(a, pl[kk2], o_acc[ds]);
      }
    }
    if (t + 1 < ntiles) stage(t + 1, buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + xor_lane<32>(l_run);  // both halves of the row (all lanes active)
  if (!row_ok) return;
  const float inv = 1.f / l_tot;
  elem* op = out + (static_cast<int64_t>(q0 + tok) * num_q_heads + hq) * D;
  // lane value j of dim-subtile ds is dim 32 ds + 8 (j/4) + 4 half + j%4
#pragma unroll
  for (int ds = 0; ds < S::DSUB; ++ds)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = ds * 32 + j4 * 8 + half * 4;
      uint2 w;
      w.x = pack2<ST>(o_acc[ds][j4 * 4 + 0] * inv, o_acc[ds][j4 * 4 + 1] * inv);
      w.y = pack2<ST>(o_acc[ds][j4 * 4 + 2] * inv, o_acc[ds][j4 * 4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + d0) = w;
    }
}

template <typename ST, int D, int BS, int G>
hipError_t launch_t(const PrefillArgs& a, hipStream_t st) {
  using S = PrefillShape<ST, D, BS, G>;
  using elem = typename ST::elem;
  const int tiles = (a.max_q_len + S::TOK - 1) / S::TOK;
  if (tiles == 0 || a.num_seqs == 0) return hipSuccess;
  const size_t lds = 2 * S::STAGE * sizeof(elem);
  static bool lds_attr_set = false;  // above 64 KiB of dynamic LDS must be allowed explicitly
  if (!lds_attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<ST, D, BS, G>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    lds_attr_set = true;
  }
  dim3 grid(tiles, a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((prefill_kernel<ST, D, BS, G>), grid, dim3(kThreads), lds, st,
                     static_cast<const elem*>(a.q), static_cast<const elem*>(a.k_cache),
                     static_cast<const elem*>(a.v_cache), a.block_tables, a.max_blocks_per_seq, a.context_lens,
                     a.cu_q_lens, a.num_blocks, a.num_kv_heads, a.scale * kLog2e, static_cast<elem*>(a.out));
  return hipGetLastError();
}

template <typename ST, int D, int BS>
hipError_t by_group(const PrefillArgs& a, hipStream_t st) {
  switch (a.group) {
    case 1: return launch_t<ST, D, BS, 1>(a, st);
    case 2: return launch_t<ST, D, BS, 2>(a, st);
    case 4: return launch_t<ST, D, BS, 4>(a, st);
    case 8: return launch_t<ST, D, BS, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename ST, int D>
hipError_t by_block(const PrefillArgs& a, hipStream_t st) {
  switch (a.block_size) {
    case 16: return by_group<ST, D, 16>(a, st);
    case 32: return by_group<ST, D, 32>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename ST>
hipError_t by_dim(const PrefillArgs& a, hipStream_t st) {
  switch (a.head_dim) {
    case 64: return by_block<ST, 64>(a, st);
    case 128: return by_block<ST, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case 1: return by_dim<F16>(a, st);
    case 2: return by_dim<BF16>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
