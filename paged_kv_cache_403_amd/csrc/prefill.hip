// Chunked-prefill attention over the paged cache, on the gfx950 matrix cores.
//
// A chunk of n new tokens of a sequence (already appended, so the context
// holds L >= n tokens) attends causally: row i sits at position L - n + i and
// sees keys 0..L - n + i (5x10.cn/post/462, "分块预填充"; lshu.cn/news/11644,
// "整体架构": long prompts are split into chunks over several iterations).
// Prefill is bound by the matrix units ("性能关键路径与瓶颈"), so both
// contractions run as v_mfma_f32_32x32x16_{bf16,f16}:
//
//  * one workgroup = (sequence, KV head, tile of 256 rows); a row is a (token,
//    q head of the group) pair, so the G q heads sharing a KV head share every
//    K/V tile; eight wavefronts (two per SIMD, so one's softmax overlaps the
//    other's matrix work) own 32 rows each;
//  * the sequence's block-table entries are staged in LDS once; keys come in
//    tiles of 64 gathered through them (64/BS blocks), double buffered in
//    LDS: K as [key][dim], V as [dim][key] -- the pool keeps V transposed
//    inside each block, so the PV operand is read with 16-byte LDS loads;
//  * S^T = K Q^T with Q held in registers as the B operand; K rows are fed to
//    the A operand in the order that makes each lane's accumulator hold 8
//    consecutive keys of its own row per 16-key step, which is exactly the
//    B-operand layout of O^T = V^T P^T -- probabilities never leave the lane;
//  * online softmax per row in the exp2 domain (fp32 state).  The reference
//    max only moves when a score exceeds it by 2^8 (probabilities stay below
//    256), so rescaling the accumulators is rare and skipped by whole
//    wavefronts when no row needs it;
//  * causal masking only on tiles that cross a row's diagonal; a wavefront
//    skips tiles that lie wholly above its rows' diagonals;
//  * P enters PV rounded to the storage type.  On a sequence's first key
//    tile -- where rows with only a few keys can give outputs of large
//    magnitude -- it enters as two 16-bit parts (nearest value and
//    remainder, two MFMAs), so such rows keep only their output rounding;
//  * workgroup ids are mapped so that all row tiles of one (sequence, KV
//    head) run on the same XCD and share its L2.
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace pa {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // rows per workgroup
constexpr int kKeys = 64;           // keys per tile
constexpr int kXcds = 8;            // MI355X: workgroups go round robin over 8 XCDs
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.f;  // log2 units the running max may lag the true max
constexpr int kSortMax = 4096;  // items per XCD ordered longest first (more keep index order)

// ST: the matrix (activation) type; PT: the pool's element type (ST, or FP8
// codes widened to ST while staging)
template <typename ST, typename PT, int D, int BS, int G>
struct PrefillShape {
  static constexpr int KPAD = D + 8;       // K tile row stride (elements)
  static constexpr int VPAD = kKeys + 8;   // V^T tile row stride (elements)
  static constexpr int K_ELEMS = kKeys * KPAD;
  static constexpr int V_ELEMS = D * VPAD;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int CPE = 16 / PT::bytes;          // pool elements per 16-byte chunk
  static constexpr int CHUNKS = kKeys * D / CPE;     // 16-byte pool chunks per K (and per V) tile
  static constexpr int PER_THREAD = CHUNKS / kThreads;
  static constexpr int BLOCKS = kKeys / BS;          // cache blocks per tile
  static constexpr int CPB = BS * D / CPE;           // chunks per block tile
  static constexpr int TOK = kRows / G;              // tokens per workgroup tile
  static constexpr int KSTEPS = D / 16;
  static constexpr int DSUB = D / 32;
  static_assert(PER_THREAD >= 1 && PER_THREAD * kThreads == CHUNKS, "tile chunks");
  static_assert(BLOCKS * BS == kKeys, "blocks per tile");
  static_assert(BS % CPE == 0 || CPE == 8, "a V chunk stays inside one block's dim row");
};

// KS: the key-split instance (nsplit key ranges, partials to the
// workspace); the other one runs each row tile's keys whole, as if nsplit
// were 1 at compile time.
template <typename ST, typename PT, int D, int BS, int G, bool KS>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(
    const typename ST::elem* __restrict__ q, const typename PT::elem* __restrict__ kc,
    const typename PT::elem* __restrict__ vc, const int32_t* __restrict__ tables, int max_blocks,
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ cu_q, int num_blocks, int num_kv_heads,
    int num_units, int row_tiles, int max_context, float scale_log2, float v_scale,
    typename ST::elem* __restrict__ out, int nsplit, float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  using S = PrefillShape<ST, PT, D, BS, G>;
  using elem = typename ST::elem;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  elem* smem = reinterpret_cast<elem*>(smem_raw);
  int32_t* tbl = reinterpret_cast<int32_t*>(smem + 2 * S::STAGE);

  const int tid = threadIdx.x;
  // Workgroup -> (unit = sequence * KV heads + head, row tile).  Workgroup w
  // runs on XCD w % 8 as slot w / 8; the XCD owns units x, x + 8, ..., so
  // all row tiles of a unit share one L2.  Within an XCD the slots take the
  // items in decreasing number of key tiles (ties by index): the dispatcher
  // hands slots to compute units in order, so this is longest-first
  // scheduling of the uneven contexts.
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int xunits = num_units > xcd ? (num_units - xcd + kXcds - 1) / kXcds : 0;
  const int nsp = KS ? nsplit : 1;
  const int nitems = xunits * row_tiles * nsp;  // (unit, row tile, key range)
  if (slot >= nitems) return;
  int item = slot;
  if (nitems <= kSortMax) {
    int* cost = reinterpret_cast<int*>(tbl);  // the table area is free until the item is known
    __shared__ int chosen;
    for (int e = tid; e < nitems; e += kThreads) {
      const int u = xcd + kXcds * (e / (row_tiles * nsp));
      const int su = u / num_kv_heads;
      const int nu = cu_q[su + 1] - cu_q[su];
      const int Lu = min(ctx_lens[su], max_context);
      const int t0 = ((e / nsp) % row_tiles) * S::TOK;
      const int ke = e % nsp;
      // key tiles the row tile reads (0: no rows), and this item's share
      const int tt = (nu <= 0 || t0 >= nu || Lu < nu) ? 0 : (Lu - nu + min(nu, t0 + S::TOK) - 1) / kKeys + 1;
      cost[e] = (ke + 1) * tt / nsp - ke * tt / nsp;
    }
    __syncthreads();
    for (int e = tid; e < nitems; e += kThreads) {
      const int c = cost[e];
      int rank = 0;
      for (int f = 0; f < nitems; ++f) {
        const int cf = cost[f];
        rank += (cf > c || (cf == c && f < e)) ? 1 : 0;
      }
      if (rank == slot) chosen = e;
    }
    __syncthreads();
    item = chosen;
    __syncthreads();  // cost[] is overwritten by the block table below
  }
  const int unit = xcd + kXcds * (item / (row_tiles * nsp));
  const int s = unit / num_kv_heads;
  const int g = unit - s * num_kv_heads;
  const int tile = (item / nsp) % row_tiles;
  const int ksplit = item % nsp;

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;  // which 8 of 16 along the contraction
  const int nl = lane & 31;    // this lane's row within the wave

  const int q0 = cu_q[s];
  const int n = cu_q[s + 1] - q0;
  int L = ctx_lens[s];
  PA_DEBUG_COUNT(PA_DBG_CONTEXT_LEN, n > 0 && tile * S::TOK < n && (L > max_context || L < n));
  L = L > max_context ? max_context : L;
  const int tok0 = tile * S::TOK;
  if (n <= 0 || tok0 >= n || L < n) return;
  const int num_q_heads = num_kv_heads * G;

  // this lane's row
  const int r = wave * 32 + nl;
  const int tok = tok0 + r / G;
  const int hq = g * G + r % G;
  const bool row_ok = tok < n;
  const int pos = L - n + (row_ok ? tok : n - 1);  // last key this row sees
  // last key any row of this wavefront sees (rows past the chunk see n - 1)
  const int wave_pos = L - n + min(n - 1, tok0 + (wave * 32 + 31) / G);

  const int tok_last = min(n, tok0 + S::TOK) - 1;
  const int kmax = L - n + tok_last;  // last key any row of the tile sees
  const int ntiles = kmax / kKeys + 1;
  // this item's key tiles (all of them without a split)
  const int t_lo = KS ? ksplit * ntiles / nsp : 0;
  const int t_hi = KS ? (ksplit + 1) * ntiles / nsp : ntiles;
  const int diag0 = L - n + tok0;  // keys above this may be masked for some row
  const int nblk_valid = (L + BS - 1) / BS;
  // partial rows of this item in the workspace (key-split instance)
  const int64_t prow = (static_cast<int64_t>(q0 + tok) * num_q_heads + hq) * nsp + ksplit;
  if (KS && t_lo >= t_hi) {
    // more key ranges than the row tile has key tiles: an empty partial
    if (row_ok && half == 0) *reinterpret_cast<float2*>(ws_ml + 2 * prow) = float2{-INFINITY, 0.f};
    return;
  }
  // From here on the item has at least one key tile (ntiles >= 1 since
  // L >= n), so the prologue and the first tile run unconditionally; a
  // guarded prologue would leave the Q loads outstanding on one path, and
  // the wait for them would then sit inside the tile loop.

  // block-table entries of every tile, out-of-range ids replaced by block 0
  {
    const int32_t* trow = tables + static_cast<int64_t>(s) * max_blocks;
    const int nt = ntiles * S::BLOCKS;
    for (int i = tid; i < nt; i += kThreads) {
      int b = i < nblk_valid ? trow[i] : 0;
      PA_DEBUG_COUNT(PA_DBG_BLOCK_ID, b < 0 || b >= num_blocks);
      tbl[i] = (b >= 0 && b < num_blocks) ? b : 0;
    }
  }

  // Q as the B operand of S^T = K Q^T: lane holds q[row][16 kk + 8 half .. +8]
  u32x4 qb[S::KSTEPS];
  {
    const elem* qp = q + (static_cast<int64_t>(q0 + (row_ok ? tok : 0)) * num_q_heads + hq) * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < S::KSTEPS; ++kk) qb[kk] = row_ok ? load16(qp + kk * 16) : u32x4{0, 0, 0, 0};
  }

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
      const int blk = tbl[t * S::BLOCKS + b];
      const int64_t base = static_cast<int64_t>(blk) * blk_stride + head_k + static_cast<int64_t>(cc) * S::CPE;
      kst[i] = load16(kc + base);
      vst[i] = load16(vc + base);
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
      // K chunk: key row within block, CPE dims; V^T chunk: one dim, CPE
      // consecutive keys of the block
      const int krow = cc / (D / S::CPE);
      const int kdc = cc % (D / S::CPE);
      const int vdim = cc / (BS / S::CPE);
      const int vkc = cc % (BS / S::CPE);
      constexpr int W = S::CPE / 8;  // 16-byte LDS rows per chunk once widened
      u32x4 kv[W], vv[W];
      if constexpr (W == 1) {
        kv[0] = kst[i];
        vv[0] = vst[i];
      } else {
        // sixteen E4M3 codes -> sixteen 16-bit values, exactly
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            kv[h][2 * e] = widen_fp8_pair<ST, false>(kst[i][2 * h + e]);
            kv[h][2 * e + 1] = widen_fp8_pair<ST, true>(kst[i][2 * h + e]);
            vv[h][2 * e] = widen_fp8_pair<ST, false>(vst[i][2 * h + e]);
            vv[h][2 * e + 1] = widen_fp8_pair<ST, true>(vst[i][2 * h + e]);
          }
      }
      if (tail) {
        const int key_k = t * kKeys + b * BS + krow;
        const int key_v = t * kKeys + b * BS + vkc * S::CPE;
#pragma unroll
        for (int w = 0; w < W; ++w) {
          if (key_k >= L) kv[w] = u32x4{0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = key_v + 8 * w + 2 * e;
            const uint32_t lo = key < L ? 0x0000ffffu : 0u;
            const uint32_t hi = key + 1 < L ? 0xffff0000u : 0u;
            vv[w][e] &= (lo | hi);
          }
        }
      }
#pragma unroll
      for (int w = 0; w < W; ++w) {
        store16(kl + (b * BS + krow) * S::KPAD + kdc * S::CPE + 8 * w, kv[w]);
        store16(vl + vdim * S::VPAD + b * BS + vkc * S::CPE + 8 * w, vv[w]);
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o_acc[S::DSUB];
#pragma unroll
  for (int ds = 0; ds < S::DSUB; ++ds) o_acc[ds] = f32x16{};

  __syncthreads();  // block table in LDS
  fetch(t_lo);
  stage(t_lo, 0);
  __syncthreads();

  const int arow = key_perm(nl);
  // one key tile; `first` marks the sequence's first tile (tile 0), the
  // only one whose probabilities enter PV in two parts.  It runs once for
  // the item's first tile and then in a loop with first = false, so the
  // loop body carries no first-tile path.
  auto tile_step = [&](int t, bool first) __attribute__((always_inline)) {
    const int buf = (t - t_lo) & 1;
    if (t + 1 < t_hi) fetch(t + 1);
    const elem* kl = smem + buf * S::STAGE;
    const elem* vl = kl + S::K_ELEMS;

    const bool active = t * kKeys <= wave_pos;  // some row of this wavefront sees a key of this tile
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    float mx = -INFINITY;
    if (active) {
      // S^T for the two 32-key subtiles.  The sixteen K operands are read
      // from LDS ahead of the products, in two batches of eight (the group
      // barriers below hold the scheduler to that order instead of pairing
      // each read with its product), so the wave waits for LDS twice per
      // tile rather than once per product.
      u32x4 ka[S::KSTEPS][2];
#pragma unroll
      for (int kk = 0; kk < S::KSTEPS; ++kk)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          ka[kk][ks] = *reinterpret_cast<const u32x4*>(kl + (ks * 32 + arow) * S::KPAD + kk * 16 + half * 8);
#pragma unroll
      for (int kk = 0; kk < S::KSTEPS; ++kk)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) sacc[ks] = mfma32<ST>(ka[kk][ks], qb[kk], sacc[ks]);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 12, 0);
      // lane value j of subtile ks is key t*64 + 32 ks + 16 (j/8) + 8 half + j%8
      const int kbase = t * kKeys + half * 8;
      if (t * kKeys + kKeys - 1 > diag0) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const int key = kbase + ks * 32 + (jj >> 3) * 16 + (jj & 7);
            sacc[ks][jj] = key <= pos ? sacc[ks][jj] : -INFINITY;
          }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, sacc[ks][jj]);
      mx = halves_max(mx) * scale_log2;
    }
    // The next tile goes from registers to LDS between the score and the
    // softmax phases: its buffer was released by the previous iteration's
    // barrier, and LDS is otherwise idle while the exponentials run.
    if (t + 1 < t_hi) stage(t + 1, buf ^ 1);
    if (active) {
      // the reference max moves only when the tile's max passes it by kLazy
      const bool move = mx > m_run + kLazy;
      const bool rescale = move && m_run > -INFINITY;  // accumulators hold earlier keys
      const float m_new = move ? mx : m_run;
      const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      m_run = m_new;
      // a row that has seen no key yet (only possible in a key range after
      // the first: all of its keys so far lie past its diagonal) keeps
      // probabilities of 0 instead of exp2(-inf + inf)
      const float m_ref = (KS && m_new == -INFINITY) ? 0.f : m_new;
      float psum = 0.f;
      // P^T as B operand, one per 16-key step
      u32x4 pb[4], pl[4];
      const bool split = first;  // first tile: probabilities as two 16-bit parts
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int a8 = 0; a8 < 2; ++a8) {
          float p[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            p[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[ks][a8 * 8 + u], scale_log2, -m_ref));
            psum += p[u];
          }
          uint32_t hi[4];
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) hi[w2] = pack2<ST>(p[2 * w2], p[2 * w2 + 1]);
          pb[ks * 2 + a8] = u32x4{hi[0], hi[1], hi[2], hi[3]};
          if (split) {
            uint32_t lo[4];
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
              float h0, h1;
              widen2<ST>(hi[w2], h0, h1);
              lo[w2] = pack2<ST>(p[2 * w2] - h0, p[2 * w2 + 1] - h1);
            }
            pl[ks * 2 + a8] = u32x4{lo[0], lo[1], lo[2], lo[3]};
          }
        }
      l_run = l_run * alpha + psum;
      if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
        for (int ds = 0; ds < S::DSUB; ++ds) o_acc[ds] *= alpha;
      }
      // O^T += V^T P^T
#pragma unroll
      for (int kk2 = 0; kk2 < 4; ++kk2) {
#pragma unroll
        for (int ds = 0; ds < S::DSUB; ++ds) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(vl + (ds * 32 + nl) * S::VPAD + kk2 * 16 + half * 8);
          o_acc[ds] = mfma32<ST>(a, pb[kk2], o_acc[ds]);
          if (split) o_acc[ds] = mfma32<ST>(a, pl[kk2], o_acc[ds]);
        }
      }
    }
    __syncthreads();
  };
  tile_step(t_lo, t_lo == 0);
  for (int t = t_lo + 1; t < t_hi; ++t) tile_step(t, false);

  const float l_tot = halves_sum(l_run);  // both halves of the row
  if (!row_ok) return;
  if constexpr (KS) {
    // partials of this key range: O unnormalised, (max, sum); lane value j
    // of dim-subtile ds is dim 32 ds + 8 (j/4) + 4 half + j%4
    float* po = ws_o + prow * D;
#pragma unroll
    for (int ds = 0; ds < S::DSUB; ++ds)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4)
        *reinterpret_cast<float4*>(po + ds * 32 + j4 * 8 + half * 4) =
            float4{o_acc[ds][j4 * 4 + 0], o_acc[ds][j4 * 4 + 1], o_acc[ds][j4 * 4 + 2], o_acc[ds][j4 * 4 + 3]};
    if (half == 0) *reinterpret_cast<float2*>(ws_ml + 2 * prow) = float2{m_run, l_tot};
    return;
  }
  const float inv = v_scale / l_tot;
  elem* op = out + (static_cast<int64_t>(q0 + tok) * num_q_heads + hq) * D;
  // lane value j of dim-subtile ds is dim 32 ds + 8 (j/4) + 4 half + j%4
#pragma unroll
  for (int ds = 0; ds < S::DSUB; ++ds)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = ds * 32 + j4 * 8 + half * 4;
      uint2 wv;
      wv.x = pack2<ST>(o_acc[ds][j4 * 4 + 0] * inv, o_acc[ds][j4 * 4 + 1] * inv);
      wv.y = pack2<ST>(o_acc[ds][j4 * 4 + 2] * inv, o_acc[ds][j4 * 4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + d0) = wv;
    }
}

// Log-sum-exp merge of the key ranges' partials: a thread per (row, 4
// dimensions); rows are (token, q head) of the chunks, rows past the last
// chunk's token are not the kernel's.  A range without keys (sum 0) carries
// no weight.
constexpr int kMergeThreads = 256;
template <typename ST, int D>
__global__ __launch_bounds__(kMergeThreads) void prefill_merge_kernel(const float* __restrict__ ws_o,
                                                                      const float* __restrict__ ws_ml,
                                                                      const int32_t* __restrict__ cu_q, int num_seqs,
                                                                      int num_q_heads, int nsplit, float v_scale,
                                                                      typename ST::elem* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kMergeThreads + threadIdx.x;
  const int64_t row = idx / (D / 4);
  const int d0 = static_cast<int>(idx % (D / 4)) * 4;
  if (row >= static_cast<int64_t>(cu_q[num_seqs]) * num_q_heads) return;
  float M = -INFINITY;
  for (int k = 0; k < nsplit; ++k) {
    const float2 ml = *reinterpret_cast<const float2*>(ws_ml + 2 * (row * nsplit + k));
    if (ml.y > 0.f) M = fmaxf(M, ml.x);
  }
  float4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int k = 0; k < nsplit; ++k) {
    const float2 ml = *reinterpret_cast<const float2*>(ws_ml + 2 * (row * nsplit + k));
    if (ml.y > 0.f) {
      const float w = __builtin_amdgcn_exp2f(ml.x - M);
      const float4 o = *reinterpret_cast<const float4*>(ws_o + (row * nsplit + k) * D + d0);
      num.x = __builtin_fmaf(o.x, w, num.x);
      num.y = __builtin_fmaf(o.y, w, num.y);
      num.z = __builtin_fmaf(o.z, w, num.z);
      num.w = __builtin_fmaf(o.w, w, num.w);
      den = __builtin_fmaf(ml.y, w, den);
    }
  }
  const float inv = den > 0.f ? v_scale / den : 0.f;
  uint2 wv;
  wv.x = pack2<ST>(num.x * inv, num.y * inv);
  wv.y = pack2<ST>(num.z * inv, num.w * inv);
  *reinterpret_cast<uint2*>(out + row * D + d0) = wv;
}

template <typename ST, typename PT, int D, int BS, int G>
hipError_t launch_t(const PrefillArgs& a, hipStream_t st) {
  using S = PrefillShape<ST, PT, D, BS, G>;
  using elem = typename ST::elem;
  const int row_tiles = (a.max_q_len + S::TOK - 1) / S::TOK;
  if (row_tiles == 0 || a.num_seqs == 0) return hipSuccess;
  const int units = a.num_seqs * a.num_kv_heads;
  const int nsplit = a.key_splits > 1 ? a.key_splits : 1;
  if (nsplit > 1 && (!a.ws_o || !a.ws_ml)) return hipErrorInvalidValue;
  const int64_t grid = static_cast<int64_t>((units + kXcds - 1) / kXcds) * kXcds * row_tiles * nsplit;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const int max_tiles = (a.max_context_len + kKeys - 1) / kKeys;
  const int per_xcd = (units + kXcds - 1) / kXcds * row_tiles * nsplit;
  const size_t tbl_entries = std::max<size_t>(static_cast<size_t>(max_tiles) * S::BLOCKS,
                                              per_xcd <= kSortMax ? static_cast<size_t>(per_xcd) : 0);
  const size_t lds = 2 * S::STAGE * sizeof(elem) + tbl_entries * sizeof(int32_t);
  if (lds > kPrefillMaxLds) return hipErrorInvalidValue;
  // above 64 KiB of dynamic LDS must be allowed explicitly; a function-local
  // static is set once, also when several host threads launch at once
  static const hipError_t lds_attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<ST, PT, D, BS, G, false>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kPrefillMaxLds));
  if (lds_attr != hipSuccess) return lds_attr;
  static const hipError_t lds_attr_ks =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<ST, PT, D, BS, G, true>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kPrefillMaxLds));
  if (lds_attr_ks != hipSuccess) return lds_attr_ks;
  using pelem = typename PT::elem;
  auto kernel = nsplit > 1 ? prefill_kernel<ST, PT, D, BS, G, true> : prefill_kernel<ST, PT, D, BS, G, false>;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), lds, st,
                     static_cast<const elem*>(a.q), static_cast<const pelem*>(a.k_cache),
                     static_cast<const pelem*>(a.v_cache), a.block_tables, a.max_blocks_per_seq, a.context_lens,
                     a.cu_q_lens, a.num_blocks, a.num_kv_heads, units, row_tiles, a.max_context_len,
                     a.scale * kLog2e * a.k_scale, a.v_scale, static_cast<elem*>(a.out), nsplit, a.ws_o, a.ws_ml);
  if (nsplit == 1) return hipGetLastError();
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = static_cast<int64_t>(a.total_q) * a.num_kv_heads * G * (D / 4);
  const int64_t blocks = (threads + kMergeThreads - 1) / kMergeThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_merge_kernel<ST, D>), dim3(static_cast<unsigned>(blocks)), dim3(kMergeThreads), 0, st,
                     a.ws_o, a.ws_ml, a.cu_q_lens, a.num_seqs, a.num_kv_heads * G, nsplit, a.v_scale,
                     static_cast<elem*>(a.out));
  return hipGetLastError();
}

template <typename ST, typename PT, int D, int BS>
hipError_t by_group(const PrefillArgs& a, hipStream_t st) {
  switch (a.group) {
    case 1: return launch_t<ST, PT, D, BS, 1>(a, st);
    case 2: return launch_t<ST, PT, D, BS, 2>(a, st);
    case 4: return launch_t<ST, PT, D, BS, 4>(a, st);
    case 8: return launch_t<ST, PT, D, BS, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename ST, int D>
hipError_t by_block(const PrefillArgs& a, hipStream_t st) {
  switch (a.block_size) {
    case 8: return by_group<ST, ST, D, 8>(a, st);
    case 16: return by_group<ST, ST, D, 16>(a, st);
    case 32: return by_group<ST, ST, D, 32>(a, st);
    case 64: return by_group<ST, ST, D, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

// FP8 pools: head_dim 128, blocks of 16 tokens or more
template <typename ST>
hipError_t by_block_fp8(const PrefillArgs& a, hipStream_t st) {
  if (a.head_dim != 128) return hipErrorInvalidValue;
  switch (a.block_size) {
    case 16: return by_group<ST, FP8, 128, 16>(a, st);
    case 32: return by_group<ST, FP8, 128, 32>(a, st);
    case 64: return by_group<ST, FP8, 128, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename ST>
hipError_t by_dim(const PrefillArgs& a, hipStream_t st) {
  if (a.kv_fp8) return by_block_fp8<ST>(a, st);
  switch (a.head_dim) {
    case 64: return by_block<ST, 64>(a, st);
    case 128: return by_block<ST, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t prefill_lds_bytes(int32_t dtype, int32_t head_dim, int32_t block_size, int32_t max_context_len) {
  (void)dtype;  // both matrix-core types are 16-bit
  const size_t stage = static_cast<size_t>(kKeys) * (head_dim + 8) + static_cast<size_t>(head_dim) * (kKeys + 8);
  const size_t max_tiles = (static_cast<size_t>(max_context_len) + kKeys - 1) / kKeys;
  const size_t blocks_per_tile = block_size >= kKeys ? 1 : kKeys / block_size;
  // table entries of every tile, or the item costs of the longest-first
  // ordering if more
  return 2 * stage * 2 + std::max<size_t>(max_tiles * blocks_per_tile, kSortMax) * sizeof(int32_t);
}

int32_t prefill_choose_splits(int32_t num_seqs, int32_t num_kv_heads, int32_t group, int32_t max_q_len,
                              int32_t max_context_len) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || group <= 0 || max_q_len <= 0 || max_context_len <= 0) return 1;
  const int64_t tok = kRows / group;  // tokens per row tile
  const int64_t row_tiles = (max_q_len + tok - 1) / tok;
  const int64_t units = static_cast<int64_t>(num_seqs) * num_kv_heads;
  const int64_t grid = (units + kXcds - 1) / kXcds * kXcds * row_tiles;
  if (grid >= kPrefillTargetItems) return 1;
  int64_t k = (kPrefillTargetItems + grid - 1) / grid;
  const int64_t tiles = (static_cast<int64_t>(max_context_len) + kKeys - 1) / kKeys;
  k = std::min<int64_t>(k, std::max<int64_t>(1, tiles / 4));
  return static_cast<int32_t>(std::min<int64_t>(k, kPrefillMaxSplits));
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case 1: return by_dim<F16>(a, st);
    case 2: return by_dim<BF16>(a, st);
  }
  return hipErrorInvalidValue;
}

PA_DEBUG_UNIT(prefill)

}  // namespace pa
