// Prefix-grouped decode: sequences of one batch that share the physical
// blocks of a prompt prefix read those blocks once for all of them.
//
// Within a batch, requests forked from one prompt keep the prompt's blocks
// by reference and only copy a block on their first write to it
// (lshu.cn/news/11644, "收益分析"); the same page names prefix caching
// within the batch as one of the few decode-side savings, decode being
// bound by the KV bytes it reads ("性能关键路径与瓶颈").  Plain decode still
// reads the shared blocks once per sequence.  Here the decode of a step is
// split by keys, which attention allows because partial results over
// disjoint key sets combine exactly through their log-sum-exp (the same
// merge as split-K decode):
//
//  * a planner (one workgroup) cuts the batch into chunks of consecutive
//    sequences -- the caller's groups, split so that a chunk's q rows
//    (members x q heads per KV head) fit one 32-row matrix tile -- and
//    measures on the block tables themselves how many leading full blocks
//    each member has in common with the chunk's longest sequence (its
//    reference).  The caller's grouping is only a hint: a sequence that
//    shares nothing gets a shared length of 0 and is decoded alone;
//  * one persistent kernel then walks two work lists.  A shared-prefix item
//    is a (chunk, KV head, partition): all of the chunk's rows run over the
//    reference's blocks on the matrix cores, S^T = K Q^T and O^T = V^T P^T
//    with v_mfma_f32_32x32x16, each row masked at its own shared length.  A
//    suffix item is a (sequence, KV head, partition) of the sequence's own
//    tokens, decoded like split decode.  Prefix items come first (they are
//    the longest), so suffix items fill in behind them;
//  * private tails of at most 64 keys are not items of their own: the last
//    prefix partition of the chunk takes them as extra masked tiles (most
//    forks diverge only a few tokens before the step);
//  * every item leaves (max, sum, output) partials in workspace slots (a
//    sequence whose only slot is one suffix partition writes its output
//    directly); a merge kernel combines each sequence's slots by
//    log-sum-exp.  Merging inside the persistent kernel instead, by the
//    last item of each sequence, needs device-scope release fences (an L2
//    write-back per item on this chip) and measured many times slower.
//
// The result equals plain decode over each sequence's own table: a member
// reads only blocks whose table entries equal its own.
#include <algorithm>
#include <atomic>
#include <climits>

#include "common.h"
#include "decode_item.h"
#include "launch.h"
#include "mfma.h"

namespace pa {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kTile = 32;  // keys per matrix tile
constexpr int kSufBuckets = 32;  // size classes of the suffix work list
constexpr int kFoldTail = 64;  // private tails up to this many keys ride along with the shared prefix

// Inclusive scan of x over the workgroup (kPlanThreads threads) under the
// associative `op`; `total` receives the reduction over all threads.
template <typename T, typename Op>
__device__ __forceinline__ T block_scan(T x, T ident, Op op, T* wave_tot, T& total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_up(x, o, 64);
    if (lane >= o) x = op(x, y);
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  T before = ident, all = ident;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    const T t = wave_tot[w];
    if (w < wave) before = op(before, t);
    all = op(all, t);
  }
  __syncthreads();  // wave_tot is rewritten by the next scan
  total = all;
  return op(before, x);
}

struct PlanParams {
  const int32_t* group_start;
  const int32_t* tables;
  const int32_t* ctx_lens;
  int32_t* seq_start;
  int32_t* slot_base;
  int32_t* nslots;
  int32_t* pre_items;
  int32_t* pre_count;
  int32_t* suf_items;
  int32_t* suf_count;
  int num_groups, num_seqs, max_context, max_blocks, block_size, part_tokens, chunk_max;
};

__global__ __launch_bounds__(kPlanThreads) void grouped_plan_kernel(PlanParams P) {
  __shared__ int ref_of[kGroupedMaxSeqs];  // chunk start, then the chunk's reference
  __shared__ int share[kGroupedMaxSeqs];   // shared tokens (block multiple); a reference holds its chunk's max
  __shared__ int len[kGroupedMaxSeqs];     // clamped context lengths
  __shared__ int wtot_i[kPlanWaves];
  __shared__ int bucket_count[kSufBuckets];
  const int S = P.num_seqs, tid = threadIdx.x, BS = P.block_size;

  // 1. run starts: sequence 0 and every in-range group start
  for (int s = tid; s < S; s += kPlanThreads) {
    ref_of[s] = s == 0;
    len[s] = clamp_len(P.ctx_lens[s], P.max_context);
  }
  __syncthreads();
  for (int g = tid; g < P.num_groups; g += kPlanThreads) {
    const int st = P.group_start[g];
    if (st > 0 && st < S) ref_of[st] = 1;
  }
  __syncthreads();

  // 2. run start of each sequence (running max of flagged indices), then
  //    runs cut into chunks of at most chunk_max members
  int carry = 0;
  for (int base = 0; base < S; base += kPlanThreads) {
    const int s = base + tid;
    const int v = (s < S && ref_of[s]) ? s : 0;
    int pass_max = 0;
    const int run = max(carry, block_scan(v, 0, [](int a, int b) { return max(a, b); }, wtot_i, pass_max));
    if (s < S) ref_of[s] = run + ((s - run) / P.chunk_max) * P.chunk_max;
    carry = max(carry, pass_max);
  }
  __syncthreads();

  // 3. each chunk's reference: its longest member (the first of equals),
  //    found by the chunk's first sequence and parked in `share` (not yet
  //    in use), then copied to every member
  for (int s = tid; s < S; s += kPlanThreads) {
    if (ref_of[s] != s) continue;
    int n = 1, best = s;
    while (n < P.chunk_max && s + n < S && ref_of[s + n] == s) {
      if (len[s + n] > len[best]) best = s + n;
      ++n;
    }
    share[s] = best;
  }
  __syncthreads();
  for (int s = tid; s < S; s += kPlanThreads) ref_of[s] = share[ref_of[s]];
  __syncthreads();

  // 4. leading full blocks each member has in common with its reference.
  //    `lpm` adjacent lanes share a sequence (as many as the batch leaves
  //    room for) and compare 8 entries each per step, interleaved.
  int lpm = 1;
  while (lpm < 64 && S * lpm * 2 <= kPlanThreads) lpm *= 2;
  for (int base = 0; base < S * lpm; base += kPlanThreads) {
    const int v = base + tid, s = v / lpm, sub = v % lpm;
    const int ref = s < S ? ref_of[s] : 0;
    const int lim = (s < S && ref != s) ? min(len[s], len[ref]) / BS : 0;
    const int32_t* a = P.tables + static_cast<int64_t>(s < S ? s : 0) * P.max_blocks;
    const int32_t* b = P.tables + static_cast<int64_t>(ref) * P.max_blocks;
    int common = 0;
    while (common < lim) {  // the same trip count for the lpm lanes of a sequence
      int first = INT_MAX;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = common + sub + lpm * e;
        if (j < lim && a[j] != b[j]) first = min(first, j);
      }
      for (int o = 1; o < lpm; o <<= 1) first = min(first, __shfl_xor(first, o, 64));
      if (first != INT_MAX) {
        common = first;
        break;
      }
      common += 8 * lpm;
    }
    if (s < S && sub == 0) share[s] = min(common, lim) * BS;
  }
  __syncthreads();
  for (int s = tid; s < S; s += kPlanThreads) {
    const int ref = ref_of[s];
    if (ref != s && share[s] > 0) atomicMax(&share[ref], share[s]);
  }
  __syncthreads();

  // 5. work lists.  Prefix items (first member, members, partition,
  //    reference) for each chunk with a shared prefix, emitted by the
  //    chunk's first sequence; suffix items (sequence, partition) over each
  //    sequence's own tokens are counted per size class here and placed in
  //    step 6.
  int carry2 = 0;
  const int PT = P.part_tokens;
  // size class of a suffix item of t tokens
  auto suf_bucket = [&](int t) { return static_cast<int>((static_cast<int64_t>(t - 1) * kSufBuckets) / PT); };
  for (int k = tid; k < kSufBuckets; k += kPlanThreads) bucket_count[k] = 0;
  __syncthreads();
  for (int base = 0; base < S; base += kPlanThreads) {
    const int s = base + tid;
    int own_pre = 0, np = 0, sh = 0, sb = 0, ref = 0;
    if (s < S) {
      ref = ref_of[s];
      sh = share[s];
      sb = (share[ref] + PT - 1) / PT;
      if (s == 0 || ref_of[s - 1] != ref) own_pre = sb;  // first of its chunk
      const int tail = len[s] - sh;
      np = tail <= 0 || (sb > 0 && tail <= kFoldTail) ? 0 : (tail + PT - 1) / PT;
    }
    int total = 0;
    const int pfirst = carry2 + block_scan(own_pre, 0, [](int a, int b) { return a + b; }, wtot_i, total) - own_pre;
    if (s < S) {
      P.seq_start[s] = sh;
      P.slot_base[s] = sb;
      P.nslots[s] = sb + np;
      if (own_pre > 0) {
        int n = 1;
        while (n < P.chunk_max && s + n < S && ref_of[s + n] == ref) ++n;
        for (int p = 0; p < own_pre; ++p) {
          int32_t* it = P.pre_items + 4 * (pfirst + p);
          it[0] = s;
          it[1] = n;
          it[2] = p;
          it[3] = ref;
        }
      }
      if (np > 1) atomicAdd(&bucket_count[kSufBuckets - 1], np - 1);
      if (np > 0) atomicAdd(&bucket_count[suf_bucket(len[s] - sh - (np - 1) * PT)], 1);
    }
    carry2 += total;
  }
  __syncthreads();

  // 6. suffix items in falling size (a counting sort over size classes):
  //    the persistent kernel deals positions out round robin, so the short
  //    items come last and fill in behind the long ones
  if (tid == 0) {
    int acc = 0;
    for (int k = kSufBuckets - 1; k >= 0; --k) {
      const int c = bucket_count[k];
      bucket_count[k] = acc;
      acc += c;
    }
    *P.pre_count = carry2;
    *P.suf_count = acc;
  }
  __syncthreads();
  for (int s = tid; s < S; s += kPlanThreads) {
    const int sh = share[s];
    const int sb = (share[ref_of[s]] + PT - 1) / PT;
    const int tail = len[s] - sh;
    const int np = tail <= 0 || (sb > 0 && tail <= kFoldTail) ? 0 : (tail + PT - 1) / PT;
    if (np > 1) {
      const int first = atomicAdd(&bucket_count[kSufBuckets - 1], np - 1);
      for (int p = 0; p < np - 1; ++p) {
        P.suf_items[2 * (first + p)] = s;
        P.suf_items[2 * (first + p) + 1] = p;
      }
    }
    if (np > 0) {
      const int at = atomicAdd(&bucket_count[suf_bucket(tail - (np - 1) * PT)], 1);
      P.suf_items[2 * at] = s;
      P.suf_items[2 * at + 1] = np - 1;
    }
  }
}

struct GroupedParams {
  DecodeParams dec;          // the suffix work list in items / n_items
  const int32_t* seq_start;  // shared tokens per sequence; a reference holds its chunk's maximum
  const int32_t* slot_base;
  const int32_t* nslots;
  const int32_t* pre_items;  // (first member, members, partition, reference)
  const int32_t* pre_count;
};

template <int D>
struct PrefixLds {
  float o[kWaves][32][D + 4];  // per-wave unnormalised O rows
  float m[kWaves][32];
  float l[kWaves][32];
  float c[kWaves][32];  // merge weights
  float inv[32];
};

template <int G, int D, int BS>
union GroupedLds {
  DecodeLds<G, D, BS> dec;
  PrefixLds<D> pre;
};

// Eight pool elements from p as one MFMA operand of the 16-bit type AT:
// one 16-byte load, or 8 E4M3 codes widened exactly.
template <typename ST, typename AT>
__device__ __forceinline__ u32x4 load8_operand(const typename ST::elem* p) {
  if constexpr (ST::bytes == 1) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    const uint32_t w0 = w[0], w1 = w[1];
    return u32x4{widen_fp8_pair<AT, false>(w0), widen_fp8_pair<AT, true>(w0), widen_fp8_pair<AT, false>(w1),
                 widen_fp8_pair<AT, true>(w1)};
  } else {
    return load16_nt(p);
  }
}

// A shared-prefix item: the rows r = member * G + h of one chunk over one
// partition of the shared prefix, keys read through the reference's table;
// wave w takes key tiles w, w + 4, ...  Writes slot `part` of every member.
// ST: the pool's element type; AT: the activation (matrix) type.
template <typename ST, int D, int BS, int G, typename AT>
__device__ __forceinline__ void prefix_item(PrefixLds<D>& sh, const GroupedParams& GP, int item, int kvh, int& first,
                                            int& members) {
  static_assert(D % 32 == 0 && D >= 64, "head_dim");
  static_assert(BS == 8 || BS == 16 || BS == 32 || BS == 64, "block size");
  constexpr int KS = D / 16;      // contraction steps of S^T = K Q^T
  constexpr int DT = D / 32;      // 32-wide column tiles of O^T
  using elem = typename ST::elem;
  using qelem = typename AT::elem;
  const DecodeParams& P = GP.dec;
  const qelem* __restrict__ q = static_cast<const qelem*>(P.q);
  const elem* __restrict__ kc = static_cast<const elem*>(P.kc);
  const elem* __restrict__ vc = static_cast<const elem*>(P.vc);
  const int hk = P.num_kv_heads, hq = hk * G;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 31;   // row of this lane (B operand column / accumulator column)
  const int hf = lane >> 5;  // half: k-elements 8*hf.. of each step
  const int64_t blk_stride = static_cast<int64_t>(hk) * BS * D;

  first = __builtin_amdgcn_readfirstlane(GP.pre_items[4 * item]);
  members = __builtin_amdgcn_readfirstlane(GP.pre_items[4 * item + 1]);
  const int part = __builtin_amdgcn_readfirstlane(GP.pre_items[4 * item + 2]);
  const int ref = __builtin_amdgcn_readfirstlane(GP.pre_items[4 * item + 3]);
  const int share_max = __builtin_amdgcn_readfirstlane(GP.seq_start[ref]);
  const int tok0 = part * P.part_tokens;
  const int tok1 = min(share_max, tok0 + P.part_tokens);
  const int ntiles = (tok1 - tok0 + kTile - 1) / kTile;
  const int mem = r / G, hh = r - mem * G;
  const bool row_ok = mem < members;
  const int row_lim = row_ok ? GP.seq_start[first + mem] : 0;

  // Q^T as the B operand: row r, dims 8 * (2k + hf) ..
  u32x4 qb[KS];
  const qelem* qrow = q + (static_cast<int64_t>(first + (row_ok ? mem : 0)) * hq + kvh * G + hh) * D + 8 * hf;
#pragma unroll
  for (int k = 0; k < KS; ++k) qb[k] = row_ok ? load16(qrow + 16 * k) : u32x4{0, 0, 0, 0};

  // the partition's block ids, one per lane (64 * BS >= part_tokens)
  const int32_t* trow = P.tables + static_cast<int64_t>(ref) * P.max_blocks + tok0 / BS;
  const int nblk = (tok1 - tok0 + BS - 1) / BS;
  int bid = lane < nblk ? trow[lane] : 0;
  bid = (bid >= 0 && bid < P.num_blocks) ? bid : 0;

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // K rows in A-operand order (key_perm) and V^T rows for the PV steps.
  // Keys at or past tok1 (the last tile's end when the shared length is not
  // a multiple of 32) are masked out of the scores, but their V rows still
  // meet a zero probability in the PV products, and 0 * NaN is NaN: unused
  // slots may hold NaN, so such 8-key groups (tok1 is a block multiple, so
  // a group is wholly in or out) read the partition's first keys instead.
  const int kkey = key_perm(r);
  auto load_tile = [&](int t, u32x4* kr, u32x4* vr) __attribute__((always_inline)) {
    // keys are counted from the partition's start (a block boundary)
    const int kabs = t * kTile + kkey;
    const int kb = __shfl(bid, kabs / BS, 64);
    const elem* kp =
        kc + static_cast<int64_t>(kb) * blk_stride + (static_cast<int64_t>(kvh) * BS + kabs % BS) * D + 8 * hf;
#pragma unroll
    for (int k = 0; k < KS; ++k) kr[k] = load8_operand<ST, AT>(kp + 16 * k);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int key0 = 16 * k + 8 * hf;  // first of this lane's 8 keys in the step
      const bool in = tok0 + t * kTile + key0 < tok1;
      const int key = in ? t * kTile + key0 : 0;
      const int vb = __shfl(bid, key / BS, 64);
      const elem* vp = vc + static_cast<int64_t>(vb) * blk_stride + (static_cast<int64_t>(kvh) * D + r) * BS + key % BS;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vr[dt * 2 + k] = load8_operand<ST, AT>(vp + dt * 32 * BS);
    }
  };

  // One key tile: scores, online softmax, PV.  P enters the PV products as
  // two 16-bit parts (nearest value and remainder), so the weights keep
  // about 16 bits: rows with only a few shared keys can have outputs as
  // large as single V entries, where one 16-bit rounding of P would show.
  auto compute = [&](int key0, int lim, const u32x4* kr, const u32x4* vr) __attribute__((always_inline)) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int k = 0; k < KS; ++k) s = mfma32<AT>(kr[k], qb[k], s);

    float x[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = key0 + key_perm(8 * (e >> 2) + 4 * hf + (e & 3));
      x[e] = key < lim ? s[e] * P.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, x[e]);
    }
    tmax = halves_max(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      x[e] = __builtin_amdgcn_exp2f(x[e] - m_use);
      psum += x[e];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    u32x4 hi[2], lo[2];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float a0 = x[8 * k + 2 * c], a1 = x[8 * k + 2 * c + 1];
        const uint32_t h = pack2<AT>(a0, a1);
        float h0, h1;
        widen2<AT>(h, h0, h1);
        hi[k][c] = h;
        lo[k][c] = pack2<AT>(a0 - h0, a1 - h1);
      }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      o[dt] *= alpha;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        o[dt] = mfma32<AT>(vr[dt * 2 + k], hi[k], o[dt]);
        o[dt] = mfma32<AT>(vr[dt * 2 + k], lo[k], o[dt]);
      }
    }
  };

  // two register buffers alternate, the next tile's loads in flight while
  // the current one is computed (at the end the last tile is requested
  // again: a cache hit)
  const int my_tiles = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;
  const int last = wave + (my_tiles - 1) * kWaves;
  u32x4 k0[KS], v0[2 * DT], k1[KS], v1[2 * DT];
  if (my_tiles > 0) load_tile(wave, k0, v0);
  for (int i = 0; i < my_tiles; i += 2) {
    const int t = wave + i * kWaves;
    load_tile(min(t + kWaves, last), k1, v1);
    compute(tok0 + t * kTile, row_lim, k0, v0);
    if (i + 1 < my_tiles) {
      load_tile(min(t + 2 * kWaves, last), k0, v0);
      compute(tok0 + (t + kWaves) * kTile, row_lim, k1, v1);
    }
  }

  // The last partition also takes the members' short private tails (keys
  // share..L-1 read through the member's own table, at most kFoldTail of
  // them): one tile per 32 keys, scored for all rows but kept only for the
  // member's own.  Tiles go round robin over the waves.
  if (part == (share_max + P.part_tokens - 1) / P.part_tokens - 1) {
    // lane m holds member m's shared length and context length
    const int tl0 = lane < members ? GP.seq_start[first + lane] : 0;
    const int tlL = lane < members ? clamp_len(P.ctx_lens[first + lane], P.max_context) : 0;
    int g = 0;  // running tile index over the members
    for (int m = 0; m < members; ++m) {
      const int t0 = __builtin_amdgcn_readlane(tl0, m);
      const int Lm = __builtin_amdgcn_readlane(tlL, m);
      const int tail = Lm - t0;
      if (tail <= 0 || tail > kFoldTail) continue;
      const int32_t* mrow = P.tables + static_cast<int64_t>(first + m) * P.max_blocks;
      for (int key0 = t0; key0 < Lm; key0 += kTile, ++g) {
        if (g % kWaves != wave) continue;
        // keys past the tail read the tail's last block again (masked)
        const int kb0 = mrow[min(key0 + kkey, Lm - 1) / BS];
        const int kb = (kb0 >= 0 && kb0 < P.num_blocks) ? kb0 : 0;
        const elem* kp = kc + static_cast<int64_t>(kb) * blk_stride +
                         (static_cast<int64_t>(kvh) * BS + (key0 + kkey) % BS) * D + 8 * hf;
#pragma unroll
        for (int k = 0; k < KS; ++k) k0[k] = load8_operand<ST, AT>(kp + 16 * k);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int key = key0 + 16 * k + 8 * hf;
          const int vb0 = mrow[min(key, Lm - 1) / BS];
          const int vb = (vb0 >= 0 && vb0 < P.num_blocks) ? vb0 : 0;
          const elem* vp =
              vc + static_cast<int64_t>(vb) * blk_stride + (static_cast<int64_t>(kvh) * D + r) * BS + key % BS;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) v0[dt * 2 + k] = load8_operand<ST, AT>(vp + dt * 32 * BS);
        }
        // keys at or past Lm: unused slots that may hold NaN, zeroed (their
        // zero probabilities would not cancel a NaN)
        if (key0 + kTile > Lm) {
#pragma unroll
          for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const int key = key0 + 16 * k + 8 * hf + 2 * c;
              const uint32_t keep = (key < Lm ? 0x0000ffffu : 0u) | (key + 1 < Lm ? 0xffff0000u : 0u);
#pragma unroll
              for (int dt = 0; dt < DT; ++dt) v0[dt * 2 + k][c] &= keep;
            }
        }
        compute(key0, mem == m ? Lm : 0, k0, v0);
      }
    }
  }

  // merge the four wavefronts' states of each row into the members' slots
  const float l_tot = halves_sum(l_run);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float4 v4 = {o[dt][4 * j], o[dt][4 * j + 1], o[dt][4 * j + 2], o[dt][4 * j + 3]};
      *reinterpret_cast<float4*>(&sh.o[wave][r][dt * 32 + 8 * j + 4 * hf]) = v4;
    }
  if (hf == 0) {
    sh.m[wave][r] = m_run;
    sh.l[wave][r] = l_tot;
  }
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < 32) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (sh.l[w][tid] > 0.f) M = fmaxf(M, sh.m[w][tid]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float c = sh.l[w][tid] > 0.f ? __builtin_amdgcn_exp2f(sh.m[w][tid] - M) : 0.f;
      sh.c[w][tid] = c;
      L += c * sh.l[w][tid];
    }
    // (an FP8 pool's V scale enters here, as in the decode items)
    sh.inv[tid] = L > 0.f ? (ST::bytes == 1 ? P.v_scale : 1.f) / L : 0.f;
    const int mm = tid / G;
    if (mm < members) {
      const int64_t pidx = (static_cast<int64_t>(first + mm) * hq + kvh * G + tid % G) * P.max_parts + part;
      P.ws_ml[2 * pidx] = M;
      P.ws_ml[2 * pidx + 1] = L;
    }
  }
  __syncthreads();
  for (int e = tid; e < 32 * D; e += kThreads) {
    const int row = e / D, d = e - row * D;
    const int mm = row / G;
    if (mm >= members) continue;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc = __builtin_fmaf(sh.c[w][row], sh.o[w][row][d], acc);
    const int64_t pidx = (static_cast<int64_t>(first + mm) * hq + kvh * G + row % G) * P.max_parts + part;
    P.ws_o[pidx * D + d] = acc * sh.inv[row];
  }
}

// The persistent kernel: prefix items, then suffix items, each times the KV
// heads.  A suffix item that is its sequence's only slot writes the output
// directly; every other item leaves partials for the merge kernel.
template <typename ST, int D, int BS, int G, typename AT>
__global__ __launch_bounds__(kThreads, 2) void grouped_decode_kernel(GroupedParams GP) {
  __shared__ GroupedLds<G, D, BS> sh;
  const DecodeParams& P = GP.dec;
  const int hk = P.num_kv_heads;
  const int n_pre = __builtin_amdgcn_readfirstlane(*GP.pre_count) * hk;
  const int n_all = n_pre + __builtin_amdgcn_readfirstlane(*P.n_items) * hk;
  for (int it = blockIdx.x; it < n_all; it += gridDim.x) {
    __syncthreads();  // the previous item is done with LDS
    if (it < n_pre) {
      const int item = it / hk;
      int first, members;
      prefix_item<ST, D, BS, G, AT>(sh.pre, GP, item, it - item * hk, first, members);
    } else {
      const int j = it - n_pre, item = j / hk;
      const int s = __builtin_amdgcn_readfirstlane(P.items[2 * item]);
      const int part = __builtin_amdgcn_readfirstlane(P.items[2 * item + 1]);
      const int L = clamp_len(P.ctx_lens[s], P.max_context);
      const bool only = __builtin_amdgcn_readfirstlane(GP.nslots[s]) == 1 &&
                        __builtin_amdgcn_readfirstlane(GP.slot_base[s]) == 0;
      decode_item<ST, D, BS, G, AT>(sh.dec, P, s, j - item * hk, part, L,
                                    __builtin_amdgcn_readfirstlane(GP.seq_start[s]),
                                __builtin_amdgcn_readfirstlane(GP.slot_base[s]), !only);
    }
  }
}

// Log-sum-exp merge of each (sequence, KV head)'s slots: grid (KV head,
// sequence), G rows of D outputs.  The slot weights of the G rows go to LDS
// first (G * max_parts floats of dynamic LDS), so the output loop's loads are
// independent.  Slots without keys (sum 0) carry no weight; a row with none
// (context 0) is written as zeros.  Rows written directly by the decode
// kernel are skipped.
template <typename AT, int D, int G>
__global__ __launch_bounds__(kThreads) void grouped_merge_kernel(DecodeParams P, const int32_t* __restrict__ nslots,
                                                                const int32_t* __restrict__ slot_base) {
  extern __shared__ float w_sh[];  // [G][max_parts]
  __shared__ float M_sh[G];
  const int kvh = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int ns = min(nslots[s], P.max_parts);
  if (ns == 1 && slot_base[s] == 0) return;
  const int hq = P.num_kv_heads * G, mp = P.max_parts;
  const int64_t qh0 = static_cast<int64_t>(s) * hq + kvh * G;
  const float* ml = P.ws_ml + 2 * qh0 * mp;  // the G rows' slots are contiguous
  for (int i = tid; i < G * ns; i += kThreads) {
    const int h = i / ns, p = i - h * ns;
    const float l = ml[2 * (h * mp + p) + 1];
    w_sh[h * mp + p] = l > 0.f ? ml[2 * (h * mp + p)] : -INFINITY;
  }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int p = 0; p < ns; ++p) M = fmaxf(M, w_sh[tid * mp + p]);
    M_sh[tid] = M;
  }
  __syncthreads();
  for (int i = tid; i < G * ns; i += kThreads) {
    const int h = i / ns, p = i - h * ns;
    const float m = w_sh[h * mp + p];
    w_sh[h * mp + p] = m == -INFINITY ? 0.f : ml[2 * (h * mp + p) + 1] * __builtin_amdgcn_exp2f(m - M_sh[h]);
  }
  __syncthreads();
  typename AT::elem* out = static_cast<typename AT::elem*>(P.out);
  for (int e = tid; e < G * D; e += kThreads) {
    const int h = e / D, d = e - h * D;
    const float* o = P.ws_o + (qh0 + h) * mp * D + d;
    const float* w = w_sh + h * mp;
    float num = 0.f, den = 0.f;
    for (int p = 0; p < ns; ++p) {
      num = __builtin_fmaf(w[p], o[static_cast<int64_t>(p) * D], num);
      den += w[p];
    }
    out[(qh0 + h) * D + d] = narrow<AT>(den > 0.f ? num / den : 0.f);
  }
}

// Workgroups of the persistent kernel that fit on the device at once.
template <typename ST, int D, int BS, int G, typename AT>
int grouped_grid() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cached[kMaxDev];  // 0 = not yet queried; racing writers store the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) dev = 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&grouped_decode_kernel<ST, D, BS, G, AT>), kThreads, 0) !=
            hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    n = cus * per_cu;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <typename ST, int D, int BS, int G, typename AT>
hipError_t launch_t(const GroupedArgs& g, hipStream_t st) {
  const DecodeArgs& a = g.d;
  PlanParams pp{};
  pp.group_start = g.group_start;
  pp.tables = a.block_tables;
  pp.ctx_lens = a.context_lens;
  pp.seq_start = g.seq_start;
  pp.slot_base = g.slot_base;
  pp.nslots = g.nslots;
  pp.pre_items = g.pre_items;
  pp.pre_count = g.pre_count;
  pp.suf_items = a.ws_items;
  pp.suf_count = a.ws_count;
  pp.num_groups = g.num_groups;
  pp.num_seqs = a.num_seqs;
  pp.max_context = a.max_context_len;
  pp.max_blocks = a.max_blocks_per_seq;
  pp.block_size = BS;
  pp.part_tokens = a.part_tokens;
  pp.chunk_max = 32 / G;
  hipLaunchKernelGGL(grouped_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, pp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  GroupedParams P{};
  P.dec.q = a.q;
  P.dec.kc = a.k_cache;
  P.dec.vc = a.v_cache;
  P.dec.tables = a.block_tables;
  P.dec.ctx_lens = a.context_lens;
  P.dec.items = a.ws_items;
  P.dec.n_items = a.ws_count;
  P.dec.out = a.out;
  P.dec.ws_ml = a.ws_ml;
  P.dec.ws_o = a.ws_o;
  P.dec.scale_log2 = a.scale * kLog2e * a.k_scale;
  P.dec.v_scale = a.v_scale;
  P.dec.max_blocks = a.max_blocks_per_seq;
  P.dec.max_context = a.max_context_len;
  P.dec.num_blocks = a.num_blocks;
  P.dec.num_kv_heads = a.num_kv_heads;
  P.dec.part_tokens = a.part_tokens;
  P.dec.max_parts = a.num_parts;
  P.seq_start = g.seq_start;
  P.slot_base = g.slot_base;
  P.nslots = g.nslots;
  P.pre_items = g.pre_items;
  P.pre_count = g.pre_count;
  // both item lists are bounded by sequences x partitions of the longest context
  const int64_t parts =
      std::max<int64_t>(1, (static_cast<int64_t>(a.max_context_len) + a.part_tokens - 1) / a.part_tokens);
  const int64_t upper = (a.num_seqs / 2 + a.num_seqs) * parts * a.num_kv_heads;
  const int grid =
      static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(upper, grouped_grid<ST, D, BS, G, AT>())));
  hipLaunchKernelGGL((grouped_decode_kernel<ST, D, BS, G, AT>), dim3(grid), dim3(kThreads), 0, st, P);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((grouped_merge_kernel<AT, D, G>), dim3(a.num_kv_heads, a.num_seqs), dim3(kThreads),
                     static_cast<size_t>(G) * a.num_parts * sizeof(float), st, P.dec, g.nslots, g.slot_base);
  return hipGetLastError();
}

template <typename ST, int D, int BS, typename AT>
hipError_t by_group(const GroupedArgs& a, hipStream_t st) {
  switch (a.d.group) {
    case 1: return launch_t<ST, D, BS, 1, AT>(a, st);
    case 2: return launch_t<ST, D, BS, 2, AT>(a, st);
    case 4: return launch_t<ST, D, BS, 4, AT>(a, st);
    case 8: return launch_t<ST, D, BS, 8, AT>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename ST, int D, typename AT>
hipError_t by_block(const GroupedArgs& a, hipStream_t st) {
  switch (a.d.block_size) {
    case 8:
      if constexpr (ST::bytes == 1) return hipErrorInvalidValue;  // FP8 pools hold blocks of 16 tokens or more
      else return by_group<ST, D, 8, AT>(a, st);
    case 16: return by_group<ST, D, 16, AT>(a, st);
    case 32: return by_group<ST, D, 32, AT>(a, st);
    case 64: return by_group<ST, D, 64, AT>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename ST>
hipError_t by_dim(const GroupedArgs& a, hipStream_t st) {
  switch (a.d.head_dim) {
    case 64: return by_block<ST, 64, ST>(a, st);
    case 128: return by_block<ST, 128, ST>(a, st);
  }
  return hipErrorInvalidValue;
}

// FP8 pools (head_dim 128) with 16-bit activations
template <typename AT>
hipError_t by_act_fp8(const GroupedArgs& a, hipStream_t st) {
  if (a.d.head_dim != 128) return hipErrorInvalidValue;
  return by_block<FP8, 128, AT>(a, st);
}

}  // namespace

hipError_t launch_decode_grouped(const GroupedArgs& a, hipStream_t st) {
  if (a.d.dtype == 3) {
    switch (a.d.act_dtype) {
      case 1: return by_act_fp8<F16>(a, st);
      case 2: return by_act_fp8<BF16>(a, st);
    }
    return hipErrorInvalidValue;
  }
  switch (a.d.dtype) {
    case 1: return by_dim<F16>(a, st);
    case 2: return by_dim<BF16>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
