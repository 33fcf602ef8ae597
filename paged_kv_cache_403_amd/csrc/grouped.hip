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
//  * a persistent kernel walks the shared-prefix items.  An item is a
//    (chunk, KV head, partition): all of the chunk's rows run over the
//    reference's blocks on the matrix cores, S^T = K Q^T and O^T = V^T P^T
//    with v_mfma_f32_32x32x16, each row masked at its own shared length.
//    K and V travel from HBM straight into per-wavefront rings in LDS
//    (global_load_lds), so the loads in flight do not hold registers;
//  * a second persistent kernel walks the suffix items: a (sequence, KV
//    head, partition) of the sequence's own tokens, decoded like split
//    decode and at its occupancy (one kernel for both lists has to hold
//    both paths' registers, and measured slower on both);
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
constexpr int kPreItemInts = 8;  // first member, members, partition, reference, shared length, 3 unused

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

  // 1. run starts: sequence 0 and every in-range group start (the lengths
  //    and the group starts load in the same round)
  for (int s = tid; s < S; s += kPlanThreads) ref_of[s] = s == 0;
  __syncthreads();
  for (int i = tid; i < max(S, P.num_groups); i += kPlanThreads) {
    const int L = i < S ? P.ctx_lens[i] : 0;
    const int st = i < P.num_groups ? P.group_start[i] : 0;
    if (i < S) len[i] = clamp_len(L, P.max_context);
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

  // 4. leading full blocks each member has in common with its reference:
  //    the first differing table entry.  `lpm` adjacent lanes share a
  //    sequence (as many as the batch leaves room for) and compare 16
  //    entries each per step, interleaved, until a step finds a difference.
  int lpm = 1;
  while (lpm < 64 && S * lpm * 2 <= kPlanThreads) lpm *= 2;
  for (int base = 0; base < S * lpm; base += kPlanThreads) {
    const int v = base + tid, s = v / lpm, sub = v % lpm;
    const int ref = s < S ? ref_of[s] : 0;
    const int lim = (s < S && ref != s) ? min(len[s], len[ref]) / BS : 0;
    const int32_t* a = P.tables + static_cast<int64_t>(s < S ? s : 0) * P.max_blocks;
    const int32_t* b = P.tables + static_cast<int64_t>(ref) * P.max_blocks;
    int first = lim;
    for (int j0 = 0; j0 < lim; j0 += 16 * lpm) {  // the same trip count for the lpm lanes of a sequence
      // entries past lim re-read entry lim - 1 (unconditional loads, all in
      // flight at once) and are not compared
      int av[16], bv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = min(j0 + sub + lpm * e, lim - 1);
        av[e] = a[j];
        bv[e] = b[j];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = j0 + sub + lpm * e;
        if (j < lim && av[e] != bv[e]) first = min(first, j);
      }
      for (int o = 1; o < lpm; o <<= 1) first = min(first, __shfl_xor(first, o, 64));
      if (first < lim) break;
    }
    if (s < S && sub == 0) share[s] = first * BS;
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
          int32_t* it = P.pre_items + kPreItemInts * (pfirst + p);
          it[0] = s;
          it[1] = n;
          it[2] = p;
          it[3] = ref;
          it[4] = share[ref];
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
  if (tid < 64) {  // exclusive scan of the class counts from the largest class down, by one wavefront
    const int k = kSufBuckets - 1 - tid;
    const int c = tid < kSufBuckets ? bucket_count[k] : 0;
    int x = c;
#pragma unroll
    for (int o = 1; o < kSufBuckets; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (tid >= o) x += y;
    }
    if (tid < kSufBuckets) bucket_count[k] = x - c;
    if (tid == kSufBuckets - 1) {
      *P.pre_count = carry2;
      *P.suf_count = x;
    }
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
  const int32_t* pre_items;  // kPreItemInts each: first member, members, partition, reference, shared length
  const int32_t* pre_count;
};

// Geometry of a shared-prefix item.  Each wavefront walks its own key tiles
// of 32 keys (as in the split decode items: tiles w, w + 4, ...) and streams
// them from HBM straight into a ring of its own in LDS (global_load_lds, 16
// bytes per lane) in parts of 64 dimensions: the K parts of a tile, then
// its V parts.  The loads in flight sit in LDS, not in registers, and a
// wavefront waits only for its own loads; two workgroups per compute unit
// (two wavefronts per SIMD) let one wavefront's matrix and softmax work
// cover the other's waits.
template <typename ST, int D>
struct PrefixGeom {
  static constexpr int DT = D / 32;            // 32-wide column tiles of O^T
  static constexpr int KS = D / 16;            // contraction steps of S^T = K Q^T
  static constexpr int KSPLIT = D / 64;        // K parts (and V parts) of a tile
  static constexpr int NP = 2 * KSPLIT;        // parts of a tile
  static constexpr int PROW = 64 * ST::bytes;  // bytes of a K row's part
  static constexpr int CPP = PROW / 16;        // 16-byte chunks per K row part
  static constexpr int LCPP = ilog2(CPP);
  static constexpr int KPC = 16 / ST::bytes;   // keys per 16-byte chunk of a V^T row
  static constexpr int PART = kTile * PROW;    // bytes of a part (K or V)
  static constexpr int NIP = PART / 1024;      // 1 KiB load instructions per part
  static constexpr int RW = 16 * 1024 / PART;  // parts in a wavefront's ring
  static_assert(D % 64 == 0 && NIP >= 1, "parts of 64 dimensions");
  static_assert(RW >= 3 && (RW - 2) * NIP < 64, "ring depth");
};

constexpr int kMaxTailTiles = 64;  // 32 members x at most 2 tiles of a short private tail

template <typename ST, int D, int BS>
struct PrefixLds {
  using Geo = PrefixGeom<ST, D>;
  static constexpr int NBT = kTile / BS > 0 ? kTile / BS : 1;  // blocks under a tile
  union {
    u32x4 ring[kWaves][Geo::RW * Geo::PART / 16];
    struct {
      float o[kWaves][32][D + 4];  // per-wave unnormalised O rows
      float m[kWaves][32];
      float l[kWaves][32];
      float c[kWaves][32];  // merge weights
      float inv[32];
    } mg;
  };
  int tail_member[kMaxTailTiles];  // tail tiles of the last partition: member,
  int tail_key0[kMaxTailTiles];    // first key,
  int tail_len[kMaxTailTiles];     // member's context length,
  int tail_blk[kMaxTailTiles][NBT];  // blocks of the tile's keys
};

// One 16-byte load per lane from HBM into LDS: lane l's bytes land at
// lds + 16 l (the LDS address is the wavefront's, the global one each
// lane's own).  Counted in vmcnt like any load; the compiler neither waits
// for it before LDS reads of those bytes nor orders them after it, so
// readers wait explicitly (wait_vm).
__device__ __forceinline__ void load_to_lds(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(lds), 16, 0, 0);
}

// Wait until at most N of this wave's vector memory operations are
// outstanding (they complete in issue order).  The "memory" clobber keeps
// the compiler from moving LDS reads of the loaded bytes above the wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// ... at most k * STEP, for a wave-uniform k <= K
template <int STEP, int K>
__device__ __forceinline__ void wait_vm_steps(int k) {
  if constexpr (K == 0) {
    wait_vm<0>();
  } else {
    if (k >= K) {
      wait_vm<K * STEP>();
      return;
    }
    wait_vm_steps<STEP, K - 1>(k);
  }
}
// This wave's LDS reads have returned (before a load overwrites what they read).
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Eight elements of a tile in LDS as one MFMA operand of the 16-bit type
// AT: 16 bytes, or 8 E4M3 codes (8 bytes) widened exactly.
template <typename ST, typename AT>
__device__ __forceinline__ u32x4 lds_operand(const char* p) {
  if constexpr (ST::bytes == 1) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    const uint32_t w0 = w[0], w1 = w[1];
    return u32x4{widen_fp8_pair<AT, false>(w0), widen_fp8_pair<AT, true>(w0), widen_fp8_pair<AT, false>(w1),
                 widen_fp8_pair<AT, true>(w1)};
  } else {
    return *reinterpret_cast<const u32x4*>(p);
  }
}

// A shared-prefix item: the rows r = member * G + h of one chunk over one
// partition of the shared prefix, keys read through the reference's table;
// wave w takes key tiles w, w + 4, ...  Writes slot `part` of every member.
// ST: the pool's element type; AT: the activation (matrix) type.
//
// LDS layout of a part: K as 32 rows (key order) of 64 dimensions whose
// 16-byte chunks are rotated by XOR with the low bits of the lane that
// reads the row, so that the lanes of a read phase hit distinct banks; V^T
// of 64 dimensions as [key chunk][dim] 16-byte chunks (KPC keys of one
// dimension each), which the operand reads sweep contiguously.
template <typename ST, int D, int BS, int G, typename AT>
__device__ __forceinline__ void prefix_item(PrefixLds<ST, D, BS>& sh, const GroupedParams& GP, int item, int kvh) {
  using Geo = PrefixGeom<ST, D>;
  static_assert(BS == 8 || BS == 16 || BS == 32 || BS == 64, "block size");
  constexpr int DT = Geo::DT, KS = Geo::KS, RW = Geo::RW, NIP = Geo::NIP, PART = Geo::PART;
  constexpr int KSPLIT = Geo::KSPLIT, NP = Geo::NP, CPP = Geo::CPP, KPC = Geo::KPC, LCPP = Geo::LCPP;
  constexpr int EB = ST::bytes;
  static_assert(BS % (64 / CPP) == 0 && BS % KPC == 0, "a load instruction stays inside one block");
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

  // What the item needs from HBM comes in three rounds: the item itself;
  // then the rows' shared lengths, q, the partition's block ids and (last
  // partition) the members' lengths; then the first K/V loads and the
  // private tails' block ids.
  const int32_t* itp = GP.pre_items + kPreItemInts * item;
  const int first = __builtin_amdgcn_readfirstlane(itp[0]);
  const int members = __builtin_amdgcn_readfirstlane(itp[1]);
  const int part = __builtin_amdgcn_readfirstlane(itp[2]);
  const int ref = __builtin_amdgcn_readfirstlane(itp[3]);
  const int share_max = __builtin_amdgcn_readfirstlane(itp[4]);
  const int tok0 = part * P.part_tokens;
  const int tok1 = min(share_max, tok0 + P.part_tokens);
  const int ntiles = (tok1 - tok0 + kTile - 1) / kTile;
  const int mem = r / G, hh = r - mem * G;
  const bool row_ok = mem < members;
  const bool last_part = part == (share_max + P.part_tokens - 1) / P.part_tokens - 1;
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

  // The last partition also takes the members' short private tails (keys
  // share..L-1 read through the member's own table, at most kFoldTail of
  // them): one tile per 32 keys, scored for all rows but kept only for the
  // member's own.  Lane m counts member m's tiles.
  const bool lane_mem = last_part && lane < members;
  const int t0 = lane_mem ? GP.seq_start[first + lane] : 0;
  const int Lm = lane_mem ? clamp_len(P.ctx_lens[first + lane], P.max_context) : 0;
  const int nt = (Lm - t0 > 0 && Lm - t0 <= kFoldTail) ? (Lm - t0 + kTile - 1) / kTile : 0;
  int incl = nt;  // inclusive prefix sum over the lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  const int ntail = __builtin_amdgcn_readlane(incl, 63);
  PA_DEBUG_COUNT(PA_DBG_BLOCK_ID, bid < 0 || bid >= P.num_blocks);
  bid = (bid >= 0 && bid < P.num_blocks) ? bid : 0;
  const int total = ntiles + ntail;
  const int my_tiles = total > wave ? (total - wave + kWaves - 1) / kWaves : 0;
  const int nparts = NP * my_tiles;

  // chunk rotation of K row `key`: the low bits of the lane that reads it
  // (lane key_perm(key) of each half), folded so that rows sharing a
  // 256-byte bank line in a read phase differ too
  auto swz = [](int key) __attribute__((always_inline)) {
    const int m = key_perm(key);
    return (m ^ (m >> LCPP)) & (CPP - 1);
  };
  // per-lane byte offsets, inside a block, of the 1 KiB load instructions
  // of a K part and of a V part of dimensions 0..63 (a tile starting at a
  // block's first key; a 64-key block adds 32 rows for its second tile)
  // (V instruction i covers key chunk i of dims `lane`: its offset is
  // voff0 plus a constant)
  uint32_t koff[NIP];
#pragma unroll
  for (int i = 0; i < NIP; ++i) {
    const int p = 64 * i + lane;
    const int key = p >> LCPP;
    const int c = (p & (CPP - 1)) ^ swz(key);
    koff[i] = static_cast<uint32_t>(((kvh * BS + key % BS) * D + c * KPC) * EB);
  }
  const uint32_t voff0 = static_cast<uint32_t>((kvh * D + lane) * BS * EB);

  char* const ring = reinterpret_cast<char*>(&sh.ring[wave][0]);
  const char* const kbase = reinterpret_cast<const char*>(kc);
  const char* const vbase = reinterpret_cast<const char*>(vc);
  const int64_t blk_bytes = blk_stride * EB;

  // Loads of part h of this wave (tile h / NP; part h % NP: K of
  // dimensions 64 q.. for q = h % NP < KSPLIT, else V of dimensions
  // 64 (q - KSPLIT)..) into ring slot h % RW.  Every instruction stays
  // inside one block, so its block id is wave-uniform.  V keys past the
  // shared length in the last shared tile come from the partition's first
  // block (unused slots may hold NaN, which a zero probability would not
  // cancel); a tail tile's keys past the member's length read that
  // member's last block, and zero_v_past clears their V.
  auto issue = [&](int h) __attribute__((always_inline)) {
    const int jt = h / NP, q = h - jt * NP;
    const int t = wave + kWaves * jt;
    const bool is_v = q >= KSPLIT;
    const int dim0 = 64 * (is_v ? q - KSPLIT : q);
    int blk[NIP];
    int row0;  // first row of the tile in its block (64-key blocks)
    if (t < ntiles) {
      const int rel0 = kTile * t;  // partition-relative
      row0 = BS == 64 ? rel0 % BS : 0;
#pragma unroll
      for (int i = 0; i < NIP; ++i) {
        const int key = is_v ? (64 * i / 64) * KPC : (64 * i) >> LCPP;  // first key of instruction i
        const int b = (rel0 + key) / BS;
        blk[i] = __builtin_amdgcn_readlane(bid, (is_v && b >= nblk) ? 0 : b);
      }
    } else {
      const int e = t - ntiles;
      row0 = BS == 64 ? __builtin_amdgcn_readfirstlane(sh.tail_key0[e]) % BS : 0;
#pragma unroll
      for (int i = 0; i < NIP; ++i) {
        const int key = is_v ? (64 * i / 64) * KPC : (64 * i) >> LCPP;
        blk[i] = __builtin_amdgcn_readfirstlane(sh.tail_blk[e][key / BS]);
      }
    }
    char* dst = ring + (h % RW) * PART;
    const char* base = is_v ? vbase + (static_cast<int64_t>(dim0) * BS + row0) * EB
                            : kbase + (static_cast<int64_t>(row0) * D + dim0) * EB;
#pragma unroll
    for (int i = 0; i < NIP; ++i) {
      const uint32_t off = is_v ? voff0 + static_cast<uint32_t>(((i * KPC) % BS) * EB) : koff[i];
      load_to_lds(base + static_cast<int64_t>(blk[i]) * blk_bytes + off, dst + i * 1024);
    }
  };

  // per-lane LDS offsets of the operands inside a part: K row key_perm(r),
  // unit 2k + hf of the part's steps (16-bit: chunk 2k + hf; E4M3: half hf
  // of chunk k), rotated; V^T dims 32 dt + r of the part, keys 16 k + 8 hf ..
  int kread[KS / KSPLIT];
#pragma unroll
  for (int k = 0; k < KS / KSPLIT; ++k) {
    const int krow = key_perm(r) * Geo::PROW, ksw = swz(key_perm(r));
    kread[k] = EB == 2 ? krow + (((2 * k + hf) ^ ksw) << 4) : krow + ((k ^ ksw) << 4) + 8 * hf;
  }
  const int vread = ((EB == 2 ? hf * 64 : 0) + r) * 16 + (EB == 1 ? 8 * hf : 0);

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x16{};
  // m_run: the row's reference maximum, moved up only when a tile's scores
  // pass it by more than 2^kLazyLog2 (so probabilities stay below 256, well
  // inside fp32 and the two-part 16-bit P); O and l are rescaled only then,
  // and only in waves where some row moved.
  constexpr float kLazyLog2 = 8.f;
  float m_run = -INFINITY, l_run = 0.f;
  u32x4 hi[2], lo[2];
  float alpha = 1.f;
  bool rescale = false;

  // S^T += K Q^T over the KS / KSPLIT steps of K part `qk` at `kp`
  auto s_part = [&](f32x16& s, const char* kp, int qk) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < KS / KSPLIT; ++k)
      s = mfma32<AT>(lds_operand<ST, AT>(kp + kread[k]), qb[qk * (KS / KSPLIT) + k], s);
  };
  // The online softmax of a tile's scores (keys at or past `lim` masked);
  // the probabilities leave as two 16-bit parts (nearest value and
  // remainder), so the weights keep about 16 bits: rows with only a few
  // shared keys can have outputs as large as single V entries, where one
  // 16-bit rounding of P would show.
  auto softmax = [&](const f32x16& s, int key0, int lim) __attribute__((always_inline)) {
    float x[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = key0 + key_perm(8 * (e >> 2) + 4 * hf + (e & 3));
      x[e] = key < lim ? s[e] * P.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, x[e]);
    }
    tmax = halves_max(tmax);
    const bool up = tmax > m_run + kLazyLog2;
    rescale = __builtin_amdgcn_ballot_w64(up) != 0;
    if (rescale) {
      const float m_new = up ? tmax : m_run;
      alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      x[e] = __builtin_amdgcn_exp2f(x[e] - m_use);
      psum += x[e];
    }
    l_run += psum;
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
  };
  // Zero, in the V part at `vp`, the keys at or past `vlim` of a tail tile
  // starting at key0 (unused slots may hold NaN, which a zero probability
  // would not cancel).
  auto zero_v_past = [&](char* vp, int key0, int vlim) __attribute__((always_inline)) {
    for (int idx = lane; idx < (kTile / KPC) * 64; idx += 64) {
      const int k0 = key0 + (idx / 64) * KPC;  // first key of the chunk
      if (k0 + KPC <= vlim) continue;
      u32x4* p = reinterpret_cast<u32x4*>(vp + idx * 16);
      u32x4 v = *p;
#pragma unroll
      for (int b = 0; b < 16; ++b)  // byte b holds key k0 + b / EB
        if (k0 + b / EB >= vlim) v[b / 4] &= ~(0xffu << (8 * (b % 4)));
      *p = v;
    }
  };
  // O^T += V^T P^T for the column tiles of V part `qv` at `vp`
  auto pv_part = [&](const char* vp, int qv) __attribute__((always_inline)) {
#pragma unroll
    for (int dl = 0; dl < 2; ++dl) {
      const int dt = 2 * qv + dl;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const u32x4 v = lds_operand<ST, AT>(vp + vread + ((EB == 2 ? 2 * k : k) * 64 + 32 * dl) * 16);
        o[dt] = mfma32<AT>(v, hi[k], o[dt]);
        o[dt] = mfma32<AT>(v, lo[k], o[dt]);
      }
    }
  };

  // The first loads of shared tiles go out before wave 0 lists the tail
  // tiles (with their block ids) in LDS; the tail tiles' loads after.
  int issued = 0;
  const int prologue = min(RW - 1, nparts);
  for (; issued < prologue && wave + kWaves * (issued / NP) < ntiles; ++issued) issue(issued);
  if (last_part) {
    if (wave == 0) {
      const int32_t* mrow = P.tables + static_cast<int64_t>(first + (lane < members ? lane : 0)) * P.max_blocks;
      for (int j = 0; j < nt; ++j) {
        const int e = incl - nt + j, k0 = t0 + j * kTile;
        sh.tail_member[e] = lane;
        sh.tail_key0[e] = k0;
        sh.tail_len[e] = Lm;
        // keys past the member's length read its last block (masked)
#pragma unroll
        for (int b = 0; b < PrefixLds<ST, D, BS>::NBT; ++b) {
          const int id = mrow[min(k0 + b * BS, Lm - 1) / BS];
          PA_DEBUG_COUNT(PA_DBG_BLOCK_ID, id < 0 || id >= P.num_blocks);
          sh.tail_blk[e][b] = (id >= 0 && id < P.num_blocks) ? id : 0;
        }
      }
    }
    __syncthreads();
  }
  for (; issued < prologue; ++issued) issue(issued);

  // The walk: before part h is used, parts up to h + RW - 1 are requested
  // (the newest into the slot of part h - 1, whose reads have returned);
  // then this wave waits for its own loads of h.
  int h = 0;
  auto next = [&]() __attribute__((always_inline)) -> char* {
    wait_vm_steps<NIP, RW - 2>(issued - h - 1);
    wait_lds();
    if (issued < nparts) issue(issued++);
    return ring + (h++ % RW) * PART;
  };
  for (int j = 0; j < my_tiles; ++j) {
    const int t = wave + kWaves * j;
    int key0, lim, vlim;
    const bool tail_tile = t >= ntiles;
    if (!tail_tile) {
      key0 = tok0 + t * kTile;
      lim = row_lim;
      vlim = INT_MAX;
    } else {
      const int e = t - ntiles;
      const int tm = __builtin_amdgcn_readfirstlane(sh.tail_member[e]);
      vlim = __builtin_amdgcn_readfirstlane(sh.tail_len[e]);
      key0 = __builtin_amdgcn_readfirstlane(sh.tail_key0[e]);
      lim = mem == tm ? vlim : 0;
    }
    f32x16 s = f32x16{};
#pragma unroll
    for (int qk = 0; qk < KSPLIT; ++qk) s_part(s, next(), qk);
    softmax(s, key0, lim);
    if (rescale) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
#pragma unroll
    for (int qv = 0; qv < KSPLIT; ++qv) {
      char* vp = next();
      if (tail_tile && key0 + kTile > vlim) zero_v_past(vp, key0, vlim);
      pv_part(vp, qv);
    }
  }

  // merge the four wavefronts' states of each row into the members' slots
  const float l_tot = halves_sum(l_run);
  __syncthreads();  // every wave is done with its ring, which the merge buffers reuse
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float4 v4 = {o[dt][4 * j], o[dt][4 * j + 1], o[dt][4 * j + 2], o[dt][4 * j + 3]};
      *reinterpret_cast<float4*>(&sh.mg.o[wave][r][dt * 32 + 8 * j + 4 * hf]) = v4;
    }
  if (hf == 0) {
    sh.mg.m[wave][r] = m_run;
    sh.mg.l[wave][r] = l_tot;
  }
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < 32) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (sh.mg.l[w][tid] > 0.f) M = fmaxf(M, sh.mg.m[w][tid]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float c = sh.mg.l[w][tid] > 0.f ? __builtin_amdgcn_exp2f(sh.mg.m[w][tid] - M) : 0.f;
      sh.mg.c[w][tid] = c;
      L += c * sh.mg.l[w][tid];
    }
    // (an FP8 pool's V scale enters here, as in the decode items)
    sh.mg.inv[tid] = L > 0.f ? (ST::bytes == 1 ? P.v_scale : 1.f) / L : 0.f;
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
    for (int w = 0; w < kWaves; ++w) acc = __builtin_fmaf(sh.mg.c[w][row], sh.mg.o[w][row][d], acc);
    const int64_t pidx = (static_cast<int64_t>(first + mm) * hq + kvh * G + row % G) * P.max_parts + part;
    P.ws_o[pidx * D + d] = acc * sh.mg.inv[row];
  }
}

// Shared-prefix items times the KV heads, two workgroups per compute unit.
template <typename ST, int D, int BS, int G, typename AT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_prefix_kernel(GroupedParams GP) {
  __shared__ PrefixLds<ST, D, BS> sh;
  const int hk = GP.dec.num_kv_heads;
  const int n = __builtin_amdgcn_readfirstlane(*GP.pre_count) * hk;
  for (int it = blockIdx.x; it < n; it += gridDim.x) {
    __syncthreads();  // the previous item is done with LDS
    const int item = it / hk;
    prefix_item<ST, D, BS, G, AT>(sh, GP, item, it - item * hk);
  }
}

// Suffix items times the KV heads: each sequence's own tokens, decoded as
// the split decode items are (and held to the same wavefronts per SIMD).  An item that is its sequence's only slot
// writes the output directly; every other one leaves partials for the merge
// kernel.
template <typename ST, int D, int BS, int G, typename AT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(decode_waves_per_eu<ST, D, BS, G, true>(), 8)))
void grouped_suffix_kernel(GroupedParams GP) {
  __shared__ DecodeLds<G, D, BS> sh;
  const DecodeParams& P = GP.dec;
  const int hk = P.num_kv_heads;
  const int n = __builtin_amdgcn_readfirstlane(*P.n_items) * hk;
  for (int it = blockIdx.x; it < n; it += gridDim.x) {
    __syncthreads();  // the previous item is done with LDS
    const int item = it / hk;
    const int s = __builtin_amdgcn_readfirstlane(P.items[2 * item]);
    const int part = __builtin_amdgcn_readfirstlane(P.items[2 * item + 1]);
    const int L = clamp_len(P.ctx_lens[s], P.max_context);
    const bool only = __builtin_amdgcn_readfirstlane(GP.nslots[s]) == 1 &&
                      __builtin_amdgcn_readfirstlane(GP.slot_base[s]) == 0;
    decode_item<ST, D, BS, G, AT, split_tile_buffers<ST, D, BS, G>()>(
        sh, P, s, it - item * hk, part, L, __builtin_amdgcn_readfirstlane(GP.seq_start[s]),
        __builtin_amdgcn_readfirstlane(GP.slot_base[s]), !only);
  }
}

// Log-sum-exp merge of each (sequence, KV head)'s slots: grid (KV head,
// sequence), G rows of D outputs.  A thread owns 4 columns of one row and
// the slots p = grp, grp + NGRP, ...: it requests their partial outputs
// first (up to KREG of them in registers), while wave 0 turns the slots'
// (max, sum) pairs into weights in LDS (G * max_parts floats of dynamic
// LDS) -- per row, the lanes of one LPR-lane segment take every LPR-th
// slot and reduce with shuffles.  Slots without keys (sum 0) carry no
// weight; a row with none (context 0) is written as zeros.  Rows written
// directly by the suffix kernel are skipped.
template <typename AT, int D, int G>
__global__ __launch_bounds__(kThreads) void grouped_merge_kernel(DecodeParams P, const int32_t* __restrict__ nslots,
                                                                const int32_t* __restrict__ slot_base) {
  constexpr int C4 = D / 4;             // float4 columns of a row
  constexpr int ROWT = G * C4;          // threads covering the G rows once
  static_assert(kThreads % ROWT == 0, "slot groups");
  constexpr int NGRP = kThreads / ROWT;  // slot groups
  constexpr int KREG = 8;                // slots per thread held in registers
  constexpr int LPR = 64 / G;            // lanes of wave 0 per row in the weight phase
  extern __shared__ float w_sh[];        // [G][max_parts]
  __shared__ float4 part_sh[NGRP][ROWT];
  __shared__ float den_sh[G];
  const int kvh = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int ns = min(nslots[s], P.max_parts);
  if (ns == 1 && slot_base[s] == 0) return;
  const int hq = P.num_kv_heads * G, mp = P.max_parts;
  const int64_t qh0 = static_cast<int64_t>(s) * hq + kvh * G;
  const int grp = tid / ROWT, rt = tid - grp * ROWT, h = rt / C4, c4 = rt - h * C4;

  const float* orow = P.ws_o + (qh0 + h) * mp * D + 4 * c4;
  float4 ov[KREG];
#pragma unroll
  for (int k = 0; k < KREG; ++k) {
    const int p = grp + NGRP * k;
    ov[k] = p < ns ? *reinterpret_cast<const float4*>(orow + static_cast<int64_t>(p) * D) : float4{0.f, 0.f, 0.f, 0.f};
  }

  if (tid < 64) {
    const int hw = tid / LPR, pl = tid - hw * LPR;
    const float* ml = P.ws_ml + 2 * (qh0 + hw) * mp;
    float M = -INFINITY;
    for (int p = pl; p < ns; p += LPR)
      if (ml[2 * p + 1] > 0.f) M = fmaxf(M, ml[2 * p]);
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    float den = 0.f;
    for (int p = pl; p < ns; p += LPR) {
      const float l = ml[2 * p + 1];
      const float w = l > 0.f ? l * __builtin_amdgcn_exp2f(ml[2 * p] - M) : 0.f;
      w_sh[hw * mp + p] = w;
      den += w;
    }
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) den += __shfl_xor(den, o, 64);
    if (pl == 0) den_sh[hw] = den;
  }
  __syncthreads();

  const float* w = w_sh + h * mp;
  float4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < KREG; ++k) {
    const int p = grp + NGRP * k;
    const float wp = p < ns ? w[p] : 0.f;
    num.x = __builtin_fmaf(wp, ov[k].x, num.x);
    num.y = __builtin_fmaf(wp, ov[k].y, num.y);
    num.z = __builtin_fmaf(wp, ov[k].z, num.z);
    num.w = __builtin_fmaf(wp, ov[k].w, num.w);
  }
  for (int p = grp + NGRP * KREG; p < ns; p += NGRP) {  // slots past the registers
    const float4 v = *reinterpret_cast<const float4*>(orow + static_cast<int64_t>(p) * D);
    num.x = __builtin_fmaf(w[p], v.x, num.x);
    num.y = __builtin_fmaf(w[p], v.y, num.y);
    num.z = __builtin_fmaf(w[p], v.z, num.z);
    num.w = __builtin_fmaf(w[p], v.w, num.w);
  }
  part_sh[grp][rt] = num;
  __syncthreads();
  if (grp == 0) {
    float4 t = part_sh[0][rt];
#pragma unroll
    for (int g2 = 1; g2 < NGRP; ++g2) {
      const float4 u = part_sh[g2][rt];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
    }
    const float den = den_sh[h];
    const float inv = den > 0.f ? 1.f / den : 0.f;
    typename AT::elem* out = static_cast<typename AT::elem*>(P.out) + (qh0 + h) * D + 4 * c4;
    out[0] = narrow<AT>(t.x * inv);
    out[1] = narrow<AT>(t.y * inv);
    out[2] = narrow<AT>(t.z * inv);
    out[3] = narrow<AT>(t.w * inv);
  }
}

// Workgroups of a persistent kernel that fit on the device at once (Tag
// tells the kernels apart for the per-device cache).
template <typename Tag>
int resident_workgroups(const void* kernel) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cached[kMaxDev];  // 0 = not yet queried; racing writers store the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) dev = 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess || per_cu <= 0)
      per_cu = 1;
    n = cus * per_cu;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
template <typename ST, int D, int BS, int G, typename AT, bool PREFIX>
struct GroupedTag {};

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
  // Item lists: at most (sequences / 2 chunks) x partitions prefix items
  // (a chunk with a shared prefix has two members or more) and sequences x
  // partitions suffix items, each times the KV heads.  The prefix kernel
  // runs first; a sequence's prefix and suffix slots meet in the merge.
  const int64_t parts =
      std::max<int64_t>(1, (static_cast<int64_t>(a.max_context_len) + a.part_tokens - 1) / a.part_tokens);
  const int64_t upper_pre = std::max<int64_t>(1, a.num_seqs / 2) * parts * a.num_kv_heads;
  const int64_t upper_suf = static_cast<int64_t>(a.num_seqs) * parts * a.num_kv_heads;
  auto pre_kernel = grouped_prefix_kernel<ST, D, BS, G, AT>;
  auto suf_kernel = grouped_suffix_kernel<ST, D, BS, G, AT>;
  const int grid_pre = static_cast<int>(std::max<int64_t>(
      1, std::min<int64_t>(upper_pre, resident_workgroups<GroupedTag<ST, D, BS, G, AT, true>>(
                                          reinterpret_cast<const void*>(pre_kernel)))));
  const int grid_suf = static_cast<int>(std::max<int64_t>(
      1, std::min<int64_t>(upper_suf, resident_workgroups<GroupedTag<ST, D, BS, G, AT, false>>(
                                          reinterpret_cast<const void*>(suf_kernel)))));
  hipLaunchKernelGGL(pre_kernel, dim3(grid_pre), dim3(kThreads), 0, st, P);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(suf_kernel, dim3(grid_suf), dim3(kThreads), 0, st, P);
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

PA_DEBUG_UNIT(grouped)

}  // namespace pa
