// Host block manager of the paged KV cache (CPU only; no HIP calls).
//
// Bookkeeping as lshu.cn/news/11644 describes it ("方案：页式内存管理",
// "收益分析"): a global pool of fixed-size blocks, a block table per
// sequence, a free pool from which a block is taken only when a sequence's
// last block is full, all blocks returned when the sequence ends, and
// read-only sharing of prefix blocks with copy-on-write at the divergence.
//
// Conventions the pages leave open: the free pool is FIFO (front out, back
// in); a fork shares ceil(keep / block_size) blocks; a write into a block
// with more than one holder moves the writer to a fresh block and emits the
// pair (shared, fresh) for a whole-block copy; a write that opens a new block
// never copies.  Appends are all-or-nothing.
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include <algorithm>

#include "block_manager_impl.h"
#include "pagedattn.h"

using pa_host::Seq;

extern "C" {

pa_bm* pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order, int32_t free_len) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  pa_bm* bm = new (std::nothrow) pa_bm();
  if (!bm) return nullptr;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
  if (free_order) {
    if (free_len < 0 || free_len > num_blocks) {
      delete bm;
      return nullptr;
    }
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < free_len; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return nullptr;
      }
      seen[b] = 1;
      bm->free_list.push_back(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) bm->free_list.push_back(b);
  }
  return bm;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

int pa_bm_add_seq(pa_bm* bm, int32_t seq) {
  if (!bm || bm->seqs.count(seq)) return PA_EINVAL;
  bm->seqs.emplace(seq, Seq{});
  return PA_OK;
}

int pa_bm_fork(pa_bm* bm, int32_t parent, int32_t child, int32_t keep) {
  if (!bm || parent == child || bm->seqs.count(child)) return PA_EINVAL;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end() || keep < 0 || keep > it->second.len) return PA_EINVAL;
  const int64_t nblk = (static_cast<int64_t>(keep) + bm->block_size - 1) / bm->block_size;
  Seq c;
  c.table.assign(it->second.table.begin(), it->second.table.begin() + nblk);
  for (int32_t b : c.table) ++bm->ref[b];
  c.len = keep;
  bm->seqs.emplace(child, std::move(c));
  return PA_OK;
}

int pa_bm_append(pa_bm* bm, int32_t seq, int32_t n_tokens, int64_t* slots_out, int32_t* cow_pairs_out,
                 int32_t cow_cap, int32_t* n_cow_out) {
  if (!bm || n_tokens < 0 || (n_tokens > 0 && !slots_out) || cow_cap < 0) return PA_EINVAL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_EINVAL;
  Seq& s = it->second;
  const int64_t need = bm->blocks_needed(s, n_tokens);
  if (need > static_cast<int64_t>(bm->free_list.size())) return PA_ENOMEM;
  // at most one copy per append: only the block holding position len can be shared
  if (need > 0 && s.len % bm->block_size != 0 && bm->ref[s.table[s.len / bm->block_size]] > 1 &&
      (cow_cap < 1 || !cow_pairs_out))
    return PA_EINVAL;
  int32_t n_cow = 0;
  const int64_t bs = bm->block_size;
  for (int32_t t = 0; t < n_tokens; ++t) {
    const int64_t pos = s.len;
    const int64_t i = pos / bs, off = pos % bs;
    if (off == 0) {
      s.table.push_back(bm->take());
    } else {
      const int32_t blk = s.table[i];
      if (bm->ref[blk] > 1) {
        const int32_t fresh = bm->take();
        cow_pairs_out[2 * n_cow] = blk;
        cow_pairs_out[2 * n_cow + 1] = fresh;
        ++n_cow;
        bm->drop(blk);
        s.table[i] = fresh;
      }
    }
    slots_out[t] = static_cast<int64_t>(s.table[i]) * bs + off;
    s.len = pos + 1;
  }
  if (n_cow_out) *n_cow_out = n_cow;
  return PA_OK;
}

int pa_bm_append_batch(pa_bm* bm, const int32_t* seqs, const int32_t* n_tokens, int32_t num_seqs,
                       int64_t* slots_out, int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow_out,
                       int32_t* n_done_out) {
  if (!bm || num_seqs < 0 || (num_seqs > 0 && (!seqs || !n_tokens))) return PA_EINVAL;
  int64_t slot_off = 0;
  int32_t cow_total = 0, done = 0;
  int rc = PA_OK;
  for (int32_t i = 0; i < num_seqs; ++i) {
    int32_t nc = 0;
    rc = pa_bm_append(bm, seqs[i], n_tokens[i], slots_out ? slots_out + slot_off : nullptr,
                      cow_pairs_out ? cow_pairs_out + 2 * cow_total : nullptr, cow_cap - cow_total, &nc);
    if (rc != PA_OK) break;
    slot_off += n_tokens[i];
    cow_total += nc;
    ++done;
  }
  if (n_cow_out) *n_cow_out = cow_total;
  if (n_done_out) *n_done_out = done;
  return rc;
}

int pa_bm_free_seq(pa_bm* bm, int32_t seq) {
  if (!bm) return PA_EINVAL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_EINVAL;
  for (int32_t b : it->second.table) bm->drop(b);
  bm->seqs.erase(it);
  return PA_OK;
}

int pa_bm_table(const pa_bm* bm, int32_t seq, int32_t* out, int32_t cap, int32_t* len_out) {
  if (!bm) return PA_EINVAL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_EINVAL;
  const auto& t = it->second.table;
  if (len_out) *len_out = static_cast<int32_t>(t.size());
  if (static_cast<int64_t>(t.size()) > cap || (!out && !t.empty())) return PA_EINVAL;
  if (!t.empty()) std::memcpy(out, t.data(), t.size() * sizeof(int32_t));
  return PA_OK;
}

int pa_bm_tables(const pa_bm* bm, const int32_t* seqs, int32_t num_seqs, int32_t* out, int32_t max_blocks,
                 int32_t pad_block, int32_t* lens_out) {
  if (!bm || num_seqs < 0 || max_blocks < 0 || (num_seqs > 0 && (!seqs || !out))) return PA_EINVAL;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return PA_EINVAL;
    const auto& t = it->second.table;
    if (static_cast<int64_t>(t.size()) > max_blocks) return PA_EINVAL;
    int32_t* row = out + static_cast<int64_t>(i) * max_blocks;
    for (int32_t j = 0; j < max_blocks; ++j) row[j] = j < static_cast<int32_t>(t.size()) ? t[j] : pad_block;
    if (lens_out) lens_out[i] = static_cast<int32_t>(it->second.len);
  }
  return PA_OK;
}

int pa_bm_seq_len(const pa_bm* bm, int32_t seq, int32_t* len_out) {
  if (!bm || !len_out) return PA_EINVAL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_EINVAL;
  *len_out = static_cast<int32_t>(it->second.len);
  return PA_OK;
}

int32_t pa_bm_num_free(const pa_bm* bm) { return bm ? static_cast<int32_t>(bm->free_list.size()) : -1; }

int32_t pa_bm_free_list(const pa_bm* bm, int32_t* out, int32_t cap) {
  if (!bm || !out || cap < 0) return -1;
  int32_t n = 0;
  for (int32_t b : bm->free_list) {
    if (n >= cap) break;
    out[n++] = b;
  }
  return n;
}

int pa_bm_usage(const pa_bm* bm, int64_t* blocks_in_use, int64_t* slots_filled) {
  if (!bm || !blocks_in_use || !slots_filled) return PA_EINVAL;
  // filled slots of each held block: the most any holder has written into it
  std::vector<int32_t> filled(bm->num_blocks, 0);
  for (const auto& kv : bm->seqs) {
    const Seq& q = kv.second;
    for (size_t j = 0; j < q.table.size(); ++j) {
      const int64_t f = std::min<int64_t>(bm->block_size, q.len - static_cast<int64_t>(j) * bm->block_size);
      int32_t& slot = filled[q.table[j]];
      slot = std::max<int32_t>(slot, static_cast<int32_t>(std::max<int64_t>(f, 0)));
    }
  }
  int64_t held = 0, used = 0;
  for (int32_t b = 0; b < bm->num_blocks; ++b) {
    if (bm->ref[b] > 0) {
      ++held;
      used += filled[b];
    }
  }
  *blocks_in_use = held;
  *slots_filled = used;
  return PA_OK;
}

int32_t pa_bm_refcount(const pa_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

}  // extern "C"
