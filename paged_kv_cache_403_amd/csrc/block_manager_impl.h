// Host block manager state, shared by the block manager's C ABI
// (block_manager.cpp) and the scheduler loop (scheduler.cpp).
#pragma once

#include <cstdint>
#include <deque>
#include <unordered_map>
#include <vector>

#include "pagedattn.h"

namespace pa_host {

struct Seq {
  std::vector<int32_t> table;
  int64_t len = 0;
};

}  // namespace pa_host

struct pa_bm {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> ref;  // per physical block
  std::unordered_map<int32_t, pa_host::Seq> seqs;

  int32_t take() {
    int32_t b = free_list.front();
    free_list.pop_front();
    ref[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--ref[b] == 0) free_list.push_back(b);
  }
  // blocks an append of n tokens to s would take from the free pool
  int64_t blocks_needed(const pa_host::Seq& s, int64_t n) const {
    if (n <= 0) return 0;
    const int64_t bs = block_size, p0 = s.len, p1 = s.len + n;  // positions [p0, p1)
    // positions p with p % bs == 0 in [p0, p1)
    int64_t fresh = (p1 + bs - 1) / bs - (p0 + bs - 1) / bs;
    int64_t cow = 0;
    if (p0 % bs != 0 && ref[s.table[p0 / bs]] > 1) cow = 1;
    return fresh + cow;
  }
};

