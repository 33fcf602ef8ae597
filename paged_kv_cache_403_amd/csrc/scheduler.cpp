// Host scheduler loop around the paged cache (CPU only, no HIP calls).
//
// One call is one iteration of the centralized scheduler the pages describe
// (lshu.cn/news/11644, "整体架构"): look at the free block pool, pull as many
// waiting requests as fit, give them blocks, prefill long prompts in chunks
// over several iterations, batch the current token of every running
// request, run the step, update, and return a finished request's blocks to
// the pool at once.  Requests join and leave at every iteration (continuous
// batching; 5x10.cn/post/462, "技术架构深度分析").  The caller runs the kernels
// of each returned batch (append, chunked prefill, decode) before the next
// call; blocks freed by the next call are reused only by work enqueued after
// it on the same stream.
//
// Rules the pages leave open (the host reference in the tests follows the
// same ones):
//  * a token budget per iteration (max_batched_tokens) and a cap on running
//    requests; decode tokens are scheduled first (one per running request
//    whose prompt is cached, oldest admission first), then the next chunk of
//    the prompts still being prefilled (oldest first), then new requests in
//    arrival order;
//  * a chunk is as long as the prompt's remainder, the budget left and the
//    pool's room allow; a request is admitted only if its first chunk is not
//    empty, and once one waiting request cannot start no later one does;
//  * a decode token that needs a block when the pool is empty preempts the
//    newest running request not yet scheduled in this iteration (itself if
//    there is none): its blocks are freed and it goes back to the front of
//    the waiting queue, to be prefilled again from its first token;
//  * the iteration that caches a prompt's last token also yields the
//    request's first new token; each decode iteration yields one more; a
//    request that has produced max_new_tokens is finished, and its blocks
//    are freed at the start of the next iteration.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "block_manager_impl.h"
#include "pagedattn.h"

namespace {

enum class State { kWaiting, kPrefill, kDecode, kFinished };

struct Req {
  int32_t prompt = 0;
  int32_t max_new = 0;
  int32_t cached = 0;     // tokens in the cache
  int32_t generated = 0;  // new tokens produced
  State state = State::kWaiting;
};

}  // namespace

struct pa_sched {
  pa_bm* bm = nullptr;
  int32_t budget = 0;
  int32_t max_running = 0;
  std::unordered_map<int32_t, Req> reqs;
  std::deque<int32_t> waiting;   // arrival order, preempted requests in front
  std::vector<int32_t> running;  // admission order
  std::vector<int32_t> to_free;  // finished in the previous iteration

  // tokens a sequence holding `len` tokens can take from its last block and
  // the free pool
  int64_t capacity(int64_t len) const {
    const int64_t bs = bm->block_size;
    const int64_t room = len % bs == 0 ? 0 : bs - len % bs;
    return room + static_cast<int64_t>(bm->free_list.size()) * bs;
  }
};

namespace {

void preempt(pa_sched* s, int32_t id) {
  Req& r = s->reqs[id];
  pa_bm_free_seq(s->bm, id);
  r.cached = 0;
  r.generated = 0;
  r.state = State::kWaiting;
  s->running.erase(std::find(s->running.begin(), s->running.end(), id));
  s->waiting.push_front(id);
}

}  // namespace

extern "C" {

pa_sched* pa_sched_create(pa_bm* bm, int32_t max_batched_tokens, int32_t max_running) {
  if (!bm || max_batched_tokens <= 0 || max_running <= 0) return nullptr;
  pa_sched* s = new (std::nothrow) pa_sched();
  if (!s) return nullptr;
  s->bm = bm;
  s->budget = max_batched_tokens;
  s->max_running = max_running;
  return s;
}

void pa_sched_destroy(pa_sched* s) { delete s; }

int pa_sched_add(pa_sched* s, int32_t req, int32_t prompt_len, int32_t max_new_tokens) {
  if (!s || req < 0 || prompt_len <= 0 || max_new_tokens <= 0 || s->reqs.count(req) || s->bm->seqs.count(req))
    return PA_EINVAL;
  Req r;
  r.prompt = prompt_len;
  r.max_new = max_new_tokens;
  s->reqs.emplace(req, r);
  s->waiting.push_back(req);
  return PA_OK;
}

int32_t pa_sched_unfinished(const pa_sched* s) {
  if (!s) return -1;
  int32_t n = 0;
  for (const auto& kv : s->reqs) n += kv.second.state != State::kFinished;
  return n;
}

int pa_sched_step(pa_sched* s, int32_t* reqs_out, int32_t* n_new_out, int32_t cap, int64_t* slots_out,
                  int64_t slot_cap, int32_t* pairs_out, int32_t pair_cap, int32_t* finished_out,
                  int32_t* preempted_out, int32_t list_cap, pa_sched_batch* out) {
  if (!s || !out || cap < 0 || slot_cap < 0 || pair_cap < 0 || list_cap < 0) return PA_EINVAL;
  // worst case sizes, so that a too-small output can be reported before any state changes
  if (cap < static_cast<int32_t>(std::min<size_t>(s->reqs.size(), static_cast<size_t>(s->max_running))) ||
      slot_cap < s->budget || list_cap < static_cast<int32_t>(s->reqs.size()) || !reqs_out || !n_new_out ||
      !slots_out || !finished_out || !preempted_out)
    return PA_EINVAL;
  *out = pa_sched_batch{};
  pa_bm* bm = s->bm;

  // finished requests of the previous iteration give their blocks back
  for (int32_t id : s->to_free) pa_bm_free_seq(bm, id);
  s->to_free.clear();

  int32_t left = s->budget, n = 0, n_pre = 0, n_pairs = 0, n_preempt = 0;
  int64_t n_slots = 0;
  auto emit = [&](int32_t id, int32_t count) -> int {
    int32_t nc = 0;
    const int rc = pa_bm_append(bm, id, count, slots_out + n_slots, pairs_out ? pairs_out + 2 * n_pairs : nullptr,
                                pair_cap - n_pairs, &nc);
    if (rc != PA_OK) return rc;
    reqs_out[n] = id;
    n_new_out[n] = count;
    ++n;
    n_slots += count;
    n_pairs += nc;
    s->reqs[id].cached += count;
    left -= count;
    return PA_OK;
  };

  // 1. one decode token per running request with a cached prompt
  std::vector<int32_t> done_this_step;
  for (size_t i = 0; i < s->running.size() && left > 0;) {
    const int32_t id = s->running[i];
    Req& r = s->reqs[id];
    if (r.state != State::kDecode) {
      ++i;
      continue;
    }
    bool self_preempted = false;
    while (bm->blocks_needed(bm->seqs[id], 1) > static_cast<int64_t>(bm->free_list.size())) {
      // newest running request not yet scheduled in this iteration
      const int32_t victim = s->running.size() > i + 1 ? s->running.back() : id;
      preempted_out[n_preempt++] = victim;
      preempt(s, victim);
      if (victim == id) {
        self_preempted = true;
        break;
      }
    }
    if (self_preempted) continue;  // running[i] is now the next request
    const int rc = emit(id, 1);
    if (rc != PA_OK) return rc;
    done_this_step.push_back(id);
    ++i;
  }
  const int32_t n_dec = n;

  // 2. the next chunk of prompts being prefilled
  for (size_t i = 0; i < s->running.size() && left > 0; ++i) {
    const int32_t id = s->running[i];
    Req& r = s->reqs[id];
    if (r.state != State::kPrefill) continue;
    const int64_t chunk = std::min<int64_t>({r.prompt - r.cached, left, s->capacity(r.cached)});
    if (chunk <= 0) break;
    const int rc = emit(id, static_cast<int32_t>(chunk));
    if (rc != PA_OK) return rc;
    ++n_pre;
    done_this_step.push_back(id);
  }

  // 3. admission, arrival order
  while (!s->waiting.empty() && left > 0 && static_cast<int32_t>(s->running.size()) < s->max_running) {
    const int32_t id = s->waiting.front();
    Req& r = s->reqs[id];
    const int64_t chunk = std::min<int64_t>({r.prompt, left, s->capacity(0)});
    if (chunk <= 0) break;
    s->waiting.pop_front();
    if (pa_bm_add_seq(bm, id) != PA_OK) return PA_EINVAL;
    r.state = State::kPrefill;
    s->running.push_back(id);
    const int rc = emit(id, static_cast<int32_t>(chunk));
    if (rc != PA_OK) return rc;
    ++n_pre;
    done_this_step.push_back(id);
  }

  // 4. what the step yields: a first token when a prompt's last token is
  //    cached, one token per decode; finished requests leave the batch now
  //    and free their blocks at the next call
  int32_t n_fin = 0;
  for (int32_t id : done_this_step) {
    Req& r = s->reqs[id];
    if (r.state == State::kPrefill && r.cached == r.prompt) {
      r.state = State::kDecode;
      r.generated = 1;
    } else if (r.state == State::kDecode && r.cached > r.prompt) {
      ++r.generated;
    }
    if (r.state == State::kDecode && r.generated >= r.max_new) {
      r.state = State::kFinished;
      s->running.erase(std::find(s->running.begin(), s->running.end(), id));
      s->to_free.push_back(id);
      finished_out[n_fin++] = id;
    }
  }
  out->num_decode = n_dec;
  out->num_prefill = n_pre;
  out->num_slots = n_slots;
  out->num_pairs = n_pairs;
  out->num_finished = n_fin;
  out->num_preempted = n_preempt;
  return PA_OK;
}

}  // extern "C"
