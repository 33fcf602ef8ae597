"""Reference scheduler loop (host), one call = one iteration.

The steps of the centralized scheduler in lshu.cn/news/11644, "整体架构":
check the free block pool, pull as many waiting requests as fit, allocate
their blocks, prefill long prompts in chunks over several iterations, batch
the current token of every running request, run the step, update, and free
a finished request's blocks at once.  The pages fix no policy; these are
the readings (the library's scheduler follows the same ones):

* a token budget per iteration and a cap on running requests;
* decode tokens first -- one per running request whose prompt is cached,
  oldest admission first -- then the next chunk of each prompt still being
  prefilled (oldest first), then new requests in arrival order;
* a chunk is as long as the prompt's remainder, the budget left and the
  pool's room (free blocks plus room in the last block) allow; admission
  stops at the first waiting request whose first chunk would be empty;
* a decode token that needs a block while the pool is empty preempts the
  newest running request not yet scheduled this iteration (itself if none):
  its blocks are freed and it returns to the front of the queue, to be
  prefilled again from its first token;
* the iteration that caches a prompt's last token yields the first new
  token, each decode iteration one more; at max_new_tokens the request is
  finished and its blocks are freed at the start of the next iteration.
"""
from collections import deque

from .block_manager import BlockManager


class Request:
    def __init__(self, rid, prompt, max_new):
        self.rid, self.prompt, self.max_new = rid, prompt, max_new
        self.cached = 0
        self.generated = 0
        self.state = "waiting"


class Scheduler:
    def __init__(self, bm: BlockManager, budget: int, max_running: int):
        self.bm, self.budget, self.max_running = bm, budget, max_running
        self.reqs = {}
        self.waiting = deque()
        self.running = []
        self.to_free = []

    def add(self, rid, prompt, max_new):
        self.reqs[rid] = Request(rid, prompt, max_new)
        self.waiting.append(rid)

    def unfinished(self):
        return sum(r.state != "finished" for r in self.reqs.values())

    def _room(self, seq_len):
        bs = self.bm.block_size
        last = (bs - seq_len % bs) % bs
        return last + len(self.bm.free) * bs

    def _preempt(self, rid):
        r = self.reqs[rid]
        self.bm.free_seq(rid)
        r.cached, r.generated, r.state = 0, 0, "waiting"
        self.running.remove(rid)
        self.waiting.appendleft(rid)

    def step(self):
        """Returns (decode ids, prefill (id, n) list, slots, pairs, finished, preempted)."""
        for rid in self.to_free:
            self.bm.free_seq(rid)
        self.to_free = []
        left = self.budget
        decodes, prefills, slots, pairs, preempted, done = [], [], [], [], [], []

        def grow(rid, n):
            s, p = self.bm.append(rid, n)
            slots.extend(s)
            pairs.extend(p)
            self.reqs[rid].cached += n
            done.append(rid)

        # one decode token per running request whose prompt is cached
        i = 0
        while i < len(self.running) and left > 0:
            rid = self.running[i]
            r = self.reqs[rid]
            if r.state != "decode":
                i += 1
                continue
            needs_block = self.bm.lens[rid] % self.bm.block_size == 0
            skipped = False
            while needs_block and not self.bm.free:
                victim = self.running[-1] if len(self.running) > i + 1 else rid
                preempted.append(victim)
                self._preempt(victim)
                if victim == rid:
                    skipped = True
                    break
            if skipped:
                continue
            grow(rid, 1)
            decodes.append(rid)
            left -= 1
            i += 1
        # the next chunk of prompts being prefilled
        for rid in list(self.running):
            if left <= 0:
                break
            r = self.reqs[rid]
            if r.state != "prefill":
                continue
            n = min(r.prompt - r.cached, left, self._room(r.cached))
            if n <= 0:
                break
            grow(rid, n)
            prefills.append((rid, n))
            left -= n
        # admission in arrival order
        while self.waiting and left > 0 and len(self.running) < self.max_running:
            rid = self.waiting[0]
            r = self.reqs[rid]
            n = min(r.prompt, left, self._room(0))
            if n <= 0:
                break
            self.waiting.popleft()
            self.bm.add_seq(rid)
            r.state = "prefill"
            self.running.append(rid)
            grow(rid, n)
            prefills.append((rid, n))
            left -= n
        # what the step yields
        finished = []
        for rid in done:
            r = self.reqs[rid]
            if r.state == "prefill" and r.cached == r.prompt:
                r.state, r.generated = "decode", 1
            elif r.state == "decode" and r.cached > r.prompt:
                r.generated += 1
            if r.state == "decode" and r.generated >= r.max_new:
                r.state = "finished"
                self.running.remove(rid)
                self.to_free.append(rid)
                finished.append(rid)
        return decodes, prefills, slots, pairs, finished, preempted
