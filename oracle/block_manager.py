"""Reference block manager (host bookkeeping of the paged KV cache).

Follows lshu.cn/news/11644, "方案：页式内存管理": every sequence owns a block
table (logical block i -> physical block id); all sequences draw from one
global pool; when a sequence grows by a token and its last block still has
room the token goes there, otherwise a block is taken from the free pool and
its id appended to the table; when a sequence finishes all of its blocks go
back to the free pool at once.  "收益分析" adds read-only sharing of
identical prefix blocks with copy-on-write at the later divergence.

Conventions the pages leave open (fixed here so the C++ manager can be
checked against this one bit for bit):

* the free pool is a FIFO: blocks are handed out from the front, returned
  blocks go to the back (the printed free pool [2, 4, 6, 8, ...] is read
  front first);
* a fork shares the parent's first ceil(keep / block_size) blocks and bumps
  each one's reference count;
* writing a token into a block whose reference count is above one first
  replaces that table entry by a fresh block and records the pair
  (shared block, fresh block) for a whole-block copy; the old block loses one
  reference.  A write that starts a new block never copies;
* a token's slot is block_id * block_size + position % block_size.
"""
from collections import deque


class OutOfBlocks(Exception):
    pass


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.block_size = int(block_size)
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        self.num_blocks = int(num_blocks)
        self.free = deque(order)
        self.ref = {}  # physical block -> reference count (only blocks in use)
        self.tables = {}  # seq -> list of physical blocks
        self.lens = {}  # seq -> tokens held

    # -- helpers -----------------------------------------------------------------
    def _take(self) -> int:
        if not self.free:
            raise OutOfBlocks()
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def _drop(self, b: int):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            del self.ref[b]
            self.free.append(b)

    # -- operations --------------------------------------------------------------
    def add_seq(self, seq: int):
        if seq in self.tables:
            raise ValueError(f"sequence {seq} exists")
        self.tables[seq] = []
        self.lens[seq] = 0

    def fork(self, parent: int, child: int, keep: int):
        if child in self.tables:
            raise ValueError(f"sequence {child} exists")
        if not 0 <= keep <= self.lens[parent]:
            raise ValueError("keep out of range")
        nblk = -(-keep // self.block_size)
        shared = self.tables[parent][:nblk]
        for b in shared:
            self.ref[b] += 1
        self.tables[child] = list(shared)
        self.lens[child] = keep

    def append(self, seq: int, n: int):
        """Grow `seq` by n tokens.  Returns (slots, cow_pairs)."""
        slots, pairs = [], []
        table = self.tables[seq]
        # all-or-nothing: count the blocks the append takes before touching state
        pos0 = self.lens[seq]
        need = sum(1 for p in range(pos0, pos0 + n) if p % self.block_size == 0)
        if n > 0 and pos0 % self.block_size != 0 and self.ref[table[pos0 // self.block_size]] > 1:
            need += 1
        if need > len(self.free):
            raise OutOfBlocks()
        for _ in range(n):
            pos = self.lens[seq]
            i, off = divmod(pos, self.block_size)
            if off == 0:
                # last block full (or no block yet): take one from the free pool
                assert i == len(table)
                table.append(self._take())
            else:
                blk = table[i]
                if self.ref[blk] > 1:
                    fresh = self._take()
                    pairs.append((blk, fresh))
                    self._drop(blk)
                    table[i] = fresh
            slots.append(table[i] * self.block_size + off)
            self.lens[seq] = pos + 1
        return slots, pairs

    def free_seq(self, seq: int):
        for b in self.tables.pop(seq):
            self._drop(b)
        del self.lens[seq]

    def table(self, seq: int):
        return list(self.tables[seq])
