"""Reference data movement for the paged pool, and a driver that replays a
workload's cache operations through the reference block manager.

Pool layout (the pages do not fix one): separate K and V arrays, each
[num_blocks][num_kv_heads][block_size][head_dim] in the storage type.  The
token at slot s lives at [s // block_size, :, s % block_size, :].

* append: the step's K/V of each new token are written into its slot before
  attention runs (zzmblog.top vLLM guide, "Transformer推理与KV缓存": decode
  computes only the current token's K,V and appends it to the cache, then
  attends).  A negative slot means "skip this token".
* copy: a shared block about to be written is first copied whole, K and V,
  to the fresh block that replaces it (lshu.cn/news/11644, "收益分析":
  copy-on-write on divergence).  Pairs are applied in order.
"""
from dataclasses import dataclass

import numpy as np

from .block_manager import BlockManager
from .storage import host_dtype, kv_encode


class Pool:
    """dtype: the pool's element type.  An "fp8" pool stores E4M3 codes of
    the appended activation values (act_dtype) divided by k_scale / v_scale
    (storage.kv_encode)."""

    def __init__(self, num_blocks, num_kv_heads, block_size, head_dim, dtype, fill_bits=None, act_dtype=None,
                 k_scale=1.0, v_scale=1.0):
        hd = host_dtype(dtype)
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        self.dtype = dtype
        self.act_dtype = act_dtype or dtype
        self.k_scale, self.v_scale = k_scale, v_scale
        self.block_size = block_size
        self.k = np.zeros(shape, dtype=hd)
        self.v = np.zeros(shape, dtype=hd)
        if fill_bits is not None:
            self.k[...] = fill_bits
            self.v[...] = fill_bits

    def write(self, slots, k_new, v_new):
        slots = np.asarray(slots, dtype=np.int64)
        keep = slots >= 0
        blk, off = np.divmod(slots[keep], self.block_size)
        k_new, v_new = np.asarray(k_new)[keep], np.asarray(v_new)[keep]
        if self.dtype == "fp8":
            k_new = kv_encode(k_new, self.act_dtype, self.k_scale)
            v_new = kv_encode(v_new, self.act_dtype, self.v_scale)
        # pool[blk, :, off, :] selects one [heads][head_dim] row per token
        self.k[blk, :, off, :] = k_new
        self.v[blk, :, off, :] = v_new

    def copy(self, pairs):
        for src, dst in pairs:
            self.k[dst] = self.k[src]
            self.v[dst] = self.v[src]


@dataclass
class StepState:
    """Everything the step needs, as the reference computes it."""

    bm: BlockManager
    pool: Pool
    slot_mapping: np.ndarray  # int64 [sum n_new], batch order
    cow_pairs: np.ndarray  # int32 [n][2]
    tables: np.ndarray  # int32 [S][max_blocks], padded with the poison block
    context_lens: np.ndarray  # int32 [S]
    q_lens: np.ndarray  # int32 [S]
    setup_slots: np.ndarray  # int64, all pre-step appends in issue order


def run_workload(wl, fill_bits=None, with_pool=True) -> StepState:
    """Replay setup and step operations of a `workloads.Workload`.

    The pool starts filled with `fill_bits` (a sentinel in unused slots), the
    pre-step cache is built, then the step's block-manager calls run and the
    step's copies and appends are applied, in that order.  with_pool=False
    replays only the bookkeeping (slots, copy pairs, tables, lengths) and
    leaves `pool` None -- for workloads too large to hold twice in host
    memory."""
    sp = wl.spec
    bm = BlockManager(sp.num_blocks, sp.block_size, wl.free_order)
    pool = (Pool(sp.num_blocks, sp.num_kv_heads, sp.block_size, sp.head_dim, sp.kv_dtype or sp.dtype, fill_bits,
                 act_dtype=sp.dtype, k_scale=sp.k_scale, v_scale=sp.v_scale) if with_pool else None)
    setup_slots = []
    for op in wl.setup_ops():
        if op.kind == "add":
            bm.add_seq(op.seq)
        elif op.kind == "fork":
            bm.fork(op.parent, op.seq, op.keep)
        else:
            slots, pairs = bm.append(op.seq, op.n)
            if pool is not None:
                pool.copy(pairs)
                pool.write(slots, op.k, op.v)
            setup_slots.extend(slots)
    step_slots, step_pairs = [], []
    for op in wl.step_ops():
        slots, pairs = bm.append(op.seq, op.n)
        step_slots.extend(slots)
        step_pairs.extend(pairs)
    if pool is not None:
        k_new, v_new = wl.step_kv()
        pool.copy(step_pairs)
        pool.write(step_slots, k_new, v_new)
    batch = wl.batch
    maxb = max(len(bm.tables[p.seq_id]) for p in batch)
    tables = np.full((len(batch), max(maxb, 1)), sp.poison_block, dtype=np.int32)
    for r, p in enumerate(batch):
        t = bm.tables[p.seq_id]
        tables[r, : len(t)] = t
    return StepState(
        bm=bm,
        pool=pool,
        slot_mapping=np.asarray(step_slots, dtype=np.int64),
        cow_pairs=np.asarray(step_pairs, dtype=np.int32).reshape(-1, 2),
        tables=tables,
        context_lens=np.asarray([bm.lens[p.seq_id] for p in batch], dtype=np.int32),
        q_lens=np.asarray([p.n_new for p in batch], dtype=np.int32),
        setup_slots=np.asarray(setup_slots, dtype=np.int64),
    )
