"""Pins of the reference block manager and pool data movement.

* the worked block-table example printed in lshu.cn/news/11644
  ("方案：页式内存管理"), stored in tests/golden/block_table_example.json;
* allocator invariants over random operation sequences, and a content check:
  every sequence read back through its block table must equal its logical
  token list tracked by a trivially simple list model (this catches a wrong
  slot formula, a missing copy-on-write copy, a block freed too early, ...).
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.block_manager import BlockManager, OutOfBlocks
from oracle.cache import Pool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_table_example.json")


def check_page_example(BM=BlockManager):
    g = json.load(open(GOLDEN))
    bs = g["block_size"]
    bm = BM(len(g["free_order_that_rebuilds_the_example"]), bs, g["free_order_that_rebuilds_the_example"])
    bm.add_seq("A")
    sa, _ = bm.append("A", g["A"]["tokens"])
    bm.add_seq("B")
    sb, _ = bm.append("B", g["B"]["tokens"])
    assert bm.table("A") == g["A"]["table"]
    assert bm.table("B") == g["B"]["table"]
    assert list(bm.free)[:4] == g["free_pool_front_after_setup"]
    for pos, slot in g["expected_slots"]["A"].items():
        assert sa[int(pos)] == slot
    for pos, slot in g["expected_slots"]["B"].items():
        assert sb[int(pos)] == slot
    s, pairs = bm.append("A", 1)
    assert s == [g["append_A_one_token"]["slot"]] and pairs == []
    assert bm.table("A") == g["append_A_one_token"]["table"]
    s, pairs = bm.append("B", 1)
    assert s == [g["append_B_one_token"]["slot"]] and pairs == []
    assert bm.table("B") == g["append_B_one_token"]["table"]
    s, _ = bm.append("B", 14)
    exp = g["append_B_to_65_tokens"]
    assert s[-2] == exp["last_slot_in_block_14"] and s[-1] == exp["slot_of_token_64"]
    assert bm.table("B") == exp["table"]
    before = len(bm.free)
    bm.free_seq("A")
    assert list(bm.free)[before:] == g["free_A_returns"]


def test_page_worked_example():
    check_page_example()


def test_out_of_blocks_is_all_or_nothing():
    bm = BlockManager(3, 4)
    bm.add_seq(0)
    bm.append(0, 9)  # 3 blocks
    with pytest.raises(OutOfBlocks):
        bm.append(0, 4)  # would need a 4th block
    assert bm.lens[0] == 9 and len(bm.table(0)) == 3
    s, _ = bm.append(0, 3)  # fits in the last block
    assert len(s) == 3


def test_cow_on_shared_partial_block_and_no_copy_when_block_aligned():
    bm = BlockManager(8, 4, list(range(8)))
    bm.add_seq("root")
    bm.append("root", 6)  # blocks 0 (full), 1 (2 of 4)
    bm.fork("root", "a", 6)
    bm.fork("root", "b", 4)
    assert bm.ref[0] == 3 and bm.ref[1] == 2
    s, pairs = bm.append("a", 1)  # writes into shared block 1 -> copy to 2
    assert pairs == [(1, 2)] and s == [2 * 4 + 2] and bm.table("a") == [0, 2]
    s, pairs = bm.append("b", 1)  # block aligned: fresh block, no copy
    assert pairs == [] and s == [3 * 4 + 0] and bm.table("b") == [0, 3]
    s, pairs = bm.append("root", 1)  # last holder of block 1 writes in place
    assert pairs == [] and s == [1 * 4 + 2]


# ---- random operation sequences ---------------------------------------------------

OPS = st.lists(
    st.tuples(st.sampled_from(["add", "fork", "append", "append", "append", "free"]),
              st.integers(0, 5), st.integers(0, 5), st.integers(0, 40)),
    min_size=1, max_size=40)


def replay_and_check(ops, nb=24, bs=4, BM=BlockManager, PoolCls=Pool):
    bm = BM(nb, bs, list(np.random.default_rng(nb).permutation(nb)))
    pool = PoolCls(nb, 1, bs, 1, "f32", fill_bits=-1.0)
    model = {}  # seq -> list of token ids (the logical contents)
    next_id = 0
    for kind, a, b, n in ops:
        if kind == "add" and a not in model:
            bm.add_seq(a)
            model[a] = []
        elif kind == "fork" and a in model and b not in model:
            keep = min(n, len(model[a]))
            bm.fork(a, b, keep)
            model[b] = list(model[a][:keep])
        elif kind == "append" and a in model:
            try:
                slots, pairs = bm.append(a, n)
            except OutOfBlocks:
                continue
            ids = np.arange(next_id, next_id + n, dtype=np.float32)
            next_id += n
            pool.copy(pairs)
            # every write lands in a block this sequence holds alone
            for s in slots:
                assert bm.ref[s // bs] == 1
            pool.write(slots, ids.reshape(n, 1, 1), ids.reshape(n, 1, 1))
            model[a].extend(ids.tolist())
        elif kind == "free" and a in model:
            bm.free_seq(a)
            del model[a]
        # invariants after every operation
        refs = {}
        for seq, t in bm.tables.items():
            for blk in t:
                refs[blk] = refs.get(blk, 0) + 1
        assert refs == bm.ref
        assert sum(bm.ref.values()) == sum(len(t) for t in bm.tables.values())
        free = list(bm.free)
        assert len(set(free)) == len(free)
        assert not (set(free) & set(bm.ref))
        assert len(free) + len(bm.ref) == nb
        for seq, toks in model.items():
            t = bm.table(seq)
            assert bm.lens[seq] == len(toks)
            assert len(t) == -(-len(toks) // bs)  # waste under one block
            got = [pool.k[t[p // bs], 0, p % bs, 0] for p in range(len(toks))]
            assert got == toks
    for seq in list(model):
        bm.free_seq(seq)
    assert len(bm.free) == nb and not bm.ref


@settings(max_examples=300, deadline=None)
@given(OPS)
def test_random_operation_sequences(ops):
    replay_and_check(ops)


def test_pool_write_and_copy_touch_only_their_targets():
    rng = np.random.default_rng(7)
    pool = Pool(6, 2, 4, 3, "bf16", fill_bits=0x7FC0)
    before_k, before_v = pool.k.copy(), pool.v.copy()
    k_new = rng.integers(0, 2**15, size=(3, 2, 3)).astype(np.uint16)
    v_new = rng.integers(0, 2**15, size=(3, 2, 3)).astype(np.uint16)
    slots = [5, -1, 22]
    pool.write(slots, k_new, v_new)
    assert (pool.k[1, :, 1, :] == k_new[0]).all() and (pool.v[5, :, 2, :] == v_new[2]).all()
    mask = np.ones(pool.k.shape, bool)
    mask[1, :, 1, :] = False
    mask[5, :, 2, :] = False
    assert (pool.k[mask] == before_k[mask]).all() and (pool.v[mask] == before_v[mask]).all()
    pool.copy([(1, 3), (3, 4)])  # in order: 4 receives 1's contents via 3
    assert (pool.k[4] == pool.k[1]).all() and (pool.v[3] == pool.v[1]).all()
    assert (pool.k[0] == before_k[0]).all()
