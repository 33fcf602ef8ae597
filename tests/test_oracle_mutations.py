"""Planted mistakes in the oracle (CPU only) must each fail a pin.

Each case patches one piece of the reference with a plausible slip and checks
that at least one of the pin checks raises.  This shows the pins are strong
enough to catch a dropped term, a wrong index or a transposed mapping.
"""
import numpy as np
import pytest

from oracle import attention as A
from oracle import block_manager as BMmod
from oracle import cache as C
from oracle import storage as S

from test_oracle_attention import check_causal_bruteforce, check_gather, check_sdpa
from test_oracle_block_manager import check_page_example, replay_and_check

SMALL_CAUSAL = [(C_, n, bs) for bs in (1, 4) for C_ in (0, 3, 7) for n in (1, 3, 5)]
RANDOM_OPS = [("add", 0, 0, 0), ("append", 0, 0, 7), ("fork", 0, 1, 6), ("append", 1, 0, 3),
              ("append", 0, 0, 2), ("fork", 1, 2, 9), ("append", 2, 0, 5), ("free", 0, 0, 0),
              ("append", 1, 0, 4), ("add", 3, 0, 0), ("append", 3, 0, 9)]


def _all_pins():
    check_page_example(BM=BMmod.BlockManager)
    replay_and_check(RANDOM_OPS, BM=BMmod.BlockManager, PoolCls=C.Pool)
    for name in ("gqa_shared_prefix", "mixed_chunked_prefill", "tiny_decode"):
        check_gather(name)
        check_sdpa(name)
    check_causal_bruteforce(SMALL_CAUSAL)


def test_unpatched_oracle_passes_all_pins():
    _all_pins()


class _NoCowBM(BMmod.BlockManager):
    """Slip: writes into a shared block in place (no copy-on-write)."""

    def append(self, seq, n):
        saved = dict(self.ref)
        self.ref = {b: 1 for b in self.ref}
        try:
            return super().append(seq, n)
        finally:
            for b, r in saved.items():
                if b in self.ref:
                    self.ref[b] = r


class _SlotOffByBlockBM(BMmod.BlockManager):
    """Slip: slot = block id + position % block_size (forgot the block_size factor)."""

    def append(self, seq, n):
        slots, pairs = super().append(seq, n)
        return [(s // self.block_size) + (s % self.block_size) for s in slots], pairs


class _LifoBM(BMmod.BlockManager):
    """Slip: hands blocks out from the back of the free pool."""

    def _take(self):
        if not self.free:
            raise BMmod.OutOfBlocks()
        b = self.free.pop()
        self.ref[b] = 1
        return b


def _gather_next_slot(pk, pv, table, L, dtype, kv=None):
    """Slip: reads the slot after the right one inside each block."""
    bs = pk.shape[2]
    j = np.arange(L)
    blk = np.asarray(table)[j // bs]
    off = (j + 1) % bs
    return S.to_f64(pk[blk, :, off, :], dtype), S.to_f64(pv[blk, :, off, :], dtype)


MUTATIONS = {
    "gqa_map_modulo": lambda mp: mp.setattr(A, "kv_head_of", lambda h, hq, hkv: h % hkv),
    "chunk_rows_top_aligned": lambda mp: mp.setattr(A, "query_positions", lambda L, n: np.arange(n)),
    "mask_excludes_diagonal": lambda mp: mp.setattr(
        A, "visible_keys", lambda L, pos: np.arange(L)[None, :] < np.asarray(pos)[:, None]),
    "bf16_wrong_shift": lambda mp: mp.setattr(
        A, "to_f64", lambda a, d: (np.asarray(a, np.uint32) << 15).view(np.float32).astype(np.float64)
        if d == "bf16" else S.to_f64(a, d)),
    "no_copy_on_write": lambda mp: (mp.setattr(C, "BlockManager", _NoCowBM),
                                    mp.setattr(BMmod, "BlockManager", _NoCowBM)),
    "slot_missing_block_factor": lambda mp: (mp.setattr(C, "BlockManager", _SlotOffByBlockBM),
                                             mp.setattr(BMmod, "BlockManager", _SlotOffByBlockBM)),
    "free_pool_from_back": lambda mp: mp.setattr(BMmod.BlockManager, "_take", _LifoBM._take),
    "copy_skipped": lambda mp: mp.setattr(C.Pool, "copy", lambda self, pairs: None),
    "gather_wrong_offset": lambda mp: mp.setattr(A, "gather", _gather_next_slot),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    MUTATIONS[name](monkeypatch)
    caught = False
    try:
        _all_pins()
    except AssertionError:
        caught = True
    assert caught, f"no pin caught the planted mistake {name}"


def test_merge_without_weights_is_caught():
    """Slip in the split-K merge: averaging partial outputs unweighted."""
    import workloads

    wl = workloads.make("long_splitk_decode", reduced=True)
    st = C.run_workload(wl)
    args = (wl.step_q(), st.pool.k, st.pool.v, st.tables, st.context_lens, st.q_lens, wl.spec.scale, wl.spec.dtype)
    ref, _ = A.paged_attention(*args)
    m, l, o = A.split_partials(*args, partition=512)
    bad = np.where((l > 0)[..., None], o, 0).sum(-2) / np.maximum((l > 0).sum(-1), 1)[..., None]
    assert np.abs(bad - ref).max() > 1e-6
    good, _ = A.merge_partials(m, l, o)
    assert np.abs(good - ref).max() <= 1e-12
