"""Chunked prefill with the row tiles' keys split over several workgroups
(pa_prefill_chunk_split) against the oracle.

Each key range leaves partial results per row, combined by log-sum-exp, so
ranges that start past a row's diagonal (the row sees none of their keys),
ranges without any key tile (more ranges than the row tile has tiles) and
the first tile's two-part probabilities must all come out as the unsplit
kernel's.  Rows are checked at the tolerance of the activation type."""
import numpy as np
import pytest

import workloads
from fullsize_check import check_rows, chunk_edges
from gpu_harness import TOL, run_step
from oracle import attention as A
from oracle.cache import run_workload
from oracle.storage import to_f64

pytestmark = pytest.mark.gpu


def _oracle(wl):
    st = run_workload(wl, fill_bits=None)
    out, _ = A.paged_attention(wl.step_q(), st.pool.k, st.pool.v, st.tables, st.context_lens, st.q_lens,
                               wl.spec.scale, wl.spec.dtype, kv=wl.spec.kv)
    return out


def _err(res, ref, dtype):
    return float(np.abs(to_f64(res.out, dtype) - ref).max())


# (Hq, Hkv, D, BS, dtype, FP8 pool)
SHAPES = [
    (32, 8, 128, 16, "bf16", False), (16, 2, 64, 32, "f16", False), (8, 8, 128, 64, "bf16", False),
    (64, 8, 128, 16, "f16", False), (32, 8, 128, 16, "bf16", True), (16, 8, 128, 8, "f16", False),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_split_prefill_ragged_chunks(shape):
    hq, hkv, d, bs, dt, fp8 = shape
    ctx = [1, 9, 64, 65, 130, 300, 700, 1500]
    n = [1, 9, 33, 64, 100, 70, 300, 257]
    wl = workloads.custom(hq, hkv, d, bs, dt, ctx, n_new=n, seed=hq + d + bs)
    if fp8:
        wl = workloads.with_fp8_kv(wl)
    print(f"[gpu] split prefill {shape}", flush=True)
    ref = _oracle(wl)
    for k in (0, 2, 3, 8):
        res = run_step(wl, keep_pool=False, prefill_all=True, key_splits=k)
        err = _err(res, ref, dt)
        assert err <= TOL[dt], (shape, k, err)


def test_split_prefill_matches_unsplit_on_the_mixed_batch():
    wl = workloads.make("mixed_chunked_prefill", reduced=True)
    print("[gpu] split prefill on the reduced mixed batch", flush=True)
    ref = _oracle(wl)
    a = run_step(wl, keep_pool=False)
    for k in (2, 5):
        b = run_step(wl, keep_pool=False, key_splits=k)
        assert _err(b, ref, wl.spec.dtype) <= TOL[wl.spec.dtype], k
        assert np.abs(to_f64(a.out, wl.spec.dtype) - to_f64(b.out, wl.spec.dtype)).max() <= TOL[wl.spec.dtype], k


def test_split_prefill_one_long_chunk():
    """One 512-token chunk on a 6000-token context: the case the split is
    for (few workgroups without it); every row against the oracle."""
    wl = workloads.custom(32, 8, 128, 16, "bf16", [6000], n_new=[512], seed=5)
    print("[gpu] split prefill, one long chunk", flush=True)
    ref = _oracle(wl)
    for k in (0, 4, 8):
        res = run_step(wl, keep_pool=False, key_splits=k)
        assert _err(res, ref, "bf16") <= TOL["bf16"], k


def test_split_prefill_nan_in_unused_slots_does_not_leak():
    wl = workloads.custom(32, 8, 128, 16, "bf16", [20, 100, 333], n_new=[20, 37, 64], seed=9)
    print("[gpu] split prefill NaN poison", flush=True)
    a = run_step(wl, fill=float("nan"), keep_pool=False, key_splits=4)
    b = run_step(wl, keep_pool=False, key_splits=4)
    assert np.isfinite(to_f64(a.out, "bf16")).all()
    assert np.array_equal(a.out, b.out)


@pytest.mark.parametrize("n_chunks,cached", [(1, 4096), (1, 16384), (2, 4096), (2, 16384)])
def test_split_prefill_fullsize_few_chunks(n_chunks, cached):
    """The few-chunk batches bench.py times (512-token chunks, 32 q / 8 KV
    heads, head_dim 128, bf16, 16-token blocks) at the split the library
    chooses: the first and last row of every chunk and 14 random ones, every
    q head, against the definition."""
    wl = workloads.custom(32, 8, 128, 16, "bf16", [cached + 512] * n_chunks, n_new=[512] * n_chunks,
                          seed=cached + n_chunks, name="few_chunk_prefill")
    print(f"[gpu] split prefill full size: {n_chunks} x 512 on {cached} cached", flush=True)
    res = run_step(wl, keep_pool=False, key_splits=0)
    worst, n, where = check_rows(wl, res.out, TOL["bf16"], rows_of=chunk_edges(np.random.default_rng(cached), 14))
    assert n >= n_chunks * 2 * 32, n  # first and last rows at least, every q head
    print(f"[gpu]   {n} rows, worst |err| {worst:.3g} at {where}", flush=True)
