"""Decode shapes walked on the matrix cores (8 q heads per KV head; FP8 pools
of 16-token blocks at 4) against the oracle.

That walk reads key tiles of 32 tokens, so with 16-token blocks a tile can
begin before the partition it serves (partitions of an odd number of
blocks, and grouped decode's suffix items, which start at a shared length
that is any multiple of the block size): those tokens are masked out.  The
last tile of a context is masked at its end, and the V values of unused
slots must not reach the output even when they hold NaN.
"""
import numpy as np
import pytest

import workloads
from gpu_harness import TOL, run_step
from oracle import attention as A
from oracle.cache import run_workload
from oracle.storage import to_f64

pytestmark = pytest.mark.gpu

# (Hq, Hkv, D, BS, activation dtype, FP8 pool)
SHAPES = [
    (64, 8, 128, 16, "bf16", False), (64, 8, 128, 32, "f16", False), (16, 2, 128, 16, "f16", False),
    (64, 8, 128, 16, "bf16", True), (64, 8, 128, 32, "f16", True), (64, 8, 128, 64, "bf16", True),
    (32, 8, 128, 16, "bf16", True), (8, 2, 128, 16, "f16", True),
]
LENS = [1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 100, 300, 517]


def _workload(shape, seed):
    hq, hkv, d, bs, dt, fp8 = shape
    wl = workloads.custom(hq, hkv, d, bs, dt, LENS, seed=seed)
    return workloads.with_fp8_kv(wl) if fp8 else wl


def _oracle(wl):
    st = run_workload(wl, fill_bits=None)
    out, _ = A.paged_attention(wl.step_q(), st.pool.k, st.pool.v, st.tables, st.context_lens, st.q_lens,
                               wl.spec.scale, wl.spec.dtype, kv=wl.spec.kv)
    return out


def _err(res, ref, dtype):
    return float(np.abs(to_f64(res.out, dtype) - ref).max())


@pytest.mark.parametrize("shape", SHAPES)
def test_matrix_core_decode_partitions(shape):
    """One pass, the library's partitions, and partitions of one and of three
    blocks (tiles that start before their partition)."""
    bs, dt = shape[3], shape[4]
    wl = _workload(shape, seed=bs + shape[0])
    print(f"[gpu] matrix-core decode {shape}", flush=True)
    ref = _oracle(wl)
    for part in (0, -1, bs, 3 * bs):
        res = run_step(wl, partition_size=part, keep_pool=False)
        err = _err(res, ref, dt)
        assert err <= TOL[dt], (shape, part, err)


@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[3], SHAPES[6]])
def test_matrix_core_decode_nan_in_unused_slots(shape):
    wl = _workload(shape, seed=7)
    print(f"[gpu] matrix-core decode NaN poison {shape}", flush=True)
    for part in (0, 3 * shape[3]):
        a = run_step(wl, fill=float("nan"), partition_size=part, keep_pool=False)
        b = run_step(wl, partition_size=part, keep_pool=False)
        assert np.isfinite(to_f64(a.out, shape[4])).all(), part
        assert np.array_equal(a.out, b.out), part


@pytest.mark.parametrize("fp8", [False, True])
def test_matrix_core_grouped_suffixes(fp8):
    """Grouped decode at 8 q heads per KV head: shared lengths of 1, 3 and 4
    blocks, so suffix items start inside a 32-token tile."""
    bs = 16
    groups = [
        (3 * bs + 5, [3 * bs + 6, 3 * bs + 40, 200, 3 * bs + 5]),
        (bs + 2, [bs + 3, 90, 33]),
        (4 * bs, [4 * bs + 1, 9 * bs, 300]),
        (0, [7, 40]),
    ]
    wl = workloads.custom_shared(64, 8, 128, bs, "bf16", groups, seed=11)
    if fp8:
        wl = workloads.with_fp8_kv(wl)
    print(f"[gpu] matrix-core grouped decode fp8={fp8}", flush=True)
    ref = _oracle(wl)
    for part in (0, 32, 64):
        res = run_step(wl, partition_size=part, keep_pool=False, grouped=True,
                       group_start=workloads.group_starts(wl))
        err = _err(res, ref, "bf16")
        assert err <= TOL["bf16"], (part, err)
