"""GPU parity of the FP8 (E4M3) KV pool against the oracle.

Bit-exact: the pool's codes after the step's copies and appends (the append
quantises 16-bit rows with the fp32 reciprocal of each scale, as the oracle
does).  Within the activation type's tolerance (fp16 2e-3, bf16 8e-3 max
|err|): decode outputs against the oracle's attention over the codes times
the scales -- the quantisation itself is part of the definition, so only the
kernel's fp32 arithmetic and the output rounding separate the two.
"""
import numpy as np
import pytest
import torch

import workloads
from fullsize_check import check_rows
from gpu_harness import TOL, run_step
from oracle import attention as A
from oracle.cache import run_workload
from oracle.storage import kv_encode, to_f64
from test_gpu_parity import _check_pool

pytestmark = pytest.mark.gpu


def _oracle(wl):
    st = run_workload(wl, fill_bits=None)
    out, _ = A.paged_attention(wl.step_q(), st.pool.k, st.pool.v, st.tables, st.context_lens, st.q_lens,
                               wl.spec.scale, wl.spec.dtype, kv=wl.spec.kv)
    return st, out


def _err(res, ref, dtype):
    return float(np.abs(to_f64(res.out, dtype) - ref).max())


@pytest.mark.parametrize("part", [0, 64, -1])
@pytest.mark.parametrize("name", ["mha_decode_7b", "gqa_shared_prefix", "long_splitk_decode"])
def test_reduced_fp8_parity(name, part):
    wl = workloads.with_fp8_kv(workloads.make(name, reduced=True))
    print(f"[gpu] fp8 {name} reduced part={part}", flush=True)
    st, ref = _oracle(wl)
    res = run_step(wl, partition_size=part)
    assert res.k_pool.dtype == np.uint8
    assert np.array_equal(res.tables, st.tables)
    _check_pool(res, st)
    err = _err(res, ref, wl.spec.dtype)
    print(f"[gpu]   max|err| = {err:.3e}", flush=True)
    assert err <= TOL[wl.spec.dtype]


FP8_SHAPES = [  # (Hq, Hkv, D, BS, activation dtype): q heads per KV head 1, 2, 4, 4, 8, 8, 4, 8
    (16, 16, 128, 16, "f16"), (16, 8, 128, 32, "bf16"), (32, 8, 128, 16, "bf16"), (16, 4, 128, 32, "f16"),
    (64, 8, 128, 16, "f16"), (8, 1, 128, 32, "bf16"),
    # 64-token blocks: whole-block tiles at 4 q heads, 32-token parts at 8
    (32, 8, 128, 64, "f16"), (64, 8, 128, 64, "bf16"),
]


@pytest.mark.parametrize("shape", FP8_SHAPES)
def test_fp8_shapes_and_ragged_lengths(shape):
    hq, hkv, d, bs, dt = shape
    lens = [1, bs - 1, bs, bs + 1, 3 * bs, 5 * bs + 7, 300]
    wl = workloads.with_fp8_kv(workloads.custom(hq, hkv, d, bs, dt, lens, seed=hq * 5 + bs))
    print(f"[gpu] fp8 shape {shape}", flush=True)
    st, ref = _oracle(wl)
    for part in (0, 2 * bs):
        res = run_step(wl, partition_size=part, keep_pool=part == 0)
        if part == 0:
            _check_pool(res, st)
        assert _err(res, ref, dt) <= TOL[dt], (shape, part)


def test_fp8_nan_codes_in_unused_slots_do_not_leak():
    wl = workloads.with_fp8_kv(workloads.make("mha_decode_7b", reduced=True))
    a = run_step(wl, fill=float("nan"), keep_pool=False)
    b = run_step(wl, keep_pool=False)
    assert np.isfinite(to_f64(a.out, wl.spec.dtype)).all()
    assert np.array_equal(a.out, b.out)


def test_fp8_fullsize_all_rows():
    """The 7B-shaped MHA decode batch at full size with an FP8 pool, in the
    launch configuration bench.py times: every row (all q heads) against
    attention over the quantised logical K/V (fp64)."""
    wl = workloads.with_fp8_kv(workloads.make("mha_decode_7b"))
    sp = wl.spec
    print("[gpu] fp8 full size mha_decode_7b", flush=True)
    res = run_step(wl, partition_size=-1, keep_pool=False)
    worst, n, where = check_rows(wl, res.out, TOL[sp.dtype])
    print(f"[gpu]   {n} rows, max|err| = {worst:.3e} at {where}", flush=True)


def test_fp8_mixed_prefill_reduced_parity():
    """Chunked prefill (and the decode side) of the mixed step over an FP8
    pool: every output row against the oracle's attention over the codes
    times the scales."""
    wl = workloads.with_fp8_kv(workloads.make("mixed_chunked_prefill", reduced=True))
    print("[gpu] fp8 mixed_chunked_prefill reduced", flush=True)
    st, ref = _oracle(wl)
    res = run_step(wl, partition_size=-1)
    _check_pool(res, st)
    err = _err(res, ref, wl.spec.dtype)
    print(f"[gpu]   max|err| = {err:.3e}", flush=True)
    assert err <= TOL[wl.spec.dtype]


FP8_PREFILL_SHAPES = [  # (Hq, Hkv, BS, activation dtype): q heads per KV head 1, 2, 4, 8; every block size
    (8, 8, 16, "f16"), (16, 8, 32, "bf16"), (16, 4, 64, "bf16"), (16, 2, 16, "f16"), (32, 8, 64, "f16"),
]


@pytest.mark.parametrize("shape", FP8_PREFILL_SHAPES)
def test_fp8_prefill_shapes_and_ragged_chunks(shape):
    """Chunks of ragged lengths (one row, a partial tile, several 64-key
    tiles with a tail) on cached contexts that start mid-block."""
    hq, hkv, bs, dt = shape
    lens = [1, 70, 200, 331]
    n_new = [1, 37, 130, 64]
    wl = workloads.with_fp8_kv(workloads.custom(hq, hkv, 128, bs, dt, lens, n_new=n_new, seed=hq * 7 + bs))
    print(f"[gpu] fp8 prefill shape {shape}", flush=True)
    st, ref = _oracle(wl)
    res = run_step(wl, prefill_all=True)
    _check_pool(res, st)
    err = _err(res, ref, dt)
    print(f"[gpu]   max|err| = {err:.3e}", flush=True)
    assert err <= TOL[dt], shape


def test_fp8_prefill_nan_codes_in_unused_slots_do_not_leak():
    wl = workloads.with_fp8_kv(workloads.make("mixed_chunked_prefill", reduced=True))
    a = run_step(wl, fill=float("nan"), keep_pool=False)
    b = run_step(wl, keep_pool=False)
    assert np.isfinite(to_f64(a.out, wl.spec.dtype)).all()
    assert np.array_equal(a.out, b.out)


def test_fp8_mixed_fullsize_all_rows():
    """The mixed chunked-prefill step at full size on an FP8 pool, in the
    launch configuration bench.py times: every chunk row and every decode
    row (all q heads) against attention over the quantised logical K/V
    (fp64)."""
    wl = workloads.with_fp8_kv(workloads.make("mixed_chunked_prefill"))
    sp = wl.spec
    print("[gpu] fp8 full size mixed_chunked_prefill", flush=True)
    res = run_step(wl, partition_size=-1, keep_pool=False)
    worst, n, where = check_rows(wl, res.out, TOL[sp.dtype])
    print(f"[gpu]   {n} rows, max|err| = {worst:.3e} at {where}", flush=True)
