"""GPU parity for block sizes 8 and 64 (zzmblog.top vLLM guide, "核心参数调优":
8 for many short sequences, 32/64 for long contexts) on top of 16 and 32:
pool contents bit-exact, decode (one pass and split) and chunked prefill
within the dtype tolerance, an FP8 pool at 64, and the 7B-shaped batch at
full size (sampled rows)."""
import numpy as np
import pytest

import workloads
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


DECODE_SHAPES = [  # (Hq, Hkv, D, dtype)
    (8, 8, 64, "f32"), (8, 2, 128, "f32"), (16, 4, 64, "f16"), (32, 4, 128, "bf16"), (16, 2, 128, "f16"),
    (8, 8, 128, "bf16"),
]


@pytest.mark.parametrize("bs", [8, 64])
@pytest.mark.parametrize("shape", DECODE_SHAPES)
def test_decode_block_sizes(shape, bs):
    hq, hkv, d, dt = shape
    lens = [1, bs - 1, bs, bs + 1, 3 * bs + 5, 300, 700]
    wl = workloads.custom(hq, hkv, d, bs, dt, lens, seed=hq + d + bs)
    print(f"[gpu] decode {shape} block_size {bs}", flush=True)
    st, ref = _oracle(wl)
    for part in (0, 2 * bs, -1):
        res = run_step(wl, partition_size=part, keep_pool=part == 0)
        if part == 0:
            _check_pool(res, st)
        assert _err(res, ref, dt) <= TOL[dt], (shape, bs, part)


@pytest.mark.parametrize("bs", [8, 64])
@pytest.mark.parametrize("shape", [(8, 8, 128, "bf16"), (16, 2, 64, "f16"), (32, 8, 128, "bf16")])
def test_prefill_block_sizes(shape, bs):
    hq, hkv, d, dt = shape
    ctx = [1, 9, 64, 65, 130, 300]
    n = [1, 9, 33, 64, 100, 70]
    wl = workloads.custom(hq, hkv, d, bs, dt, ctx, n_new=n, seed=hq * 3 + bs)
    print(f"[gpu] prefill {shape} block_size {bs}", flush=True)
    st, ref = _oracle(wl)
    res = run_step(wl, keep_pool=True, prefill_all=True)
    _check_pool(res, st)
    assert _err(res, ref, dt) <= TOL[dt]


def test_fp8_pool_block_size_64():
    wl = workloads.with_fp8_kv(workloads.custom(32, 8, 128, 64, "bf16", [1, 63, 64, 65, 200, 640], seed=3))
    st, ref = _oracle(wl)
    for part in (0, 128):
        res = run_step(wl, partition_size=part, keep_pool=part == 0)
        if part == 0:
            _check_pool(res, st)
        assert _err(res, ref, "bf16") <= TOL["bf16"]


@pytest.mark.parametrize("bs", [8, 64])
def test_fullsize_decode_block_sizes(bs):
    wl = workloads.with_block_size(workloads.make("mha_decode_7b"), bs)
    sp = wl.spec
    print(f"[gpu] full size {sp.name}", flush=True)
    res = run_step(wl, partition_size=-1, keep_pool=False)
    rng = np.random.default_rng(bs)
    worst = 0.0
    for r in sorted(set(int(x) for x in rng.integers(0, len(wl.batch), size=10))):
        p = wl.batch[r]
        h = int(rng.integers(sp.num_q_heads))
        K, V = wl.logical_kv(p.seq_id)
        ref = A.attention_rows(wl.q[p.seq_id][0:1, h], K[:, h], V[:, h], [p.context_len - 1], sp.scale, sp.dtype)[0]
        err = float(np.abs(to_f64(res.out[r, h], sp.dtype) - ref).max())
        worst = max(worst, err)
        assert err <= TOL[sp.dtype], (r, h, err)
    print(f"[gpu]   sampled max|err| = {worst:.3e}", flush=True)
