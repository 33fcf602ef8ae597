"""pa_decode_noalloc -- split decode with its scratch in the library's fixed
device array -- against pa_decode with a caller workspace, through the C
ABI: two calls in a row (the second with a smaller batch, fewer partitions
and a different partition size, so it runs over what the first left in the
array), each bit for bit equal to pa_decode on the same inputs (the same
kernels and partitioning), and within the decode tolerance of the oracle."""
import numpy as np
import pytest
import torch

import paged_kv_cache_403_amd as P
import workloads
from gpu_harness import TOL
from oracle import attention as A
from oracle.cache import run_workload
from oracle.storage import to_f64
from paged_kv_cache_403_amd.runtime import PagedKVCache, to_device, to_host

pytestmark = pytest.mark.gpu


def _setup(wl):
    sp = wl.spec
    cache = PagedKVCache(sp.num_blocks, sp.num_kv_heads, sp.block_size, sp.head_dim, sp.dtype, "cuda",
                         wl.free_order, fill_value=1.0e4)
    cache.apply_ops(wl.setup_ops())
    batch = wl.batch
    plan = cache.prepare_step([p.seq_id for p in batch], [p.n_new for p in batch], sp.poison_block)
    k_new, v_new = wl.step_kv()
    P.pa_kv_append(cache.desc, to_device(k_new, sp.dtype, "cuda"), to_device(v_new, sp.dtype, "cuda"),
                   plan.slot_mapping)
    q = to_device(wl.step_q(), sp.dtype, "cuda")
    return cache, plan, q


def _oracle(wl):
    st = run_workload(wl, fill_bits=None)
    out, _ = A.paged_attention(wl.step_q(), st.pool.k, st.pool.v, st.tables, st.context_lens, st.q_lens,
                               wl.spec.scale, wl.spec.dtype)
    return out


CALLS = [  # (Hq, Hkv, D, BS, dtype, context lengths, partition tokens): the second is smaller
    (32, 8, 128, 32, "bf16", [5000, 4999, 1200, 37], 64),
    (32, 8, 128, 32, "bf16", [900, 33], 32),
]


def test_noalloc_matches_workspace_decode_twice():
    wls = [workloads.custom(hq, hkv, d, bs, dt, lens, seed=70 + i)
           for i, (hq, hkv, d, bs, dt, lens, _) in enumerate(CALLS)]
    prepared = [_setup(wl) for wl in wls]
    for i, ((*_, part), wl, (cache, plan, q)) in enumerate(zip(CALLS, wls, prepared)):
        sp = wl.spec
        max_ctx = int(plan.host_lens.max())
        print(f"[gpu] no-alloc call {i}: {len(wl.batch)} seqs, max context {max_ctx}, partition {part}", flush=True)
        got = torch.full_like(q, 7.0)
        P.pa_decode_noalloc(cache.desc, q, got, plan.block_tables, plan.context_lens, max_ctx, sp.scale, part)
        torch.cuda.synchronize()
        ws = torch.empty(P.pa_decode_workspace_bytes(len(wl.batch), sp.num_q_heads, sp.head_dim, max_ctx, part),
                         dtype=torch.uint8, device="cuda")
        want = torch.full_like(q, 7.0)
        P.pa_decode(cache.desc, q, want, plan.block_tables, plan.context_lens, max_ctx, sp.scale, part, ws)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), i
        err = float(np.abs(to_f64(to_host(got), sp.dtype) - _oracle(wl)).max())
        print(f"[gpu]   bit-equal to pa_decode; max|err| vs oracle {err:.3e}", flush=True)
        assert err <= TOL[sp.dtype]


def test_noalloc_refuses_a_split_beyond_its_array():
    """More scratch than the fixed array holds: PA_EWORKSPACE before any
    launch, with the bytes needed and the limit in the message."""
    wl = workloads.custom(32, 8, 128, 32, "bf16", [64, 64], seed=3)
    cache, plan, q = _setup(wl)
    out = torch.zeros_like(q)
    # 600 sequences x 32 heads x 4096 partitions of 32 tokens: far past 32 MiB
    big_q = torch.zeros(600, 32, 128, dtype=torch.bfloat16, device="cuda")
    tabs = torch.zeros(600, 4096, dtype=torch.int32, device="cuda")
    lens = torch.ones(600, dtype=torch.int32, device="cuda")
    with pytest.raises(P.PagedAttnError, match="needs .* bytes of scratch"):
        P.pa_decode_noalloc(cache.desc, big_q, torch.empty_like(big_q), tabs, lens, 4096 * 32, 0.1, 32)
    # the library still works afterwards
    P.pa_decode_noalloc(cache.desc, q, out, plan.block_tables, plan.context_lens, int(plan.host_lens.max()),
                        wl.spec.scale, 32)
    torch.cuda.synchronize()
