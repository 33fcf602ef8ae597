"""The library's launches under HIP graph capture.

A mixed step -- copy-on-write copies, the append of every new token,
chunked prefill and split decode (planner, walk and merge) --, a
prefix-grouped decode call and a key-split prefill (partials and merge) are
each captured once in a graph and replayed with
fresh queries in the graph's input buffers.  Between replays the same work
runs eagerly with synchronisations around it; every replay must give the
eager outputs bit for bit.  The outputs are filled with NaN before each
replay, so a launch that the capture lost would show.  Nothing the library
enqueues is a memset or an allocation, and all of its one-time set-up
(attribute and occupancy queries) happens in the eager warm-up.
"""
import numpy as np
import pytest
import torch

import bench
import workloads

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _new_queries(st, gen):
    for name in ("q_dec", "q_pre"):
        if hasattr(st, name):
            q = getattr(st, name)
            q.copy_(torch.randn(q.shape, generator=gen).to(q.dtype))


def test_mixed_step_graph_replays_match_eager():
    wl = workloads.make("mixed_chunked_prefill", reduced=True)
    print(f"[gpu] graph: {wl.spec.name} reduced, split decode at 32-token partitions", flush=True)
    st = bench.Step(wl, 32)
    assert len(st.dec) and len(st.pre)
    gen = torch.Generator().manual_seed(4035)
    st.step()  # every launch path once, outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.step()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        _new_queries(st, gen)
        torch.cuda.synchronize()
        st.step()
        torch.cuda.synchronize()
        want_dec, want_pre = st.out_dec.clone(), st.out_pre.clone()
        st.out_dec.fill_(float("nan"))
        st.out_pre.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(st.out_dec), _bits(want_dec)), r
        assert torch.equal(_bits(st.out_pre), _bits(want_pre)), r
        assert not torch.isnan(want_dec.float()).any() and not torch.isnan(want_pre.float()).any()
    print(f"[gpu] graph: {REPLAYS} replays bit-equal to eager", flush=True)


def test_grouped_decode_graph_replays_match_eager():
    import paged_kv_cache_403_amd as P

    wl = workloads.make("gqa_shared_prefix", reduced=True)
    print(f"[gpu] graph: {wl.spec.name} reduced, grouped decode", flush=True)
    st = bench.Step(wl, -1)
    st.copy_append()
    sp = wl.spec
    hint = torch.from_numpy(bench.group_starts(wl, st.dec)).to("cuda")
    part = 256
    ws = torch.empty(P.pa_decode_grouped_workspace_bytes(len(st.dec), sp.num_q_heads, sp.head_dim, st.max_dec, part),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(st.q_dec)

    def grouped():
        P.pa_decode_grouped(st.cache.desc, st.q_dec, out, st.tab_dec, st.len_dec, st.max_dec, sp.scale, hint, part,
                            ws)

    gen = torch.Generator().manual_seed(4036)
    grouped()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        grouped()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        _new_queries(st, gen)
        torch.cuda.synchronize()
        grouped()
        torch.cuda.synchronize()
        want = out.clone()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(want)), r
        assert not torch.isnan(want.float()).any()
    print(f"[gpu] graph: {REPLAYS} grouped replays bit-equal to eager", flush=True)


def test_split_prefill_graph_replays_match_eager():
    """Key-split prefill (partials into the workspace, then the merge) on
    one 512-token chunk over 2048 cached tokens, at the library's split."""
    import paged_kv_cache_403_amd as P

    wl = workloads.custom(32, 8, 128, 16, "bf16", [2048 + 512], n_new=[512], seed=5, name="one_chunk")
    sp = wl.spec
    st = bench.Step(wl, 0)
    st.copy_append()
    k = P.pa_prefill_choose_splits(st.cache.desc, len(st.pre), sp.num_q_heads, st.maxq_pre, st.maxc_pre)
    assert k > 1
    print(f"[gpu] graph: split prefill, {k} key splits", flush=True)
    ws = torch.empty(P.pa_prefill_workspace_bytes(st.q_pre.shape[0], sp.num_q_heads, sp.head_dim, k),
                     dtype=torch.uint8, device="cuda")

    def split():
        P.pa_prefill_chunk_split(st.cache.desc, st.q_pre, st.out_pre, st.cu_pre, st.len_pre, st.tab_pre,
                                 st.maxq_pre, st.maxc_pre, sp.scale, k, ws)

    gen = torch.Generator().manual_seed(4037)
    split()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        split()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        _new_queries(st, gen)
        torch.cuda.synchronize()
        split()
        torch.cuda.synchronize()
        want = st.out_pre.clone()
        st.out_pre.fill_(float("nan"))
        ws.fill_(0xFF)  # NaN partials: a replay must rewrite every one it reads
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(st.out_pre), _bits(want)), r
        assert not torch.isnan(want.float()).any()
    print(f"[gpu] graph: {REPLAYS} split-prefill replays bit-equal to eager", flush=True)
