#!/usr/bin/env python3
"""Benchmark of the paged KV-cache attention hot path on one MI355X.

A step is one pass of the hot path over one batch: the block manager's slot
mapping and copy-on-write pairs for the step's new tokens (host, prepared once
since repeating the step is idempotent), then on one HIP stream the
copy-on-write block copies, the KV append through the slot mapping, and the
attention kernels (paged decode for one-token sequences, chunked prefill for
chunks).  Inputs are resident in HBM before the timed region.

Headline workload: 7B-shaped MHA decode (64 sequences, contexts U{128..2048},
32 q = 32 KV heads, head_dim 128, fp16, block_size 16).  `value` is the
step's algorithmic bytes (K/V read, q/out, tables, append) over the step time.
Secondary measurements: chunked prefill on the mixed workload (8 chunks of
512 tokens on cached contexts U{0..4096}, 32/8 heads, bf16) in TFLOP/s;
plain vs prefix-grouped decode on the shared-prefix workload (256 sequences
in groups of 8 forked from 512-token prompts, 32/8 heads, bf16), where the
grouped path reads each shared block once; the headline decode batch again
with an FP8 (E4M3) pool, whose K/V bytes are half; and that batch on pools
of block size 8, 16, 32 and 64 with each pool's unused share.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16/fp16 matrix peak
METRIC = "paged decode KV-read GB/s (% HBM peak) + seqs/s; prefill TFLOP/s (% MFMA)"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def decode_bytes(lens, num_q_heads, num_kv_heads, head_dim, block_size, eb, kv_eb=None):
    """Algorithmic bytes of decode: K/V read (kv_eb bytes per element, eb if
    None), q read and out written (eb), table entries and lengths."""
    import numpy as np

    lens = np.asarray(lens, dtype=np.int64)
    kv = int(lens.sum()) * num_kv_heads * head_dim * (kv_eb or eb) * 2
    qo = len(lens) * num_q_heads * head_dim * eb * 2
    meta = int(((lens + block_size - 1) // block_size).sum()) * 4 + len(lens) * 4
    return int(kv + qo + meta), int(kv)


def prefill_flops(cached, n_new, num_q_heads, head_dim):
    """QK^T and PV over the causal (unmasked) region only: per chunk of n rows
    on C cached tokens, Hq * 4 * D * (n*C + n(n+1)/2)."""
    tot = 0
    for c, n in zip(cached, n_new):
        c, n = int(c), int(n)
        tot += num_q_heads * 4 * head_dim * (n * c + n * (n + 1) // 2)
    return tot


class Step:
    """Device state of one workload's step, ready to be replayed."""

    def __init__(self, wl, partition_size, device="cuda"):
        import numpy as np
        import torch

        import paged_kv_cache_403_amd as P
        from paged_kv_cache_403_amd.runtime import PagedKVCache, to_device

        self.P = P
        sp = wl.spec
        self.wl = wl
        t0 = time.time()
        self.cache = PagedKVCache(sp.num_blocks, sp.num_kv_heads, sp.block_size, sp.head_dim, sp.dtype, device,
                                  wl.free_order, fill_value=1.0e4, kv_dtype=sp.kv_dtype or None, k_scale=sp.k_scale,
                                  v_scale=sp.v_scale)
        self.cache.apply_ops(wl.setup_ops())
        batch = wl.batch
        self.plan = self.cache.prepare_step([p.seq_id for p in batch], [p.n_new for p in batch], sp.poison_block)
        k_new, v_new = wl.step_kv()
        self.k_new = to_device(k_new, sp.dtype, device)
        self.v_new = to_device(v_new, sp.dtype, device)
        q_all = wl.step_q()
        n_new = self.plan.n_new
        starts = np.concatenate([[0], np.cumsum(n_new)])
        dec = np.array([i for i in range(len(batch)) if n_new[i] == 1], dtype=np.int64)
        pre = np.array([i for i in range(len(batch)) if n_new[i] > 1], dtype=np.int64)
        self.dec, self.pre = dec, pre
        self.partition_size = partition_size
        if len(dec):
            self.q_dec = to_device(q_all[starts[dec]], sp.dtype, device)
            self.out_dec = torch.empty_like(self.q_dec)
            idx = torch.from_numpy(dec).to(device)
            self.tab_dec = self.plan.block_tables[idx].contiguous()
            self.len_dec = self.plan.context_lens[idx].contiguous()
            self.max_dec = int(self.plan.host_lens[dec].max())
            wsb = P.pa_decode_workspace_bytes(len(dec), sp.num_q_heads, sp.head_dim, self.max_dec, partition_size)
            self.ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device=device) if wsb else None
            self.part_used = int(P.pa_decode_choose_partition(self.cache.desc, len(dec), sp.num_q_heads, self.max_dec)
                              if partition_size == -1 else partition_size)
            self.dec_bytes, self.dec_kv_bytes = decode_bytes(self.plan.host_lens[dec], sp.num_q_heads,
                                                             sp.num_kv_heads, sp.head_dim, sp.block_size,
                                                             sp.elem_bytes, sp.kv_elem_bytes)
        else:
            self.dec_bytes = self.dec_kv_bytes = 0
        if len(pre):
            rows = np.concatenate([np.arange(starts[i], starts[i + 1]) for i in pre])
            self.q_pre = to_device(q_all[rows], sp.dtype, device)
            self.out_pre = torch.empty_like(self.q_pre)
            cu = np.concatenate([[0], np.cumsum(n_new[pre])]).astype(np.int32)
            self.cu_pre = torch.from_numpy(cu).to(device)
            idx = torch.from_numpy(pre).to(device)
            self.tab_pre = self.plan.block_tables[idx].contiguous()
            self.len_pre = self.plan.context_lens[idx].contiguous()
            self.maxq_pre = int(n_new[pre].max())
            self.maxc_pre = int(self.plan.host_lens[pre].max())
            cached = self.plan.host_lens[pre] - n_new[pre]
            self.pre_flops = prefill_flops(cached, n_new[pre], sp.num_q_heads, sp.head_dim)
        else:
            self.pre_flops = 0
        T = int(n_new.sum())
        eb, kb = sp.elem_bytes, sp.kv_elem_bytes
        self.append_bytes = T * sp.num_kv_heads * sp.head_dim * (eb + kb) * 2 + T * 8
        npairs = len(self.plan.host_pairs)
        self.copy_bytes = npairs * sp.num_kv_heads * sp.block_size * sp.head_dim * kb * 4 + npairs * 8
        torch.cuda.synchronize()
        log(f"{sp.name}: setup {time.time() - t0:.1f}s, {len(dec)} decode seqs, {len(pre)} chunks, "
            f"{npairs} copy pairs")

    def copy_append(self):
        self.P.pa_copy_blocks(self.cache.desc, self.plan.cow_pairs)
        self.P.pa_kv_append(self.cache.desc, self.k_new, self.v_new, self.plan.slot_mapping)

    def decode(self):
        sp = self.wl.spec
        self.P.pa_decode(self.cache.desc, self.q_dec, self.out_dec, self.tab_dec, self.len_dec, self.max_dec,
                         sp.scale, self.partition_size, self.ws)

    def prefill(self):
        sp = self.wl.spec
        self.P.pa_prefill_chunk(self.cache.desc, self.q_pre, self.out_pre, self.cu_pre, self.len_pre, self.tab_pre,
                                self.maxq_pre, self.maxc_pre, sp.scale)


SETTLE_S = 0.1  # untimed repetitions before any warm-up and timing


def settle(fn, seconds=SETTLE_S):
    """Repeat fn for `seconds` of wall time: the clocks take tens of ms of
    sustained matrix work to reach their steady state."""
    import torch

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_loop(fn, iters):
    """Average time of `iters` back-to-back calls of fn, from one pair of
    HIP events around the loop on the stream the library launches on
    (torch's current stream), in ms."""
    import torch

    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def time_steps(st, steps, warmup):
    """Time `steps` whole steps between one pair of events, after SETTLE_S
    seconds of the same step and `warmup` more steps; then each kernel group
    alone over as many back-to-back repetitions (its average launch time).
    Events between the groups of every step would add their own cost (each
    record is a marker packet with a cache write-back) to the step time, so
    the step loop carries none."""
    import torch

    def one():
        st.copy_append()
        if len(st.pre):
            st.prefill()
        if len(st.dec):
            st.decode()

    settle(one)
    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    total_ms = time_loop(one, steps)
    wall = time.perf_counter() - t0
    ca = time_loop(st.copy_append, steps)
    pf = time_loop(st.prefill, steps) if len(st.pre) else 0.0
    dc = time_loop(st.decode, steps) if len(st.dec) else 0.0
    return total_ms, wall * 1e3 / steps, ca, pf, dc


def cpu_baseline(wl, budget_s=15.0, min_s=10.0):
    """The fp64 oracle on the host cores, on the same workload: sequences of
    the batch in order (the whole batch again, if it takes less than min_s)
    until about budget_s of work, in GB/s of the same algorithmic decode
    bytes."""
    import numpy as np

    from oracle import attention as A
    from oracle.cache import run_workload

    sp = wl.spec
    st = run_workload(wl)
    q = wl.step_q()
    rows = np.concatenate([[0], np.cumsum(st.q_lens)])
    nseq = len(st.context_lens)
    done, t_used, byts = 0, 0.0, 0
    while t_used < (budget_s if done < nseq else min_s):
        s = done % nseq
        t0 = time.perf_counter()
        A.paged_attention(q[rows[s]:rows[s + 1]], st.pool.k, st.pool.v, st.tables[s:s + 1],
                          st.context_lens[s:s + 1], st.q_lens[s:s + 1], sp.scale, sp.dtype)
        t_used += time.perf_counter() - t0
        b, _ = decode_bytes(st.context_lens[s:s + 1], sp.num_q_heads, sp.num_kv_heads, sp.head_dim,
                            sp.block_size, sp.elem_bytes)
        byts += b
        done += 1
    try:
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    except Exception:
        threads = os.cpu_count()
    return {"value": round(byts / t_used / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} sequence passes over the {nseq} sequences of {sp.name} (fp64 NumPy oracle, "
                      f"{t_used:.1f}s of oracle time), decode bytes of those sequences over that time"}


DECODE_KERNEL_SOURCES = ("paged_kv_cache_403_amd/csrc/decode.hip", "paged_kv_cache_403_amd/csrc/decode_item.h",
                         "paged_kv_cache_403_amd/csrc/common.h")


def sources_sha256(paths):
    """One SHA-256 over the files a kernel is compiled from, in order."""
    import hashlib

    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(kernel_sources):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, each scaled by
    what the counter reads for a plain device copy of known size), or None
    when the kernel's sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "decode_kernel_mha_decode_7b_hbm_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        sha = sources_sha256(kernel_sources)
    except OSError:
        return None
    if rec.get("kernel_sources_sha256") != sha:
        return None
    return int(rec["hbm_bytes_per_launch"])


def decode_group_starts(wl, dec):
    """Runs of consecutive decode sequences forked from one prompt (or a
    prompt followed by its forks): the grouping hint of grouped decode."""
    import numpy as np

    batch = wl.batch
    root = [batch[i].parent if batch[i].parent >= 0 else batch[i].seq_id for i in dec]
    starts = [0] + [i for i in range(1, len(root)) if root[i] != root[i - 1]] + [len(root)]
    return np.array(starts, dtype=np.int32)


def time_decode(st, iters, warmup):
    """Average decode launch time (HIP events on the library's stream), us."""
    import torch

    settle(st.decode)
    for _ in range(warmup):
        st.decode()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        st.decode()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters * 1e3


def measure_block_sizes(name, iters, warmup, sizes=(8, 16, 32, 64)):
    """The same decode batch on pools of several block sizes: decode time
    and rate, and the pool's unused share from the library's block manager
    (1 - filled slots / slots of the blocks held) next to what reserving the
    batch's longest context for every sequence would leave unused."""
    import numpy as np

    import workloads

    base = workloads.make(name)
    rows = []
    for bs in sizes:
        wl = base if bs == base.spec.block_size else workloads.with_block_size(base, bs)
        st = Step(wl, -1)
        st.copy_append()
        us = time_decode(st, iters, warmup)
        held, used = st.cache.bm.usage()
        rows.append({"block_size": bs, "decode_us": round(us, 2),
                     "achieved_gbs": round(st.dec_bytes / (us * 1e-6) / 1e9, 1),
                     "decode_partition_tokens": st.part_used, "blocks_in_use": held,
                     "paged_waste": round(1.0 - used / (held * bs), 5)})
        log(f"{name} block_size {bs}: decode {us:.1f} us, unused share {rows[-1]['paged_waste']:.4f}")
    lens = np.array([p.context_len for p in base.batch], dtype=np.int64)
    static = 1.0 - float(lens.sum()) / float(len(lens) * lens.max())
    return {"workload": name, "sizes": rows, "static_reservation_waste": round(static, 4),
            "static_reservation_tokens": int(lens.max())}


def measure_long(name, iters, warmup):
    """Split-K decode of a few very long sequences: the library's partition
    choice and 512-token partitions, HIP-event launch times (planner, walk
    and merge together) and the rate of the decode's algorithmic bytes."""
    import torch

    import workloads

    wl = workloads.make(name)
    st = Step(wl, -1)
    st.copy_append()
    rows = []
    for part in (-1, 512):
        st.partition_size = part
        if part != -1:
            st.part_used = part
        wsb = st.P.pa_decode_workspace_bytes(len(st.dec), wl.spec.num_q_heads, wl.spec.head_dim, st.max_dec,
                                             part)
        st.ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device="cuda") if wsb else None
        us = time_decode(st, iters, warmup)
        rows.append({"partition_tokens": st.part_used, "decode_us": round(us, 2),
                     "achieved_gbs": round(st.dec_bytes / (us * 1e-6) / 1e9, 1),
                     "frac": round(st.dec_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
        log(f"{name}: {st.part_used}-token partitions, decode {us:.1f} us = {rows[-1]['achieved_gbs']:.0f} GB/s")
    return {"workload": name, "bytes_per_launch": st.dec_bytes, "runs": rows}


def time_prefill(st, iters, warmup):
    """Average prefill launch time (HIP events on the library's stream), us."""
    import torch

    settle(st.prefill)
    for _ in range(warmup):
        st.prefill()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        st.prefill()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters * 1e3


def measure_serving_loop(n_requests=1024, budget=8192, max_running=256):
    """The host scheduler loop (pa_sched_*) driving the kernels over a
    synthetic arrival trace, as a serving engine would each iteration: the
    scheduler picks decode tokens and prompt chunks under a token budget and
    hands out slots, then one pa_kv_append, one pa_prefill_chunk and one
    pa_decode run on the iteration's batch.  Shapes of the mixed workload
    (32 q / 8 KV heads, head_dim 128, bf16, block_size 16); prompts lognormal
    around 512 tokens (cap 4096), 1..64 new tokens each; a pool that holds
    every request.  K/V/q rows are synthetic values (their contents do not
    change the work).  Reports tokens per second through the whole loop
    (host scheduling, table uploads and kernels, wall clock) and the part of
    that time the GPU was busy (events around each iteration's kernels)."""
    import numpy as np
    import torch

    import paged_kv_cache_403_amd as P
    import workloads
    from paged_kv_cache_403_amd.runtime import PagedKVCache

    hq, hkv, d, bs, dt = 32, 8, 128, 16, "bf16"
    trace = workloads.arrival_trace(n_requests, seed=3, median_prompt=512, max_prompt=4096, max_new=64,
                                    mean_gap=0.25)
    nb = sum(-(-(p + m) // bs) for _, _, p, m in trace) + 1
    g = torch.Generator(device="cuda").manual_seed(403)
    rows = budget + max_running
    kbuf = torch.randn(rows, hkv, d, device="cuda", dtype=torch.bfloat16, generator=g)
    vbuf = torch.randn(rows, hkv, d, device="cuda", dtype=torch.bfloat16, generator=g)
    qbuf = torch.randn(rows, hq, d, device="cuda", dtype=torch.bfloat16, generator=g)
    obuf = torch.empty_like(qbuf)
    max_ctx = max(p + m for _, _, p, m in trace)
    wsb = P.pa_decode_workspace_bytes(max_running, hq, d, max_ctx, -1)
    ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device="cuda")
    scale = 1.0 / np.sqrt(d)

    def run():
        cache = PagedKVCache(nb, hkv, bs, d, dt, "cuda", np.arange(nb - 1, dtype=np.int32), fill_value=0.0)
        sched = P.Scheduler(cache.bm, budget, max_running)
        k, it, tokens = 0, 0, 0
        cached = {}
        events = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (k < len(trace) or sched.unfinished() > 0) and it < 100000:
            while k < len(trace) and trace[k][0] <= it:
                sched.add(*trace[k][1:])
                k += 1
            decodes, prefills, slots, pairs, finished, pre = sched.step()
            it += 1
            entries = [(rid, 1) for rid in decodes] + list(prefills)
            if not entries:
                continue
            for rid in pre:  # preempted: prefilled again from the start
                cached[rid] = 0
            T = int(sum(n for _, n in entries))
            tokens += T
            ids = np.array([rid for rid, _ in entries], np.int32)
            for rid, n in entries:
                cached[rid] = cached.get(rid, 0) + n
            lens = np.array([cached[rid] for rid, _ in entries], np.int32)
            mb = int(max(-(-int(lens.max()) // bs), 1))
            tables, _ = cache.bm.tables(ids, mb, nb - 1)
            slots_d = torch.from_numpy(slots).cuda()
            tables_d = torch.from_numpy(tables).cuda()
            lens_d = torch.from_numpy(lens).cuda()
            nd = len(decodes)
            if prefills:
                n_new = np.array([n for _, n in prefills], np.int32)
                cu_d = torch.from_numpy(np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)).cuda()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            if len(pairs):
                P.pa_copy_blocks(cache.desc, torch.from_numpy(pairs).cuda())
            P.pa_kv_append(cache.desc, kbuf[:T], vbuf[:T], slots_d)
            if nd:
                P.pa_decode(cache.desc, qbuf[:nd], obuf[:nd], tables_d[:nd], lens_d[:nd], int(lens[:nd].max()),
                            scale, -1, ws)
            if prefills:
                npre = int(n_new.sum())
                P.pa_prefill_chunk(cache.desc, qbuf[nd:nd + npre], obuf[nd:nd + npre], cu_d, lens_d[nd:],
                                   tables_d[nd:], int(n_new.max()), int(lens[nd:].max()), scale)
            b.record()
            events.append((a, b))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return it, tokens, wall, sum(x.elapsed_time(y) for x, y in events)

    run()  # warm-up pass over the same trace
    it, tokens, wall, gpu_ms = run()
    res = {"requests": n_requests, "iterations": it, "tokens": tokens, "wall_s": round(wall, 4),
           "tokens_per_s": round(tokens / wall, 1), "gpu_busy_ms": round(gpu_ms, 2),
           "gpu_share": round(gpu_ms / (wall * 1e3), 3), "token_budget": budget, "max_running": max_running}
    log(f"serving loop: {n_requests} requests, {it} iterations, {tokens} tokens in {wall:.3f} s = "
        f"{tokens / wall:.0f} tokens/s (GPU busy {gpu_ms:.1f} ms)")
    return res


def measure_fp8(name, ref_us, iters, warmup, prefill_name=None):
    """Decode of the same batch with an FP8 (E4M3) pool and 16-bit
    activations: time, algorithmic bytes (1-byte K/V), rate, and the speedup
    over the 16-bit pool's decode time ref_us."""
    import workloads

    wl = workloads.with_fp8_kv(workloads.make(name))
    st = Step(wl, -1)
    st.copy_append()
    us = time_decode(st, iters, warmup)
    gbs = st.dec_bytes / (us * 1e-6) / 1e9
    log(f"{wl.spec.name}: decode {us:.1f} us, {gbs:.0f} GB/s, x{ref_us / us:.2f} over the 16-bit pool")
    res = {"workload": wl.spec.name, "kv_dtype": "fp8 e4m3", "act_dtype": wl.spec.dtype,
           "k_scale": wl.spec.k_scale, "v_scale": wl.spec.v_scale, "decode_us": round(us, 2),
           "bytes_per_launch": st.dec_bytes, "achieved_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
           "speedup_vs_16bit_pool": round(ref_us / us, 3), "decode_partition_tokens": st.part_used}
    if prefill_name:
        # chunked prefill over an FP8 pool (the codes widened while staging)
        wlp = workloads.with_fp8_kv(workloads.make(prefill_name))
        stp = Step(wlp, -1)
        stp.copy_append()
        pus = time_prefill(stp, max(5, iters // 2), warmup)
        tf = stp.pre_flops / (pus * 1e-6) / 1e12
        log(f"{wlp.spec.name}: prefill {pus:.1f} us = {tf:.1f} TFLOP/s")
        res["prefill"] = {"workload": wlp.spec.name, "prefill_us": round(pus, 2), "tflops": round(tf, 2),
                          "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    return res


def measure_grouped(name, iters, warmup, fp8=False):
    """Plain split decode against prefix-grouped decode on one workload's
    decode batch: HIP-event times on the library's stream, and the K/V bytes
    each must read (logical: every sequence's context; unique: each
    physical block once)."""
    import torch

    import workloads

    wl = workloads.make(name)
    if fp8:
        wl = workloads.with_fp8_kv(wl)
    st = Step(wl, -1)
    sp = wl.spec
    P = st.P
    st.copy_append()
    hint = torch.from_numpy(decode_group_starts(wl, st.dec)).to("cuda")
    n = len(st.dec)
    part = 1024
    wsb = P.pa_decode_grouped_workspace_bytes(n, sp.num_q_heads, sp.head_dim, st.max_dec, part)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(st.q_dec)

    def grouped():
        P.pa_decode_grouped(st.cache.desc, st.q_dec, out, st.tab_dec, st.len_dec, st.max_dec, sp.scale, hint, part,
                            ws)

    def timed(fn):
        settle(fn)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters * 1e3

    plain_us = timed(st.decode)
    grouped_us = timed(grouped)
    torch.cuda.synchronize()
    diff = float((out.float() - st.out_dec.float()).abs().max())
    tabs, lens = st.plan.host_tables[st.dec], st.plan.host_lens[st.dec]
    blocks = set()
    for row, L in zip(tabs, lens):
        blocks.update(int(b) for b in row[:(int(L) + sp.block_size - 1) // sp.block_size])
    unique = len(blocks) * sp.num_kv_heads * sp.block_size * sp.head_dim * sp.kv_elem_bytes * 2
    log(f"{sp.name}: plain decode {plain_us:.1f} us, grouped decode {grouped_us:.1f} us "
        f"(unique K/V {unique / 1e6:.1f} MB of {st.dec_kv_bytes / 1e6:.1f} MB logical)")
    return {"workload": sp.name, "plain_decode_us": round(plain_us, 2), "plain_partition_tokens": st.part_used,
            "grouped_decode_us": round(grouped_us, 2), "grouped_partition_tokens": part,
            "speedup": round(plain_us / grouped_us, 3), "logical_kv_bytes": st.dec_kv_bytes,
            "unique_kv_bytes": unique, "grouped_unique_gbs": round(unique / (grouped_us * 1e-6) / 1e9, 1),
            "plain_logical_gbs": round(st.dec_kv_bytes / (plain_us * 1e-6) / 1e9, 1),
            "max_abs_diff_vs_plain": diff}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mha_decode_7b")
    ap.add_argument("--partition", type=int, default=-1, help="decode partition tokens (0 one pass, -1 auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill measurement")
    ap.add_argument("--no-grouped", action="store_true", help="skip the plain vs grouped decode measurement")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 KV-pool decode measurement")
    ap.add_argument("--no-block-sizes", action="store_true", help="skip the block-size sweep")
    ap.add_argument("--no-long", action="store_true", help="skip the long-context split-K measurement")
    ap.add_argument("--no-serving", action="store_true", help="skip the scheduler-loop measurement")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (the known-size reference for "
                         "the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log(f"device {torch.cuda.get_device_name(0)}")
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes 3 times")
        return
    wl = workloads.make(args.workload)
    sp = wl.spec
    st = Step(wl, args.partition)
    ms, wall_ms, ca_ms, pf_ms, dc_ms = time_steps(st, args.steps, args.warmup)
    step_bytes = st.dec_bytes + st.append_bytes + st.copy_bytes
    value = step_bytes / (ms * 1e-3) / 1e9
    n_seqs = len(wl.batch)
    log(f"{sp.name}: {ms * 1e3:.1f} us/step (wall {wall_ms * 1e3:.1f}), decode {dc_ms * 1e3:.1f} us, "
        f"copy+append {ca_ms * 1e3:.1f} us, {value:.0f} GB/s")
    dom_bytes, dom_ms, bound = st.dec_bytes, dc_ms, "hbm"
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sp.dtype,
        "data": "synthetic",
        "config": {
            "workload": sp.name, "num_seqs": n_seqs, "num_q_heads": sp.num_q_heads,
            "num_kv_heads": sp.num_kv_heads, "head_dim": sp.head_dim, "block_size": sp.block_size,
            "context_tokens": int(st.plan.host_lens.sum()), "max_context": int(st.plan.host_lens.max()),
            "decode_partition_tokens": getattr(st, "part_used", None), "parallelism": "none (1 GPU)",
        },
        "seqs_per_s": round(n_seqs / (ms * 1e-3), 1),
        "breakdown_us": {"copy_append": round(ca_ms * 1e3, 2), "prefill": round(pf_ms * 1e3, 2),
                         "decode": round(dc_ms * 1e3, 2)},
        "roofline": {"bound": bound, "achieved": round(dom_bytes / (dom_ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_bytes / (dom_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic(DECODE_KERNEL_SOURCES),
                     "kernel": "decode_kernel", "bytes_per_launch": dom_bytes},
    }
    if not args.no_prefill:
        wl5 = workloads.make("mixed_chunked_prefill")
        st5 = Step(wl5, -1)
        ms5, _, ca5, pf5, dc5 = time_steps(st5, max(5, args.steps // 5), 2)
        tf = st5.pre_flops / (pf5 * 1e-3) / 1e12
        dec_gbs = st5.dec_bytes / (dc5 * 1e-3) / 1e9
        log(f"mixed_chunked_prefill: step {ms5 * 1e3:.1f} us, prefill {pf5 * 1e3:.1f} us = {tf:.1f} TFLOP/s, "
            f"decode {dc5 * 1e3:.1f} us = {dec_gbs:.0f} GB/s")
        result["prefill"] = {
            "workload": "mixed_chunked_prefill", "ms_per_step": round(ms5, 5),
            "prefill_us": round(pf5 * 1e3, 2), "flops": st5.pre_flops,
            "tflops": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "decode_us": round(dc5 * 1e3, 2), "decode_gbs": round(dec_gbs, 1), "copy_append_us": round(ca5 * 1e3, 2),
        }
    if not args.no_grouped:
        result["shared_prefix"] = measure_grouped("gqa_shared_prefix", max(10, args.steps // 2), 3)
        if not args.no_fp8:
            result["shared_prefix"]["fp8_kv"] = measure_grouped("gqa_shared_prefix", max(10, args.steps // 2), 3,
                                                                fp8=True)
    if not args.no_fp8 and sp.dtype in ("f16", "bf16"):
        result["fp8_kv"] = measure_fp8(args.workload, dc_ms * 1e3, max(10, args.steps // 2), 3,
                                       None if args.no_prefill else "mixed_chunked_prefill")
    if not args.no_block_sizes:
        result["block_sizes"] = measure_block_sizes(args.workload, max(10, args.steps // 2), 3)
    if not args.no_long:
        result["long_split"] = measure_long("long_splitk_decode", max(10, args.steps // 2), 3)
    if not args.no_serving:
        result["serving_loop"] = measure_serving_loop()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
