#!/usr/bin/env python3
"""Benchmark of the paged KV-cache attention hot path on one MI355X.

A step is one pass of the hot path over one batch: the block manager's slot
mapping and copy-on-write pairs for the step's new tokens (host, prepared once
since repeating the step is idempotent), then on one HIP stream the
copy-on-write block copies, the KV append through the slot mapping, and the
attention kernels (paged decode for one-token sequences, chunked prefill for
chunks).  Inputs are resident in HBM before the timed region.

Headline workload: the long-context split-K decode batch (4 sequences of
131072 tokens, 32 q / 8 KV heads, head_dim 128, bf16, block_size 32,
partitions of 512 tokens merged by log-sum-exp): the largest of the five
synthetic configurations, and one that fits one GPU.  `value` is the step's
algorithmic bytes (K/V read, q/out, tables, lengths, append) over the median
step time.

Timing (every figure): each iteration has its own pair of HIP events on the
stream the library launches on (torch's current stream); between iterations,
outside the timed region, a 512 MiB scratch buffer is written and another
512 MiB read, so no K/V byte of the previous iteration is left in the 256 MB
Infinity Cache and no dirty flush line is written back during the next one;
after 0.1 s of the same work (clocks settle) and W warm-up iterations, the
median of K iterations is reported (back-to-back "warm" loop means are given
beside the decode figures for comparison).

Beside the headline: every configuration's step with its kernel times and
rates (tiny decode latency; the 7B-shaped MHA decode; the shared-prefix batch
through plain and prefix-grouped decode, rates on unique and logical bytes,
and its copy-on-write copies; the long batch at the library's partition
choice; the mixed chunked-prefill step), the FP8 pool, the block-size sweep,
decode at 8 q heads per KV head, prefill of one or two chunks with and
without the key split, and the fp64 oracle's rate on the host cores for each
configuration.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16/fp16 matrix peak
METRIC = "paged decode KV-read GB/s (% HBM peak) + seqs/s; prefill TFLOP/s (% MFMA)"
HEADLINE = "long_splitk_decode"
FLUSH_BYTES = 512 << 20
SETTLE_S = 0.1  # untimed repetitions before any warm-up and timing


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


class Timer:
    """Median of per-iteration HIP-event times with the cache flushed between
    iterations (outside the timed region)."""

    def __init__(self, device="cuda", flush=True):
        import torch

        self.torch = torch
        self.flush_on = flush
        if flush:
            self.wbuf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=device)
            self.rbuf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=device)
            self.sink = torch.zeros((), dtype=torch.float32, device=device)
            self.k = 0

    def flush(self):
        if self.flush_on:
            self.k += 1
            self.wbuf.fill_(self.k)
            self.sink += self.rbuf.sum()

    def settle(self, fn, seconds=SETTLE_S):
        torch = self.torch
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(8):
                fn()
            torch.cuda.synchronize()

    def median_us(self, fn, iters, warmup, settle=True):
        """Median and all per-iteration times (us) of fn."""
        torch = self.torch
        if settle:
            self.settle(fn)
        for _ in range(warmup):
            self.flush()
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        torch.cuda.synchronize()
        for a, b in ev:
            self.flush()
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) * 1e3 for a, b in ev]
        return statistics.median(ts), ts

    def warm_us(self, fn, iters):
        """Mean of a back-to-back loop between one event pair (no flush)."""
        torch = self.torch
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / iters


def spread(ts):
    q = statistics.quantiles(ts, n=10) if len(ts) >= 10 else [min(ts), max(ts)]
    return {"p10_us": round(q[0], 2), "p90_us": round(q[-1], 2), "min_us": round(min(ts), 2)}


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
        self.part_used = None
        if len(dec):
            self.q_dec = to_device(q_all[starts[dec]], sp.dtype, device)
            self.out_dec = torch.empty_like(self.q_dec)
            idx = torch.from_numpy(dec).to(device)
            self.tab_dec = self.plan.block_tables[idx].contiguous()
            self.len_dec = self.plan.context_lens[idx].contiguous()
            self.max_dec = int(self.plan.host_lens[dec].max())
            self.set_partition(partition_size)
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
        self.npairs = len(self.plan.host_pairs)
        self.copy_bytes = self.npairs * sp.num_kv_heads * sp.block_size * sp.head_dim * kb * 4 + self.npairs * 8
        self.step_bytes = self.dec_bytes + self.append_bytes + self.copy_bytes
        torch.cuda.synchronize()
        log(f"{sp.name}: setup {time.time() - t0:.1f}s, {len(dec)} decode seqs, {len(pre)} chunks, "
            f"{self.npairs} copy pairs")

    def set_partition(self, partition_size):
        import torch

        sp = self.wl.spec
        self.partition_size = partition_size
        wsb = self.P.pa_decode_workspace_bytes(len(self.dec), sp.num_q_heads, sp.head_dim, self.max_dec,
                                               partition_size)
        self.ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device="cuda") if wsb else None
        self.part_used = int(self.P.pa_decode_choose_partition(self.cache.desc, len(self.dec), sp.num_q_heads,
                                                               self.max_dec)
                             if partition_size == -1 else partition_size)

    def copy(self):
        self.P.pa_copy_blocks(self.cache.desc, self.plan.cow_pairs)

    def append(self):
        self.P.pa_kv_append(self.cache.desc, self.k_new, self.v_new, self.plan.slot_mapping)

    def copy_append(self):
        self.copy()
        self.append()

    def decode(self):
        sp = self.wl.spec
        self.P.pa_decode(self.cache.desc, self.q_dec, self.out_dec, self.tab_dec, self.len_dec, self.max_dec,
                         sp.scale, self.partition_size, self.ws)

    def prefill(self):
        sp = self.wl.spec
        self.P.pa_prefill_chunk(self.cache.desc, self.q_pre, self.out_pre, self.cu_pre, self.len_pre, self.tab_pre,
                                self.maxq_pre, self.maxc_pre, sp.scale)

    def step(self):
        self.copy_append()
        if len(self.pre):
            self.prefill()
        if len(self.dec):
            self.decode()


def gbs(nbytes, us):
    return nbytes / (us * 1e-6) / 1e9


def decode_entry(st, timer, iters, warmup, name="decode"):
    """Flushed median of the decode launch (planner, walk and merge for a
    split), its rate, and the back-to-back warm mean."""
    us, ts = timer.median_us(st.decode, iters, warmup)
    warm = timer.warm_us(st.decode, max(10, iters // 2))
    rate = gbs(st.dec_bytes, us)
    log(f"{st.wl.spec.name}: {name} {us:.1f} us = {rate:.0f} GB/s ({rate / HBM_PEAK_GBS:.1%}); warm {warm:.1f} us")
    return {"us": round(us, 2), **spread(ts), "warm_us": round(warm, 2), "bytes": st.dec_bytes,
            "kv_bytes": st.dec_kv_bytes, "gbs": round(rate, 1), "frac": round(rate / HBM_PEAK_GBS, 4),
            "seqs_per_s": round(len(st.dec) / (us * 1e-6), 1), "partition_tokens": st.part_used}


def unique_kv_bytes(st):
    """K/V bytes of the decode batch counting each physical block once."""
    sp = st.wl.spec
    tabs, lens = st.plan.host_tables[st.dec], st.plan.host_lens[st.dec]
    blocks = set()
    for row, L in zip(tabs, lens):
        blocks.update(int(b) for b in row[:(int(L) + sp.block_size - 1) // sp.block_size])
    return len(blocks) * sp.num_kv_heads * sp.block_size * sp.head_dim * sp.kv_elem_bytes * 2


def group_starts(wl, dec):
    """Runs of consecutive decode sequences forked from one prompt (or a
    prompt followed by its forks): the grouping hint of grouped decode."""
    import numpy as np

    batch = wl.batch
    root = [batch[i].parent if batch[i].parent >= 0 else batch[i].seq_id for i in dec]
    starts = [0] + [i for i in range(1, len(root)) if root[i] != root[i - 1]] + [len(root)]
    return np.array(starts, dtype=np.int32)


def grouped_entry(st, timer, iters, warmup, part=1024):
    """Prefix-grouped decode of the step's decode batch: flushed median, the
    rate on unique K/V bytes (each physical block once: what the method must
    move) and on logical bytes, and the largest difference from plain decode."""
    import torch

    sp = st.wl.spec
    P = st.P
    hint = torch.from_numpy(group_starts(st.wl, st.dec)).to("cuda")
    n = len(st.dec)
    wsb = P.pa_decode_grouped_workspace_bytes(n, sp.num_q_heads, sp.head_dim, st.max_dec, part)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(st.q_dec)

    def grouped():
        P.pa_decode_grouped(st.cache.desc, st.q_dec, out, st.tab_dec, st.len_dec, st.max_dec, sp.scale, hint, part,
                            ws)

    us, ts = timer.median_us(grouped, iters, warmup)
    warm = timer.warm_us(grouped, max(10, iters // 2))
    st.decode()
    torch.cuda.synchronize()
    diff = float((out.float() - st.out_dec.float()).abs().max())
    uniq = unique_kv_bytes(st)
    meta = st.dec_bytes - st.dec_kv_bytes
    rate = gbs(uniq + meta, us)
    log(f"{sp.name}: grouped decode {us:.1f} us, {rate:.0f} GB/s on unique bytes ({rate / HBM_PEAK_GBS:.1%}); "
        f"warm {warm:.1f} us")
    return {"us": round(us, 2), **spread(ts), "warm_us": round(warm, 2), "partition_tokens": part,
            "unique_kv_bytes": uniq, "unique_bytes": uniq + meta, "unique_gbs": round(rate, 1),
            "unique_frac": round(rate / HBM_PEAK_GBS, 4), "logical_gbs": round(gbs(st.dec_bytes, us), 1),
            "max_abs_diff_vs_plain": diff}


def run_config(name, timer, iters, warmup, partition=-1, fp8=False):
    """One configuration's step and its parts, all flushed medians."""
    import workloads

    wl = workloads.make(name)
    if fp8:
        wl = workloads.with_fp8_kv(wl)
    sp = wl.spec
    st = Step(wl, partition)
    step_us, ts = timer.median_us(st.step, iters, warmup)
    res = {"workload": sp.name, "num_seqs": len(wl.batch), "dtype": sp.dtype,
           "kv_dtype": sp.kv_dtype or sp.dtype, "block_size": sp.block_size,
           "step_us": round(step_us, 2), **{"step_" + k: v for k, v in spread(ts).items()},
           "step_bytes": st.step_bytes, "step_gbs": round(gbs(st.step_bytes, step_us), 1)}
    if st.npairs:
        cus, _ = timer.median_us(st.copy, iters, warmup, settle=False)
        res["cow_copy"] = {"pairs": st.npairs, "bytes": st.copy_bytes, "us": round(cus, 2),
                           "gbs": round(gbs(st.copy_bytes, cus), 1)}
    aus, _ = timer.median_us(st.append, iters, warmup, settle=False)
    res["append"] = {"tokens": int(st.plan.n_new.sum()), "bytes": st.append_bytes, "us": round(aus, 2)}
    if len(st.pre):
        pus, pts = timer.median_us(st.prefill, iters, warmup)
        tf = st.pre_flops / (pus * 1e-6) / 1e12
        res["prefill"] = {"chunks": len(st.pre), "us": round(pus, 2), **spread(pts), "flops": st.pre_flops,
                          "tflops": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                          "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
        log(f"{sp.name}: prefill {pus:.1f} us = {tf:.1f} TFLOP/s ({tf / MFMA_BF16_PEAK_TFLOPS:.1%})")
    if len(st.dec):
        res["decode"] = decode_entry(st, timer, iters, warmup)
    log(f"{sp.name}: step {step_us:.1f} us")
    return res, st


def measure_block_sizes(name, timer, iters, warmup, sizes=(8, 16, 32, 64)):
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
        d = decode_entry(st, timer, iters, warmup)
        held, used = st.cache.bm.usage()
        rows.append({"block_size": bs, "decode_us": d["us"], "gbs": d["gbs"], "partition_tokens": st.part_used,
                     "blocks_in_use": held, "paged_waste": round(1.0 - used / (held * bs), 5)})
        log(f"{name} block_size {bs}: unused share {rows[-1]['paged_waste']:.4f}")
    lens = np.array([p.context_len for p in base.batch], dtype=np.int64)
    static = 1.0 - float(lens.sum()) / float(len(lens) * lens.max())
    return {"workload": name, "sizes": rows, "static_reservation_waste": round(static, 4),
            "static_reservation_tokens": int(lens.max())}


def measure_gqa8(timer, iters, warmup):
    """Decode at 8 q heads per KV head (the matrix-core walk): 4 sequences of
    65536 tokens, 64 q / 8 KV heads, head_dim 128, 16-token blocks, the
    library's partitions, on a bf16 pool and on an FP8 pool."""
    import workloads

    rows = []
    for fp8 in (False, True):
        wl = workloads.custom(64, 8, 128, 16, "bf16", [65536] * 4, name="long_gqa8_decode")
        if fp8:
            wl = workloads.with_fp8_kv(wl)
        st = Step(wl, -1)
        st.copy_append()
        rows.append({"kv_dtype": "fp8" if fp8 else "bf16", **decode_entry(st, timer, iters, warmup)})
        del st
    return {"workload": "long_gqa8_decode: 4 x 65536 tokens, 64 q / 8 KV heads, head_dim 128, bf16 activations, "
                        "block_size 16", "rows": rows}


def measure_prefill_split(timer, iters, warmup):
    """Prefill of few chunks, where one workgroup per (row tile, KV head)
    leaves most compute units idle: one and two 512-token chunks on 4096 and
    16384 cached tokens (32 q / 8 KV heads, head_dim 128, bf16, 16-token
    blocks; the one chunk on 16384 also over an FP8 pool), the whole-keys
    launch against the key split the library chooses (pa_prefill_chunk_split
    with key_splits 0)."""
    import torch

    import workloads

    rows = []
    cases = [(c, False) for c in ((4096,), (16384,), (4096, 4096), (16384, 16384))] + [((16384,), True)]
    for cached, fp8 in cases:
        wl = workloads.custom(32, 8, 128, 16, "bf16", [c + 512 for c in cached], n_new=[512] * len(cached),
                              name="few_chunk_prefill")
        if fp8:
            wl = workloads.with_fp8_kv(wl)
        sp = wl.spec
        st = Step(wl, 0)
        st.copy_append()
        P = st.P
        k = P.pa_prefill_choose_splits(st.cache.desc, len(st.pre), sp.num_q_heads, st.maxq_pre, st.maxc_pre)
        ws = torch.empty(max(P.pa_prefill_workspace_bytes(st.q_pre.shape[0], sp.num_q_heads, sp.head_dim, k), 16),
                         dtype=torch.uint8, device="cuda")

        def split():
            P.pa_prefill_chunk_split(st.cache.desc, st.q_pre, st.out_pre, st.cu_pre, st.len_pre, st.tab_pre,
                                     st.maxq_pre, st.maxc_pre, sp.scale, k, ws)

        whole_us, _ = timer.median_us(st.prefill, iters, warmup)
        split_us, _ = timer.median_us(split, iters, warmup)
        row = {"chunks": len(cached), "cached_tokens": cached[0], "kv_dtype": "fp8" if fp8 else "bf16",
               "key_splits": k, "flops": st.pre_flops,
               "whole_us": round(whole_us, 2), "split_us": round(split_us, 2)}
        for tag, us in (("whole", whole_us), ("split", split_us)):
            tf = st.pre_flops / (us * 1e-6) / 1e12
            row[tag + "_tflops"] = round(tf, 2)
            row[tag + "_frac"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
        log(f"few-chunk prefill {len(cached)} x 512 on {cached[0]} ({row['kv_dtype']} pool): whole {whole_us:.1f} us, "
            f"{k} key splits {split_us:.1f} us")
        rows.append(row)
        del st, ws
        torch.cuda.empty_cache()
    return {"workload": "few_chunk_prefill: 1 or 2 chunks of 512 tokens on 4096 or 16384 cached tokens, 32 q / 8 KV "
                        "heads, head_dim 128, bf16 activations (bf16 pool; one row over an FP8 pool), block_size 16",
            "peak": MFMA_BF16_PEAK_TFLOPS, "rows": rows}


# ---- the fp64 oracle on the host -----------------------------------------------------

def host_info():
    """CPU model, threads the oracle's BLAS uses, and the BLAS build."""
    import numpy as np

    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    threads = None
    try:
        import threadpoolctl

        info = [x for x in threadpoolctl.threadpool_info() if x.get("user_api") == "blas"]
        if info:
            threads = int(info[0]["num_threads"])
    except Exception:
        pass
    if threads is None:
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    blas = {}
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = {"name": b.get("name"), "version": b.get("version"),
                "config": (b.get("openblas configuration") or "")[:120]}
    except Exception:
        pass
    return {"cpu_model": model, "threads": threads, "affinity_cpus": len(os.sched_getaffinity(0)), "blas": blas}


def oracle_rate(name, budget_s):
    """The fp64 NumPy oracle (gather through the tables, then plain softmax
    attention) over the configuration's sequences in batch order until about
    budget_s seconds of oracle time: decode rows in GB/s of the same
    algorithmic bytes, chunk rows in GFLOP/s of the same algorithmic flops."""
    import numpy as np

    import workloads
    from oracle import attention as A
    from oracle.cache import run_workload

    wl = workloads.make(name)
    sp = wl.spec
    st = run_workload(wl)
    q = wl.step_q()
    rows = np.concatenate([[0], np.cumsum(st.q_lens)])
    nseq = len(st.context_lens)
    t_dec = t_pre = 0.0
    b_dec = f_pre = 0
    done = 0
    while t_dec + t_pre < budget_s and done < 64 * nseq:
        s = done % nseq
        t0 = time.perf_counter()
        A.paged_attention(q[rows[s]:rows[s + 1]], st.pool.k, st.pool.v, st.tables[s:s + 1],
                          st.context_lens[s:s + 1], st.q_lens[s:s + 1], sp.scale, sp.dtype)
        dt = time.perf_counter() - t0
        n, L = int(st.q_lens[s]), int(st.context_lens[s])
        if n == 1:
            t_dec += dt
            b_dec += decode_bytes([L], sp.num_q_heads, sp.num_kv_heads, sp.head_dim, sp.block_size,
                                  sp.elem_bytes)[0]
        else:
            t_pre += dt
            f_pre += prefill_flops([L - n], [n], sp.num_q_heads, sp.head_dim)
        done += 1
    res = {"workload": name, "sequence_passes": done, "of_sequences": nseq,
           "oracle_s": round(t_dec + t_pre, 2)}
    if t_dec:
        res["decode_gbs"] = round(b_dec / t_dec / 1e9, 4)
    if t_pre:
        res["prefill_gflops"] = round(f_pre / t_pre / 1e9, 3)
    log(f"oracle {name}: {done} sequence passes in {t_dec + t_pre:.1f} s")
    return res


# ---- HBM traffic from the committed counter summary ------------------------------------

DECODE_KERNEL_SOURCES = ("paged_kv_cache_403_amd/csrc/decode.hip", "paged_kv_cache_403_amd/csrc/decode_item.h",
                         "paged_kv_cache_403_amd/csrc/common.h")
COUNTERS = "profiles/split_decode_long_splitk_decode_p512_hbm_counters.json"


def sources_sha256(paths):
    """One SHA-256 over the files a kernel is compiled from, in order."""
    import hashlib

    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic():
    """HBM bytes per launch of the headline decode (its three kernels) from
    the committed rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, each
    scaled by what the counter reads for a plain device copy of known size),
    or None when the kernels' sources have changed since the counters were
    taken."""
    try:
        with open(os.path.join(ROOT, COUNTERS)) as f:
            rec = json.load(f)
        sha = sources_sha256(DECODE_KERNEL_SOURCES)
    except OSError:
        return None
    if rec.get("kernel_sources_sha256") != sha:
        return None
    return int(rec["hbm_bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--partition", type=int, default=None,
                    help="decode partition tokens (0 one pass, -1 library choice; default: the workload's "
                         "stated partitions, else -1)")
    ap.add_argument("--headline-only", action="store_true", help="time the headline step only")
    ap.add_argument("--grouped", action="store_true",
                    help="also time prefix-grouped decode of the workload's decode batch")
    ap.add_argument("--no-flush", action="store_true", help="no cache flush between timed iterations")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the other configurations")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 KV-pool measurements")
    ap.add_argument("--no-block-sizes", action="store_true", help="skip the block-size sweep")
    ap.add_argument("--no-gqa8", action="store_true", help="skip the 8-q-heads-per-KV-head decode batch")
    ap.add_argument("--no-prefill-split", action="store_true",
                    help="skip the few-chunk prefill batches (whole keys against the key split)")
    ap.add_argument("--oracle-s", type=float, default=12.0, help="oracle seconds for the headline baseline")
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
    timer = Timer(flush=not args.no_flush)
    wl = workloads.make(args.workload)
    sp = wl.spec
    part = args.partition if args.partition is not None else (sp.partition_size or -1)
    st = Step(wl, part)
    K, W = args.steps, args.warmup
    # the timed steps: W warm-ups, then K steps each between its own events
    timer.settle(st.step)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_us, ts = timer.median_us(st.step, K, W, settle=False)
    wall = time.perf_counter() - t0
    value = gbs(st.step_bytes, step_us)
    n_seqs = len(wl.batch)
    log(f"{sp.name}: step {step_us:.1f} us median of {K} (wall {wall * 1e3 / K:.1f} ms per step with flush), "
        f"{value:.0f} GB/s")
    head = decode_entry(st, timer, K, W) if len(st.dec) else None
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "settle_s": SETTLE_S,
        "ms_per_step": round(step_us / 1e3, 5),
        "step_timing": {"statistic": "median", **spread(ts),
                        "flush": None if args.no_flush else "write 512 MiB + read 512 MiB between iterations"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sp.dtype,
        "data": "synthetic",
        "config": {
            "workload": sp.name, "num_seqs": n_seqs, "num_q_heads": sp.num_q_heads,
            "num_kv_heads": sp.num_kv_heads, "head_dim": sp.head_dim, "block_size": sp.block_size,
            "context_tokens": int(st.plan.host_lens.sum()), "max_context": int(st.plan.host_lens.max()),
            "decode_partition_tokens": st.part_used, "parallelism": "none (1 GPU)",
        },
        "seqs_per_s": round(n_seqs / (step_us * 1e-6), 1),
        "step_bytes": st.step_bytes,
    }
    if head is not None:
        result["decode"] = head
        result["roofline"] = {
            "bound": "hbm", "achieved": head["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": head["frac"],
            "traffic": counter_traffic(),
            "kernel": ("pa_decode: decode_plan_kernel + decode_persistent_kernel + decode_reduce_kernel"
                       if st.part_used and st.part_used < st.max_dec else "pa_decode: decode_kernel"),
            "bytes_per_launch": st.dec_bytes, "launch_us": head["us"]}
    if args.grouped:
        result["grouped"] = grouped_entry(st, timer, K, W)
    if not args.headline_only:
        configs = {}
        if not args.no_configs:
            for name in workloads.CONFIG_NAMES:
                if name == sp.name:
                    continue
                res, cst = run_config(name, timer, K, W)
                if name == "gqa_shared_prefix":
                    res["grouped"] = grouped_entry(cst, timer, K, W)
                configs[name] = res
                del cst
                torch.cuda.empty_cache()
            if sp.name == HEADLINE and "partition_tokens" in (head or {}):
                st.set_partition(-1)
                configs[HEADLINE + "_library_partition"] = {"decode": decode_entry(st, timer, K, W)}
        result["configs"] = configs
        if not args.no_fp8:
            fp8 = {}
            for name in ("mha_decode_7b", "gqa_shared_prefix", "mixed_chunked_prefill"):
                res, cst = run_config(name, timer, K, W, fp8=True)
                if name == "gqa_shared_prefix":
                    res["grouped"] = grouped_entry(cst, timer, K, W)
                fp8[name] = res
                del cst
                torch.cuda.empty_cache()
            result["fp8_kv"] = fp8
        if not args.no_block_sizes:
            result["block_sizes"] = measure_block_sizes("mha_decode_7b", timer, max(20, K // 2), W)
        if not args.no_gqa8:
            result["gqa8"] = measure_gqa8(timer, max(20, K // 2), W)
        if not args.no_prefill_split:
            result["prefill_split"] = measure_prefill_split(timer, max(20, K // 2), W)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        hi = host_info()
        base = oracle_rate(sp.name, args.oracle_s)
        result["cpu_baseline"] = {
            "value": base.get("decode_gbs"), "unit": "GB/s", "cores": hi["threads"], "kind": "oracle",
            "sample": f"{base['sequence_passes']} sequence passes over the {base['of_sequences']} sequences of "
                      f"{sp.name} (fp64 NumPy oracle, {base['oracle_s']} s of oracle time), decode bytes of those "
                      f"sequences over that time",
            "host": hi}
        if not args.headline_only and not args.no_configs:
            result["cpu_baseline"]["per_config"] = [oracle_rate(n, 4.0) for n in workloads.CONFIG_NAMES
                                                    if n != sp.name]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
