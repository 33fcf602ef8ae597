"""Seeded synthetic workloads for paged KV-cache attention.

This module only *draws inputs*: sequence lengths, the order in which the
physical block pool hands out blocks, the logical K/V values of every
sequence, the query rows, and the order of cache operations (add a sequence,
fork it from a shared prefix holder, append tokens).  It holds none of the
method's arithmetic: no block-table or slot computation, no attention, no
copy-on-write decision.  Both the CPU oracle and the HIP path consume the same
drawn inputs and each applies its own block manager and kernels to them.

Workloads follow the problem statement of the PagedAttention pages (fixed
block size in tokens, per-sequence block tables, context lengths that include
the token appended in the step, read-only shared prefix blocks), with the
sizes of the five synthetic configurations:

  tiny_decode            4 seqs, lens {1,15,16,33}, BS 16, 2/2 heads, D 64, fp32
  mha_decode_7b          64 seqs, lens U{128..2048}, BS 16, 32/32 heads, D 128, fp16
  gqa_shared_prefix      256 seqs in groups of 8 sharing a 512-token prefix,
                         lens lognormal(median 512, sigma 1, cap 8192),
                         BS 16, 32/8 heads, D 128, bf16
  long_splitk_decode     4 seqs x 131072 tokens, BS 32, 32/8 heads, D 128,
                         bf16, 512-token partitions
  mixed_chunked_prefill  8 chunks of 512 tokens on cached contexts U{0..4096}
                         plus 120 decode seqs with lens U{256..4096},
                         BS 16, 32/8 heads, D 128, bf16

Values are fp32 N(0,1) draws rounded to the storage type with round to
nearest even.  Storage representations on the host: fp32 -> float32,
fp16 -> float16, bf16 -> uint16 bit patterns (NumPy has no bfloat16).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

SEED_ROOT = 403

# storage type name -> (host numpy dtype of the stored bits/values, bytes)
STORAGE = {"f32": (np.float32, 4), "f16": (np.float16, 2), "bf16": (np.uint16, 2)}

# value draws are made in fixed-size chunks, each from its own child seed, so
# the result does not depend on how many threads fill it
_CHUNK = 1 << 22

CONFIG_NAMES = (
    "tiny_decode",
    "mha_decode_7b",
    "gqa_shared_prefix",
    "long_splitk_decode",
    "mixed_chunked_prefill",
)


@dataclass(frozen=True)
class Spec:
    """Shape of one paged-cache workload (structure only)."""

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str  # "f32" | "f16" | "bf16"
    num_blocks: int  # physical blocks in the pool, the poison block included
    partition_size: int = 0  # decode split-K partition in tokens, 0 = one pass
    kv_dtype: str = ""  # pool element type when it differs from dtype: "fp8" (E4M3 codes)
    k_scale: float = 1.0  # FP8 pool: value = code * scale
    v_scale: float = 1.0

    @property
    def kv(self):
        """(kv_dtype, k_scale, v_scale) of an FP8 pool, else None."""
        return (self.kv_dtype, self.k_scale, self.v_scale) if self.kv_dtype else None

    @property
    def kv_elem_bytes(self) -> int:
        return 1 if self.kv_dtype == "fp8" else self.elem_bytes

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def poison_block(self) -> int:
        """Reserved block that table padding points at; never handed out."""
        return self.num_blocks - 1

    @property
    def elem_bytes(self) -> int:
        return STORAGE[self.dtype][1]


@dataclass
class SeqPlan:
    """One sequence of the workload.

    parent/keep: the sequence is forked from `parent` sharing its first
    `keep` tokens (parent == -1: a fresh sequence, keep == 0).
    pre_len: tokens in the cache before the step (shared ones included).
    n_new: tokens appended in the step; they are also the query rows.
    in_batch: False for prefix holders that only own shared blocks.
    """

    seq_id: int
    parent: int
    keep: int
    pre_len: int
    n_new: int
    in_batch: bool

    @property
    def context_len(self) -> int:
        return self.pre_len + self.n_new


@dataclass
class Op:
    """A cache operation in the order the workload issues it."""

    kind: str  # "add" | "fork" | "append"
    seq: int
    parent: int = -1
    keep: int = 0
    n: int = 0
    k: np.ndarray | None = None  # [n][Hkv][D] storage repr, for "append"
    v: np.ndarray | None = None


@dataclass
class Workload:
    spec: Spec
    seqs: list  # SeqPlan, setup order (prefix holders first, then the batch)
    free_order: np.ndarray  # int32 permutation of 0..num_blocks-2
    own_k: dict  # seq_id -> [pre_len - keep + n_new][Hkv][D]
    own_v: dict
    q: dict  # seq_id -> [n_new][Hq][D]
    seed: tuple = ()
    notes: dict = field(default_factory=dict)

    # ---- views (structure only) -------------------------------------------------
    @property
    def batch(self) -> list:
        return [p for p in self.seqs if p.in_batch]

    def plan(self, seq_id: int) -> SeqPlan:
        for p in self.seqs:
            if p.seq_id == seq_id:
                return p
        raise KeyError(seq_id)

    def setup_ops(self):
        """Operations that build the pre-step cache, in issue order."""
        ops = []
        for p in self.seqs:
            if p.parent < 0:
                ops.append(Op("add", p.seq_id))
            else:
                ops.append(Op("fork", p.seq_id, parent=p.parent, keep=p.keep))
            n_own = p.pre_len - p.keep
            if n_own > 0:
                ops.append(Op("append", p.seq_id, n=n_own,
                              k=self.own_k[p.seq_id][:n_own], v=self.own_v[p.seq_id][:n_own]))
        return ops

    def step_ops(self):
        """The step's appends, one per batch sequence in batch order."""
        ops = []
        for p in self.batch:
            n_own = p.pre_len - p.keep
            ops.append(Op("append", p.seq_id, n=p.n_new,
                          k=self.own_k[p.seq_id][n_own:], v=self.own_v[p.seq_id][n_own:]))
        return ops

    def logical_kv(self, seq_id: int):
        """Full logical K/V of a sequence: inherited prefix then own tokens."""
        p = self.plan(seq_id)
        if p.parent < 0:
            return self.own_k[seq_id], self.own_v[seq_id]
        pk, pv = self.logical_kv(p.parent)
        return (np.concatenate([pk[: p.keep], self.own_k[seq_id]]),
                np.concatenate([pv[: p.keep], self.own_v[seq_id]]))

    def step_q(self):
        """Query rows of the batch, concatenated in batch order: [sum n_new][Hq][D]."""
        return np.concatenate([self.q[p.seq_id] for p in self.batch])

    def step_kv(self):
        """New tokens' K/V concatenated in batch order: [sum n_new][Hkv][D]."""
        ks, vs = [], []
        for p in self.batch:
            n_own = p.pre_len - p.keep
            ks.append(self.own_k[p.seq_id][n_own:])
            vs.append(self.own_v[p.seq_id][n_own:])
        return np.concatenate(ks), np.concatenate(vs)


# ---- value draws ----------------------------------------------------------------

def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values -> storage representation, round to nearest even."""
    if dtype == "f32":
        return x.astype(np.float32, copy=False)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
        # finite inputs only: add half an ulp of bf16, ties to the even result
        r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        return (r >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dtype)


def _round_fast(x: np.ndarray, dtype: str) -> np.ndarray:
    """Same rounding as round_to_storage, through torch's multi-threaded casts."""
    if dtype == "f32":
        return x
    import torch

    t = torch.from_numpy(x)
    if dtype == "f16":
        return t.to(torch.float16).numpy()
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _threads(threads=None):
    return threads or min(16, len(os.sched_getaffinity(0)))


def normal_values_many(requests, dtype: str, threads: int | None = None):
    """N(0,1) fp32 draws for several streams at once: requests is a list of
    (key, shape); each stream is filled in fixed-size chunks, chunk c from the
    seed (key..., c), so values do not depend on the thread count."""
    outs, jobs = [], []
    for key, shape in requests:
        n = int(np.prod(shape))
        buf = np.empty(n, dtype=np.float32)
        outs.append((buf, shape))
        for c in range((n + _CHUNK - 1) // _CHUNK):
            jobs.append((key, c, buf, c * _CHUNK, min(n, (c + 1) * _CHUNK)))

    def fill(job):
        key, c, buf, a, b = job
        g = np.random.default_rng(np.random.SeedSequence(list(key) + [c]))
        g.standard_normal(b - a, dtype=np.float32, out=buf[a:b])

    nt = _threads(threads)
    if len(jobs) > 1 and nt > 1:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(fill, jobs))
    else:
        for j in jobs:
            fill(j)
    return [_round_fast(buf, dtype).reshape(shape) for buf, shape in outs]


def normal_values(key: tuple, shape, dtype: str, threads: int | None = None) -> np.ndarray:
    """N(0,1) fp32 draws for the stream `key`, rounded to `dtype`."""
    return normal_values_many([(key, shape)], dtype, threads)[0]


def _stream(cfg_key, *parts):
    return (SEED_ROOT,) + tuple(cfg_key) + tuple(parts)


def synthesize(spec: Spec, plans: list, cfg_key: tuple, notes=None) -> Workload:
    """Draw the pool order and every value for a list of sequence plans."""
    H, D = spec.num_kv_heads, spec.head_dim
    g = np.random.default_rng(np.random.SeedSequence(list(_stream(cfg_key, 1))))
    free_order = g.permutation(spec.num_blocks - 1).astype(np.int32)
    reqs, slots = [], []
    for p in plans:
        n_own = p.context_len - p.keep
        reqs.append((_stream(cfg_key, 2, p.seq_id), (n_own, H, D)))
        slots.append(("k", p.seq_id))
        reqs.append((_stream(cfg_key, 3, p.seq_id), (n_own, H, D)))
        slots.append(("v", p.seq_id))
    for p in plans:
        if p.in_batch:
            reqs.append((_stream(cfg_key, 4, p.seq_id), (p.n_new, spec.num_q_heads, D)))
            slots.append(("q", p.seq_id))
    vals = normal_values_many(reqs, spec.dtype)
    own_k, own_v, q = {}, {}, {}
    dst = {"k": own_k, "v": own_v, "q": q}
    for (kind, sid), arr in zip(slots, vals):
        dst[kind][sid] = arr
    return Workload(spec, plans, free_order, own_k, own_v, q, seed=tuple(cfg_key), notes=notes or {})


def pool_blocks_needed(plans: list, block_size: int) -> int:
    """Upper bound of blocks the plans can occupy (a partially shared last
    block may be replaced by a private copy, counted once more)."""
    need = 0
    for p in plans:
        need += -(-p.context_len // block_size) - (p.keep // block_size)
    return need


def sized_pool(plans, block_size, fixed=None) -> int:
    """Pool = needed + 10% + 1 (the +1 is the poison block)."""
    if fixed is not None:
        return fixed
    need = pool_blocks_needed(plans, block_size)
    return need + -(-need // 10) + 1


# ---- the five configurations ----------------------------------------------------

def _decode_plans(ctx_lens):
    return [SeqPlan(i, -1, 0, int(L) - 1, 1, True) for i, L in enumerate(ctx_lens)]


def make(name: str, reduced: bool = False, seed: int = 0) -> Workload:
    """Build a named configuration.  `reduced=True` keeps the shape (heads,
    head_dim, block size, dtype, sharing structure) but shrinks the batch and
    lengths so the fp64 oracle finishes in seconds while still spanning many
    blocks, several partitions and ragged tails."""
    k = CONFIG_NAMES.index(name) + 1
    key = (k, seed, 1 if reduced else 0)
    lg = np.random.default_rng(np.random.SeedSequence(list(_stream(key, 0))))
    if name == "tiny_decode":
        plans = _decode_plans([1, 15, 16, 33])
        spec = Spec(name, 2, 2, 64, 16, "f32", num_blocks=16)
        return synthesize(spec, plans, key)
    if name == "mha_decode_7b":
        S, lo, hi = (64, 128, 2048) if not reduced else (6, 1, 300)
        lens = lg.integers(lo, hi, size=S, endpoint=True)
        plans = _decode_plans(lens)
        spec = Spec(name, 32, 32, 128, 16, "f16", num_blocks=sized_pool(plans, 16))
        return synthesize(spec, plans, key)
    if name == "gqa_shared_prefix":
        groups, per, prefix, cap = (32, 8, 512, 8192) if not reduced else (2, 4, 64, 400)
        median = prefix
        S = groups * per
        lens = np.clip(np.rint(np.exp(lg.normal(math.log(median), 1.0, size=S))), 1, cap).astype(np.int64)
        plans = []
        for gi in range(groups):
            plans.append(SeqPlan(S + gi, -1, 0, prefix, 0, False))
        for s in range(S):
            L = int(lens[s])
            plans.append(SeqPlan(s, S + s // per, min(L - 1, prefix), L - 1, 1, True))
        spec = Spec(name, 32, 8, 128, 16, "bf16", num_blocks=sized_pool(plans, 16))
        return synthesize(spec, plans, key, notes={"groups": groups, "group_size": per,
                                                   "prefix_tokens": prefix})
    if name == "long_splitk_decode":
        S, L, P = (4, 131072, 512) if not reduced else (2, 1500, 512)
        plans = _decode_plans([L] * S)
        spec = Spec(name, 32, 8, 128, 32, "bf16", num_blocks=sized_pool(plans, 32), partition_size=P)
        return synthesize(spec, plans, key)
    if name == "mixed_chunked_prefill":
        n_chunk, chunk, cmax, n_dec, dlo, dhi = ((8, 512, 4096, 120, 256, 4096) if not reduced
                                                 else (3, 70, 200, 5, 1, 300))
        cached = lg.integers(0, cmax, size=n_chunk, endpoint=True)
        dec = lg.integers(dlo, dhi, size=n_dec, endpoint=True)
        plans = [SeqPlan(i, -1, 0, int(c), chunk, True) for i, c in enumerate(cached)]
        plans += [SeqPlan(n_chunk + i, -1, 0, int(L) - 1, 1, True) for i, L in enumerate(dec)]
        spec = Spec(name, 32, 8, 128, 16, "bf16", num_blocks=sized_pool(plans, 16))
        return synthesize(spec, plans, key, notes={"num_chunks": n_chunk, "chunk_tokens": chunk})
    raise ValueError(name)


def custom(num_q_heads, num_kv_heads, head_dim, block_size, dtype, ctx_lens, n_new=None,
           seed=0, partition_size=0, num_blocks=None, name="custom") -> Workload:
    """Independent fresh sequences with given context lengths (tests)."""
    n_new = n_new if n_new is not None else [1] * len(ctx_lens)
    plans = [SeqPlan(i, -1, 0, int(L) - int(n), int(n), True) for i, (L, n) in enumerate(zip(ctx_lens, n_new))]
    spec = Spec(name, num_q_heads, num_kv_heads, head_dim, block_size, dtype,
                num_blocks=sized_pool(plans, block_size, num_blocks), partition_size=partition_size)
    return synthesize(spec, plans, (99, seed, num_q_heads, num_kv_heads, head_dim, block_size,
                                    ["f32", "f16", "bf16"].index(dtype)))


def custom_shared(num_q_heads, num_kv_heads, head_dim, block_size, dtype, groups, seed=0, holder_in_batch=False,
                  name="custom_shared") -> Workload:
    """Decode sequences in groups that fork one prefix holder each (tests).

    groups: list of (prefix_len, [context lengths of the members]).  A member
    keeps min(L - 1, prefix_len) tokens of its holder's prefix, as in the
    shared-prefix configuration; prefix_len 0 makes the members fresh
    sequences.  holder_in_batch: the holder decodes in the step too, just
    before its members (context prefix_len + 1)."""
    plans = []
    n_batch = sum(len(m) for _, m in groups) + (sum(1 for p, _ in groups if p > 0) if holder_in_batch else 0)
    sid, hid = 0, n_batch
    for prefix, members in groups:
        parent = -1
        if prefix > 0:
            if holder_in_batch:
                plans.append(SeqPlan(sid, -1, 0, prefix, 1, True))
                parent, sid = sid, sid + 1
            else:
                plans.append(SeqPlan(hid, -1, 0, prefix, 0, False))
                parent, hid = hid, hid + 1
        for L in members:
            if parent >= 0:
                plans.append(SeqPlan(sid, parent, min(int(L) - 1, prefix), int(L) - 1, 1, True))
            else:
                plans.append(SeqPlan(sid, -1, 0, int(L) - 1, 1, True))
            sid += 1
    spec = Spec(name, num_q_heads, num_kv_heads, head_dim, block_size, dtype,
                num_blocks=sized_pool(plans, block_size))
    return synthesize(spec, plans, (98, seed, num_q_heads, num_kv_heads, head_dim, block_size,
                                    ["f32", "f16", "bf16"].index(dtype), 1 if holder_in_batch else 0))


def group_starts(wl: Workload):
    """Runs of consecutive batch sequences forked from one holder (or the
    holder followed by its forks), as the [num_groups + 1] start list a
    grouped decode takes as its hint."""
    batch = wl.batch
    root = []
    for p in batch:
        root.append(p.parent if p.parent >= 0 else p.seq_id)
    starts = [0]
    for i in range(1, len(batch)):
        if root[i] != root[i - 1]:
            starts.append(i)
    starts.append(len(batch))
    return np.array(starts, dtype=np.int32)


# Per-tensor scales of the FP8 variants: N(0,1) draws (|x| up to ~5.5 in
# these batches) divided by them stay inside E4M3's +-448 and use most of
# its exponent range; K and V differ so a swapped scale shows.
FP8_K_SCALE = 0.0125
FP8_V_SCALE = 0.0175


def with_fp8_kv(wl: Workload, k_scale: float = FP8_K_SCALE, v_scale: float = FP8_V_SCALE) -> Workload:
    """The same workload (plans, pool order, every drawn value) with an FP8
    E4M3 pool: activations (q, output, the appended K/V rows) keep the
    workload's 16-bit type, the pool stores codes of K / k_scale and
    V / v_scale."""
    if wl.spec.dtype not in ("f16", "bf16"):
        raise ValueError("FP8 pools take 16-bit activations")
    spec = replace(wl.spec, name=wl.spec.name + "_fp8", kv_dtype="fp8", k_scale=k_scale, v_scale=v_scale)
    return replace(wl, spec=spec)


def with_block_size(wl: Workload, block_size: int) -> Workload:
    """The same sequences and values on a pool of another block size: the
    pool is re-sized for it and its free order drawn again (from a stream of
    its own), everything else is kept."""
    spec = replace(wl.spec, name=f"{wl.spec.name}_bs{block_size}", block_size=block_size,
                   num_blocks=sized_pool(wl.seqs, block_size))
    g = np.random.default_rng(np.random.SeedSequence(list(_stream(wl.seed, 1, block_size))))
    return replace(wl, spec=spec, free_order=g.permutation(spec.num_blocks - 1).astype(np.int32))


def arrival_trace(n_requests: int, seed: int = 0, median_prompt: int = 160, max_prompt: int = 1500,
                  max_new: int = 48, mean_gap: float = 0.7):
    """Synthetic request arrivals for the scheduler loop: (arrival
    iteration, request id, prompt tokens, new tokens to produce), in
    arrival order.  Prompts lognormal (sigma 1) around median_prompt,
    capped; new tokens uniform in 1..max_new; gaps between arrivals
    exponential with mean mean_gap iterations (several may share one)."""
    g = np.random.default_rng(np.random.SeedSequence([SEED_ROOT, 77, seed]))
    prompts = np.clip(np.rint(np.exp(g.normal(math.log(median_prompt), 1.0, size=n_requests))), 1, max_prompt)
    news = g.integers(1, max_new, size=n_requests, endpoint=True)
    t = np.floor(np.cumsum(g.exponential(mean_gap, size=n_requests))).astype(np.int64)
    return [(int(t[i]), i, int(prompts[i]), int(news[i])) for i in range(n_requests)]
