"""Pins of the reference attention against things other than itself.

* gather: reading a sequence through its block table returns exactly the
  logical K/V the workload drew for it (bit for bit, storage representation);
* torch's scaled_dot_product_attention (CPU, float64, grouped-query mode, an
  explicit causal mask aligned to the end of the context) agrees to 1e-12 on
  every configuration's reduced shape;
* a brute-force causal check: the full score matrix with an explicit mask,
  soft-maxed with scipy, exhaustively over small context/chunk/block sizes;
* softmax invariants: one key returns its value exactly, zero query or equal
  keys give the mean of the values, outputs lie in the values' hull, weights
  sum to one;
* split-K: merging per-partition states by log-sum-exp reproduces the unsplit
  result for partitions of one block, 64 tokens and the whole context;
* storage decoding agrees with torch's bfloat16 / float16 widening for every
  finite bit pattern.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import workloads
from oracle import attention as A
from oracle.cache import run_workload
from oracle.storage import to_f64


def _state(name, reduced=True):
    wl = workloads.make(name, reduced=reduced)
    return wl, run_workload(wl)


def _sdpa_reference(wl, st):
    """torch SDPA per sequence on the logical (contiguous) K/V."""
    sp = wl.spec
    outs = []
    for p in wl.batch:
        K, V = wl.logical_kv(p.seq_id)
        K = torch.from_numpy(to_f64(K, sp.dtype)).permute(1, 0, 2)[None]  # [1][Hkv][L][D]
        V = torch.from_numpy(to_f64(V, sp.dtype)).permute(1, 0, 2)[None]
        q = torch.from_numpy(to_f64(wl.q[p.seq_id], sp.dtype)).permute(1, 0, 2)[None]  # [1][Hq][n][D]
        L, n = p.context_len, p.n_new
        rows = torch.arange(n)[:, None] + (L - n)
        mask = torch.arange(L)[None, :] <= rows
        o = torch.nn.functional.scaled_dot_product_attention(
            q, K, V, attn_mask=mask, scale=sp.scale, enable_gqa=True)
        outs.append(o[0].permute(1, 0, 2).numpy())
    return np.concatenate(outs)


def check_gather(name):
    wl, st = _state(name)
    for r, p in enumerate(wl.batch):
        K, V = wl.logical_kv(p.seq_id)
        L = int(st.context_lens[r])
        assert L == p.context_len
        bs = wl.spec.block_size
        j = np.arange(L)
        blk = st.tables[r][j // bs]
        assert (st.pool.k[blk, :, j % bs, :] == K).all()
        assert (st.pool.v[blk, :, j % bs, :] == V).all()


def check_sdpa(name):
    wl, st = _state(name)
    out, _ = A.paged_attention(wl.step_q(), st.pool.k, st.pool.v, st.tables, st.context_lens,
                               st.q_lens, wl.spec.scale, wl.spec.dtype)
    ref = _sdpa_reference(wl, st)
    err = np.abs(out - ref).max()
    assert err <= 1e-12, err


@pytest.mark.parametrize("name", workloads.CONFIG_NAMES)
def test_gather_returns_logical_kv(name):
    check_gather(name)


@pytest.mark.parametrize("name", workloads.CONFIG_NAMES)
def test_matches_torch_sdpa(name):
    check_sdpa(name)


def check_causal_bruteforce(cases=None):
    cases = cases or [(C, n, bs) for bs in (1, 2, 4, 16) for C in range(0, 13, 3) for n in range(1, 7)]
    for C, n, bs in cases:
        wl = workloads.custom(2, 1, 4, bs, "f32", [C + n], n_new=[n], seed=C * 100 + n * 10 + bs)
        st = run_workload(wl)
        out, lse = A.paged_attention(wl.step_q(), st.pool.k, st.pool.v, st.tables, st.context_lens,
                                     st.q_lens, wl.spec.scale, "f32")
        K, V = wl.logical_kv(0)
        K, V = to_f64(K, "f32"), to_f64(V, "f32")
        q = to_f64(wl.q[0], "f32")
        L = C + n
        for h in range(2):
            S = wl.spec.scale * np.einsum("id,jd->ij", q[:, h], K[:, 0])
            mask = np.zeros((n, L), bool)
            for i in range(n):
                for j in range(L):
                    mask[i, j] = j <= C + i
            S = np.where(mask, S, -np.inf)
            P = scipy.special.softmax(S, axis=1)
            ref = P @ V[:, 0]
            assert np.abs(out[:, h] - ref).max() <= 1e-12
            assert np.abs(lse[:, h] - scipy.special.logsumexp(S, axis=1)).max() <= 1e-12


def test_causal_bruteforce():
    check_causal_bruteforce()


def test_single_key_returns_its_value_exactly():
    wl, st = _state("tiny_decode", reduced=False)
    out, lse = A.paged_attention(wl.step_q(), st.pool.k, st.pool.v, st.tables, st.context_lens,
                                 st.q_lens, wl.spec.scale, "f32")
    assert st.context_lens[0] == 1
    V = to_f64(wl.logical_kv(0)[1], "f32")
    for h in range(2):
        assert (out[0, h] == V[0, A.kv_head_of(h, 2, 2)]).all()


def test_zero_query_and_equal_keys_give_mean_value():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((37, 8))
    V = rng.standard_normal((37, 8))
    o, lse, p = A.attend(np.zeros(8), K, V, 0.3)
    assert np.abs(o - V.mean(0)).max() <= 1e-14 and abs(lse - math.log(37)) <= 1e-14
    Keq = np.repeat(K[:1], 37, axis=0)
    o, _, _ = A.attend(rng.standard_normal(8), Keq, V, 0.3)
    assert np.abs(o - V.mean(0)).max() <= 1e-14


def test_weights_sum_to_one_and_output_in_hull():
    rng = np.random.default_rng(4)
    for L in (1, 2, 15, 16, 17, 513):
        K = rng.standard_normal((L, 16)) * 3
        V = rng.standard_normal((L, 16))
        o, _, p = A.attend(rng.standard_normal(16) * 3, K, V, 1 / 4)
        assert abs(p.sum() - 1) <= 1e-14 * L and (p >= 0).all()
        assert (o >= V.min(0) - 1e-12).all() and (o <= V.max(0) + 1e-12).all()


@pytest.mark.parametrize("name", ["long_splitk_decode", "mixed_chunked_prefill", "gqa_shared_prefix"])
def test_split_merge_identity(name):
    wl, st = _state(name)
    args = (wl.step_q(), st.pool.k, st.pool.v, st.tables, st.context_lens, st.q_lens, wl.spec.scale, wl.spec.dtype)
    ref, ref_lse = A.paged_attention(*args)
    for P in (wl.spec.block_size, 64, int(st.context_lens.max())):
        m, l, o = A.split_partials(*args, partition=P)
        out, lse = A.merge_partials(m, l, o)
        scale = np.abs(ref).max()
        assert np.abs(out - ref).max() <= 1e-13 * max(1.0, scale)
        assert np.abs(lse - ref_lse).max() <= 1e-12


def test_storage_decoding_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = to_f64(bits, "bf16")
    fin = np.isfinite(ref)
    assert (got[fin] == ref[fin]).all() and (np.isnan(got) == np.isnan(ref)).all()
    h = bits.view(np.float16)
    ref16 = torch.from_numpy(h.copy()).to(torch.float64).numpy()
    fin = np.isfinite(ref16)
    assert (to_f64(h, "f16")[fin] == ref16[fin]).all()


def test_generator_rounding_matches_torch():
    x = np.random.default_rng(5).standard_normal(1 << 16).astype(np.float32) * 7
    x[:4] = [1.0 + 2**-8, 1.0 + 3 * 2**-8, -(1.0 + 2**-8), 0.0]  # exact ties
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (workloads.round_to_storage(x, "bf16") == ref).all()


def test_workload_generation_is_deterministic():
    a = workloads.make("gqa_shared_prefix", reduced=True)
    b = workloads.make("gqa_shared_prefix", reduced=True)
    assert (a.free_order == b.free_order).all()
    for s in a.own_k:
        assert (a.own_k[s] == b.own_k[s]).all() and (a.own_v[s] == b.own_v[s]).all()
    for s in a.q:
        assert (a.q[s] == b.q[s]).all()
    x = workloads.normal_values((1, 2, 3), (5, 1 << 20), "f16", threads=1)
    y = workloads.normal_values((1, 2, 3), (5, 1 << 20), "f16", threads=8)
    assert (x == y).all()


@pytest.mark.parametrize("name", ["mha_decode_7b", "gqa_shared_prefix", "mixed_chunked_prefill"])
def test_sampled_rows_match_batched_reference(name):
    """attention_rows on a sequence's logical K/V (the sampled form the
    full-size GPU tests use) reproduces paged_attention's rows, and the
    bookkeeping-only replay matches the full one."""
    wl, st = _state(name)
    sp = wl.spec
    ref, _ = A.paged_attention(wl.step_q(), st.pool.k, st.pool.v, st.tables, st.context_lens, st.q_lens,
                               sp.scale, sp.dtype)
    light = run_workload(wl, with_pool=False)
    assert light.pool is None
    for a, b in [(light.slot_mapping, st.slot_mapping), (light.cow_pairs, st.cow_pairs), (light.tables, st.tables),
                 (light.context_lens, st.context_lens), (light.setup_slots, st.setup_slots)]:
        assert np.array_equal(a, b)
    G = sp.num_q_heads // sp.num_kv_heads
    row = 0
    for p in wl.batch:
        K, V = wl.logical_kv(p.seq_id)
        for h in (0, sp.num_q_heads - 1):
            pos = p.context_len - p.n_new + np.arange(p.n_new)
            got = A.attention_rows(wl.q[p.seq_id][:, h], K[:, h // G], V[:, h // G], pos, sp.scale, sp.dtype)
            assert np.abs(got - ref[row:row + p.n_new, h]).max() <= 1e-12
        row += p.n_new
