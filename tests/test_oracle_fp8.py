"""Pins of the oracle's FP8 (E4M3) KV format against things other than
itself: torch's float8_e4m3fn type (decode of every code, and its
round-to-nearest-even cast on in-range values), closed forms of the format
(largest value, smallest normal and subnormal, NaN codes), exact ties, and
saturation."""
import numpy as np
import pytest
import torch

import workloads
from oracle import attention as A
from oracle.cache import run_workload
from oracle.storage import E4M3, kv_encode, kv_values, quantize_e4m3, to_f64


def test_decode_table_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(E4M3))
    assert np.array_equal(np.flatnonzero(nan), [0x7F, 0xFF])
    assert np.array_equal(ref[~nan], E4M3[~nan])


def test_closed_forms():
    assert E4M3[0x7E] == 448.0 and E4M3[0xFE] == -448.0
    assert E4M3[0x08] == 2.0 ** -6  # smallest normal
    assert E4M3[0x01] == 2.0 ** -9  # smallest subnormal
    assert E4M3[0x07] == 7 * 2.0 ** -9
    assert E4M3[0x38] == 1.0 and E4M3[0x39] == 1.125
    assert E4M3[0x00] == 0.0 and np.signbit(E4M3[0x80])


def test_every_value_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(quantize_e4m3(E4M3[codes].astype(np.float32)), codes)


def test_ties_go_to_the_even_code_and_saturation():
    pos = E4M3[:127]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)  # exact in fp32
    got = quantize_e4m3(mids)
    lo = np.arange(126)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want)
    assert quantize_e4m3(np.float32(2.0 ** -10)) == 0  # half the smallest subnormal: tie to 0
    assert quantize_e4m3(np.float32(1000.0)) == 0x7E
    assert quantize_e4m3(np.float32(-1e30)) == 0xFE
    assert quantize_e4m3(np.float32(np.inf)) == 0x7E
    assert quantize_e4m3(np.float32(-0.0)) == 0x80
    assert quantize_e4m3(np.float32(np.nan)) & 0x7F == 0x7F


def test_quantizer_matches_torch_cast_in_range():
    g = np.random.default_rng(7)
    x = np.concatenate([g.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 120.0)]).astype(np.float32)
    x = x[np.abs(x) <= 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(quantize_e4m3(x), ref)


def test_kv_encode_is_an_fp32_multiply_then_nearest():
    x = np.array([0.3, -1.7, 2.0, 5.5], dtype=np.float32)
    codes = kv_encode(x.astype(np.float16), "f16", 0.0125)
    y = x.astype(np.float16).astype(np.float32) * (np.float32(1) / np.float32(0.0125))
    assert np.array_equal(codes, quantize_e4m3(y))
    v = kv_values(codes, 0.0125)
    assert np.all(np.abs(v - x.astype(np.float16).astype(np.float64)) <= np.abs(x) * 2.0 ** -4 + 1e-12)


@pytest.mark.parametrize("name", ["mha_decode_7b", "gqa_shared_prefix", "long_splitk_decode"])
def test_fp8_pool_holds_codes_of_the_logical_values(name):
    wl = workloads.with_fp8_kv(workloads.make(name, reduced=True))
    sp = wl.spec
    st = run_workload(wl)
    assert st.pool.k.dtype == np.uint8
    for r, p in enumerate(wl.batch[:4]):
        K, V = wl.logical_kv(p.seq_id)
        L = p.context_len
        j = np.arange(L)
        blk, off = st.tables[r][j // sp.block_size], j % sp.block_size
        assert np.array_equal(st.pool.k[blk, :, off, :], kv_encode(K, sp.dtype, sp.k_scale))
        assert np.array_equal(st.pool.v[blk, :, off, :], kv_encode(V, sp.dtype, sp.v_scale))
        # attention over the pool equals attention over the dequantised logical rows
        q = wl.q[p.seq_id][:, 0]
        Kd, Vd = kv_values(kv_encode(K[:, 0], sp.dtype, sp.k_scale), sp.k_scale), \
            kv_values(kv_encode(V[:, 0], sp.dtype, sp.v_scale), sp.v_scale)
        z = sp.scale * (Kd @ to_f64(q, sp.dtype)[-1])
        w = np.exp(z - z.max())
        ref = (w / w.sum()) @ Vd
        got = A.attention_rows(q[-1:], kv_encode(K[:, 0], sp.dtype, sp.k_scale),
                               kv_encode(V[:, 0], sp.dtype, sp.v_scale), [L - 1], sp.scale, sp.dtype, sp.kv)[0]
        assert np.abs(got - ref).max() < 1e-12
