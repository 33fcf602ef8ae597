"""The binding refuses tensors of the wrong type, shape or device before any
launch: the kernels size every access from the pool descriptor and the
counts, so a mismatched tensor would be read or written past its end.

CPU only: the descriptors point nowhere (the calls must fail before the
library is reached), and the tensors are host tensors whose type or shape is
wrong, so the error names that, not the missing device.
"""
import pytest
import torch

import paged_kv_cache_403_amd as P

FAKE = 0x1000


def _cache(dtype=P.PA_BF16, act=None, hkv=8, d=128, bs=16):
    c = P.pa_cache(FAKE, FAKE, 64, hkv, bs, d, dtype)
    c.act_dtype = act if act is not None else dtype
    c.k_scale = c.v_scale = 1.0
    return c


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_append_checks():
    c = _cache()
    k = torch.zeros(5, 8, 128, dtype=torch.bfloat16)
    slots = torch.zeros(5, dtype=torch.int64)
    _raises("slot_mapping must be torch.int64", P.pa_kv_append, c, k, k, slots.to(torch.int32))
    _raises("k_new must have shape", P.pa_kv_append, c, k[:4], k, slots)  # fewer rows than slots
    _raises("v_new must have shape", P.pa_kv_append, c, k, torch.zeros(5, 8, 64, dtype=torch.bfloat16), slots)
    _raises("k_new must be torch.bfloat16", P.pa_kv_append, c, k.half(), k, slots)
    # an FP8 pool takes rows of its activation type
    f8 = _cache(P.PA_FP8_E4M3, act=P.PA_F16)
    _raises("k_new must be torch.float16", P.pa_kv_append, f8, k, k, slots)
    # right types and shapes: only the missing device remains
    _raises("must be a device tensor", P.pa_kv_append, c, k, k, slots)


def test_copy_checks():
    c = _cache()
    _raises("pairs must be torch.int32", P.pa_copy_blocks, c, torch.zeros(3, 2, dtype=torch.int64))
    _raises("pairs must have shape", P.pa_copy_blocks, c, torch.zeros(3, 3, dtype=torch.int32))


def _dec_args(S=4, hq=32, d=128, dt=torch.bfloat16, mb=8):
    q = torch.zeros(S, hq, d, dtype=dt)
    return q, torch.zeros_like(q), torch.zeros(S, mb, dtype=torch.int32), torch.zeros(S, dtype=torch.int32)


@pytest.mark.parametrize("entry", ["decode", "grouped"])
def test_decode_checks(entry):
    c = _cache()

    def call(q, out, tab, lens):
        if entry == "decode":
            return P.pa_decode(c, q, out, tab, lens, 100, 0.1)
        return P.pa_decode_grouped(c, q, out, tab, lens, 100, 0.1, None)

    q, out, tab, lens = _dec_args()
    _raises("out must be torch.bfloat16", call, q, out.float(), tab, lens)  # fp32 out, bf16 pool
    _raises("out must have shape", call, q, out[:3], tab, lens)  # out smaller than q
    _raises("q must be torch.bfloat16", call, q.half(), out, tab, lens)
    _raises("q must have shape", call, torch.zeros(4, 32, 64, dtype=torch.bfloat16), out, tab, lens)
    _raises("block_tables must be torch.int32", call, q, out, tab.long(), lens)
    _raises("block_tables must have shape", call, q, out, tab[:3], lens)
    _raises("context_lens must be torch.int32", call, q, out, tab, lens.long())
    _raises("context_lens must have shape", call, q, out, tab, lens[:2])
    if entry == "grouped":
        _raises("group_start must be torch.int32", P.pa_decode_grouped, c, q, out, tab, lens, 100, 0.1,
                torch.zeros(3, dtype=torch.int64))
    _raises("must be a device tensor", call, q, out, tab, lens)


@pytest.mark.parametrize("entry", ["whole", "split"])
def test_prefill_checks(entry):
    c = _cache()
    q, out, tab, lens = _dec_args(S=10)
    tab, lens = tab[:2], lens[:2]
    cu = torch.tensor([0, 5, 10], dtype=torch.int32)
    f = P.pa_prefill_chunk if entry == "whole" else P.pa_prefill_chunk_split
    _raises("out must have shape", f, c, q, out[:9], cu, lens, tab, 5, 100, 0.1)
    _raises("cu_q_lens must be torch.int32", f, c, q, out, cu.long(), lens, tab, 5, 100, 0.1)
    _raises("cu_q_lens must have shape", f, c, q, out, cu[:2], lens, tab, 5, 100, 0.1)
    _raises("block_tables must have shape", f, c, q, out, cu, lens, tab[:1], 5, 100, 0.1)
    _raises("must be a device tensor", f, c, q, out, cu, lens, tab, 5, 100, 0.1)
