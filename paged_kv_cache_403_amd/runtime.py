"""A device pool plus its host block manager.

`PagedKVCache` owns the K/V pool tensors (K tiles [block_size][head_dim], V
tiles [head_dim][block_size]) and a `BlockManager`; it replays cache
operations (add / fork / append with token data) through the C ABI, and
prepares a step: the batch's slot mapping and copy-on-write pairs (host), the
padded block tables and context lengths (copied to the device).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import binding as B

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_device(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Host storage representation (float32 / float16 / uint16 bf16 bits) -> device tensor."""
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device, non_blocking=False)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host storage representation."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@dataclass
class StepPlan:
    seqs: np.ndarray  # int32 batch sequence ids
    n_new: np.ndarray  # int32 tokens appended per sequence
    slot_mapping: torch.Tensor  # int64 device [sum n_new]
    cow_pairs: torch.Tensor  # int32 device [n][2]
    block_tables: torch.Tensor  # int32 device [S][max_blocks]
    context_lens: torch.Tensor  # int32 device [S]
    host_slots: np.ndarray
    host_pairs: np.ndarray
    host_tables: np.ndarray
    host_lens: np.ndarray
    max_context_len: int


class PagedKVCache:
    """dtype: the activation type (q, out, appended rows).  kv_dtype "fp8"
    makes the pool E4M3 codes (uint8) with scales k_scale / v_scale; a
    fill_value then fills unused slots with the NaN code if it is NaN, else
    with the largest finite code."""

    def __init__(self, num_blocks, num_kv_heads, block_size, head_dim, dtype: str, device="cuda",
                 free_order=None, fill_value=None, kv_dtype=None, k_scale=1.0, v_scale=1.0):
        self.dtype = dtype
        self.kv_dtype = kv_dtype or dtype
        self.device = torch.device(device)
        td = torch.uint8 if self.kv_dtype == "fp8" else TORCH_DTYPE[dtype]
        self.k = torch.empty((num_blocks, num_kv_heads, block_size, head_dim), dtype=td, device=self.device)
        self.v = torch.empty((num_blocks, num_kv_heads, head_dim, block_size), dtype=td, device=self.device)
        if fill_value is not None:
            fill = (0x7F if np.isnan(fill_value) else 0x7E) if self.kv_dtype == "fp8" else fill_value
            self.k.fill_(fill)
            self.v.fill_(fill)
        if self.kv_dtype == "fp8":
            self.desc = B.make_cache(self.k, self.v, TORCH_DTYPE[dtype], k_scale, v_scale)
        else:
            self.desc = B.make_cache(self.k, self.v)
        self.bm = B.BlockManager(num_blocks, block_size, free_order)
        self.block_size = block_size
        self.num_blocks = num_blocks

    # -- data movement through the library ------------------------------------------
    def _flush(self, slots, ks, vs):
        if not slots:
            return
        s = torch.from_numpy(np.concatenate(slots)).to(self.device)
        k = to_device(np.concatenate(ks), self.dtype, self.device)
        v = to_device(np.concatenate(vs), self.dtype, self.device)
        B.pa_kv_append(self.desc, k, v, s)
        slots.clear()
        ks.clear()
        vs.clear()

    def apply_ops(self, ops):
        """Replay add / fork / append operations in order.  Appends are
        batched into one library call until a copy-on-write pair has to run
        (it must see every earlier write and precede every later one)."""
        slots, ks, vs, all_slots = [], [], [], []
        for op in ops:
            if op.kind == "add":
                self.bm.add_seq(op.seq)
            elif op.kind == "fork":
                self.bm.fork(op.parent, op.seq, op.keep)
            elif op.kind == "append":
                s, pairs = self.bm.append(op.seq, op.n)
                if len(pairs):
                    self._flush(slots, ks, vs)
                    B.pa_copy_blocks(self.desc, torch.from_numpy(np.ascontiguousarray(pairs)).to(self.device))
                slots.append(s)
                ks.append(op.k)
                vs.append(op.v)
                all_slots.append(s)
            else:
                raise ValueError(op.kind)
        self._flush(slots, ks, vs)
        return np.concatenate(all_slots) if all_slots else np.zeros(0, np.int64)

    def prepare_step(self, seqs, n_new, pad_block: int, max_blocks: int | None = None) -> StepPlan:
        """Host side of a step: grow each sequence by its new tokens (slot
        mapping and copy pairs), then the padded tables and lengths."""
        seqs = np.asarray(seqs, dtype=np.int32)
        n_new = np.asarray(n_new, dtype=np.int32)
        slots, pairs = self.bm.append_batch(seqs, n_new)
        lens = np.array([self.bm.seq_len(int(s)) for s in seqs], dtype=np.int32)
        need = int(max(-(-int(lens.max()) // self.block_size), 1)) if len(lens) else 1
        mb = max(need, max_blocks or 0)
        tables, _ = self.bm.tables(seqs, mb, pad_block)
        dev = self.device
        return StepPlan(
            seqs=seqs, n_new=n_new,
            slot_mapping=torch.from_numpy(slots.copy()).to(dev),
            cow_pairs=torch.from_numpy(np.ascontiguousarray(pairs)).to(dev),
            block_tables=torch.from_numpy(tables).to(dev),
            context_lens=torch.from_numpy(lens).to(dev),
            host_slots=slots.copy(), host_pairs=pairs.copy(), host_tables=tables, host_lens=lens,
            max_context_len=int(lens.max()) if len(lens) else 0,
        )
