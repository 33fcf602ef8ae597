"""Memory-waste figures the pages quote, as plain definitions.  Test
infrastructure: only tests/ and the benchmark's reporting use it.

* Static reservation (lshu.cn/news/11644, "问题：KV Cache 的内存困境"): every
  sequence of a batch reserves `reserved` slots up front; the unused share
  is 1 - sum(L) / (S * reserved) -- 2048 slots for sequences that average
  256 tokens leave about 87% unused.
* Paged blocks (m.ypxx.net, "2.1 PagedAttention分页注意力核心机制"; lshu,
  "收益分析"): blocks are taken as tokens arrive, so only the last block of
  a sequence is partly empty; a block shared by several sequences is held
  once.  The unused share is 1 - filled slots / (blocks held * block_size),
  a block's filled slots being the most any of its holders has written
  into it.
"""
import numpy as np


def static_waste(lens, reserved: int) -> float:
    lens = np.asarray(lens, dtype=np.int64)
    return 1.0 - float(lens.sum()) / float(len(lens) * reserved)


def paged_usage(tables: dict, lens: dict, block_size: int):
    """(blocks held, filled slots) over the sequences' tables (seq -> block
    list) and lengths (seq -> tokens)."""
    filled = {}
    for s, table in tables.items():
        L = int(lens[s])
        for j, b in enumerate(table):
            f = max(0, min(block_size, L - j * block_size))
            filled[b] = max(filled.get(b, 0), f)
    return len(filled), sum(filled.values())


def paged_waste(tables: dict, lens: dict, block_size: int) -> float:
    held, used = paged_usage(tables, lens, block_size)
    return 1.0 - used / (held * block_size) if held else 0.0
