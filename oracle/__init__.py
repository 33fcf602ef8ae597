"""Plain fp64 CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only `tests/`, `__graft_entry__.smoke()`
and the `cpu_baseline` leg of `bench.py` use it.  It shares no code with the
HIP library (no kernels, headers, helpers, tables or constants); the only
module both sides use is `workloads`, which draws seeded inputs and holds
none of the method's arithmetic.

What it computes, and the passages it follows (pages cited by title/host and
section):

* `storage`   exact decoding of fp32 / fp16 / bf16 storage to fp64.
* `block_manager`  the paged cache's bookkeeping: a global pool of fixed-size
  blocks, a per-sequence block table mapping logical blocks to physical ones,
  a free pool handed out from the front, a new block taken only when the last
  one is full, all blocks returned when a sequence ends, and read-only shared
  prefix blocks that are copied on the first write (lshu.cn/news/11644,
  "方案：页式内存管理" and "收益分析"; zzmblog.top vLLM guide,
  "PagedAttention核心设计").
* `cache`     data movement into the pool: token K/V scattered to slots,
  whole blocks copied for copy-on-write.
* `attention` attention read through the block tables, which the pages state
  gives the same K/V sequence as a contiguous cache (lshu.cn/news/11644,
  "方案：页式内存管理", last paragraph; 5x10.cn/post/462, "技术架构深度分析":
  the memory system does not change model outputs).  It is therefore written
  as the plain definition: gather, then softmax(scale * q K^T) V in fp64, with
  decode appending the current token before attending (zzmblog.top vLLM
  guide, "Transformer推理与KV缓存") and chunked prefill attending causally
  to the cached context plus the chunk (lshu.cn/news/11644, scheduler loop
  under "整体架构"; 5x10.cn/post/462, "分块预填充").
* `attention.split_partials` / `merge_partials`: per-partition softmax state
  merged by the log-sum-exp identity (the pages are silent on split-K; this is
  the textbook identity, pinned against the unsplit result).

Parity pins live in tests/test_oracle_*.py (run with -m "not gpu").
Parity unpinned: the free-list order convention (any order is a correct
allocator; this one is fixed by convention so both sides agree bit-exactly).
"""

from . import storage, block_manager, cache, attention  # noqa: F401
