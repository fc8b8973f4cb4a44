"""Plain CPU oracle for paged attention over a block-table KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product library (``paged_kv_cache_73_amd``)
imports, calls or links this package; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP path: it has its own bf16 decoder, its own indexing and its own block manager.

Everything here is deliberately slow and literal: float64 arithmetic, the
"gather the pages into a contiguous array, then run an ordinary two-pass softmax"
strategy (what the pages call stage A), and pure-Python bookkeeping for the block
manager.  Each function names the passage of the source pages it follows:

* "Paged attention 与 online softmax" (dilfish.github.io, chapter 11): §11.1 block
  table, address and pool size; §11.2 the block-merge rule; §11.3 sharing,
  copy-on-write and reference counts.
* "结合nanovllm的FlashAttention和PagedAttention主要原理概述" (meredith2328.github.io):
  problems 题目2 (online softmax trace), 题目3 (FlashAttention tile example),
  题目4 (waste), 题目5 (block table), 题目6 (prefix reference counts).
* "从零开始写Qwen3（六）PagedAttention" (mlqm.cn reprint): sections KVCache大小计算,
  分页自注意力的改进, fast-attn 库的使用 and 自己来实现 (slot_mapping write).
* "Sayfalı dikkat" (Hugging Face transformers docs, Turkish): the varlen path
  ("Değişken uzunluklu yol") and decode path ("Çözme yolu") examples.

Parity status of every function is listed in the module docstrings; none is
"parity unpinned" except the causal rule with a cached prefix, which no page
prints a value for and which is pinned by brute force only.
"""

from . import attention, blocks  # noqa: F401
