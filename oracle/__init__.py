"""Plain CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (``paged_kv_cache_kvcache_amd``) never imports it and
shares no code with it; the two meet only through the seeded input generators
in ``workloads/``, which hold none of the method's arithmetic.

What is here, and where each definition comes from:

* ``allocator``  -- the block manager: fixed 256-token blocks handed out from a
  FIFO free pool (intelliparadigm.com Nano-vLLM article, §2.1 动态分块内存管理),
  per-block reference counts ("1200行代码挑战vLLM", §2 内存管理策略), prefix
  reuse keyed by a hash of the prompt ("1200行代码挑战vLLM", §性能优化 1. 前缀缓存),
  lazy release (intelliparadigm.com article, §7.2 关键优化点).  Pure Python.
* ``attention``  -- kv_store, paged decode and paged causal prefill, written as
  the textbook definition of softmax attention over keys gathered through the
  block table (ocdem.com nano-vllm article, §2.1 PagedAttention; score = Q·Kᵀ
  as in the intelliparadigm.com article, §2.2 混合精度计算流水线).  NumPy fp64.

Every function is pinned by ``tests/test_oracle*.py`` against values that do
not come from the oracle itself: published FNV-1a vectors, closed forms, a
hand-worked example, PyTorch's fp64 SDPA on the CPU, and pure-Python brute
force.  Numeric parity against the pages themselves is unpinned: the pages print
no attention values.
"""

from . import allocator, attention  # noqa: F401
