"""CPU oracle for paged decode and prefill attention: TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 implementation of what the paged attention path computes,
written from the pages and checked against what they (and mathematics) fix.
Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it.  The product path (the C-ABI library, its kernels
and its Python binding) never imports, calls or links anything here, and
nothing here imports the product.

Pages cited (by title, with section / code block):
  [P1] "KV Cache 优化与内存管理深度解析：PagedAttention 原理与实践"
       (aiattnstudio.link/posts/kv-cache-paged-attention)
  [P2] "5.KV Cache 管理 & PagedAttention" (lowentro.cn notes; an interview
       question bank, cited by question number and sub-section)
  [P3] "paged-attention-and-vllm-inference" (astro-blog-cod.pages.dev)

Modules:
  attention      decode attention: plain definition (O1) and the block-wise
                 online-softmax / partition-merge routes (O2)
  cache_write    writing new K/V tokens into cache slots (O3)
  fp8            OCP E4M3FN decode table and round-to-nearest-even,
                 saturating quantiser
  sizing         KV-cache memory closed form and block-count arithmetic (O4)
  allocator      a Python model of the ref-counted LIFO block allocator (O4)
  prefix_cache   a Python model of the prefix cache keyed by token prefixes
  prefill        causal multi-token (prefill) attention over the cache (O5)

Parity status: every function here is pinned by a test under tests/ that
does not re-type its formula; see the module docstrings.
"""
