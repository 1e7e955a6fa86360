"""CPU oracle for the paged KV-cache hot path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The GPU library never
calls it and shares no code with it; the two meet only in the seeded inputs of
``pa_inputs``.

It is plain and slow on purpose: float64 NumPy over a contiguous copy of each
sequence's K/V, a pure-Python block allocator, and pool writes done one token
or one block at a time.

Pages cited (title, site, section heading as printed):
  [youngju] "vLLM 내부 구조 (2) — PagedAttention은 KV 캐시를 왜 페이지로
            쪼갰는가", youngju.dev
  [icarus]  "PagedAttention", icarus.shaojiemike.top
  [ttlab]   "llm-kv-cache-02-serving-engine-kv", ttlab.hopto.org

Modules:
  encoding       fp32 -> bf16 / fp16 bit patterns and back
  block_manager  free list, block tables, refcounts, fork, copy-on-write
  pool           the physical block pool as bit patterns; append; block copy
  attention      gather through the block table; decode; causal prefill chunk
  run            drives a ``pa_inputs`` scenario through all of the above
  capacity       KV slots that hold tokens, paged against max-length reservation
  scheduler      chunked prefill: each step's prefill chunks under a token budget

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (printed examples, closed forms, invariants, torch's
scaled_dot_product_attention in float64, brute force on tiny pools).  The
allocation order of free blocks is a chosen policy (the pages allow any free
block); it is pinned by the pages' printed block-table example and by
agreement with the library's allocator, not by the pages alone.
"""
