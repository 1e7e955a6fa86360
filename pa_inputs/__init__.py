"""Seeded synthetic inputs for the paged KV-cache hot path.

This package is shared by the CPU oracle's tests and by the GPU-side callers
(tests, bench, smoke).  It holds shape tables and random draws only: no slot
arithmetic, no gather, no attention.  Every number that the method computes is
computed separately on each side.

The workload shapes follow the pages' own examples:
  * "PagedAttention" (icarus.shaojiemike.top), section "KV Cache 为什么难管理"
    -- K/V for every layer, KV head, token and head dimension;
  * "llm-kv-cache-02-serving-engine-kv" (ttlab.hopto.org), sections 2-5 --
    16-token blocks, a 22,048-token KV capacity with 512+128-token requests,
    a 3,000-token shared prefix with 32-token tails, 3,500-token inputs fed
    in 1,024-token chunks.
"""

from .configs import CONFIGS, config  # noqa: F401
from . import gen  # noqa: F401
from .scenario import build_scenario, Scenario  # noqa: F401
