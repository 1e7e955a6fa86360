"""Shape tables of the five synthetic workloads (and a beam-search one).

Sizes only.  Which sequences exist, how long they are and what values their
K/V hold are drawn in ``gen`` and laid out as an op list in ``scenario``.
"""

import copy
import math

# Each entry: dtype of the pool / q / out, head layout, block size, pool size
# and the length recipe.  ``ctx`` is the number of tokens a sequence already
# holds before the step's append (the decode then attends over ctx + 1).
CONFIGS = {
    1: dict(
        name="tiny-fp32-decode",
        dtype="f32",
        B=4,
        ctx=("fixed", [1, 16, 17, 100]),
        H_q=4,
        H_kv=4,
        d=64,
        bs=16,
        num_blocks=64,
        kind="decode",
    ),
    2: dict(
        name="qwen3-1.7b-layer-decode-b32",
        dtype="bf16",
        B=32,
        ctx=("uniform", 512, 640),
        H_q=16,
        H_kv=8,
        d=128,
        bs=16,
        num_blocks=1378,  # 22,048 tokens of KV capacity at 16 tokens per block
        kind="decode",
    ),
    3: dict(
        name="13b-mha-layer-decode-b64",
        dtype="bf16",
        B=64,
        ctx=("lognormal", 400.0, 0.8, 16, 2048),
        H_q=40,
        H_kv=40,
        d=128,
        bs=16,  # swept over 8 / 16 / 32
        num_blocks=None,  # 64 * (2048 // bs + 1): room for the longest context + 1
        # Device allocation per KV head for timing runs (the block manager
        # still hands out num_blocks): the same 0x2080000-byte stride at
        # every block size.  The default pools' strides differ per block
        # size, and 0x2040000 bytes (block 16's 8,256 blocks) alone slows
        # a 40-head decode by 7-11% at any block size.
        alloc_bytes_per_head=0x2080000,
        churn_rounds=256,
        kind="decode",
    ),
    4: dict(
        name="shared-prefix-parallel-sampling",
        dtype="bf16",
        prompts=8,
        samples=8,
        prefix=3000,
        tail=32,
        steps=16,
        H_q=32,
        H_kv=8,
        d=128,
        bs=16,
        num_blocks=2048,
        kind="fork",
    ),
    5: dict(
        name="mixed-chunked-prefill-decode",
        dtype="bf16",
        B=63,
        ctx=("uniform", 1024, 32768),
        H_q=64,
        H_kv=8,
        d=128,
        bs=16,
        ctx_before=3500,
        chunk=1024,
        num_blocks=131072,
        kind="mixed",
    ),
    # Not one of the five headline workloads: beam search, where surviving
    # beams fork from forks and shared blocks are copied on write at any depth.
    6: dict(
        name="beam-search",
        dtype="bf16",
        prompts=4,
        beam=4,
        prompt_len=200,  # 12 full blocks + 8 tokens: every first step copies on write
        steps=24,
        H_q=16,
        H_kv=8,
        d=128,
        bs=16,
        num_blocks=1024,
        kind="beam",
    ),
}


def config(cid, **overrides):
    """Return a copy of config ``cid`` with ``overrides`` applied.

    Derived fields: ``G`` (query heads per KV head), ``scale`` (1/sqrt(d) as
    an fp32 value) and, for config 3, the pool size from the block size.
    """
    c = copy.deepcopy(CONFIGS[cid])
    c.update(overrides)
    c["id"] = cid
    c["G"] = c["H_q"] // c["H_kv"]
    if c.get("num_blocks") is None:
        c["num_blocks"] = 64 * (2048 // c["bs"] + 1)
    if "scale" not in c:
        import numpy as np

        c["scale"] = float(np.float32(1.0 / math.sqrt(c["d"])))
    return c
