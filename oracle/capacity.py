"""KV memory use under paging and under max-length reservation (test
infrastructure: imported by tests only).

What the pages fix:
  * systems before paging reserved, per request, one contiguous run of the
    maximum length; what a request never used (internal fragmentation) and
    the holes between runs (external fragmentation) held no tokens; prior
    systems stored tokens in only 20.4-38.2% of their KV memory ([youngju]
    "연속 할당이 만드는 두 가지 낭비"; [ttlab] "llm-kv-cache-02-serving-engine-kv",
    section "2. PagedAttention: KV 를 블록으로 나누기", part "옛 방식의 낭비");
  * with fixed-size blocks handed out one at a time, external fragmentation
    is gone and a request wastes only the free slots of its last block, at
    most block_size - 1 ([youngju] "블록 테이블: 논리적으로 연속, 물리적으로
    흩어짐"; [ttlab] "블록과 블록 표");
  * the number of requests that can be active is about the KV capacity over
    the average KV footprint per request ([icarus] "PagedAttention", section
    "提高并发与吞吐").
"""


def paged_slots(bm, seqs):
    """Token slots the block manager holds for ``seqs``: every block of
    every table, counted once however many sequences share it."""
    blocks = set()
    for s in seqs:
        blocks.update(bm.block_table(s))
    return len(blocks) * bm.block_size


def reserved_slots(lengths, max_len):
    """Slots a max-length reservation holds: max_len per request."""
    return len(lengths) * max_len


def utilisation(tokens, slots):
    """Fraction of the held slots that store a token."""
    return tokens / slots if slots else 1.0


def waste_per_request(bm, seqs):
    """Unused slots of each sequence's blocks (its last block's free slots)."""
    return [len(bm.block_table(s)) * bm.block_size - bm.seq_len(s) for s in seqs]


def n_active(capacity_tokens, footprint_tokens):
    """Requests of a given KV footprint that fit at once in the capacity."""
    return capacity_tokens // footprint_tokens
