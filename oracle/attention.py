"""Attention over paged K/V, computed as plain softmax attention in float64.

Paging changes where K/V live and how they are found, not the mathematics:
the kernel follows the block table from logical to physical blocks, the
sequence still sees its tokens in order, and paging adds no approximation
([icarus] "Block Table 如何工作" and "不改变模型精度"; [ttlab] "블록과 블록 표").
So the oracle first gathers a contiguous copy of the sequence's K/V through its
block table and then applies the textbook definition.

Decode: the newest query of a sequence reads every visible K/V of its history
([icarus] "KV Cache 为什么难管理" and "不会降低单请求的理论读取量").
Prefill chunk: each prompt row attends causally to every earlier position and
itself; a chunk is a slice of such rows whose earlier positions are already in
the pool ([ttlab] "새 문제: 긴 프리필이 디코드를 멈춘다").

Readings (the pages do not say):
  * grouped query heads: query head h reads KV head h // (H_q / H_kv);
  * scale is a given fp32 number (1/sqrt(head_dim) in every workload here);
  * "numerically safe softmax" = subtract the row maximum before exponentiating;
  * a sequence with no visible tokens produces a zero row.
"""

import numpy as np

from . import encoding


def gather(pool, layer, table, length):
    """Contiguous K, V (float64 [kv_heads][length][head_dim]) of one sequence."""
    bs = pool.bs
    need = -(-int(length) // bs)
    if need > len(table):
        raise ValueError(f"table has {len(table)} blocks, {need} needed for {length} tokens")
    ks, vs = [], []
    for j in range(need):
        phys = int(table[j])
        n = min(bs, int(length) - j * bs)
        ks.append(pool.k[layer, :, phys, :n, :])
        vs.append(pool.v[layer, :, phys, :n, :])
    if not ks:
        shape = (pool.H, 0, pool.d)
        return np.zeros(shape), np.zeros(shape)
    k = encoding.decode(np.concatenate(ks, axis=1), pool.dtype)
    v = encoding.decode(np.concatenate(vs, axis=1), pool.dtype)
    return k, v


def softmax_weights(q, k, scale):
    """Attention weights p[h][t] for queries q [H_q][d] over keys k [H_kv][n][d]."""
    H_q, H_kv = q.shape[0], k.shape[0]
    G = H_q // H_kv
    n = k.shape[1]
    p = np.zeros((H_q, n))
    for h in range(H_q):
        s = scale * (k[h // G] @ q[h])
        if n == 0:
            continue
        e = np.exp(s - s.max())
        p[h] = e / e.sum()
    return p


def attend(q, k, v, scale):
    """out[h] = softmax(scale * K q_h) V for each query head (float64 [H_q][d])."""
    H_q, H_kv = q.shape[0], k.shape[0]
    if H_q % H_kv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = H_q // H_kv
    p = softmax_weights(q, k, scale)
    out = np.zeros((H_q, v.shape[2]))
    for h in range(H_q):
        out[h] = p[h] @ v[h // G]
    return out


def decode(pool, layer, q, tables, lengths, scale):
    """Decode attention for a batch.

    q: float64 [B][H_q][d]; tables: per-sequence lists of physical block ids;
    lengths: visible tokens per sequence (the just-appended token included).
    Returns float64 [B][H_q][d].
    """
    out = np.zeros(q.shape)
    for i in range(q.shape[0]):
        k, v = gather(pool, layer, tables[i], lengths[i])
        out[i] = attend(q[i], k, v, scale)
    return out


def causal_rows(q, k, v, ctx_before, scale, rows=None):
    """Row t of q (position ctx_before + t) attends to keys 0 .. ctx_before + t.

    q: float64 [T][H_q][d]; k, v: float64 [H_kv][>= ctx_before + T][d].
    Rows not listed in ``rows`` (None = all) are left NaN.
    """
    T = q.shape[0]
    out = np.full(q.shape, np.nan)
    for t in (range(T) if rows is None else rows):
        n = ctx_before + t + 1
        out[t] = attend(q[t], k[:, :n], v[:, :n], scale)
    return out


def prefill_chunk(pool, layer, q, table, ctx_before, scale, rows=None):
    """Causal attention of chunk rows t = 0..T-1 at positions ctx_before + t.

    Row t sees keys 0 .. ctx_before + t (itself included).  The chunk's own K/V
    must already be in the pool.  q: float64 [T][H_q][d] -> float64 [T][H_q][d].
    """
    k, v = gather(pool, layer, table, ctx_before + q.shape[0])
    return causal_rows(q, k, v, ctx_before, scale, rows)
