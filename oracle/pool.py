"""The physical block pool as raw bit patterns, and the two writes into it.

Layout: two arrays K and V, each [layers][kv_heads][blocks][block_size][head_dim]
-- the attention kernel reads K/V by layer, KV head, token and head dimension
([icarus] "类比的边界"), and the unit of allocation is a block of
``block_size`` token slots ([ttlab] "블록과 블록 표").

append:  the new token's K/V go into its slot of the current block ([icarus]
         "Block Table 如何工作").
copy:    copy-on-write duplicates a whole shared block -- every layer, every
         KV head, K and V -- before the writer diverges ([icarus] "支持块级共享";
         [ttlab] "블록을 함께 쓰기").
"""

import numpy as np

from . import encoding


class Pool:
    def __init__(self, num_layers, num_kv_heads, num_blocks, block_size, head_dim, dtype, fill_bits=None):
        self.L, self.H, self.N, self.bs, self.d = num_layers, num_kv_heads, num_blocks, block_size, head_dim
        self.dtype = dtype
        shape = (num_layers, num_kv_heads, num_blocks, block_size, head_dim)
        fill = encoding.nan_bits(dtype) if fill_bits is None else fill_bits
        self.k = np.full(shape, fill, dtype=encoding.BITS_DTYPE[dtype])
        self.v = np.full(shape, fill, dtype=encoding.BITS_DTYPE[dtype])

    def append(self, layer, k_new_bits, v_new_bits, slots):
        """Write token t's [kv_heads][head_dim] rows into slot ``slots[t]``.

        A negative slot means "no write" for that row.  Rows are written in
        token order, so a repeated slot keeps the last row.
        """
        for t, slot in enumerate(slots):
            slot = int(slot)
            if slot < 0:
                continue
            block, offset = divmod(slot, self.bs)
            self.k[layer, :, block, offset, :] = k_new_bits[t]
            self.v[layer, :, block, offset, :] = v_new_bits[t]

    def copy_blocks(self, pairs):
        """For each (src, dst) in order: block dst <- block src, all layers and heads."""
        for src, dst in pairs:
            self.k[:, :, int(dst)] = self.k[:, :, int(src)]
            self.v[:, :, int(dst)] = self.v[:, :, int(src)]
