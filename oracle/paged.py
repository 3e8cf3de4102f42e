"""Block-table (paged) layout of the cache (oracle; test infrastructure only).

Source: "10.3 - KV cache implementation details", section 7.2 (cache
management policies): the cache is allocated in fixed-size blocks (for
example 16 tokens) like virtual-memory pages; a block table maps each
sequence's logical blocks to physical blocks, so non-contiguous physical
blocks are logically contiguous for the model; section 7.3 (prefix caching):
requests that share a prefix can share its K/V. "Key-value cache" lesson
record: serving systems often manage these arrays with block-based
allocation.

Readings taken where the pages are silent (listed in the design notes):
* one pool per layer, [K|V][num_blocks][H_kv][block_size][D]: a block holds
  block_size consecutive rows of every kv head of one sequence's block;
* the block table is [B][max_context / block_size] int32; row r of sequence
  b lives in physical block table[b][r // block_size] at offset
  r % block_size;
* attention reads the logical rows [0, n_b) through the table, exactly as
  the static cache's rows (the result is the static decode of the gathered
  rows);
* an append whose target block index is outside [0, num_blocks) or whose
  rows leave [0, max_context) is skipped for that sequence (nothing
  written) and reported, like the static cache's out-of-range append;
* two sequences whose tables name the same physical blocks share those rows
  (prefix sharing); an append into a shared block writes it for both.

Element bits are stored as for the static cache (uint16 bf16 patterns).
"""

import numpy as np

_BITS = {"f32": np.uint32, "bf16": np.uint16}


class RefPagedCache:
    """Pools [L][2][num_blocks][H_kv][block_size][D] of stored bits; block tables are passed per call."""

    def __init__(self, n_layers, num_blocks, n_kv_heads, block_size, head_dim, storage, max_context):
        if max_context % block_size:
            raise ValueError("max_context must be a multiple of block_size")
        self.storage = storage
        self.block_size = block_size
        self.num_blocks = num_blocks
        self.max_context = max_context
        self.shape = (n_layers, 2, num_blocks, n_kv_heads, block_size, head_dim)
        self.pool = np.zeros(self.shape, dtype=_BITS[storage])

    def _where(self, table_row, r):
        blk = int(table_row[r // self.block_size])
        return blk, r % self.block_size

    def append(self, layer, k_new, v_new, cache_index, block_table):
        """Write rows [ci_b, ci_b + t_new) of sequence b through its table; k_new, v_new [B, H_kv, t_new, D].
        Returns the skipped sequences (rows outside [0, max_context) or a block outside the pool)."""
        k_new = np.asarray(k_new)
        v_new = np.asarray(v_new)
        t_new = k_new.shape[2]
        skipped = []
        for b, ci in enumerate(np.asarray(cache_index).tolist()):
            if ci < 0 or ci + t_new > self.max_context:
                skipped.append(b)
                continue
            where = [self._where(block_table[b], ci + i) for i in range(t_new)]
            if any(not 0 <= blk < self.num_blocks for blk, _ in where):
                skipped.append(b)
                continue
            for i, (blk, off) in enumerate(where):
                self.pool[layer, 0, blk, :, off, :] = k_new[b, :, i, :]
                self.pool[layer, 1, blk, :, off, :] = v_new[b, :, i, :]
        return skipped

    def gather(self, layer, block_table, batch):
        """The logical view through the tables: keys, values [B, H_kv, max_context, D] (rows whose block is
        outside the pool read as zero bits)."""
        _, _, nb, hkv, bs, d = self.shape
        out = np.zeros((2, batch, hkv, self.max_context, d), dtype=self.pool.dtype)
        for b in range(batch):
            for r in range(self.max_context):
                blk, off = self._where(block_table[b], r)
                if 0 <= blk < nb:
                    out[:, b, :, r, :] = self.pool[layer, :, blk, :, off, :]
        return out[0], out[1]
