"""Append of a pass's new K/V rows into the blocked cache (test infrastructure).

The paged cache (DeepSpeed-FastGen paper card by Holmes et al. 2024, "Key
points": a blocked KV cache as in PagedAttention) holds every position of a
sequence in fixed-size blocks named by its block table.  The new token i of
batch entry s sits at position ``p = context_len[s] + i``, i.e. in physical
block ``block_table[s][p // bs]`` at slot ``p % bs``.

Cache layout (a design reading; the pages give none):
    K pool: [num_blocks][Hkv][bs][D]   (key-major inside a block)
    V pool: [num_blocks][Hkv][D][bs]   (feature-major inside a block)
The copy is a bit copy, so the GPU result must equal this one bit for bit, and
every other element of both pools must stay untouched.
"""
import numpy as np


def kv_append(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              batch, block_size: int) -> None:
    """In place.  ``k_new``/``v_new``: [T][Hkv][D] in batch token order (same dtype as the pools)."""
    for s in range(batch.num_seqs):
        c = int(batch.context_len[s])
        t0 = int(batch.query_start[s])
        for i in range(int(batch.n_query[s])):
            p = c + i
            blk = int(batch.block_table[s, p // block_size])
            if blk < 0:
                raise ValueError("position has no block")
            slot = p % block_size
            k_pool[blk, :, slot, :] = k_new[t0 + i]
            v_pool[blk, :, :, slot] = v_new[t0 + i]
