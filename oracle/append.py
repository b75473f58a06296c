"""Append of a pass's new K/V rows into the blocked cache (test infrastructure).

The paged cache (DeepSpeed-FastGen paper card by Holmes et al. 2024, "Key
points": a blocked KV cache as in PagedAttention) holds every position of a
sequence in fixed-size blocks named by its block table.  The new token i of
batch entry s sits at position ``p = context_len[s] + i``, i.e. in physical
block ``block_table[s][p // bs]`` at slot ``p % bs``.

Cache layout (a design reading; the pages give none; see ``layout``):
    K pool: [num_blocks][Hkv][bs][D]         (key-major inside a block)
    V pool: [num_blocks][Hkv][bs/g][D][g]    (keys in groups of g = min(8, bs),
                                              feature-major inside a group)
The copy is a bit copy, so the GPU result must equal this one bit for bit, and
every other element of both pools must stay untouched.
"""
import numpy as np

from .layout import v_pool_shape, v_slot


def kv_append(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              batch, block_size: int) -> None:
    """In place.  ``k_new``/``v_new``: [T][Hkv][D] in batch token order (same dtype as the pools)."""
    nb, hkv, _, d = k_pool.shape
    if v_pool.shape != v_pool_shape(nb, hkv, d, block_size):
        raise ValueError(f"V pool shape {v_pool.shape} is not the layout's "
                         f"{v_pool_shape(nb, hkv, d, block_size)}")
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
            grp, j = v_slot(block_size, slot)
            v_pool[blk, :, grp, :, j] = v_new[t0 + i]
