"""Exact causal attention over a paged cache, float64 (test infrastructure).

FastGen's attention kernels derive from FlashAttention, an *exact* attention
(DeepSpeed-FastGen paper card by Holmes et al. 2024, "Key points" and
"References" 12-13): the tiling changes where numbers are computed, not the
result.  Paging ("Key points": blocked KV cache) and chunking ("Summary": long
prompts cut into chunks over several passes) change only where K/V live and
which pass computes a row.  So the oracle is the plain definition:

    for batch entry s with c = context_len[s] cached tokens and n new tokens,
    new token i (position c + i) and query head g (KV head h = g // (Hq/Hkv)):
        l_j = scale * <q_i, k_j>            for every key position j <= c + i
        o   = sum_j exp(l_j - max l) v_j / sum_j exp(l_j - max l)

Keys are gathered through the block table (position j -> block
``block_table[s][j // bs]``, slot ``j % bs``; the V pool keeps slots in groups
of min(8, bs), see ``layout``), widened exactly to float64.
Readings where the pages are silent: the new rows are appended before the
pass attends (a query sees its own chunk's earlier rows and itself);
contiguous GQA groups; ``scale`` is an argument (1/sqrt(D) in every workload).
Rows are processed in groups only to bound memory; each row's arithmetic is
the definition above.
"""
import numpy as np

from .bf16 import to_f64

ROW_GROUP = 256


def gather_history(k_pool, v_pool, table_row, length, block_size, dtype):
    """K and V of positions [0, length) of one sequence: two [Hkv][length][D] float64 arrays."""
    nb = -(-length // block_size)
    blocks = np.asarray(table_row[:nb], dtype=np.int64)
    if nb and blocks.min() < 0:
        raise ValueError("history position has no block")
    K = to_f64(k_pool[blocks], dtype)                      # [nb][Hkv][bs][D]
    V = to_f64(v_pool[blocks], dtype)                      # [nb][Hkv][bs/g][D][g]
    hkv, d = K.shape[1], K.shape[3]
    K = K.transpose(1, 0, 2, 3).reshape(hkv, nb * block_size, d)[:, :length]
    # key (block, group, index in group) -> position block*bs + group*g + index
    V = V.transpose(1, 0, 2, 4, 3).reshape(hkv, nb * block_size, d)[:, :length]
    return K, V


def ragged_attention(q, k_pool, v_pool, batch, num_q_heads: int, num_kv_heads: int,
                     scale: float, block_size: int, dtype: str, seqs=None) -> np.ndarray:
    """Return O [T][Hq][D] float64.  ``q``: [T][Hq][D] in batch token order.

    ``seqs`` optionally restricts the work to some batch entries (rows of the
    other entries are left as NaN); used to sample very large passes.
    """
    if num_q_heads % num_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    group = num_q_heads // num_kv_heads
    T = batch.num_tokens
    D = q.shape[-1]
    out = np.full((T, num_q_heads, D), np.nan)
    which = range(batch.num_seqs) if seqs is None else seqs
    for s in which:
        c = int(batch.context_len[s])
        n = int(batch.n_query[s])
        t0 = int(batch.query_start[s])
        K, V = gather_history(k_pool, v_pool, batch.block_table[s], c + n, block_size, dtype)
        Q = to_f64(q[t0:t0 + n], dtype)                    # [n][Hq][D]
        for g in range(num_q_heads):
            h = g // group
            for i0 in range(0, n, ROW_GROUP):
                i1 = min(n, i0 + ROW_GROUP)
                visible = c + i1                           # keys 0 .. c+i1-1 reach the last row
                logits = (Q[i0:i1, g, :] @ K[h, :visible, :].T) * scale
                rows = np.arange(i0, i1)[:, None]
                keys = np.arange(visible)[None, :]
                logits = np.where(keys <= c + rows, logits, -np.inf)
                m = logits.max(axis=1, keepdims=True)
                w = np.exp(logits - m)
                out[t0 + i0:t0 + i1, g, :] = (w @ V[h, :visible, :]) / w.sum(axis=1, keepdims=True)
    return out
