"""Test-side helpers: turn a generated workload into oracle inputs.

Uses the oracle (allowed in tests) to place each sequence's history into a
sentinel-filled pool, and assembles the pass's new rows in batch order.
"""
import numpy as np

import oracle
from oracle.compose import OracleBatch, SeqState, FreeList

SENT_BF16 = np.uint16(0x7FC1)          # a quiet NaN pattern
SENT_F32 = np.uint32(0x7FC00001)


def empty_pools(w):
    ks = oracle.k_pool_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size)
    vs = oracle.v_pool_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size)
    if w.dtype == "bf16":
        k = np.full(ks, SENT_BF16, np.uint16)
        v = np.full(vs, SENT_BF16, np.uint16)
    else:
        k = np.full(ks, SENT_F32, np.uint32).view(np.float32)
        v = np.full(vs, SENT_F32, np.uint32).view(np.float32)
    return k, v


def history_batch(w, states):
    """A batch whose 'new' rows are every sequence's cached history (positions 0..c-1)."""
    idx = [i for i, s in enumerate(states) if s.n_cached > 0]
    S = len(idx)
    qs = np.zeros(S + 1, np.int32)
    nq = np.zeros(S, np.int32)
    bt = np.full((S, max(1, w.table_width)), -1, np.int32)
    for k, i in enumerate(idx):
        s = states[i]
        nq[k] = s.n_cached
        qs[k + 1] = qs[k] + s.n_cached
        bt[k, :len(s.blocks)] = s.blocks
    return OracleBatch(qs, nq, np.zeros(S, np.int32), bt, np.array(idx, np.int32),
                       np.array([states[i].seq_id for i in idx], np.int64)), idx


def fill_history(w, k_pool, v_pool, states):
    hb, idx = history_batch(w, states)
    if hb.num_seqs == 0:
        return
    K = np.concatenate([w.k_rows(states[i].seq_id, 0, states[i].n_cached) for i in idx])
    V = np.concatenate([w.v_rows(states[i].seq_id, 0, states[i].n_cached) for i in idx])
    oracle.kv_append(k_pool, v_pool, K, V, hb, w.block_size)


def oracle_states(w):
    return [SeqState(s.seq_id, s.n_cached, s.prompt_len, list(s.blocks), w.table_width)
            for s in w.seqs]


def new_rows(w, batch, states):
    """Q [T][Hq][D], K/V [T][Hkv][D] of the pass in batch order."""
    Q, K, V = [], [], []
    for k in range(batch.num_seqs):
        s = states[int(batch.seq_index[k])]
        c, n = int(batch.context_len[k]), int(batch.n_query[k])
        Q.append(w.q_rows(s.seq_id, c, c + n))
        K.append(w.k_rows(s.seq_id, c, c + n))
        V.append(w.v_rows(s.seq_id, c, c + n))
    if not Q:
        dt = np.uint16 if w.dtype == "bf16" else np.float32
        z = lambda h: np.zeros((0, h, w.head_dim), dt)
        return z(w.num_q_heads), z(w.num_kv_heads), z(w.num_kv_heads)
    return np.concatenate(Q), np.concatenate(K), np.concatenate(V)


def oracle_pass(w, states=None, free=None, k_pool=None, v_pool=None, budget=None):
    """Compose + append + attention with the oracle.  Returns a dict of everything."""
    if states is None:
        states = oracle_states(w)
    if free is None:
        free = FreeList(w.free_ids)
    if k_pool is None:
        k_pool, v_pool = empty_pools(w)
        fill_history(w, k_pool, v_pool, states)
    batch, status = oracle.splitfuse_compose(states, budget or w.budget, free, w.block_size,
                                             w.table_width)
    q, kn, vn = new_rows(w, batch, states)
    oracle.kv_append(k_pool, v_pool, kn, vn, batch, w.block_size)
    out = oracle.ragged_attention(q, k_pool, v_pool, batch, w.num_q_heads, w.num_kv_heads,
                                  w.scale, w.block_size, w.dtype)
    return dict(states=states, free=free, batch=batch, status=status, q=q, k_new=kn,
                v_new=vn, k_pool=k_pool, v_pool=v_pool, out=out)
