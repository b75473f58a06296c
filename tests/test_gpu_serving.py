"""Serving loop on the GPU: every pass of a continuous-batching run, through the C ABI,
against the oracle's plain causal attention of each request computed without paging or
chunking (the SplitFuse invariance: a token's output depends only on its request's
positions, not on how passes cut the prompt, which blocks hold them, or which finished
request held those blocks before)."""
import numpy as np
import pytest
import torch

import oracle
from oracle.compose import OracleBatch
from gpu_harness import assert_close, out_to_f64, say, to_dev
from ragged_blocked_kv_splitfuse_amd import workloads as W
from ragged_blocked_kv_splitfuse_amd.runtime import PagedKVCache, num_cus
from ragged_blocked_kv_splitfuse_amd.serving import DevicePass, ServingLoop

pytestmark = pytest.mark.gpu


def unpaged_reference(v, rid, c, n):
    """Oracle attention of positions [c, c+n) of request `rid` over a contiguous pool."""
    L, bs = c + n, v.block_size
    nb = -(-L // bs)
    K = v.k_rows(rid, 0, nb * bs)                       # [nb*bs][Hkv][D]
    V = v.v_rows(rid, 0, nb * bs)
    kp = K.reshape(nb, bs, v.num_kv_heads, v.head_dim).transpose(0, 2, 1, 3).copy()
    g = min(8, bs)   # the V layout: slots in groups of min(8, bs), feature-major in a group
    vp = V.reshape(nb, bs // g, g, v.num_kv_heads, v.head_dim).transpose(0, 3, 1, 4, 2).copy()
    b = OracleBatch(np.array([0, n], np.int32), np.array([n], np.int32), np.array([c], np.int32),
                    np.arange(nb, dtype=np.int32)[None, :], np.zeros(1, np.int32),
                    np.array([rid], np.int64))
    q = v.q_rows(rid, c, L)
    return oracle.ragged_attention(q, kp, vp, b, v.num_q_heads, v.num_kv_heads, v.scale, bs,
                                   v.dtype)


@pytest.mark.parametrize("dtype,bs", [("bf16", 16), ("bf16", 64), ("f32", 16)])
def test_serving_loop_matches_unpaged_attention(dtype, bs):
    sw = W.serving_small(dtype=dtype, bs=bs)
    v = sw.values
    say(f"serving {dtype} bs={bs}: {len(sw.requests)} requests, {sw.clients} clients, "
        f"budget {sw.budget}, pool {v.num_blocks} blocks")
    cache = PagedKVCache(v.num_blocks, v.block_size, v.num_kv_heads, v.head_dim, v.dtype,
                         free_ids=v.free_ids)
    if dtype == "bf16":
        cache.k_pool.view(torch.int16).fill_(0x7FC1)
        cache.v_pool.view(torch.int16).fill_(0x7FC1)
    else:
        cache.k_pool.fill_(float("nan"))
        cache.v_pool.fill_(float("nan"))
    seen = []

    def rows(hb, running):
        Q, K, V = [], [], []
        for k in range(hb.num_seqs):
            rid, c, n = int(hb.seq_id[k]), int(hb.context_len[k]), int(hb.n_query[k])
            Q.append(v.q_rows(rid, c, c + n))
            K.append(v.k_rows(rid, c, c + n))
            V.append(v.v_rows(rid, c, c + n))
        return (to_dev(np.concatenate(Q), dtype), to_dev(np.concatenate(K), dtype),
                to_dev(np.concatenate(V), dtype))

    def check(p, hb, out):
        S = hb.num_seqs
        seen.append((hb.query_start[:S + 1].copy(), hb.n_query[:S].copy(),
                     hb.context_len[:S].copy(), hb.seq_id[:S].copy(), out_to_f64(out)))

    dp = DevicePass(cache, v.num_q_heads, v.scale, rows, num_cus(), check=check)
    loop = ServingLoop(cache.handle, v.block_size, sw.budget, sw.clients, sw.table_width)
    st = loop.run(sw.requests, device_pass=dp)
    torch.cuda.synchronize()
    say(f"{st.passes} passes, T per pass {st.tokens}")
    assert sum(st.tokens) == sum(r.stop_len for r in sw.requests)
    for p, (qs, nq, cl, sid, got) in enumerate(seen):
        ref = np.concatenate([unpaged_reference(v, int(sid[k]), int(cl[k]), int(nq[k]))
                              for k in range(len(nq))])
        assert_close(got, ref, dtype, f"pass {p} (S={len(nq)}, T={int(qs[-1])})")
    cache.close()
