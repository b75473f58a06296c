"""GPU-side test helpers: run one pass through the C ABI and compare with the oracle.

Inputs come from the seeded generator (host numpy, or torch's seeded device RNG for pools
too large for the host); expected values come from the oracle only.
"""
import sys
import time

import numpy as np
import torch

import oracle
import harness
from oracle.compose import OracleBatch
from ragged_blocked_kv_splitfuse_amd import fg
from ragged_blocked_kv_splitfuse_amd.runtime import (DeviceDescriptors, PagedKVCache,
                                                     Workspace, stream_handle)

BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
F32_MAX_ABS = 1e-5


def say(*a):
    print(f"[{time.strftime('%H:%M:%S')}]", *a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_host_bits(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def batch_of(hb: fg.HostBatch) -> OracleBatch:
    S = hb.num_seqs
    return OracleBatch(hb.query_start[:S + 1].copy(), hb.n_query[:S].copy(),
                       hb.context_len[:S].copy(), hb.block_table[:S].copy(),
                       hb.seq_index[:S].copy(), hb.seq_id[:S].copy())


def same_batch(a: OracleBatch, b: OracleBatch) -> bool:
    return all(np.array_equal(getattr(a, f), getattr(b, f)) for f in
               ("query_start", "n_query", "context_len", "block_table", "seq_index", "seq_id"))


class GpuPass:
    """Library-side state of a sequence of passes over one cache."""

    def __init__(self, w, k_pool_dev, v_pool_dev, states=None, num_cus=256):
        self.w = w
        self.cache = PagedKVCache(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                                  w.dtype, free_ids=w.free_ids, k_pool=k_pool_dev,
                                  v_pool=v_pool_dev)
        self.ss = fg.SeqStates(states if states is not None else w.fresh_states(),
                               w.table_width)
        self.desc = DeviceDescriptors()
        self.ws = Workspace()
        self.num_cus = num_cus

    def compose(self, budget=None):
        hb = fg.HostBatch(self.ss.n, self.w.table_width)
        st = fg.fg_splitfuse_compose(self.cache.handle, self.ss, budget or self.w.budget, hb)
        assert st == fg.FG_OK
        fg.fg_validate_batch(self.cache.handle, hb)
        return hb

    def run(self, hb, q, k_new, v_new):
        """append + attention on the current stream; returns (out tensor, plan info)."""
        w = self.w
        info, work = fg.fg_attention_plan(self.cache.handle, hb, w.num_q_heads, self.num_cus)
        c = self.desc.upload(hb, work if info.num_work else None)
        s = stream_handle()
        fg.fg_kv_append(self.cache.handle, c, k_new.data_ptr(), v_new.data_ptr(), s)
        out = torch.empty((hb.num_tokens, w.num_q_heads, w.head_dim), dtype=q.dtype,
                          device=q.device)
        wp, wb = self.ws.ensure(info.workspace_bytes)
        fg.fg_ragged_attention(self.cache.handle, c, info, self.desc.work_ptr, q.data_ptr(),
                               w.num_q_heads, w.scale, out.data_ptr(), wp, wb, s)
        return out, info

    def attention_only(self, hb, q):
        w = self.w
        info, work = fg.fg_attention_plan(self.cache.handle, hb, w.num_q_heads, self.num_cus)
        c = self.desc.upload(hb, work if info.num_work else None)
        out = torch.empty((hb.num_tokens, w.num_q_heads, w.head_dim), dtype=q.dtype,
                          device=q.device)
        wp, wb = self.ws.ensure(info.workspace_bytes)
        fg.fg_ragged_attention(self.cache.handle, c, info, self.desc.work_ptr, q.data_ptr(),
                               w.num_q_heads, w.scale, out.data_ptr(), wp, wb, stream_handle())
        return out

    def commit(self):
        fg.fg_splitfuse_commit(self.ss)


def errors(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got - ref)
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def assert_close(got, ref, dtype, what=""):
    mx, mean = errors(got, ref)
    say(f"{what}: max-abs {mx:.3e}, mean-abs {mean:.3e}")
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    if dtype == "bf16":
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (what, mx, mean)
    else:
        assert mx <= F32_MAX_ABS, (what, mx)
    return mx, mean


def full_pass(w, num_cus=256, budget=None):
    """Host-generated pools + one pass on GPU and in the oracle.  Returns a dict."""
    say(f"{w.name}: generating inputs")
    states = harness.oracle_states(w)
    kp, vp = harness.empty_pools(w)
    harness.fill_history(w, kp, vp, states)
    k0, v0 = kp.copy(), vp.copy()
    ob, st = oracle.splitfuse_compose(states, budget or w.budget, oracle.FreeList(w.free_ids),
                                      w.block_size, w.table_width)
    q, kn, vn = harness.new_rows(w, ob, states)
    say(f"{w.name}: GPU pass (T={ob.num_tokens}, S={ob.num_seqs})")
    gp = GpuPass(w, to_dev(k0, w.dtype), to_dev(v0, w.dtype), num_cus=num_cus)
    hb = gp.compose(budget)
    assert same_batch(batch_of(hb), ob), "library and oracle composed different passes"
    out, info = gp.run(hb, to_dev(q, w.dtype), to_dev(kn, w.dtype), to_dev(vn, w.dtype))
    torch.cuda.synchronize()
    say(f"{w.name}: oracle (records {info.num_work}, split groups {info.num_groups})")
    oracle.kv_append(kp, vp, kn, vn, ob, w.block_size)
    ref = oracle.ragged_attention(q, kp, vp, ob, w.num_q_heads, w.num_kv_heads, w.scale,
                                  w.block_size, w.dtype)
    return dict(gp=gp, hb=hb, batch=ob, out=out, ref=ref, k_pool=kp, v_pool=vp, q=q, kn=kn,
                vn=vn, info=info)


def compact_sub_batch(batch, seqs, k_dev, v_dev, q_rows_host, dtype):
    """Oracle inputs for a few batch entries of a pass whose pools live on the device: copy
    only their blocks back, relabelled 0..n-1 (the result does not depend on labels)."""
    blocks = []
    rows, qs, nq, cl = [], [0], [], []
    width = batch.block_table.shape[1]
    bt = np.full((len(seqs), width), -1, np.int32)
    for k, s in enumerate(seqs):
        c, n = int(batch.context_len[s]), int(batch.n_query[s])
        need = -(-(c + n) // int(k_dev.shape[2]))
        ids = batch.block_table[s, :need]
        bt[k, :need] = np.arange(len(blocks), len(blocks) + need)
        blocks += ids.tolist()
        t0 = int(batch.query_start[s])
        rows.append(q_rows_host[t0:t0 + n])
        qs.append(qs[-1] + n)
        nq.append(n)
        cl.append(c)
    idx = torch.tensor(blocks, dtype=torch.long, device=k_dev.device)
    kp = to_host_bits(k_dev.index_select(0, idx), dtype)
    vp = to_host_bits(v_dev.index_select(0, idx), dtype)
    sub = OracleBatch(np.array(qs, np.int32), np.array(nq, np.int32), np.array(cl, np.int32),
                      bt, np.arange(len(seqs), dtype=np.int32), np.zeros(len(seqs), np.int64))
    return sub, kp, vp, np.concatenate(rows)


def oracle_attention_by_heads(q, k_pool, v_pool, batch, num_q_heads, num_kv_heads, scale,
                              block_size, dtype, workers=None):
    """The oracle's attention, run on groups of KV heads in parallel threads (heads are
    independent, so this is the oracle's own result; numpy releases the GIL in its kernels).
    BLAS is limited to one thread per worker meanwhile."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    G = num_q_heads // num_kv_heads
    workers = workers or max(1, min(num_kv_heads, len(os.sched_getaffinity(0)), 16))
    groups = np.array_split(np.arange(num_kv_heads), workers)

    def run(hs):
        h0, h1 = int(hs[0]), int(hs[-1]) + 1
        return oracle.ragged_attention(np.ascontiguousarray(q[:, h0 * G:h1 * G]),
                                       np.ascontiguousarray(k_pool[:, h0:h1]),
                                       np.ascontiguousarray(v_pool[:, h0:h1]), batch,
                                       (h1 - h0) * G, h1 - h0, scale, block_size, dtype)

    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1, user_api="blas")
    except Exception:  # noqa: BLE001
        limit = None
    try:
        with ThreadPoolExecutor(len(groups)) as ex:
            parts = list(ex.map(run, [g for g in groups if len(g)]))
    finally:
        if limit is not None:
            limit.restore_original_limits()
    return np.concatenate(parts, axis=1)
