"""Parity at the workloads' full sizes, in the launch configuration the benchmark times
(planner sized for the device's compute units).

* LLaMA-2-7B mixed pass and Mistral-7B GQA pass: the oracle runs the whole pass.
* Decode-only pass: 32 sequences against the whole oracle, and all 256 sequences (11 GB of
  cache, generated on the device) on a sample of sequences plus a full-pool check of the
  append (exactly the new slots changed, each to its new row).
* Chunked prefill: 32 passes of 512 tokens over a 16384-token prompt against the oracle's
  last pass, the SplitFuse invariant (the last chunk's rows equal the unchunked pass's rows),
  and sampled rows of the unchunked pass against the oracle.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle
import harness
import gpu_harness as G
from oracle.compose import OracleBatch
from ragged_blocked_kv_splitfuse_amd import fg, workloads as wl
from ragged_blocked_kv_splitfuse_amd.runtime import num_cus


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _append_exact(r, w):
    dt = np.uint16 if w.dtype == "bf16" else np.uint32
    assert np.array_equal(G.to_host_bits(r["gp"].cache.k_pool, w.dtype).view(dt), r["k_pool"].view(dt))
    assert np.array_equal(G.to_host_bits(r["gp"].cache.v_pool, w.dtype).view(dt), r["v_pool"].view(dt))


@pytest.mark.parametrize("cfg", [2, 5])
def test_mixed_full_pass(cfg):
    w = wl.make(cfg)
    r = G.full_pass(w, num_cus=num_cus())
    _append_exact(r, w)
    G.assert_close(G.out_to_f64(r["out"]), r["ref"], "bf16", w.name)


def test_decode_only_32_sequences():
    w = wl.decode_only(3, num_seqs=32)
    r = G.full_pass(w, num_cus=num_cus())
    _append_exact(r, w)
    G.assert_close(G.out_to_f64(r["out"]), r["ref"], "bf16", "decode_only[32]")


def test_decode_only_full_size_sampled():
    w = wl.make(3)
    G.say(f"decode_only full: {w.num_blocks} blocks, pools {2 * w.num_blocks * 2**20 / 2**30:.1f} GiB")
    kp = torch.empty((w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim), dtype=torch.bfloat16,
                     device="cuda")
    vp = torch.empty((w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size), dtype=torch.bfloat16,
                     device="cuda")
    wl.fill_pools_device(kp, vp, seed=31337)
    k_before, v_before = kp.clone(), vp.clone()
    gp = G.GpuPass(w, kp, vp, num_cus=num_cus())
    hb = gp.compose()
    ob = G.batch_of(hb)
    states = harness.oracle_states(w)
    ob_oracle, _ = oracle.splitfuse_compose(states, w.budget, oracle.FreeList(w.free_ids),
                                            w.block_size, w.table_width)
    assert G.same_batch(ob, ob_oracle)
    q, kn, vn = harness.new_rows(w, ob_oracle, states)
    qd, knd, vnd = G.to_dev(q, "bf16"), G.to_dev(kn, "bf16"), G.to_dev(vn, "bf16")
    out, info = gp.run(hb, qd, knd, vnd)
    torch.cuda.synchronize()
    G.say(f"records {info.num_work}, groups {info.num_groups}")
    # append: exactly the new slots changed, each to its new row (device-side comparison)
    T, bs = ob.num_tokens, w.block_size
    pos = ob.context_len.astype(np.int64)               # each entry has one new token here
    blk = ob.block_table[np.arange(T), pos // bs].astype(np.int64)
    slot = pos % bs
    bi = torch.from_numpy(blk).cuda()
    si = torch.from_numpy(slot).cuda()
    assert torch.equal(kp[bi, :, si, :].view(torch.int16), knd.view(torch.int16))
    assert torch.equal(vp[bi, :, :, si].view(torch.int16), vnd.view(torch.int16))
    changed_k = int((kp.view(torch.int16) != k_before.view(torch.int16)).sum())
    changed_v = int((vp.view(torch.int16) != v_before.view(torch.int16)).sum())
    kp_fix, vp_fix = k_before.clone(), v_before.clone()
    kp_fix[bi, :, si, :] = knd
    vp_fix[bi, :, :, si] = vnd
    assert torch.equal(kp_fix.view(torch.int16), kp.view(torch.int16))
    assert torch.equal(vp_fix.view(torch.int16), vp.view(torch.int16))
    G.say(f"append: {changed_k} K and {changed_v} V elements changed, all at new slots")
    del k_before, v_before, kp_fix, vp_fix
    # attention: sampled sequences (longest, shortest and spread) against the oracle
    order = np.argsort(ob.context_len)
    pick = sorted(set(order[[0, 1, 2, -1, -2, -3]].tolist() + list(range(0, ob.num_seqs, 23))))
    sub, skp, svp, sq = G.compact_sub_batch(ob, pick, kp, vp, q, "bf16")
    ref = oracle.ragged_attention(sq, skp, svp, sub, w.num_q_heads, w.num_kv_heads, w.scale, bs, "bf16")
    got = G.out_to_f64(out)[ob.query_start[pick]]
    G.assert_close(got, ref, "bf16", f"decode_only[256] sampled {len(pick)} seqs")


def test_chunked_prefill_splitfuse():
    w = wl.make(4)
    L, chunk = 16384, w.budget
    sid = w.seqs[0].seq_id
    G.say("chunked: generating 16384 positions")
    Q = w.q_rows(sid, 0, L)
    K = w.k_rows(sid, 0, L)
    V = w.v_rows(sid, 0, L)
    kp0, vp0 = harness.empty_pools(w)                   # NaN sentinels everywhere
    # GPU: 32 passes of 512
    gp = G.GpuPass(w, G.to_dev(kp0, "bf16"), G.to_dev(vp0, "bf16"), num_cus=num_cus())
    Qd, Kd, Vd = G.to_dev(Q, "bf16"), G.to_dev(K, "bf16"), G.to_dev(V, "bf16")
    last = None
    for k in range(w.passes):
        hb = gp.compose()
        assert hb.num_seqs == 1 and hb.context_len[0] == k * chunk and hb.n_query[0] == chunk
        sl = slice(k * chunk, (k + 1) * chunk)
        out, info = gp.run(hb, Qd[sl].contiguous(), Kd[sl].contiguous(), Vd[sl].contiguous())
        gp.commit()
        last = (out, G.batch_of(hb), info)
    torch.cuda.synchronize()
    out31, b31, info31 = last
    G.say(f"pass 31: records {info31.num_work}, groups {info31.num_groups}")
    # GPU: one unchunked pass of all 16384 tokens
    gpu_u = G.GpuPass(w, G.to_dev(kp0, "bf16"), G.to_dev(vp0, "bf16"), num_cus=num_cus())
    hbu = gpu_u.compose(budget=L)
    assert hbu.num_tokens == L
    out_u, info_u = gpu_u.run(hbu, Qd, Kd, Vd)
    torch.cuda.synchronize()
    G.say(f"unchunked: records {info_u.num_work}, groups {info_u.num_groups}")
    # SplitFuse invariant on the GPU: the last chunk's rows equal the unchunked rows
    G.assert_close(G.out_to_f64(out31), G.out_to_f64(out_u[L - chunk:]), "bf16",
                   "chunked pass 31 vs unchunked rows 15872..16383")
    # oracle: the same 32 compositions, its own append, attention of pass 31
    states = harness.oracle_states(w)
    free = oracle.FreeList(w.free_ids)
    kp, vp = harness.empty_pools(w)
    for k in range(w.passes):
        ob, _ = oracle.splitfuse_compose(states, chunk, free, w.block_size, w.table_width)
        sl = slice(k * chunk, (k + 1) * chunk)
        oracle.kv_append(kp, vp, K[sl], V[sl], ob, w.block_size)
        oracle.compose.commit_pass(states)
    assert G.same_batch(ob, b31)
    ref31 = oracle.ragged_attention(Q[L - chunk:], kp, vp, ob, w.num_q_heads, w.num_kv_heads,
                                    w.scale, w.block_size, "bf16")
    G.assert_close(G.out_to_f64(out31), ref31, "bf16", "chunked pass 31 vs oracle")
    # both GPU caches hold exactly the oracle's pool after all appends
    assert np.array_equal(G.to_host_bits(gp.cache.k_pool, "bf16"), kp)
    assert np.array_equal(G.to_host_bits(gp.cache.v_pool, "bf16"), vp)
    assert np.array_equal(G.to_host_bits(gpu_u.cache.k_pool, "bf16"), kp)
    assert np.array_equal(G.to_host_bits(gpu_u.cache.v_pool, "bf16"), vp)
    # sampled rows of the unchunked pass: row i == a one-token pass at context i
    rows = sorted(set([0, 1, 2, 63, 64, 65, 127, 128, 129, 511, 512, 4095, 8191, 8192, 12345,
                       16383] + list(range(300, L, 1537))))
    bt = G.batch_of(hbu).block_table[0]
    sub = OracleBatch(np.arange(len(rows) + 1, dtype=np.int32), np.ones(len(rows), np.int32),
                      np.array(rows, np.int32), np.tile(bt, (len(rows), 1)),
                      np.zeros(len(rows), np.int32), np.zeros(len(rows), np.int64))
    # (rows share the table: the oracle only reads blocks, it never checks ownership)
    ref_u = oracle.ragged_attention(Q[rows], kp, vp, sub, w.num_q_heads, w.num_kv_heads,
                                    w.scale, w.block_size, "bf16")
    G.assert_close(G.out_to_f64(out_u)[rows], ref_u, "bf16", f"unchunked {len(rows)} sampled rows")
