"""Parity at the workloads' full sizes, in the launch configuration the benchmark times
(planner sized for the device's compute units).  Every output row is compared.

* LLaMA-2-7B mixed pass and Mistral-7B GQA pass: the oracle runs the whole pass.
* Decode-only pass: 32 sequences against the whole oracle; and all 256 sequences (11 GB of
  cache, generated on the device) against the oracle in groups of sequences copied back one
  group at a time, plus a full-pool check of the append (exactly the new slots changed, each
  to its new row).
* Chunked prefill: every one of the 32 passes of 512 tokens over a 16384-token prompt against
  the oracle's pass; the SplitFuse invariant (the last chunk's rows equal the unchunked pass's
  rows); and every row of the unchunked pass against the oracle.
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


def test_decode_only_full_size():
    w = wl.make(3)
    G.say(f"decode_only full: {w.num_blocks} blocks, pools {2 * w.num_blocks * 2**20 / 2**30:.1f} GiB")
    kp = torch.empty(oracle.k_pool_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size),
                     dtype=torch.bfloat16, device="cuda")
    vp = torch.empty(oracle.v_pool_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size),
                     dtype=torch.bfloat16, device="cuda")
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
    grp, j = oracle.v_slot(bs, slot)
    bi = torch.from_numpy(blk).cuda()
    si = torch.from_numpy(slot).cuda()
    gi, ji = torch.from_numpy(grp).cuda(), torch.from_numpy(j).cuda()
    assert torch.equal(kp[bi, :, si, :].view(torch.int16), knd.view(torch.int16))
    assert torch.equal(vp[bi, :, gi, :, ji].view(torch.int16), vnd.view(torch.int16))
    changed_k = int((kp.view(torch.int16) != k_before.view(torch.int16)).sum())
    changed_v = int((vp.view(torch.int16) != v_before.view(torch.int16)).sum())
    kp_fix, vp_fix = k_before.clone(), v_before.clone()
    kp_fix[bi, :, si, :] = knd
    vp_fix[bi, :, gi, :, ji] = vnd
    assert torch.equal(kp_fix.view(torch.int16), kp.view(torch.int16))
    assert torch.equal(vp_fix.view(torch.int16), vp.view(torch.int16))
    G.say(f"append: {changed_k} K and {changed_v} V elements changed, all at new slots")
    del k_before, v_before, kp_fix, vp_fix
    # attention: every sequence against the oracle, a group of sequences at a time (their
    # blocks copied back and relabelled; the result does not depend on block labels)
    got_all = G.out_to_f64(out)
    errs = []
    for g0 in range(0, ob.num_seqs, 32):
        pick = list(range(g0, min(ob.num_seqs, g0 + 32)))
        sub, skp, svp, sq = G.compact_sub_batch(ob, pick, kp, vp, q, "bf16")
        ref = G.oracle_attention_by_heads(sq, skp, svp, sub, w.num_q_heads, w.num_kv_heads,
                                          w.scale, bs, "bf16")
        got = got_all[ob.query_start[pick]]
        mx, mean = G.assert_close(got, ref, "bf16", f"decode_only[256] sequences {g0}..{pick[-1]}")
        errs.append(np.abs(got - ref).ravel())
        del sub, skp, svp
    d = np.concatenate(errs)
    assert d.size == ob.num_tokens * w.num_q_heads * w.head_dim
    G.assert_close(d, np.zeros_like(d), "bf16", "decode_only[256] all sequences")


def _chunked_inputs(w):
    L = w.seqs[0].prompt_len
    sid = w.seqs[0].seq_id
    G.say(f"chunked: generating {L} positions")
    return L, w.q_rows(sid, 0, L), w.k_rows(sid, 0, L), w.v_rows(sid, 0, L)


def test_chunked_prefill_every_pass():
    """32 passes of 512 tokens through the library, each pass's output against the oracle's
    pass (the oracle appends the same chunks to its own pool); both caches identical after
    every append."""
    w = wl.make(4)
    L, Q, K, V = _chunked_inputs(w)
    chunk = w.budget
    kp0, vp0 = harness.empty_pools(w)                   # NaN sentinels everywhere
    gp = G.GpuPass(w, G.to_dev(kp0, "bf16"), G.to_dev(vp0, "bf16"), num_cus=num_cus())
    Qd, Kd, Vd = G.to_dev(Q, "bf16"), G.to_dev(K, "bf16"), G.to_dev(V, "bf16")
    outs, batches = [], []
    for k in range(w.passes):
        hb = gp.compose()
        assert hb.num_seqs == 1 and hb.context_len[0] == k * chunk and hb.n_query[0] == chunk
        sl = slice(k * chunk, (k + 1) * chunk)
        out, info = gp.run(hb, Qd[sl].contiguous(), Kd[sl].contiguous(), Vd[sl].contiguous())
        gp.commit()
        outs.append(G.out_to_f64(out))
        batches.append(G.batch_of(hb))
        if k in (0, 1, 31):
            G.say(f"pass {k}: records {info.num_work}, groups {info.num_groups}")
    torch.cuda.synchronize()
    states = harness.oracle_states(w)
    free = oracle.FreeList(w.free_ids)
    kp, vp = harness.empty_pools(w)
    errs = []
    for k in range(w.passes):
        ob, _ = oracle.splitfuse_compose(states, chunk, free, w.block_size, w.table_width)
        assert G.same_batch(ob, batches[k])
        sl = slice(k * chunk, (k + 1) * chunk)
        oracle.kv_append(kp, vp, K[sl], V[sl], ob, w.block_size)
        oracle.compose.commit_pass(states)
        ref = G.oracle_attention_by_heads(Q[sl], kp, vp, ob, w.num_q_heads, w.num_kv_heads,
                                          w.scale, w.block_size, "bf16")
        G.assert_close(outs[k], ref, "bf16", f"chunked pass {k} vs oracle")
        errs.append(np.abs(outs[k] - ref).ravel())
    d = np.concatenate(errs)
    assert d.size == L * w.num_q_heads * w.head_dim
    G.assert_close(d, np.zeros_like(d), "bf16", "chunked: all 32 passes")
    assert np.array_equal(G.to_host_bits(gp.cache.k_pool, "bf16"), kp)
    assert np.array_equal(G.to_host_bits(gp.cache.v_pool, "bf16"), vp)


def test_chunked_prefill_unchunked_and_splitfuse_invariant():
    """One unchunked pass of all 16384 tokens: every row against the oracle, and the SplitFuse
    invariant on the GPU (pass 31 of the chunked run equals rows 15872..16383)."""
    w = wl.make(4)
    L, Q, K, V = _chunked_inputs(w)
    chunk = w.budget
    kp0, vp0 = harness.empty_pools(w)
    Qd, Kd, Vd = G.to_dev(Q, "bf16"), G.to_dev(K, "bf16"), G.to_dev(V, "bf16")
    gp = G.GpuPass(w, G.to_dev(kp0, "bf16"), G.to_dev(vp0, "bf16"), num_cus=num_cus())
    for k in range(w.passes):
        hb = gp.compose()
        sl = slice(k * chunk, (k + 1) * chunk)
        out31, info31 = gp.run(hb, Qd[sl].contiguous(), Kd[sl].contiguous(), Vd[sl].contiguous())
        gp.commit()
    gpu_u = G.GpuPass(w, G.to_dev(kp0, "bf16"), G.to_dev(vp0, "bf16"), num_cus=num_cus())
    hbu = gpu_u.compose(budget=L)
    assert hbu.num_tokens == L
    out_u, info_u = gpu_u.run(hbu, Qd, Kd, Vd)
    torch.cuda.synchronize()
    G.say(f"unchunked: records {info_u.num_work}, groups {info_u.num_groups}")
    G.assert_close(G.out_to_f64(out31), G.out_to_f64(out_u[L - chunk:]), "bf16",
                   "chunked pass 31 vs unchunked rows 15872..16383")
    states = harness.oracle_states(w)
    ob, _ = oracle.splitfuse_compose(states, L, oracle.FreeList(w.free_ids), w.block_size,
                                     w.table_width)
    assert G.same_batch(ob, G.batch_of(hbu))
    kp, vp = harness.empty_pools(w)
    oracle.kv_append(kp, vp, K, V, ob, w.block_size)
    assert np.array_equal(G.to_host_bits(gpu_u.cache.k_pool, "bf16"), kp)
    assert np.array_equal(G.to_host_bits(gpu_u.cache.v_pool, "bf16"), vp)
    ref = G.oracle_attention_by_heads(Q, kp, vp, ob, w.num_q_heads, w.num_kv_heads, w.scale,
                                      w.block_size, "bf16")
    G.assert_close(G.out_to_f64(out_u), ref, "bf16", f"unchunked: all {L} rows")
