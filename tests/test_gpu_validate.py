"""Validation mode (FG_VALIDATE=1) of the device entry points: valid passes run unchanged; a
corrupted device descriptor or work list is rejected with FG_E_DESC before anything is
launched (the pools stay bit-for-bit as they were, the output untouched)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import gpu_harness as G
import oracle
from ragged_blocked_kv_splitfuse_amd import fg, workloads as wl
from ragged_blocked_kv_splitfuse_amd.runtime import stream_handle


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _workload():
    return wl.custom(4242, hq=16, hkv=4, bs=16, budget=300, n_decode=3, decode_ctx=(50, 700),
                     prompts=((100, 600), (0, 200)))


def test_valid_pass_under_validation(monkeypatch):
    monkeypatch.setenv("FG_VALIDATE", "1")
    w = _workload()
    r = G.full_pass(w, num_cus=100000)          # split groups too
    dt = np.uint16
    assert np.array_equal(G.to_host_bits(r["gp"].cache.k_pool, "bf16").view(dt), r["k_pool"].view(dt))
    assert np.array_equal(G.to_host_bits(r["gp"].cache.v_pool, "bf16").view(dt), r["v_pool"].view(dt))
    G.assert_close(G.out_to_f64(r["out"]), r["ref"], "bf16", "validated pass")


def _status(fn, *a):
    try:
        fn(*a)
        return fg.FG_OK
    except fg.FgError as e:
        return e.status


def test_corrupted_descriptors_rejected(monkeypatch):
    monkeypatch.setenv("FG_VALIDATE", "1")
    w = _workload()
    kp0, vp0 = (torch.full(s, 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
                for s in (oracle.k_pool_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size),
                          oracle.v_pool_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size)))
    gp = G.GpuPass(w, kp0, vp0, num_cus=100000)
    hb = gp.compose()
    info, work = fg.fg_attention_plan(gp.cache.handle, hb, w.num_q_heads, gp.num_cus)
    T = hb.num_tokens
    q = torch.randn((T, w.num_q_heads, w.head_dim), device="cuda").to(torch.bfloat16)
    kn = torch.randn((T, w.num_kv_heads, w.head_dim), device="cuda").to(torch.bfloat16)
    vn = torch.randn_like(kn)
    out = torch.full((T, w.num_q_heads, w.head_dim), 3, dtype=torch.int16, device="cuda")
    wp, wb = gp.ws.ensure(info.workspace_bytes)
    s = stream_handle()
    k_before, v_before = kp0.clone(), vp0.clone()

    def attention(c):
        return _status(fg.fg_ragged_attention, gp.cache.handle, c, info, gp.desc.work_ptr,
                       q.data_ptr(), w.num_q_heads, w.scale, out.data_ptr(), wp, wb, s)

    cases = {
        "block id out of range": lambda bt, wk: bt.__setitem__((0, 0), w.num_blocks),
        "block shared by two sequences": lambda bt, wk: bt.__setitem__((1, 0), bt[0, 0]),
        "missing block": lambda bt, wk: bt.__setitem__((hb.num_seqs - 1, 0), -1),
    }
    for name, mut in cases.items():
        bt = hb.block_table.copy()
        mut(hb.block_table, None)
        c = gp.desc.upload(hb, work)
        hb.block_table[:] = bt
        assert _status(fg.fg_kv_append, gp.cache.handle, c, kn.data_ptr(), vn.data_ptr(), s) \
            == fg.FG_E_DESC, name
        assert attention(c) == fg.FG_E_DESC, name
        G.say(f"{name}: rejected ({fg.fg_last_error()})")
    # a corrupted work list with valid descriptors: attention rejects it, append runs
    bad = work.copy()
    ni = info.num_items * fg.FG_ITEM_INTS
    bad[ni] = info.num_items * w.num_kv_heads          # record code out of range
    c = gp.desc.upload(hb, bad)
    assert attention(c) == fg.FG_E_DESC
    G.say(f"work list: rejected ({fg.fg_last_error()})")
    torch.cuda.synchronize()
    assert torch.equal(kp0.view(torch.int16), k_before.view(torch.int16))
    assert torch.equal(vp0.view(torch.int16), v_before.view(torch.int16))
    assert bool((out == 3).all())
    # the same pass, valid: append and attention run
    c = gp.desc.upload(hb, work)
    assert _status(fg.fg_kv_append, gp.cache.handle, c, kn.data_ptr(), vn.data_ptr(), s) == fg.FG_OK
    assert attention(c) == fg.FG_OK
    torch.cuda.synchronize()
    assert not torch.equal(kp0.view(torch.int16), k_before.view(torch.int16))
