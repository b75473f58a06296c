"""fg_ragged_attention_noalloc (split partials in the library's fixed device scratch instead
of a caller workspace) against fg_ragged_attention on the same inputs: bit-identical outputs
on two calls in a row, the second with a smaller pass, both with split groups so that the
scratch is really used; the first also against the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import gpu_harness as G
from ragged_blocked_kv_splitfuse_amd import fg, workloads as wl
from ragged_blocked_kv_splitfuse_amd.runtime import stream_handle


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(w, check_oracle):
    G.say(f"no-alloc: {w.name} hq {w.num_q_heads} hkv {w.num_kv_heads} d {w.head_dim}")
    r = G.full_pass(w, num_cus=100000)                # finest splits: partials in the scratch
    gp, hb, info = r["gp"], r["hb"], r["info"]
    assert info.num_groups > 0 and 0 < info.workspace_bytes <= fg.FG_NOALLOC_WORKSPACE_BYTES
    if check_oracle:
        G.assert_close(G.out_to_f64(r["out"]), r["ref"], "bf16", "fg_ragged_attention")
    # the same plan and descriptors again (the pool already holds the appended rows)
    info2, work = fg.fg_attention_plan(gp.cache.handle, hb, w.num_q_heads, 100000)
    c = gp.desc.upload(hb, work)
    q = G.to_dev(r["q"], "bf16")
    T = hb.num_tokens
    ref = torch.empty((T, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    wp, wb = gp.ws.ensure(info2.workspace_bytes)
    fg.fg_ragged_attention(gp.cache.handle, c, info2, gp.desc.work_ptr, q.data_ptr(),
                           w.num_q_heads, w.scale, ref.data_ptr(), wp, wb, stream_handle())
    out = torch.full((T, w.num_q_heads, w.head_dim), 5, dtype=torch.int16,
                     device="cuda").view(torch.bfloat16)
    fg.fg_ragged_attention_noalloc(gp.cache.handle, c, info2, gp.desc.work_ptr, q.data_ptr(),
                                   w.num_q_heads, w.scale, out.data_ptr(), stream_handle())
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "outputs differ"
    G.assert_close(G.out_to_f64(out), r["ref"], "bf16", "fg_ragged_attention_noalloc")
    return info2.workspace_bytes


def test_noalloc_matches_workspace_call_twice():
    big = wl.custom(9101, hq=32, hkv=8, bs=64, budget=700, n_decode=10, decode_ctx=(200, 2500),
                    prompts=((600, 2000), (0, 300)))
    small = wl.custom(9102, hq=8, hkv=2, d=64, bs=16, budget=150, n_decode=3,
                      decode_ctx=(1100, 1600), prompts=((700, 900),))
    b1 = _both(big, True)
    b2 = _both(small, True)
    assert b2 < b1
