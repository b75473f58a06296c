"""Multi-pass serving loop (continuous batching over SplitFuse passes), host side.

The oracle's loop is pinned to a hand-derived trace (tests/golden/serving_hand.json) and to
properties the pages fix: every pass at the token budget while demand allows, each request's
positions processed once and in order, one token per decoding request per pass (so a request
finishes exactly O - 1 passes after its first token), blocks conserved and disjoint.  The
library's loop (native compose / commit / retire) must then reproduce the oracle's trace
exactly.
"""
import json
import os

import numpy as np
import pytest

from oracle.serving import serve
from ragged_blocked_kv_splitfuse_amd import fg
from ragged_blocked_kv_splitfuse_amd import workloads as W
from ragged_blocked_kv_splitfuse_amd.serving import ServingLoop

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "serving_hand.json")


def load_hand():
    g = json.load(open(GOLDEN))
    reqs = [W.Request(r["rid"], r["prompt_len"], r["output_len"]) for r in g["requests"]]
    return g, reqs


def oracle_trace(sw):
    v = sw.values
    return serve(sw.requests, sw.clients, sw.budget, v.free_ids, v.block_size, sw.table_width)


def native_trace(sw, keep=True):
    v = sw.values
    h = fg.fg_blocked_cache_init(v.num_blocks, v.block_size, v.num_kv_heads, v.head_dim, v.dtype,
                                 0, 0, v.free_ids)
    try:
        loop = ServingLoop(h, v.block_size, sw.budget, sw.clients, sw.table_width)
        return loop.run(sw.requests, keep_batches=keep)
    finally:
        fg.fg_blocked_cache_destroy(h)


def test_oracle_hand_trace():
    g, reqs = load_hand()
    t = serve(reqs, g["clients"], g["budget"], g["free_ids"], g["block_size"], g["table_width"])
    assert len(t.batches) == len(g["passes"])
    for b, e in zip(t.batches, g["passes"]):
        for f in ("query_start", "n_query", "context_len", "block_table", "seq_id"):
            assert np.array_equal(getattr(b, f), np.array(e[f])), f
    for k in ("first_token_pass", "finish_pass", "admit_pass"):
        assert getattr(t, k) == {int(a): b for a, b in g[k].items()}, k
    assert t.free_after == g["free_after"]


def check_stream_properties(sw, t):
    """Properties of any trace of the loop (oracle or library)."""
    v = sw.values
    reqs = {r.rid: r for r in sw.requests}
    pos = {r.rid: 0 for r in sw.requests}
    total = 0
    for p, b in enumerate(t.batches):
        T = int(b.query_start[-1])
        total += T
        running = [rid for rid in reqs if t.admit_pass[rid] <= p and
                   (rid not in t.finish_pass or t.finish_pass[rid] >= p)]
        decoding = [rid for rid in running if pos[rid] >= reqs[rid].prompt_len]
        prompt_left = sum(reqs[rid].prompt_len - pos[rid] for rid in running
                          if pos[rid] < reqs[rid].prompt_len)
        demand = len(decoding) + prompt_left
        # the budget is filled exactly while demand allows, and never padded
        assert T == min(sw.budget, demand), (p, T, demand)
        seen = set()
        for k, rid in enumerate(b.seq_id.tolist()):
            c, n = int(b.context_len[k]), int(b.n_query[k])
            assert c == pos[rid], "positions processed in order, none twice or skipped"
            pos[rid] = c + n
            ids = b.block_table[k][:-(-(c + n) // v.block_size)].tolist()
            assert not seen & set(ids), "blocks of two running requests overlap"
            seen |= set(ids)
        # every decoding request gets exactly one token (clients <= budget)
        for rid in decoding:
            k = b.seq_id.tolist().index(rid)
            assert b.n_query[k] == 1
    assert total == sum(r.stop_len for r in sw.requests)
    for r in sw.requests:
        assert pos[r.rid] == r.stop_len
        # one generated token per pass after the first
        assert t.finish_pass[r.rid] - t.first_token_pass[r.rid] == r.output_len - 1
    for c in range(sw.clients):
        mine = [sw.requests[k].rid for k in range(c, len(sw.requests), sw.clients)]
        for a, b in zip(mine, mine[1:]):
            assert t.admit_pass[b] == t.finish_pass[a] + 1
    assert t.free_after[-1] == v.num_blocks


def test_oracle_properties_small():
    sw = W.serving_small()
    check_stream_properties(sw, oracle_trace(sw))


def test_oracle_properties_512_requests():
    sw = W.serving_stream(n_requests=512, clients=32)
    check_stream_properties(sw, oracle_trace(sw))


@pytest.mark.parametrize("clients", [1, 4, 32])
def test_oracle_properties_client_counts(clients):
    sw = W.serving_stream(seed=11, n_requests=48, clients=clients, budget=512)
    check_stream_properties(sw, oracle_trace(sw))


class _Tr:
    """Library trace in the oracle's shape."""

    def __init__(self, st):
        from oracle.compose import OracleBatch
        self.batches = [OracleBatch(qs, nq, cl, bt, np.zeros(len(nq), np.int32), sid)
                        for qs, nq, cl, bt, sid in st.batches]
        self.first_token_pass, self.finish_pass = st.first_token_pass, st.finish_pass
        self.admit_pass, self.free_after = st.admit_pass, st.free_after


def same_trace(a, b):
    assert len(a.batches) == len(b.batches)
    for x, y in zip(a.batches, b.batches):
        for f in ("query_start", "n_query", "context_len", "seq_id"):
            assert np.array_equal(getattr(x, f), getattr(y, f)), f
        w = min(x.block_table.shape[1], y.block_table.shape[1])
        assert np.array_equal(x.block_table[:, :w], y.block_table[:, :w])
        assert (x.block_table[:, w:] == -1).all() and (y.block_table[:, w:] == -1).all()
    for k in ("first_token_pass", "finish_pass", "admit_pass", "free_after"):
        assert getattr(a, k) == getattr(b, k), k


def test_library_hand_trace():
    g, reqs = load_hand()
    h = fg.fg_blocked_cache_init(len(g["free_ids"]), g["block_size"], 1, 128, "bf16", 0, 0,
                                 np.array(g["free_ids"], np.int32))
    try:
        st = ServingLoop(h, g["block_size"], g["budget"], g["clients"], g["table_width"]).run(
            reqs, keep_batches=True)
    finally:
        fg.fg_blocked_cache_destroy(h)
    t = serve(reqs, g["clients"], g["budget"], g["free_ids"], g["block_size"], g["table_width"])
    same_trace(_Tr(st), t)


@pytest.mark.parametrize("make", [
    lambda: W.serving_small(),
    lambda: W.serving_stream(seed=12, n_requests=64, clients=8, budget=256),
    lambda: W.serving_stream(n_requests=512, clients=32),
])
def test_library_loop_matches_oracle(make):
    sw = make()
    same_trace(_Tr(native_trace(sw)), oracle_trace(sw))


def test_retire_partitions_and_releases_in_order():
    # three sequences owning blocks [0, 1], [2, 3], [4]; the pool's free list holds the rest
    h = fg.fg_blocked_cache_init(8, 2, 1, 128, "bf16", 0, 0, np.array([5, 6, 7], np.int32))
    try:
        arr = (fg.FgSeqState * 3)()
        store = np.full((3, 4), -1, np.int32)
        spec = [(1, 4, 4, [0, 1]), (2, 3, 5, [2, 3]), (3, 2, 2, [4])]   # id, cached, stop, blocks
        for i, (sid, c, stop, bl) in enumerate(spec):
            store[i, :len(bl)] = bl
            a = arr[i]
            a.seq_id, a.n_cached, a.prompt_len, a.n_blocks, a.max_blocks = sid, c, 1, len(bl), 4
            a.blocks = fg.ctypes.cast(store.ctypes.data + i * store.strides[0], fg.i32p)
            a.stop_len = stop
        n_live = fg.fg_splitfuse_retire(h, arr, 3)
        assert n_live == 1
        assert [arr[i].seq_id for i in range(3)] == [2, 1, 3]
        assert [arr[i].n_blocks for i in range(3)] == [2, 0, 0]
        # released: seq 1's [0, 1] then seq 3's [4]; the last released is handed out first
        assert fg.fg_blocked_cache_free_ids(h).tolist() == [4, 1, 0, 5, 6, 7]
        # a second retire finds nothing more to do
        assert fg.fg_splitfuse_retire(h, arr, 1) == 1
        # a done sequence whose block is already free: error, nothing changes
        arr[0].n_cached = 5
        arr[0].blocks[0] = 4
        with pytest.raises(fg.FgError):
            fg.fg_splitfuse_retire(h, arr, 1)
        assert arr[0].n_blocks == 2
        assert fg.fg_blocked_cache_free_ids(h).tolist() == [4, 1, 0, 5, 6, 7]
    finally:
        fg.fg_blocked_cache_destroy(h)


def test_retire_rejects_null_arguments():
    h = fg.fg_blocked_cache_init(4, 2, 1, 128, "bf16", 0, 0, None)
    try:
        n = fg.ctypes.c_int32(0)
        assert fg.lib().fg_splitfuse_retire(None, None, 0, fg.ctypes.byref(n)) == fg.FG_E_ARG
        assert fg.lib().fg_splitfuse_retire(h, None, 2, fg.ctypes.byref(n)) == fg.FG_E_ARG
        assert fg.lib().fg_splitfuse_retire(h, None, 0, None) == fg.FG_E_ARG
        assert fg.lib().fg_splitfuse_retire(h, None, 0, fg.ctypes.byref(n)) == fg.FG_OK
        assert n.value == 0
    finally:
        fg.fg_blocked_cache_destroy(h)


LATENCY_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "serving_latency_hand.json")


def test_latency_proxy_hand_timeline():
    """The effective-throughput proxy (TTFT, token pace, SLA attainment) on the hand trace with
    given pass times, against values worked out by hand."""
    from ragged_blocked_kv_splitfuse_amd.serving import (latency_summary, request_latencies,
                                                         sla_attainment)
    g, reqs = load_hand()
    lat = json.load(open(LATENCY_GOLDEN))
    h = fg.fg_blocked_cache_init(len(g["free_ids"]), g["block_size"], 1, 128, "bf16", 0, 0,
                                 np.array(g["free_ids"], np.int32))
    try:
        st = ServingLoop(h, g["block_size"], g["budget"], g["clients"], g["table_width"]).run(reqs)
    finally:
        fg.fg_blocked_cache_destroy(h)
    assert st.passes == len(lat["pass_ms"])
    ends = np.cumsum(np.array(lat["pass_ms"]) * 1e-3)
    assert np.allclose(ends * 1e3, lat["pass_end_ms"])
    ttft, pace = request_latencies(st, reqs, ends)
    for k, r in enumerate(reqs):
        assert ttft[k] * 1e3 == pytest.approx(lat["ttft_ms"][str(r.rid)], abs=1e-9)
        want = lat["pace_ms"][str(r.rid)]
        if want is None:
            assert np.isnan(pace[k])
        else:
            assert pace[k] * 1e3 == pytest.approx(want, abs=1e-9)
    for case in lat["sla"]:
        got = sla_attainment(ttft, pace, case["ttft_ms"] * 1e-3, case["pace_ms"] * 1e-3)
        assert got == pytest.approx(case["attainment"]), case
    s = latency_summary(ttft, pace, ttft_grid=(0.015,), pace_grid=(0.0045,))
    assert s["ttft_ms_mean"] == pytest.approx(9.0)
    assert s["token_pace_ms_mean"] == pytest.approx(3.75)
    assert s["sla_attainment"] == {"ttft<=0.015s,pace<=0.0045s": pytest.approx(1.0)}


def test_latency_proxy_single_pass_requests():
    """Requests served in the pass that admitted them, with one generated token: TTFT is
    exactly that pass's duration and there is no pace."""
    from ragged_blocked_kv_splitfuse_amd.serving import request_latencies, ServingStats
    reqs = [W.Request(1, 3, 1), W.Request(2, 2, 1)]
    st = ServingStats(admit_pass={1: 0, 2: 1}, first_token_pass={1: 0, 2: 1},
                      finish_pass={1: 0, 2: 1})
    ttft, pace = request_latencies(st, reqs, [0.25, 0.75])
    assert ttft.tolist() == [0.25, 0.5]
    assert np.isnan(pace).all()
