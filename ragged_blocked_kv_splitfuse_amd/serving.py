"""Multi-pass serving loop: continuous batching over Dynamic SplitFuse passes.

Requests come from closed-loop clients (DeepSpeed-FastGen paper card by Holmes et al. 2024,
"Key points": 1 to 32 concurrent clients, 512 requests; FastGen builds on continuous batching
and a blocked KV cache).  Client c sends requests c, c + C, c + 2C, ... one at a time; a
request with P prompt tokens and O generated tokens caches P + O - 1 positions and is done
after the pass that cached the last of them.  Per pass:

1. ``fg_splitfuse_compose`` fills the token budget (decode tokens first, then prompt tokens in
   arrival order, the last prompt cut to fill it) and allocates blocks;
2. the device work of the pass (``fg_kv_append`` + ``fg_ragged_attention`` through
   ``DevicePass``), or nothing for a host-only run;
3. ``fg_splitfuse_commit``, then ``fg_splitfuse_retire`` returns finished requests' blocks to
   the free list, and their clients send their next requests (joining the end of the list).

Every decision is made by the native library; this module keeps the request queues and
records when each request joined, got its first token and finished (in passes).
"""
from __future__ import annotations

import ctypes
import time
from dataclasses import dataclass, field

import numpy as np

from . import fg


class RunningSet:
    """The fg_seq_state array of the running requests.  Each struct points at its own row
    of block storage; retire moves whole structs, so entries past ``n`` always carry rows no
    live request uses, and a new request reuses the struct at index ``n``."""

    def __init__(self, capacity: int, width: int):
        self.capacity, self.width = int(capacity), int(width)
        self.storage = np.full((max(self.capacity, 1), max(self.width, 1)), -1, np.int32)
        self.arr = (fg.FgSeqState * max(self.capacity, 1))()
        base = self.storage.ctypes.data
        for i in range(self.capacity):
            self.arr[i].blocks = ctypes.cast(base + i * self.storage.strides[0], fg.i32p)
        self.n = 0

    def add(self, seq_id: int, prompt_len: int, stop_len: int, block_size: int):
        if self.n >= self.capacity:
            raise RuntimeError("running set is full")
        need = -(-stop_len // block_size)
        if need > self.width:
            raise ValueError("request needs more blocks than the table width")
        a = self.arr[self.n]
        a.seq_id, a.n_cached, a.prompt_len = int(seq_id), 0, int(prompt_len)
        a.n_blocks, a.max_blocks, a.n_scheduled, a.stop_len = 0, need, 0, int(stop_len)
        self.n += 1


@dataclass
class ServingStats:
    tokens: list = field(default_factory=list)            # T of every pass
    seqs: list = field(default_factory=list)              # S of every pass
    first_token_pass: dict = field(default_factory=dict)
    finish_pass: dict = field(default_factory=dict)
    admit_pass: dict = field(default_factory=dict)
    free_after: list = field(default_factory=list)
    batches: list = None                                  # host batch copies, if kept
    wall_s: float = 0.0

    @property
    def passes(self) -> int:
        return len(self.tokens)


class ServingLoop:
    def __init__(self, handle, block_size: int, budget: int, clients: int, table_width: int):
        self.handle = handle
        self.block_size, self.budget = int(block_size), int(budget)
        self.clients = int(clients)
        self.width = int(table_width)
        self.running = RunningSet(self.clients, self.width)
        self.batch = fg.HostBatch(self.clients, self.width)

    def run(self, requests, device_pass=None, keep_batches: bool = False,
            max_passes: int = 1_000_000) -> ServingStats:
        """Serve every request; ``device_pass(batch, running)`` runs a pass's device work."""
        C = self.clients
        queues = [list(range(c, len(requests), C)) for c in range(C)]
        client_of = {}
        st = ServingStats(batches=[] if keep_batches else None)
        rs, hb = self.running, self.batch

        def admit(c, p):
            if queues[c]:
                r = requests[queues[c].pop(0)]
                if r.prompt_len < 1 or r.output_len < 1:
                    raise ValueError("a request needs a prompt token and a generated token")
                rs.add(r.rid, r.prompt_len, r.prompt_len + r.output_len - 1, self.block_size)
                client_of[r.rid] = c
                st.admit_pass[r.rid] = p

        t0 = time.perf_counter()
        for c in range(C):
            admit(c, 0)
        p = 0
        while rs.n:
            if p >= max_passes:
                raise RuntimeError("pass limit reached")
            s = fg._check(fg.lib().fg_splitfuse_compose(self.handle, rs.arr, rs.n, self.budget,
                                                        ctypes.byref(hb.c)),
                          ok=(fg.FG_OK, fg.FG_E_NO_BLOCKS))
            if s != fg.FG_OK:
                raise RuntimeError("the pool cannot take a single token")
            st.tokens.append(hb.num_tokens)
            st.seqs.append(hb.num_seqs)
            if keep_batches:
                S = hb.num_seqs
                st.batches.append((hb.query_start[:S + 1].copy(), hb.n_query[:S].copy(),
                                   hb.context_len[:S].copy(), hb.block_table[:S].copy(),
                                   hb.seq_id[:S].copy()))
            if device_pass is not None:
                device_pass(hb, rs)
            fg._check(fg.lib().fg_splitfuse_commit(rs.arr, rs.n))
            for i in range(rs.n):
                a = rs.arr[i]
                if a.n_cached >= a.prompt_len and a.seq_id not in st.first_token_pass:
                    st.first_token_pass[a.seq_id] = p
            n_before = rs.n
            rs.n = fg.fg_splitfuse_retire(self.handle, rs.arr, n_before)
            retired = [int(rs.arr[i].seq_id) for i in range(rs.n, n_before)]
            for rid in retired:
                st.finish_pass[rid] = p
            for rid in retired:
                admit(client_of[rid], p + 1)
            st.free_after.append(fg.fg_blocked_cache_num_free(self.handle))
            p += 1
        st.wall_s = time.perf_counter() - t0
        return st


def request_latencies(stats: ServingStats, requests, pass_end_s):
    """Per-request latencies of a served stream on a timeline of pass end times.

    The effective-throughput view of serving (DeepSpeed-FastGen paper card by Holmes et al.
    2024, "Interesting ideas": throughput that counts only requests served within a
    first-token time and a steady token pace).  ``pass_end_s[p]`` is the time at which pass
    p ends, on any clock whose zero is the start of pass 0.  A request joins when the pass
    before its admission pass ends (time 0 for pass 0); its first token arrives when its
    first-token pass ends; its later tokens arrive one per pass until its finish pass.
    Returns two float64 arrays in ``requests`` order:

    * ttft: first-token pass end - join time;
    * pace: (finish pass end - first-token pass end) / (output_len - 1), the mean gap between
      generated tokens; NaN for a request with a single generated token (it has no gap).
    """
    ends = np.asarray(pass_end_s, dtype=np.float64)
    n = len(requests)
    ttft, pace = np.empty(n), np.empty(n)
    for k, r in enumerate(requests):
        a = stats.admit_pass[r.rid]
        f, e = stats.first_token_pass[r.rid], stats.finish_pass[r.rid]
        join = 0.0 if a == 0 else ends[a - 1]
        ttft[k] = ends[f] - join
        pace[k] = (ends[e] - ends[f]) / (r.output_len - 1) if r.output_len > 1 else np.nan
    return ttft, pace


def sla_attainment(ttft, pace, ttft_max: float, pace_max: float) -> float:
    """Share of requests whose first token came within ttft_max and whose token pace is within
    pace_max (a request with one generated token has no pace and meets any pace bound)."""
    ttft, pace = np.asarray(ttft), np.asarray(pace)
    if ttft.size == 0:
        return float("nan")
    ok = (ttft <= ttft_max) & (np.isnan(pace) | (pace <= pace_max))
    return float(ok.mean())


def latency_summary(ttft, pace, ttft_grid=(0.5, 1.0, 2.0), pace_grid=(0.025, 0.05, 0.1)) -> dict:
    """Mean and percentiles of TTFT and token pace (milliseconds), and SLA attainment on a grid
    of thresholds (seconds; the pages give no thresholds, so a grid is reported)."""
    ttft, pace = np.asarray(ttft), np.asarray(pace)
    pc = pace[~np.isnan(pace)]
    out = {"ttft_ms_mean": float(ttft.mean() * 1e3),
           "ttft_ms_p50": float(np.percentile(ttft, 50) * 1e3),
           "ttft_ms_p95": float(np.percentile(ttft, 95) * 1e3),
           "token_pace_ms_mean": float(pc.mean() * 1e3) if pc.size else float("nan"),
           "token_pace_ms_p95": float(np.percentile(pc, 95) * 1e3) if pc.size else float("nan")}
    out["sla_attainment"] = {f"ttft<={a}s,pace<={b}s": sla_attainment(ttft, pace, a, b)
                             for a in ttft_grid for b in pace_grid}
    return out


class Projections:
    """The dense projections of one attention layer: Q, K and V from the pass's hidden rows
    x [T][hidden] in one fused product over the stacked weights (``fg_linear_qkv_bf16``, each
    result landing in the dense layout the pass reads), and the output projection of
    attention's rows (``fg_linear_bf16``)."""

    def __init__(self, wq, wk, wv, wo, budget: int, stream=None):
        import torch
        self.wq, self.wk, self.wv, self.wo = wq, wk, wv, wo
        self.w_qkv = torch.cat((wq, wk, wv), dim=0).contiguous()
        self.hidden = int(wq.shape[1])
        self.stream = stream
        dev, dt = wq.device, wq.dtype
        mk = lambda n: torch.empty((max(int(budget), 1), int(n)), dtype=dt, device=dev)
        self.q, self.k, self.v = mk(wq.shape[0]), mk(wk.shape[0]), mk(wv.shape[0])
        self.y = mk(wo.shape[0])

    def _lin(self, x, w, y, T):
        from .runtime import stream_handle
        fg.fg_linear_bf16(x.data_ptr(), w.data_ptr(), y.data_ptr(), T, int(w.shape[1]),
                          int(w.shape[0]), stream_handle(self.stream))

    def qkv(self, x, T):
        from .runtime import stream_handle
        fg.fg_linear_qkv_bf16(x.data_ptr(), self.w_qkv.data_ptr(), self.q.data_ptr(),
                              self.k.data_ptr(), self.v.data_ptr(), T, self.hidden,
                              int(self.wq.shape[0]), int(self.wk.shape[0]),
                              stream_handle(self.stream))
        return self.q[:T], self.k[:T], self.v[:T]

    def output(self, o, T):
        self._lin(o, self.wo, self.y, T)
        return self.y[:T]

    def flops(self, T) -> int:
        return 2 * T * self.hidden * sum(int(w.shape[0]) for w in (self.wq, self.wk, self.wv)) \
            + 2 * T * int(self.wo.shape[1]) * int(self.wo.shape[0])


class DevicePass:
    """Device work of one serving pass: plan, descriptor upload, kv_append, attention.

    ``cache``: an object with ``handle`` (the library's cache handle) and ``head_dim``;
    ``rows(batch, running)`` returns the pass's (q, k_new, v_new) device tensors in batch
    order -- or, with ``proj`` (a ``Projections``), its hidden rows x, from which the pass
    computes q, k and v, and after attention the output projection.  ``check(p, batch, out)``
    (optional) sees every pass's attention output.  With ``timing``, five events per pass are
    kept in ``marks``: before the QKV projection, before kv_append, before attention, after
    attention, after the output projection (without ``proj`` the first two and the last two
    coincide)."""

    def __init__(self, cache, num_q_heads: int, scale: float, rows, num_cus: int,
                 check=None, stream=None, timing: bool = False, proj=None):
        from .runtime import DeviceDescriptors, Workspace
        self.cache, self.hq, self.scale = cache, int(num_q_heads), float(scale)
        self.rows, self.check, self.num_cus = rows, check, int(num_cus)
        self.desc, self.ws = DeviceDescriptors(), Workspace()
        self.work = np.zeros(1 << 16, np.int32)
        self.stream = stream
        self.p = 0
        self.out = None
        self.timing, self.marks = bool(timing), []
        self.proj = proj
        self.events, self.ev_next = [], 0  # timing events created ahead (reserve_events)

    def reserve_events(self, n_passes: int):
        """Create the timing events of n_passes passes now, so that creating them does not
        count in the host time of the passes that record them."""
        import torch
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(5 * int(n_passes))]
        self.ev_next = 0

    def __call__(self, hb, running):
        import torch
        from .runtime import stream_handle
        info, work = fg.fg_attention_plan(self.cache.handle, hb, self.hq, self.num_cus,
                                          self.work)
        if work is not None and work.size > self.work.size:
            self.work = np.zeros(2 * work.size, np.int32)
        c = self.desc.upload(hb, work if info.num_work else None, self.stream)
        T = hb.num_tokens
        s = stream_handle(self.stream)
        ev = None
        if self.timing:
            st = self.stream or torch.cuda.current_stream()
            if self.ev_next + 5 <= len(self.events):
                ev = self.events[self.ev_next:self.ev_next + 5]
                self.ev_next += 5
            else:
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            ev[0].record(st)
        if self.proj is not None:
            x = self.rows(hb, running)
            q, kn, vn = self.proj.qkv(x, T)
        else:
            q, kn, vn = self.rows(hb, running)
        if ev:
            ev[1].record(st)
        fg.fg_kv_append(self.cache.handle, c, kn.data_ptr(), vn.data_ptr(), s)
        if ev:
            ev[2].record(st)
        if self.out is None or self.out.shape[0] < T:
            self.out = torch.empty((max(T, 1), self.hq, self.cache.head_dim), dtype=q.dtype,
                                   device=q.device)
        out = self.out[:T]
        wp, wb = self.ws.ensure(info.workspace_bytes)
        fg.fg_ragged_attention(self.cache.handle, c, info, self.desc.work_ptr, q.data_ptr(),
                               self.hq, self.scale, out.data_ptr(), wp, wb, s)
        if ev:
            ev[3].record(st)
        if self.proj is not None:
            self.proj.output(out.view(T, -1), T)
        if ev:
            ev[4].record(st)
            self.marks.append(ev)
        if self.check is not None:
            self.check(self.p, hb, out)
        self.p += 1
