#!/usr/bin/env python3
"""Fixed-budget ragged pass on one MI355X: tokens/s of the whole hot path.

One step = one pass of the method over one synthetic batch: Dynamic SplitFuse composition
and block allocation (host, C++), upload of the ragged descriptors and work list, kv_append
(HIP) and ragged blocked attention (HIP), all through the C ABI.  Inputs are resident in
HBM before timing starts; every step recomposes the same pass from the same starting state,
so the K timed steps repeat identical work.

Default workload: LLaMA-2-7B attention shape (32 heads of 128, blocks of 64), a 2048-token
budget filled by 24 decode tokens plus prompt chunks.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama2|decode|chunked|mistral]

`--workload serving` instead runs the multi-pass serving loop (continuous batching over
SplitFuse passes) on the whole request stream -- 512 requests from `--clients` closed-loop
clients, prompt and output lengths normal with means 2600 and 60 -- once untimed and once
timed, and reports the run's tokens/s plus per-request latencies in passes and seconds.

    python bench.py --workload serving [--clients 32] [--requests 512] [--budget 2048]

`--workload sweep` times the pass over shape sweeps (sequence count at a fixed token count;
token budget for one prompt chunk and for decode tokens) and prints one JSON line with every
point.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ragged-pass tokens/s at fixed budget; KV HBM GB/s & MFMA % of peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
F32_VALU_PEAK_TFLOPS = 157.3
WORKLOADS = {"llama2": 2, "decode": 3, "chunked": 4, "mistral": 5, "serving": 0, "sweep": 0}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_traffic.json")


def kernel_source_hash():
    """Hash of the sources that decide the kernels' work: the device code, the shared internal
    header, the planner and the public header (item row sizes)."""
    h = hashlib.sha256()
    for f in (("ragged_blocked_kv_splitfuse_amd", "csrc", "fg_kernels.hip"),
              ("ragged_blocked_kv_splitfuse_amd", "csrc", "fg_internal.h"),
              ("ragged_blocked_kv_splitfuse_amd", "csrc", "fg_host.cpp"),
              ("include", "fg.h")):
        with open(os.path.join(ROOT, *f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama2", choices=sorted(WORKLOADS))
    ap.add_argument("--chunk-pass", type=int, default=31,
                    help="chunked workload: which 512-token pass (0..31) a step runs")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample (0 = skip)")
    ap.add_argument("--per-config", type=int, default=1,
                    help="also time the decode-only, chunked (pass --chunk-pass) and Mistral "
                         "passes and report them in a per_config block (0 = headline only)")
    ap.add_argument("--per-config-steps", type=int, default=20,
                    help="timed steps of each per_config pass")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--num-cus", type=int, default=0,
                    help="compute units the attention planner sizes splits for (0 = device's)")
    ap.add_argument("--clients", type=int, default=32, help="serving: closed-loop clients")
    ap.add_argument("--requests", type=int, default=512, help="serving: requests in the stream")
    ap.add_argument("--budget", type=int, default=2048, help="serving: token budget per pass")
    ap.add_argument("--model", default="llama2", choices=["llama2", "mistral"],
                    help="serving: attention shape (LLaMA-2-7B 32/32 or Mistral-7B 32/8 heads)")
    ap.add_argument("--layer", action="store_true",
                    help="serving: each pass also runs the QKV and output projections")
    ap.add_argument("--layers", type=int, default=32,
                    help="serving: layer count of the latency proxy (pass time x layers)")
    return ap.parse_args()


def setup(args, workload=None):
    import numpy as np
    import torch
    from ragged_blocked_kv_splitfuse_amd import fg, workloads as wl
    from ragged_blocked_kv_splitfuse_amd.runtime import PagedKVCache, num_cus

    cfg = WORKLOADS[workload or args.workload]
    w = wl.make(cfg, args.seed)
    init_states = w.fresh_states()
    free_ids = np.asarray(w.free_ids, np.int32)
    if cfg == 4:
        # pass k of the chunked prompt: the first 512k positions are already cached
        k = args.chunk_pass
        c = 512 * k
        nb = -(-c // w.block_size)
        order = np.asarray(w.free_ids, np.int32)
        init_states[0].n_cached = c
        init_states[0].blocks = order[:nb].tolist()
        free_ids = order[nb:]
    return prepare(w, init_states, free_ids, args.num_cus or num_cus())


def prepare(w, init_states, free_ids, cus):
    """Pools on the device (filled with seeded values), sequence states and a host batch."""
    import torch
    from ragged_blocked_kv_splitfuse_amd import fg, workloads as wl
    from ragged_blocked_kv_splitfuse_amd.runtime import PagedKVCache
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    cache = PagedKVCache(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype,
                         free_ids=free_ids)
    wl.fill_pools_device(cache.k_pool, cache.v_pool, seed=w.seed * 7919 + 1,
                         value_scale=w.value_scale)
    ss = fg.SeqStates(init_states, w.table_width)
    template = (bytes(ss.arr), ss.blocks.copy())
    hb = fg.HostBatch(ss.n, w.table_width)
    return dict(w=w, cache=cache, ss=ss, template=template, hb=hb, free_ids=free_ids,
                cus=cus, tdt=tdt)


# The profiling sweeps: (S, n, c) = sequences, new tokens each, cached tokens each.
SWEEP_S = [(S, 2048 // S, 1024) for S in (1, 4, 16, 64, 256, 1024, 2048)]
SWEEP_T_CHUNK = [(1, T, 2048) for T in (64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384)]
SWEEP_T_DECODE = [(T, 1, 1024) for T in (16, 64, 256, 1024, 2048)]


def sweep_main(args):
    """Latency and throughput of the pass (kv_append + attention) over the three shape
    families: sequence count at a fixed 2048-token pass, then the token budget for one
    prompt chunk and for decode tokens.  One JSON line holding every point."""
    import numpy as np
    import torch
    from ragged_blocked_kv_splitfuse_amd import workloads as wl
    from ragged_blocked_kv_splitfuse_amd.runtime import num_cus
    cus = args.num_cus or num_cus()
    points = []
    for family, pts in (("seqs_at_T2048", SWEEP_S), ("budget_one_chunk", SWEEP_T_CHUNK),
                        ("budget_decodes", SWEEP_T_DECODE)):
        for S_, n, c in pts:
            w = wl.uniform_pass(S_, n, c)
            P = prepare(w, w.fresh_states(), np.asarray(w.free_ids, np.int32), cus)
            r = time_pass(P, args.steps, args.warmup)
            t = r["t_attn"] + r["t_app"]
            points.append({"family": family, "S": S_, "n": n, "c": c, "T": r["T"],
                           "attention_us": r["t_attn"] * 1e6, "kv_append_us": r["t_app"] * 1e6,
                           "pass_us": t * 1e6, "tokens_per_s": r["T"] / t,
                           "step_us": r["elapsed"] / args.steps * 1e6,
                           "attn_flops": r["attn_flops"], "attn_bytes": r["attn_bytes"],
                           "mfma_frac": r["attn_flops"] / r["t_attn"] / 1e12 / BF16_PEAK_TFLOPS,
                           "hbm_frac": r["attn_bytes"] / r["t_attn"] / 1e9 / HBM_PEAK_GBS})
            print(json.dumps({"point": points[-1]}), file=sys.stderr, flush=True)
            del P, r
            torch.cuda.empty_cache()
    print(json.dumps({"metric": "pass latency and tokens/s over shape sweeps", "unit": "us",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "dtype": "bf16",
                      "data": "synthetic",
                      "config": {"workload": "uniform passes, LLaMA-2-7B attention shape",
                                 "q_heads": 32, "kv_heads": 32, "head_dim": 128,
                                 "block_size": 64},
                      "points": points}), flush=True)


def time_pass(S, steps, warmup):
    """Warm up, then time `steps` identical passes (compose + plan + upload + kv_append +
    attention) of the prepared workload.  `elapsed` is the host clock over the timed steps,
    bracketed by synchronizations.  The attention time comes from HIP events around its launch
    in every fourth timed step (and the last); the kv_append time from events around its launch
    in up to 20 further steps after the timed region (the launch stream for both)."""
    import numpy as np
    import torch
    from ragged_blocked_kv_splitfuse_amd import fg
    from ragged_blocked_kv_splitfuse_amd.runtime import DeviceDescriptors, Workspace, stream_handle

    w, cache, ss, hb = S["w"], S["cache"], S["ss"], S["hb"]
    arr_bytes, blocks0 = S["template"]
    free_ids = S["free_ids"]
    desc = DeviceDescriptors(ring=8)
    ws = Workspace()
    stream = torch.cuda.current_stream()
    sh = stream_handle(stream)
    kptr, vptr = cache.k_pool.data_ptr(), cache.v_pool.data_ptr()

    work_buf = np.zeros(1 << 20, np.int32)

    # One cache handle for the run.  Every step starts from the same state: the sequence
    # states are copied back, and the blocks the step's composition took are returned in
    # reverse order, which restores the free list exactly (it is a stack, handed out from the
    # front of free_ids).
    h = fg.fg_blocked_cache_init(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                                 w.dtype, kptr, vptr, free_ids)
    n_free0 = fg.fg_blocked_cache_num_free(h)

    def compose_and_plan():
        ctypes.memmove(ctypes.addressof(ss.arr), arr_bytes, len(arr_bytes))
        np.copyto(ss.blocks, blocks0)
        st = fg.fg_splitfuse_compose(h, ss, w.budget, hb)
        assert st == fg.FG_OK
        info, work = fg.fg_attention_plan(h, hb, w.num_q_heads, S["cus"], work_buf)
        return info, work

    def restore_free_list():
        taken = n_free0 - fg.fg_blocked_cache_num_free(h)
        if taken:
            fg.fg_blocked_cache_release(h, free_ids[taken - 1::-1])

    # pass shape and inputs
    info, work = compose_and_plan()
    T, nseq = hb.num_tokens, hb.num_seqs
    ctx = hb.context_len[:nseq].astype(np.int64)
    nq = hb.n_query[:nseq].astype(np.int64)
    restore_free_list()
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed * 104729 + 17)
    mk = lambda heads: (torch.randn((T, heads, w.head_dim), generator=g, device="cuda")
                        * w.value_scale).to(S["tdt"])
    q, k_new, v_new = mk(w.num_q_heads), mk(w.num_kv_heads), mk(w.num_kv_heads)
    out = torch.empty((T, w.num_q_heads, w.head_dim), dtype=S["tdt"], device="cuda")
    wptr, wbytes = ws.ensure(max(info.workspace_bytes, 1 << 20))

    e = 2 if w.dtype == "bf16" else 4
    kv_tokens = int((ctx + nq).sum())
    attn_bytes = kv_tokens * w.num_kv_heads * w.head_dim * e * 2 + 2 * T * w.num_q_heads * w.head_dim * e
    pairs = int((nq * ctx + nq * (nq + 1) // 2).sum())
    attn_flops = 4 * w.head_dim * w.num_q_heads * pairs
    append_bytes = 4 * T * w.num_kv_heads * w.head_dim * e

    # Every fourth timed step carries two events around the attention launch (the roofline's
    # kernel; the one after attention also guards the pinned descriptor buffers of the steps
    # since the last guard).  Each event recorded on the stream adds a marker and several us of
    # GPU idle time to its step, so the other steps carry none, and kv_append is timed in extra
    # steps after the timed region, with events around it alone.
    n_total = warmup + steps
    n_app = min(steps, 20)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_total + n_app)]
    timed_attn = []
    host_s = []   # host work per step (compose, plan, upload, launches)
    wait_s = []   # per step, time the host waited for a free descriptor buffer (flow control:
                  # the ring lets the host run 8 steps ahead of the GPU, then it waits)

    def step(i, time_append=False):
        t0 = time.perf_counter()
        w0 = desc.wait_s
        info, work = compose_and_plan()
        c = desc.upload(hb, work, stream, record=False)
        mark = not time_append and (i % 4 == 3 or i == n_total - 1)
        if time_append:
            ev[i][0].record(stream)
        fg.fg_kv_append(h, c, k_new.data_ptr(), v_new.data_ptr(), sh)
        if time_append:
            ev[i][1].record(stream)
        if mark:
            ev[i][0].record(stream)
        fg.fg_ragged_attention(h, c, info, desc.work_ptr, q.data_ptr(), w.num_q_heads, w.scale,
                               out.data_ptr(), wptr, wbytes, sh)
        if mark:
            ev[i][1].record(stream)
            if i >= warmup:
                timed_attn.append(i)
        if mark or time_append:
            desc.release(ev[i][1])
        restore_free_list()
        waited = desc.wait_s - w0
        host_s.append(time.perf_counter() - t0 - waited)
        wait_s.append(waited)
        return info

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(warmup, n_total):
        info = step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(n_total, n_total + n_app):
        step(i, time_append=True)
    torch.cuda.synchronize()
    fg.fg_blocked_cache_destroy(h)

    attn_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in timed_attn]   # attention launch only
    app_ms = [a.elapsed_time(b) for a, b in ev[n_total:]]
    return dict(info=info, T=T, nseq=nseq, nq=nq, ctx=ctx, kv_tokens=kv_tokens,
                attn_bytes=attn_bytes, attn_flops=attn_flops, append_bytes=append_bytes,
                t_attn=float(np.mean(attn_ms)) * 1e-3, t_app=float(np.mean(app_ms)) * 1e-3,
                elapsed=t1 - t0, q=q, k_new=k_new, v_new=v_new, host_s=host_s[warmup:n_total],
                wait_s=wait_s[warmup:n_total])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no "
              "multi-GPU path; the pass would shard by KV head or by sequence, with no "
              "exchange inside it.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from ragged_blocked_kv_splitfuse_amd import fg
    from ragged_blocked_kv_splitfuse_amd.runtime import DeviceDescriptors, Workspace, stream_handle

    torch.cuda.set_device(0)
    if args.workload == "serving":
        serving_main(args)
        return
    if args.workload == "sweep":
        sweep_main(args)
        return
    S = setup(args)
    r = time_pass(S, args.steps, args.warmup)
    w, cache, hb, info = S["w"], S["cache"], S["hb"], r["info"]
    T, nseq, nq, kv_tokens = r["T"], r["nseq"], r["nq"], r["kv_tokens"]
    attn_bytes, attn_flops, append_bytes = r["attn_bytes"], r["attn_flops"], r["append_bytes"]
    t_attn, t_app, elapsed = r["t_attn"], r["t_app"], r["elapsed"]
    q, k_new, v_new, host_s = r["q"], r["k_new"], r["v_new"], r["host_s"]
    wait_s = r["wait_s"]
    value = T * args.steps / elapsed

    roof = roofline(w, args.workload, attn_bytes, attn_flops, t_attn)
    per_config = None
    if args.per_config and args.workload == "llama2":
        per_config = {"llama2": config_entry(w, r, "hbm")}
        del S, r
        torch.cuda.empty_cache()
        for name, bound in (("decode", "hbm"), ("chunked", "mfma"), ("mistral", "hbm+mfma")):
            P = setup(args, name)
            rr = time_pass(P, args.per_config_steps, min(args.warmup, 3))
            per_config[name] = config_entry(P["w"], rr, bound)
            print(json.dumps({"per_config": name, **per_config[name]}), file=sys.stderr, flush=True)
            del P, rr
            torch.cuda.empty_cache()
    result = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size, "token_budget": w.budget,
                   "num_seqs": nseq, "tokens": T, "kv_tokens": kv_tokens,
                   "decode_seqs": int((nq == 1).sum()), "work_records": int(info.num_work),
                   "split_groups": int(info.num_groups)},
        "roofline": roof,
        "per_config": per_config,
        "hbm_reference": hbm_reference(append_bytes=append_bytes) if args.per_config else None,
        "mfma_reference": mfma_reference() if args.per_config else None,
        "kernels": {"attention_us": t_attn * 1e6, "kv_append_us": t_app * 1e6,
                    "kv_append_GBps": append_bytes / t_app / 1e9,
                    "gpu_only_tokens_per_s": T / (t_attn + t_app),
                    "host_us_per_step": float(np.mean(host_s)) * 1e6,
                    "host_wait_us_per_step": float(np.mean(wait_s)) * 1e6},
        "cpu_baseline": cpu_baseline(args, w, cache, hb, q, k_new, v_new) if args.cpu_seconds > 0 else None,
    }
    print(json.dumps(result), flush=True)


def serving_main(args):
    """The serving loop over the whole request stream: one untimed run, one timed run, each
    from the same initial pool state (a fresh cache handle over the same pools)."""
    import numpy as np
    import torch
    from ragged_blocked_kv_splitfuse_amd import fg, workloads as wl
    from ragged_blocked_kv_splitfuse_amd.runtime import PagedKVCache, num_cus
    from ragged_blocked_kv_splitfuse_amd.serving import (DevicePass, ServingLoop,
                                                         latency_summary, request_latencies)

    hkv = 32 if args.model == "llama2" else 8
    sw = wl.serving_stream(seed=args.seed if args.seed is not None else 6,
                           n_requests=args.requests, clients=args.clients, budget=args.budget,
                           hkv=hkv, name=f"serving_{args.model}_7b")
    v = sw.values
    tdt = torch.bfloat16
    cache = PagedKVCache(v.num_blocks, v.block_size, v.num_kv_heads, v.head_dim, v.dtype,
                         free_ids=v.free_ids)
    wl.fill_pools_device(cache.k_pool, cache.v_pool, seed=v.seed * 7919 + 1)
    g = torch.Generator(device="cuda")
    g.manual_seed(v.seed * 104729 + 17)
    mk = lambda heads: torch.randn((sw.budget, heads, v.head_dim), generator=g,
                                   device="cuda").to(tdt)
    q, kn, vn = mk(v.num_q_heads), mk(v.num_kv_heads), mk(v.num_kv_heads)
    cus = args.num_cus or num_cus()
    proj = None
    if args.layer:
        from ragged_blocked_kv_splitfuse_amd.serving import Projections
        hid = v.num_q_heads * v.head_dim
        wmk = lambda n: (torch.randn((n, hid), generator=g, device="cuda")
                         / hid ** 0.5).to(tdt)
        proj = Projections(wmk(hid), wmk(v.num_kv_heads * v.head_dim),
                           wmk(v.num_kv_heads * v.head_dim), wmk(hid), sw.budget)
        x = torch.randn((sw.budget, hid), generator=g, device="cuda").to(tdt)
        rows = lambda hb, running: x[:hb.num_tokens]
    else:
        rows = lambda hb, running: (q[:hb.num_tokens], kn[:hb.num_tokens], vn[:hb.num_tokens])

    def run(timed, passes=0):
        h = fg.fg_blocked_cache_init(v.num_blocks, v.block_size, v.num_kv_heads, v.head_dim,
                                     v.dtype, cache.k_pool.data_ptr(), cache.v_pool.data_ptr(),
                                     v.free_ids)

        class Handle:   # DevicePass wants the handle's owner: the same pools, this handle
            handle, head_dim = h, v.head_dim

        dp = DevicePass(Handle, v.num_q_heads, v.scale, rows, cus, timing=timed, proj=proj)
        if timed:
            dp.reserve_events(passes)  # the untimed run's pass count: the same stream
        try:
            loop = ServingLoop(h, v.block_size, sw.budget, sw.clients, sw.table_width)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            st = loop.run(sw.requests, device_pass=dp)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        finally:
            fg.fg_blocked_cache_destroy(h)
        return st, wall, dp.marks

    st0, wall0, _ = run(False)
    st, wall, marks = run(True, passes=len(st0.tokens))
    seg = np.array([[m[i].elapsed_time(m[i + 1]) for i in range(4)] for m in marks]) * 1e-3
    qkv_s, app, att, oproj_s = seg[:, 0], seg[:, 1], seg[:, 2], seg[:, 3]
    ends = np.array([marks[0][0].elapsed_time(m[4]) for m in marks]) * 1e-3
    T = np.array(st.tokens)
    total = int(T.sum())
    gpu_pass = seg.sum(axis=1)

    def summary(end_times):
        ttft, pace = request_latencies(st, sw.requests, end_times)
        return latency_summary(ttft, pace)

    ttft_p = [st.first_token_pass[r.rid] - st.admit_pass[r.rid] + 1 for r in sw.requests]
    serving = {"passes": st.passes, "tokens": total,
               "full_budget_passes": int((T == sw.budget).sum()),
               "mean_T": float(T.mean()), "mean_S": float(np.mean(st.seqs)),
               "gpu_s": float(gpu_pass.sum()), "wall_s": wall, "wall_s_untimed_run": wall0,
               "gpu_only_tokens_per_s": total / float(gpu_pass.sum()),
               "attention_us_mean": float(att.mean() * 1e6),
               "kv_append_us_mean": float(app.mean() * 1e6),
               "ttft_passes_mean": float(np.mean(ttft_p)), **summary(ends)}
    if proj is not None:
        gflops = sum(proj.flops(int(t)) for t in T)
        gsec = float(qkv_s.sum() + oproj_s.sum())
        serving.update({"projections_us_mean": float((qkv_s + oproj_s).mean() * 1e6),
                        "projection_tflops": gflops / gsec / 1e12,
                        "projection_mfma_frac": gflops / gsec / 1e12 / BF16_PEAK_TFLOPS})
    # Latency proxy: a model of `layers` identical layers whose pass costs `layers` times the
    # measured one (attention layer only -- no MLP, norms or sampling), on the GPU timeline.
    L = args.layers
    proxy_ends = np.cumsum(gpu_pass * L)
    proxy = {"layers": L, "includes": "kv_append + attention" + (" + QKV/O projections"
                                                                 if proj is not None else ""),
             "tokens_per_s": total / float(proxy_ends[-1]), **summary(proxy_ends)}
    result = {
        "metric": "serving-loop tokens/s (continuous SplitFuse passes, whole request stream)",
        "value": total / wall, "unit": "tokens/s", "n_gpus": 1, "steps": st.passes,
        "warmup": 1, "ms_per_step": wall / st.passes * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": sw.name, "requests": len(sw.requests), "clients": sw.clients,
                   "token_budget": sw.budget, "q_heads": v.num_q_heads,
                   "kv_heads": v.num_kv_heads, "head_dim": v.head_dim,
                   "block_size": v.block_size, "pool_blocks": v.num_blocks,
                   "prompt_mean": 2600, "output_mean": 60, "cv": 0.3,
                   "projections": proj is not None},
        "serving": serving,
        "latency_proxy": proxy,
        "roofline": None,
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def roofline(w, workload, attn_bytes, attn_flops, t_attn):
    """Roofline of the dominant kernel (attention): HBM for the decode-heavy and mixed passes,
    bf16 MFMA for the chunked pass, fp32 VALU for fp32 inputs."""
    if w.dtype == "bf16" and workload != "chunked":
        roof = {"bound": "hbm", "achieved": attn_bytes / t_attn / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    elif w.dtype == "bf16":
        roof = {"bound": "mfma", "achieved": attn_flops / t_attn / 1e12, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "alu", "achieved": attn_flops / t_attn / 1e12,
                "peak": F32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        rec = tr.get(workload)
        if rec and rec.get("kernel_source") == kernel_source_hash():
            roof["traffic"] = rec["bytes_per_launch"]
    roof["kernel"] = "attention_bf16_kernel" if w.dtype == "bf16" else "attention_f32_kernel"
    roof["algorithmic_bytes"] = attn_bytes
    roof["algorithmic_flops"] = attn_flops
    roof["mfma_frac"] = attn_flops / t_attn / 1e12 / BF16_PEAK_TFLOPS
    if w.dtype == "bf16":
        roof.update(bound_fracs(attn_bytes, attn_flops, t_attn))
    return roof


def bound_fracs(B, F, t):
    """Roofline time over measured time for both combinations of the two bounds: the larger of
    bytes / HBM peak and flops / MFMA peak, and their sum (the time if the two never overlap)."""
    tb, tf = B / (HBM_PEAK_GBS * 1e9), F / (BF16_PEAK_TFLOPS * 1e12)
    return {"max_bound_frac": max(tb, tf) / t, "additive_bound_frac": (tb + tf) / t}


def config_entry(w, r, bound):
    """One pass shape's figures: kernel times (HIP events on the launch stream), algorithmic
    bytes and flops of attention, and the fraction of the bounding roofline.  For a mixed
    pass ("hbm+mfma") the roofline time is max(bytes / HBM peak, flops / MFMA peak)."""
    t_attn, t_app = r["t_attn"], r["t_app"]
    B, F = r["attn_bytes"], r["attn_flops"]
    hbm = B / t_attn / 1e9 / HBM_PEAK_GBS
    mfma = F / t_attn / 1e12 / BF16_PEAK_TFLOPS
    t_roof = max(B / (HBM_PEAK_GBS * 1e9), F / (BF16_PEAK_TFLOPS * 1e12))
    frac = {"hbm": hbm, "mfma": mfma, "hbm+mfma": t_roof / t_attn}[bound]
    return {"workload": w.name, "tokens": r["T"], "num_seqs": r["nseq"],
            "ms": (t_attn + t_app) * 1e3, "attention_us": t_attn * 1e6,
            "kv_append_us": t_app * 1e6, "algorithmic_bytes": B, "algorithmic_flops": F,
            "append_bytes": r["append_bytes"], "bound": bound, "frac": frac, "hbm_frac": hbm,
            "mfma_frac": mfma, "kv_append_hbm_frac": r["append_bytes"] / t_app / 1e9 / HBM_PEAK_GBS,
            "gpu_only_tokens_per_s": r["T"] / (t_attn + t_app),
            "step_tokens_per_s": r["T"] * len(r["host_s"]) / r["elapsed"],
            "split_groups": int(r["info"].num_groups), "work_records": int(r["info"].num_work),
            **bound_fracs(B, F, t_attn)}


def hbm_reference(gib=4, reps=10, append_bytes=0):
    """Practical HBM rates on this device, measured beside the pass: a device-to-device copy
    of `gib` GiB (bytes read + written per second) and a read-only reduction of 2*`gib` GiB
    (torch's own kernels), both timed with events over `reps` repetitions.  With append_bytes,
    also a plain copy moving that many bytes (half read, half written, as kv_append does) with
    1 GiB of other copy traffic before each repetition, so that it starts from cold caches as
    kv_append does after an attention pass: the median event-timed duration of 20."""
    import numpy as np
    import torch
    n = gib << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    x = torch.empty(2 * n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    out = {}
    for name, fn, nbytes in (("copy", lambda: b.copy_(a), 2 * n),
                             ("read", lambda: x.sum(), 2 * n)):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name + "_GBps"] = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x
    if append_bytes:
        n2 = append_bytes // 2
        src = torch.empty(n2, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        flush_src, flush_dst = a[: 1 << 29], b[: 1 << 29]
        ts = []
        for _ in range(20):
            flush_dst.copy_(flush_src)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dst.copy_(src)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        out["append_size_cold_copy_us"] = float(np.median(ts))
        out["append_size_bytes"] = int(2 * n2)
        del src, dst, flush_src, flush_dst
    del a, b
    torch.cuda.empty_cache()
    out["how"] = (f"torch device copy of {gib} GiB (read + write bytes) and torch sum over "
                  f"{2 * gib} GiB of fp32 (read bytes), {reps} repetitions each" +
                  ("; a copy moving kv_append's bytes after 1 GiB of other traffic, median of 20"
                   if append_bytes else ""))
    return out


def mfma_reference(sizes=(8192, 16384), flops_per_size=2e13):
    """Practical bf16 matrix-core rate on this device, measured beside the pass: torch's own
    (vendor library) bf16 GEMM on square n x n x n problems, timed with events over enough
    repetitions for ~`flops_per_size` flops each after 3 warm-ups.  A plain GEMM has no
    softmax, no masking and no gathers, so this is the rate an MFMA-bound attention pass
    could at best approach on this part, against the published 2.5 PFLOP/s."""
    import torch
    out = {}
    for n in sizes:
        a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            c = a @ b
        reps = max(3, int(flops_per_size / (2 * n ** 3)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        tf = 2 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
        out[f"gemm_{n}_TFLOPs"] = tf
        out[f"gemm_{n}_frac_of_peak"] = tf / BF16_PEAK_TFLOPS
        del a, b, c
    torch.cuda.empty_cache()
    out["how"] = (f"torch bf16 matmul, square sizes {list(sizes)}, event-timed, "
                  f"~{flops_per_size:.0e} flops each after 3 warm-ups")
    return out


def host_identity():
    """CPU model, logical CPUs this process may use, and numpy's BLAS build."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            i = libs[0]
            blas = f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', '')}, " \
                   f"{i.get('architecture', '')}, {i.get('num_threads')} threads)"
    except Exception:  # noqa: BLE001
        pass
    import numpy as np
    return {"cpu_model": model, "cpus_allowed": len(os.sched_getaffinity(0)),
            "numpy": np.__version__, "blas": blas}


def cpu_baseline(args, w, cache, hb, q, k_new, v_new):
    """The oracle, as it stands, on a bounded sample of the same pass: all sequences and
    tokens, a subset of KV heads (work is linear in heads), scaled to the full pass."""
    import numpy as np
    import torch
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    from oracle.compose import OracleBatch
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    S = hb.num_seqs
    batch = OracleBatch(hb.query_start[:S + 1].copy(), hb.n_query[:S].copy(),
                        hb.context_len[:S].copy(), hb.block_table[:S].copy(),
                        hb.seq_index[:S].copy(), hb.seq_id[:S].copy())
    G = w.num_q_heads // w.num_kv_heads
    bits = (lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)) if w.dtype == "bf16" \
        else (lambda t: t.cpu().numpy())

    def run(hk):
        kp = bits(cache.k_pool[:, :hk].contiguous())
        vp = bits(cache.v_pool[:, :hk].contiguous())
        qq = bits(q[:, :hk * G].contiguous())
        kn = bits(k_new[:, :hk].contiguous())
        vn = bits(v_new[:, :hk].contiguous())
        t0 = time.perf_counter()
        oracle.kv_append(kp, vp, kn, vn, batch, w.block_size)
        oracle.ragged_attention(qq, kp, vp, batch, hk * G, hk, w.scale, w.block_size, w.dtype)
        return time.perf_counter() - t0

    t1 = run(1)
    hk = int(min(w.num_kv_heads, max(1, args.cpu_seconds // max(t1, 1e-3))))
    times = [run(hk) if hk > 1 else t1]
    while sum(times) < 0.66 * args.cpu_seconds:  # the whole pass is quick: repeat it
        times.append(run(hk))
    t = float(np.mean(times))
    full = t * w.num_kv_heads / hk
    return {"value": hb.num_tokens / full, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", **host_identity(),
            "sample": f"numpy fp64 oracle (append + attention) on {hk} of {w.num_kv_heads} KV "
                      f"heads of the same pass (all {S} sequences, {hb.num_tokens} tokens), "
                      f"{len(times)} run(s) of {t:.2f} s, scaled x{w.num_kv_heads / hk:g} to "
                      f"the full pass"}


if __name__ == "__main__":
    main()
