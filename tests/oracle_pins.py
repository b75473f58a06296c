"""Pins for the oracle: checks against things other than the oracle itself.

Each check takes the function(s) under test as arguments so that the same
check can be run against the oracle (must pass) and against deliberately
broken copies of it (must fail), see test_oracle_mutations.py.

* brute force: dense causal attention written as plain Python loops over the
  per-sequence contiguous history drawn straight from the generator (no pool,
  no block table, no numpy matmul);
* hand-derived fixtures under tests/golden/;
* closed forms (zero query -> mean of the visible V rows; the first token of a
  fresh sequence -> its own V row exactly; equal V rows -> that row; one
  dominant logit -> its V row; single query == scipy's softmax);
* invariants fixed by the method: relabelling physical blocks changes nothing,
  and processing a prompt in chunks over several passes equals one pass.
"""
import json
import math
import os

import numpy as np
from scipy.special import softmax as scipy_softmax

from oracle.bf16 import to_f64
from oracle.compose import FreeList, OracleBatch, SeqState
from ragged_blocked_kv_splitfuse_amd import workloads as wl

import harness

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def tiny_workloads():
    """Small mixed workloads: MHA and GQA, blocks of 4 and 8, fp32 and bf16, fresh and
    continuing prompts, decodes with context 0 (first token attends only itself)."""
    out = []
    out.append(wl.custom(101, dtype="f32", hq=4, hkv=2, d=8, bs=4, budget=13, n_decode=3,
                         decode_ctx=(0, 9), prompts=((0, 5), (3, 30))))
    out.append(wl.custom(102, dtype="bf16", hq=2, hkv=2, d=8, bs=8, budget=11, n_decode=2,
                         decode_ctx=(5, 17), prompts=((7, 12), (0, 9))))
    out.append(wl.custom(103, dtype="f32", hq=6, hkv=3, d=4, bs=4, budget=9, n_decode=1,
                         decode_ctx=(0, 0), prompts=((0, 20),)))
    return out


def brute_force_pass(w, res):
    """Pure-Python dense causal attention from the generator's contiguous rows."""
    batch, states = res["batch"], res["states"]
    G = w.num_q_heads // w.num_kv_heads
    T, Hq, D = batch.num_tokens, w.num_q_heads, w.head_dim
    out = np.zeros((T, Hq, D))
    for s in range(batch.num_seqs):
        st = states[int(batch.seq_index[s])]
        c, n, t0 = int(batch.context_len[s]), int(batch.n_query[s]), int(batch.query_start[s])
        K = to_f64(w.k_rows(st.seq_id, 0, c + n), w.dtype).tolist()
        V = to_f64(w.v_rows(st.seq_id, 0, c + n), w.dtype).tolist()
        Q = to_f64(w.q_rows(st.seq_id, c, c + n), w.dtype).tolist()
        for i in range(n):
            for g in range(Hq):
                h = g // G
                logits = []
                for j in range(c + i + 1):
                    acc = 0.0
                    for d in range(D):
                        acc += Q[i][g][d] * K[j][h][d]
                    logits.append(acc * w.scale)
                mx = max(logits)
                ws = [math.exp(x - mx) for x in logits]
                tot = sum(ws)
                for d in range(D):
                    out[t0 + i, g, d] = sum(ws[j] * V[j][h][d] for j in range(len(ws))) / tot
    return out


def run_pass(w, attn, append, compose):
    states = harness.oracle_states(w)
    free = compose.FreeList(w.free_ids)
    k_pool, v_pool = harness.empty_pools(w)
    # history goes in with the append under test, so a wrong slot formula in it
    # is read back consistently by a wrong gather: the hand fixtures catch that
    hb, idx = harness.history_batch(w, states)
    if hb.num_seqs:
        K = np.concatenate([w.k_rows(states[i].seq_id, 0, states[i].n_cached) for i in idx])
        V = np.concatenate([w.v_rows(states[i].seq_id, 0, states[i].n_cached) for i in idx])
        append(k_pool, v_pool, K, V, hb, w.block_size)
    batch, status = compose.splitfuse_compose(states, w.budget, free, w.block_size, w.table_width)
    q, kn, vn = harness.new_rows(w, batch, states)
    append(k_pool, v_pool, kn, vn, batch, w.block_size)
    out = attn(q, k_pool, v_pool, batch, w.num_q_heads, w.num_kv_heads, w.scale,
               w.block_size, w.dtype)
    return dict(states=states, batch=batch, status=status, out=out, q=q, k_pool=k_pool,
                v_pool=v_pool, k_new=kn, v_new=vn)


def check_bruteforce(attn, append, compose):
    worst = 0.0
    for w in tiny_workloads():
        res = run_pass(w, attn, append, compose)
        ref = brute_force_pass(w, res)
        if res["out"].shape != ref.shape:
            return float("inf")
        worst = max(worst, float(np.nanmax(np.abs(res["out"] - ref))) if ref.size else 0.0)
        if np.isnan(res["out"]).any():
            return float("inf")
    return worst


def _golden_attention():
    with open(os.path.join(GOLDEN, "attention_hand_3keys.json")) as f:
        g = json.load(f)
    return g


def check_golden_attention(attn, append):
    """Max abs error against the hand-derived outputs and slots (inf if a slot is wrong)."""
    g = _golden_attention()
    NB, bs, D = g["num_blocks"], g["block_size"], g["head_dim"]
    sent = np.uint32(0x7FC00001)
    g8 = min(8, bs)        # V slots in groups of min(8, bs), feature-major in a group
    k_pool = np.full((NB, 1, bs, D), sent, np.uint32).view(np.float32)
    v_pool = np.full((NB, 1, bs // g8, D, g8), sent, np.uint32).view(np.float32)
    rows_k = np.array(g["k_rows"], np.float32)[:, None, :]
    rows_v = np.array(g["v_rows"], np.float32)[:, None, :]
    c, n = g["context_len"], g["n_new"]
    table = np.array([g["block_table"]], np.int32)
    hist = OracleBatch(np.array([0, c], np.int32), np.array([c], np.int32),
                       np.array([0], np.int32), table, np.array([0], np.int32),
                       np.array([1], np.int64))
    append(k_pool, v_pool, rows_k[:c], rows_v[:c], hist, bs)
    batch = OracleBatch(np.array([0, n], np.int32), np.array([n], np.int32),
                        np.array([c], np.int32), table, np.array([0], np.int32),
                        np.array([1], np.int64))
    append(k_pool, v_pool, rows_k[c:], rows_v[c:], batch, bs)
    for key, val in g["expected_k_slots"].items():
        b, s = map(int, key.split(","))
        if not np.allclose(k_pool[b, 0, s, :], val, atol=0, rtol=1e-7):
            return float("inf")
    for key, val in g["expected_v_slots"].items():
        b, s = map(int, key.split(","))
        if not np.allclose(v_pool[b, 0, s // g8, :, s % g8], val, atol=0, rtol=1e-7):
            return float("inf")
    touched = {tuple(map(int, k.split(","))) for k in g["expected_k_slots"]}
    for b in range(NB):
        for s in range(bs):
            if (b, s) not in touched:
                if not (np.all(k_pool[b, 0, s, :].view(np.uint32) == sent)
                        and np.all(v_pool[b, 0, s // g8, :, s % g8].view(np.uint32) == sent)):
                    return float("inf")
    q = np.array(g["q_rows"], np.float32)[:, None, :]
    out = attn(q, k_pool, v_pool, batch, 1, 1, g["scale"], bs, "f32")
    return float(np.max(np.abs(out[:, 0, :] - np.array(g["expected_out"]))))


def _one_seq_batch(c, n, table):
    return OracleBatch(np.array([0, n], np.int32), np.array([n], np.int32),
                       np.array([c], np.int32), np.array([table], np.int32),
                       np.array([0], np.int32), np.array([7], np.int64))


def _pool_from_rows(K, V, table, bs, NB):
    """Place contiguous rows [L][H][D] into fp32 pools by hand (block-major loops)."""
    L, H, D = K.shape
    g8 = min(8, bs)        # V slots in groups of min(8, bs), feature-major in a group
    kp = np.full((NB, H, bs, D), np.nan, np.float32)
    vp = np.full((NB, H, bs // g8, D, g8), np.nan, np.float32)
    for p in range(L):
        b = table[p // bs]
        for h in range(H):
            for d in range(D):
                kp[b, h, p % bs, d] = K[p, h, d]
                vp[b, h, (p % bs) // g8, d, (p % bs) % g8] = V[p, h, d]
    return kp, vp


def check_closed_forms(attn):
    """Returns the worst error over the closed-form cases (inf on a structural failure)."""
    rng = np.random.Generator(np.random.PCG64(77))
    worst = 0.0
    H, D, bs, NB = 2, 8, 4, 12
    c, n = 9, 3
    L = c + n
    table = [11, 3, 7, 0]
    K = rng.standard_normal((L, H, D)).astype(np.float32)
    V = rng.standard_normal((L, H, D)).astype(np.float32)
    kp, vp = _pool_from_rows(K, V, table, bs, NB)
    batch = _one_seq_batch(c, n, table)

    # (a) zero query: uniform weights -> mean of the visible V rows
    q = np.zeros((n, H, D), np.float32)
    out = attn(q, kp, vp, batch, H, H, 0.3, bs, "f32")
    for i in range(n):
        ref = V[:c + i + 1].astype(np.float64).mean(axis=0)
        worst = max(worst, float(np.max(np.abs(out[i] - ref))))

    # (b) all V rows equal -> that row, whatever the logits
    Ve = np.broadcast_to(V[:1], V.shape).copy()
    kp2, vp2 = _pool_from_rows(K, Ve, table, bs, NB)
    q = rng.standard_normal((n, H, D)).astype(np.float32)
    out = attn(q, kp2, vp2, batch, H, H, 0.5, bs, "f32")
    worst = max(worst, float(np.max(np.abs(out - V[0].astype(np.float64)[None]))))

    # (c) one dominant logit: K_j = 50 q for one visible j -> o ~= V_j
    j = 4
    Kd = K.copy()
    q = rng.standard_normal((n, H, D)).astype(np.float32)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    Kd[j] = 50.0 * q[0]
    Kd[:j] *= 0.01
    Kd[j + 1:] *= 0.01
    qq = np.broadcast_to(q[:1], q.shape).copy()
    kp3, vp3 = _pool_from_rows(Kd, V, table, bs, NB)
    out = attn(qq, kp3, vp3, batch, H, H, 1.0, bs, "f32")
    # every other weight is about exp(-50): the error is far below 1e-12
    worst = max(worst, float(np.max(np.abs(out - V[j].astype(np.float64)[None]))))

    # (d) fresh sequence, first token: sees only itself -> exactly its own V row
    tbl = [5]
    K1 = rng.standard_normal((3, H, D)).astype(np.float32)
    V1 = rng.standard_normal((3, H, D)).astype(np.float32)
    kp4, vp4 = _pool_from_rows(K1, V1, tbl, bs, NB)
    q = rng.standard_normal((3, H, D)).astype(np.float32)
    out = attn(q, kp4, vp4, _one_seq_batch(0, 3, tbl), H, H, 0.7, bs, "f32")
    if not np.array_equal(out[0], V1[0].astype(np.float64)):
        return float("inf")

    # (e) single query, MHA: textbook attention through scipy's softmax
    tbl = [2, 9, 1]
    K2 = rng.standard_normal((10, H, D)).astype(np.float32)
    V2 = rng.standard_normal((10, H, D)).astype(np.float32)
    kp5, vp5 = _pool_from_rows(K2, V2, tbl, bs, NB)
    q = rng.standard_normal((1, H, D)).astype(np.float32)
    out = attn(q, kp5, vp5, _one_seq_batch(9, 1, tbl), H, H, 0.25, bs, "f32")
    for h in range(H):
        p = scipy_softmax(0.25 * (K2[:, h].astype(np.float64) @ q[0, h].astype(np.float64)))
        ref = p @ V2[:, h].astype(np.float64)
        worst = max(worst, float(np.max(np.abs(out[0, h] - ref))))
    return worst


def check_permutation_invariance(attn, append, compose):
    """Relabel physical blocks (move contents, rewrite tables): outputs must not change a bit."""
    w = wl.custom(211, dtype="bf16", hq=4, hkv=2, d=8, bs=4, budget=17, n_decode=3,
                  decode_ctx=(1, 14), prompts=((5, 40),), extra_blocks=5)
    res = run_pass(w, attn, append, compose)
    rng = np.random.Generator(np.random.PCG64(5))
    perm = rng.permutation(w.num_blocks)
    kp = np.empty_like(res["k_pool"])
    vp = np.empty_like(res["v_pool"])
    kp[perm] = res["k_pool"]
    vp[perm] = res["v_pool"]
    b = res["batch"]
    bt = np.where(b.block_table >= 0, perm[np.maximum(b.block_table, 0)], -1).astype(np.int32)
    b2 = OracleBatch(b.query_start, b.n_query, b.context_len, bt, b.seq_index, b.seq_id)
    out2 = attn(res["q"], kp, vp, b2, w.num_q_heads, w.num_kv_heads, w.scale, w.block_size,
                w.dtype)
    return bool(np.array_equal(out2, res["out"]))


def check_chunk_invariance(attn, append, compose, chunk=7):
    """One prompt: passes of `chunk` tokens vs one whole pass -> same rows."""
    L = 45
    w = wl.custom(307, dtype="f32", hq=4, hkv=2, d=8, bs=4, budget=L, n_decode=0,
                  prompts=((0, L),))
    whole = run_pass(w, attn, append, compose)
    # chunked: same workload, budget `chunk`, passes until the prompt is done
    states = harness.oracle_states(w)
    free = compose.FreeList(w.free_ids)
    k_pool, v_pool = harness.empty_pools(w)
    rows = []
    import oracle.compose as oc
    while states[0].n_cached < L:
        batch, status = compose.splitfuse_compose(states, chunk, free, w.block_size,
                                                  w.table_width)
        if batch.num_tokens == 0:
            return float("inf")
        q, kn, vn = harness.new_rows(w, batch, states)
        append(k_pool, v_pool, kn, vn, batch, w.block_size)
        rows.append(attn(q, k_pool, v_pool, batch, w.num_q_heads, w.num_kv_heads, w.scale,
                         w.block_size, w.dtype))
        oc.commit_pass(states)
    got = np.concatenate(rows)
    if got.shape != whole["out"].shape:
        return float("inf")
    return float(np.max(np.abs(got - whole["out"])))


# --------------------------------------------------------------------------
# composition
# --------------------------------------------------------------------------

def _load_compose_golden():
    with open(os.path.join(GOLDEN, "compose_hand_queue.json")) as f:
        return json.load(f)


def check_golden_compose(compose):
    g = _load_compose_golden()
    seqs = [SeqState(s["seq_id"], s["n_cached"], s["prompt_len"], list(s["blocks"]),
                     g["table_width"]) for s in g["seqs"]]
    free = compose.FreeList(g["free_ids"])
    batch, status = compose.splitfuse_compose(seqs, g["budget"], free, g["block_size"],
                                              g["table_width"])
    e = g["expected"]
    ok = (status == "ok"
          and batch.query_start.tolist() == e["query_start"]
          and batch.n_query.tolist() == e["n_query"]
          and batch.context_len.tolist() == e["context_len"]
          and batch.seq_index.tolist() == e["seq_index"]
          and batch.block_table.tolist() == e["block_table"])
    left = []
    while free.available():
        left.append(free.pop())
    return ok and left == e["free_left_in_handout_order"]


def compose_invariants(seqs_before, seqs_after, batch, status, budget, bs, free_before,
                       free_after_ids):
    """Returns a list of violated invariants (empty when all hold)."""
    bad = []
    demand = sum(1 if s.n_cached >= s.prompt_len else s.prompt_len - s.n_cached
                 for s in seqs_before)
    T = batch.num_tokens
    if T > budget:
        bad.append("budget exceeded")
    # pool large enough for everything -> exact fill
    room = len(free_before) * bs
    if room >= demand + len(seqs_before) * bs and T != min(budget, demand):
        bad.append("budget not filled although demand allowed it")
    n_of = {int(batch.seq_index[k]): int(batch.n_query[k]) for k in range(batch.num_seqs)}
    dec_idx = [i for i, s in enumerate(seqs_before) if s.n_cached >= s.prompt_len]
    pro_idx = [i for i, s in enumerate(seqs_before) if s.n_cached < s.prompt_len]
    for i in dec_idx:
        if n_of.get(i, 0) > 1:
            bad.append("decode got more than one token")
    # decodes first: a prompt gets tokens only when every decode that fits got its token
    if any(n_of.get(i, 0) > 0 for i in pro_idx):
        for i in dec_idx:
            if n_of.get(i, 0) == 0 and room >= len(seqs_before) * bs:
                bad.append("prompt served before a decode")
    # arrival order: with a pool that cannot run dry, a later prompt gets tokens only if
    # every earlier one got all it asked (with a dry pool, prompts that fit go on)
    seen_short = False
    for i in (pro_idx if room >= demand + len(seqs_before) * bs else []):
        s = seqs_before[i]
        got = n_of.get(i, 0)
        if seen_short and got > 0:
            bad.append("prompt order broken")
        if got < s.prompt_len - s.n_cached:
            seen_short = True
    # batch order is queue order, no empty entries, prefix sums
    if list(batch.seq_index) != sorted(batch.seq_index):
        bad.append("batch not in queue order")
    if np.any(batch.n_query <= 0):
        bad.append("empty batch entry")
    if not np.array_equal(np.cumsum(np.r_[0, batch.n_query]), batch.query_start):
        bad.append("query_start is not the prefix sum")
    # blocks: exactly ceil((c+n)/bs) when grown, taken from the free list in order, unshared
    used = []
    taken = []
    for k in range(batch.num_seqs):
        i = int(batch.seq_index[k])
        b, a = seqs_before[i], seqs_after[i]
        c, n = int(batch.context_len[k]), int(batch.n_query[k])
        if c != b.n_cached:
            bad.append("context_len is not the cached length")
        need = -(-(c + n) // bs)
        if len(a.blocks) != max(need, len(b.blocks)):
            bad.append("block count")
        if a.blocks[:len(b.blocks)] != b.blocks:
            bad.append("owned blocks changed")
        taken += a.blocks[len(b.blocks):]
        row = batch.block_table[k]
        if row[:len(a.blocks)].tolist() != a.blocks or np.any(row[len(a.blocks):] != -1):
            bad.append("block table row")
        used += a.blocks
    for i, s in enumerate(seqs_after):
        if i not in n_of:
            used += s.blocks
    if len(used) != len(set(used)):
        bad.append("block shared")
    # the free list is consumed in priority order: decodes (queue order), then prompts
    order = [i for i in dec_idx if i in n_of] + [i for i in pro_idx if i in n_of]
    taken = []
    for i in order:
        taken += seqs_after[i].blocks[len(seqs_before[i].blocks):]
    if taken != free_before[:len(taken)]:
        bad.append("blocks not taken from the free list in order")
    if free_after_ids != free_before[len(taken):]:
        bad.append("free list")
    if status == "no_blocks" and batch.num_seqs:
        bad.append("no_blocks status with a non-empty batch")
    if batch.num_seqs == 0 and seqs_before and status != "no_blocks":
        bad.append("empty batch without no_blocks status")
    return bad


def enumerate_tiny_queues():
    """Every queue of up to 3 requests drawn from a small menu of request kinds."""
    menu = [(0, 0), (3, 3), (4, 4), (0, 2), (0, 5), (2, 7), (4, 9)]  # (n_cached, prompt_len)
    import itertools
    for k in range(0, 4):
        for combo in itertools.product(menu, repeat=k):
            yield combo


def check_compose_exhaustive(compose, bs=4, pool_sizes=(0, 1, 2, 6), budgets=(1, 2, 3, 5, 8)):
    """Exhaustive over tiny queues, budgets and pool sizes: returns the first violation."""
    for combo in enumerate_tiny_queues():
        for nb_free in pool_sizes:
            for budget in budgets:
                next_id = 0
                seqs = []
                for j, (c, p) in enumerate(combo):
                    nb = -(-c // bs)
                    seqs.append(SeqState(j, c, p, list(range(next_id, next_id + nb)), 4))
                    next_id += nb
                free_ids = list(range(100, 100 + nb_free))
                before = [SeqState(s.seq_id, s.n_cached, s.prompt_len, list(s.blocks),
                                   s.max_blocks) for s in seqs]
                free = compose.FreeList(free_ids)
                try:
                    batch, status = compose.splitfuse_compose(seqs, budget, free, bs, 4)
                except Exception as e:  # noqa: BLE001
                    return f"raised {e!r} on {combo} budget {budget} pool {nb_free}"
                left = []
                while free.available():
                    left.append(free.pop())
                bad = compose_invariants(before, seqs, batch, status, budget, bs, free_ids, left)
                if bad:
                    return f"{bad} on {combo} budget {budget} pool {nb_free}"
    return None


def check_multipass_coverage(compose, commit):
    """Serving loop over a queue: every prompt token scheduled exactly once, in order;
    every pass is full while demand lasts."""
    rng = np.random.Generator(np.random.PCG64(9))
    bs, budget = 8, 16
    seqs = []
    for j in range(6):
        L = int(rng.integers(1, 60))
        seqs.append(SeqState(j, 0, L, [], 64))
    free = compose.FreeList(range(500))
    scheduled = {j: [] for j in range(6)}
    for _ in range(200):
        pending = [s for s in seqs if s.n_cached < s.prompt_len]
        if not pending:
            break
        demand = sum(s.prompt_len - s.n_cached for s in pending)
        batch, status = compose.splitfuse_compose(pending, budget, free, bs, 64)
        if batch.num_tokens != min(budget, demand):
            return "pass not filled"
        for k in range(batch.num_seqs):
            s = pending[int(batch.seq_index[k])]
            c, n = int(batch.context_len[k]), int(batch.n_query[k])
            scheduled[s.seq_id] += list(range(c, c + n))
        commit(pending)
    for s in seqs:
        if scheduled[s.seq_id] != list(range(s.prompt_len)):
            return f"sequence {s.seq_id} positions {scheduled[s.seq_id][:5]}..."
    return None
