"""Host side of the library through the C ABI (no GPU needed): exports, composition against
the oracle and its pins, every failure code, descriptor validation, work-list planning."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import oracle.compose as oc
import oracle_pins as pins
import harness
from oracle.compose import OracleBatch
from ragged_blocked_kv_splitfuse_amd import fg, workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "fg.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fg_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 13
    L = fg.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(fg.EXPORTS) == names


# --------------------------------------------------------------------------------------
# the C++ composition behind the oracle's interface, so the same pins can run on it
# --------------------------------------------------------------------------------------

class CFreeList:
    def __init__(self, ids):
        self.ids = [int(b) for b in ids]   # hand-out order

    def available(self):
        return len(self.ids)

    def pop(self):
        return self.ids.pop(0)


class CCompose:
    """Adapter: composition by libfg (fg_splitfuse_compose), oracle-style arguments."""
    FreeList = CFreeList

    @staticmethod
    def splitfuse_compose(seqs, budget, free, block_size, table_width):
        ids_all = list(free.ids) + [b for s in seqs for b in s.blocks]
        nb = max(ids_all + [0]) + 1
        h = fg.fg_blocked_cache_init(nb, block_size, 1, 128, "bf16", None, None, free.ids)
        try:
            ss = fg.SeqStates(seqs, table_width)
            hb = fg.HostBatch(len(seqs), table_width)
            try:
                st = fg.fg_splitfuse_compose(h, ss, budget, hb)
            except fg.FgError as e:
                raise ValueError(str(e)) from e
            for i, s in enumerate(seqs):
                s.blocks = ss.owned(i)
                s.n_scheduled = int(ss.arr[i].n_scheduled)
            free.ids = fg.fg_blocked_cache_free_ids(h).tolist()
            S = hb.num_seqs
            batch = OracleBatch(hb.query_start[:S + 1].copy(), hb.n_query[:S].copy(),
                                hb.context_len[:S].copy(), hb.block_table[:S].copy(),
                                hb.seq_index[:S].copy(), hb.seq_id[:S].copy())
        finally:
            fg.fg_blocked_cache_destroy(h)
        return batch, ("ok" if st == fg.FG_OK else "no_blocks")

    @staticmethod
    def commit_pass(seqs):
        for s in seqs:
            s.n_cached += s.n_scheduled
            s.n_scheduled = 0


def test_compose_golden():
    assert pins.check_golden_compose(CCompose)


def test_compose_exhaustive_tiny_queues():
    assert pins.check_compose_exhaustive(CCompose) is None


def test_compose_multipass_coverage():
    assert pins.check_multipass_coverage(CCompose, CCompose.commit_pass) is None


def _same_batch(a, b):
    return all(np.array_equal(getattr(a, f), getattr(b, f)) for f in
               ("query_start", "n_query", "context_len", "block_table", "seq_index", "seq_id"))


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_compose_matches_oracle_on_workloads(cfg):
    w = wl.make(cfg)
    so, sc = harness.oracle_states(w), harness.oracle_states(w)
    fo, fc = oc.FreeList(w.free_ids), CFreeList(w.free_ids)
    bo, sto = oc.splitfuse_compose(so, w.budget, fo, w.block_size, w.table_width)
    bc, stc = CCompose.splitfuse_compose(sc, w.budget, fc, w.block_size, w.table_width)
    assert sto == stc == "ok"
    assert _same_batch(bo, bc)
    assert [s.blocks for s in so] == [s.blocks for s in sc]
    left = []
    while fo.available():
        left.append(fo.pop())
    assert left == fc.ids


def test_compose_matches_oracle_random_queues():
    rng = np.random.Generator(np.random.PCG64(2024))
    for trial in range(300):
        bs = int(rng.choice([1, 2, 4, 8, 16]))
        n = int(rng.integers(0, 7))
        seqs, owned = [], 0
        for j in range(n):
            c = int(rng.integers(0, 40))
            p = int(rng.integers(0, 80)) if rng.random() < 0.6 else c
            nb = -(-c // bs)
            seqs.append((j, c, p, list(range(owned, owned + nb))))
            owned += nb
        free = list(range(owned, owned + int(rng.integers(0, 30))))
        rng.shuffle(free)
        width = max([-(-(max(p, c) + 1) // bs) for _, c, p, _ in seqs] + [1]) + 2
        budget = int(rng.integers(1, 64))
        mk = lambda: [oc.SeqState(j, c, p, list(b), width) for j, c, p, b in seqs]
        so, sc = mk(), mk()
        fo, fc = oc.FreeList(free), CFreeList(free)
        bo, sto = oc.splitfuse_compose(so, budget, fo, bs, width)
        bc, stc = CCompose.splitfuse_compose(sc, budget, fc, bs, width)
        assert sto == stc, trial
        assert _same_batch(bo, bc), trial
        assert [s.blocks for s in so] == [s.blocks for s in sc], trial


def test_commit_through_abi():
    class S:
        pass
    st = []
    for c, p in [(5, 5), (0, 9)]:
        o = S()
        o.seq_id, o.n_cached, o.prompt_len, o.blocks = 1, c, p, [0] if c else []
        st.append(o)
    h = fg.fg_blocked_cache_init(8, 8, 1, 128, "bf16", None, None, list(range(1, 8)))
    ss = fg.SeqStates(st, 4)
    hb = fg.HostBatch(2, 4)
    fg.fg_splitfuse_compose(h, ss, 6, hb)
    fg.fg_splitfuse_commit(ss)
    assert [ss.n_cached(0), ss.n_cached(1)] == [6, 5]
    assert ss.arr[0].n_scheduled == 0
    fg.fg_blocked_cache_destroy(h)


# --------------------------------------------------------------------------------------
# failure codes, forced on the CPU
# --------------------------------------------------------------------------------------

def _status(fn, *a):
    try:
        fn(*a)
        return fg.FG_OK
    except fg.FgError as e:
        return e.status


def test_init_errors():
    L = fg.lib()
    h = ctypes.c_void_p()
    assert L.fg_blocked_cache_init(None, None, None, None, -1, ctypes.byref(h)) == fg.FG_E_ARG
    assert _status(fg.fg_blocked_cache_init, 8, 3, 1, 128, "bf16", None, None) == fg.FG_E_UNSUPPORTED
    assert _status(fg.fg_blocked_cache_init, 8, 16, 1, 96, "bf16", None, None) == fg.FG_E_UNSUPPORTED
    assert _status(fg.fg_blocked_cache_init, 8, 16, 1, 256, "bf16", None, None) == fg.FG_E_UNSUPPORTED
    fg.fg_blocked_cache_destroy(fg.fg_blocked_cache_init(8, 16, 1, 64, "bf16", None, None))
    assert _status(fg.fg_blocked_cache_init, 8, 16, 1, 96, "f32", None, None) == fg.FG_E_UNSUPPORTED
    assert _status(fg.fg_blocked_cache_init, 8, 16, 1, 128, 7, None, None) == fg.FG_E_ARG
    assert _status(fg.fg_blocked_cache_init, 0, 16, 1, 128, "bf16", None, None) == fg.FG_E_ARG
    assert _status(fg.fg_blocked_cache_init, 8, 16, 0, 128, "bf16", None, None) == fg.FG_E_ARG
    assert _status(fg.fg_blocked_cache_init, 8, 16, 1, 128, "bf16", None, None, [1, 1]) == fg.FG_E_ARG
    assert _status(fg.fg_blocked_cache_init, 8, 16, 1, 128, "bf16", None, None, [8]) == fg.FG_E_ARG
    assert "listed twice" in fg.fg_last_error() or "out of range" in fg.fg_last_error()


def _one_seq(c, p, blocks, max_blocks):
    class S:
        pass
    o = S()
    o.seq_id, o.n_cached, o.prompt_len, o.blocks, o.max_blocks = 7, c, p, blocks, max_blocks
    return o


def test_compose_errors_and_no_state_change():
    h = fg.fg_blocked_cache_init(4, 8, 1, 128, "bf16", None, None, [3, 2])
    ss = fg.SeqStates([_one_seq(8, 8, [0], 4)], 4)
    hb = fg.HostBatch(1, 4)
    assert _status(fg.fg_splitfuse_compose, h, ss, 0, hb) == fg.FG_E_ARG
    small = fg.HostBatch(1, 2)   # table stride 2 < max_blocks 4
    assert _status(fg.fg_splitfuse_compose, h, ss, 4, small) == fg.FG_E_ARG
    zero = fg.HostBatch(0, 4)
    zero.c.seq_capacity = 0
    assert _status(fg.fg_splitfuse_compose, h, ss, 4, zero) == fg.FG_E_ARG
    bad = fg.SeqStates([_one_seq(9, 9, [0], 4)], 4)    # 1 block of 8 cannot hold 9 tokens
    assert _status(fg.fg_splitfuse_compose, h, bad, 4, hb) == fg.FG_E_ARG
    # pool dry: a decode at a block boundary cannot get its token
    h2 = fg.fg_blocked_cache_init(4, 8, 1, 128, "bf16", None, None, [])
    ss2 = fg.SeqStates([_one_seq(8, 8, [0], 4)], 4)
    st = fg.fg_splitfuse_compose(h2, ss2, 4, hb)
    assert st == fg.FG_E_NO_BLOCKS and hb.num_seqs == 0 and ss2.arr[0].n_blocks == 1
    for x in (h, h2):
        fg.fg_blocked_cache_destroy(x)


def test_release_errors_and_reuse_order():
    h = fg.fg_blocked_cache_init(6, 8, 1, 128, "bf16", None, None, [5, 4])
    assert _status(fg.fg_blocked_cache_release, h, [4]) == fg.FG_E_ARG      # already free
    assert _status(fg.fg_blocked_cache_release, h, [1, 1]) == fg.FG_E_ARG   # twice
    assert _status(fg.fg_blocked_cache_release, h, [9]) == fg.FG_E_ARG      # out of range
    assert fg.fg_blocked_cache_free_ids(h).tolist() == [5, 4]               # unchanged
    fg.fg_blocked_cache_release(h, [0, 1])
    assert fg.fg_blocked_cache_free_ids(h).tolist() == [1, 0, 5, 4]         # last released first
    assert fg.fg_blocked_cache_num_free(h) == 4
    # a bad id late in the list leaves nothing released (the marks made before it are undone)
    assert _status(fg.fg_blocked_cache_release, h, [2, 3, 2]) == fg.FG_E_ARG
    assert _status(fg.fg_blocked_cache_release, h, [2, 3, 7]) == fg.FG_E_ARG
    assert fg.fg_blocked_cache_free_ids(h).tolist() == [1, 0, 5, 4]
    fg.fg_blocked_cache_release(h, [2, 3])
    assert fg.fg_blocked_cache_free_ids(h).tolist() == [3, 2, 1, 0, 5, 4]
    fg.fg_blocked_cache_destroy(h)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_reverse_release_restores_the_free_list(cfg):
    # the free list is a stack handed out from the front of free_ids: returning the k blocks
    # a pass took, last taken first, restores it exactly (bench.py resets each step this way)
    w = wl.make(cfg)
    free = np.asarray(w.free_ids, np.int32)
    h = fg.fg_blocked_cache_init(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                                 w.dtype, None, None, free)
    before = fg.fg_blocked_cache_free_ids(h).copy()
    ss = fg.SeqStates(w.fresh_states(), w.table_width)
    hb = fg.HostBatch(len(w.seqs), w.table_width)
    assert fg.fg_splitfuse_compose(h, ss, w.budget, hb) == fg.FG_OK
    taken = len(before) - fg.fg_blocked_cache_num_free(h)
    assert taken > 0
    assert sorted(free[:taken].tolist()) == sorted(
        b for i in range(ss.n) for b in ss.blocks[i][:ss.arr[i].n_blocks]
        if b not in w.seqs[i].blocks)
    fg.fg_blocked_cache_release(h, free[taken - 1::-1])
    assert np.array_equal(fg.fg_blocked_cache_free_ids(h), before)
    fg.fg_blocked_cache_destroy(h)


def _batch_from(qs, nq, cl, bt):
    hb = fg.HostBatch(len(nq), len(bt[0]) if bt else 1)
    S = len(nq)
    hb.query_start[:S + 1] = qs
    hb.n_query[:S] = nq
    hb.context_len[:S] = cl
    for i, row in enumerate(bt):
        hb.block_table[i, :len(row)] = row
    hb.c.num_seqs, hb.c.num_tokens = S, qs[-1]
    return hb


def test_validate_batch():
    h = fg.fg_blocked_cache_init(8, 8, 1, 128, "bf16", None, None)
    ok = _batch_from([0, 1, 4], [1, 3], [8, 0], [[0, 1, -1], [2, -1, -1]])
    fg.fg_validate_batch(h, ok)
    cases = [
        _batch_from([0, 1, 4], [1, 3], [8, 0], [[0, 1, -1], [1, -1, -1]]),   # shared block
        _batch_from([0, 1, 4], [1, 3], [8, 0], [[0, 9, -1], [2, -1, -1]]),   # out of range
        _batch_from([0, 1, 4], [1, 3], [8, 0], [[0, -1, -1], [2, -1, -1]]),  # missing block
        _batch_from([0, 1, 5], [1, 3], [8, 0], [[0, 1, -1], [2, -1, -1]]),   # prefix sum
        _batch_from([0, 0, 3], [0, 3], [8, 0], [[0, 1, -1], [2, -1, -1]]),   # empty entry
        _batch_from([0, 1, 4], [1, 3], [30, 0], [[0, 1, 3], [2, -1, -1]]),   # beyond stride
    ]
    for hb in cases:
        assert _status(fg.fg_validate_batch, h, hb) == fg.FG_E_DESC
    fg.fg_blocked_cache_destroy(h)


def test_device_entry_points_reject_bad_arguments_without_launching():
    h = fg.fg_blocked_cache_init(8, 8, 1, 128, "bf16", None, None)
    dev = fg.FgRaggedBatch()
    dev.num_seqs, dev.num_tokens = 1, 4
    # pools were never given -> FG_E_ARG before any launch
    assert _status(fg.fg_kv_append, h, dev, 1, 1, None) == fg.FG_E_ARG
    info = fg.FgPlanInfo()
    assert _status(fg.fg_ragged_attention, h, dev, info, 0, 1, 3, 1.0, 1, 0, 0, None) == fg.FG_E_ARG
    # zero tokens: nothing to do
    dev.num_tokens = 0
    assert _status(fg.fg_kv_append, h, dev, None, None, None) == fg.FG_OK
    fg.fg_blocked_cache_destroy(h)


def test_unaligned_pointers_rejected_without_launching():
    """Every kernel moves 16 bytes per access: pools, new rows, q, out and the workspace must
    be 16-byte aligned, and a pointer that is not is refused before anything is launched
    (the pointers below are never dereferenced)."""
    assert _status(fg.fg_blocked_cache_init, 8, 64, 1, 128, "bf16", 0x1008, 0x2000) == fg.FG_E_ARG
    assert _status(fg.fg_blocked_cache_init, 8, 64, 1, 128, "bf16", 0x1000, 0x2002) == fg.FG_E_ARG
    h = fg.fg_blocked_cache_init(8, 64, 1, 128, "bf16", 0x1000, 0x2000)
    dev = fg.FgRaggedBatch()
    dev.num_seqs, dev.num_tokens = 1, 4
    dev.query_start = dev.n_query = dev.context_len = dev.block_table = \
        fg.ctypes.cast(0x3000, fg.ctypes.POINTER(fg.ctypes.c_int32))
    assert _status(fg.fg_kv_append, h, dev, 0x4008, 0x5000, None) == fg.FG_E_ARG
    assert _status(fg.fg_kv_append, h, dev, 0x4000, 0x5004, None) == fg.FG_E_ARG
    info = fg.FgPlanInfo()
    for q, out, ws in ((0x4002, 0x5000, 0x6000), (0x4000, 0x5008, 0x6000),
                       (0x4000, 0x5000, 0x6004)):
        assert _status(fg.fg_ragged_attention, h, dev, info, 0x7000, q, 1, 1.0, out, ws, 64,
                       None) == fg.FG_E_ARG
    assert "aligned" in fg.fg_last_error()
    fg.fg_blocked_cache_destroy(h)


# --------------------------------------------------------------------------------------
# attention work list
# --------------------------------------------------------------------------------------

def _compose_c(w, budget=None):
    h = fg.fg_blocked_cache_init(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                                 w.dtype, None, None, w.free_ids)
    ss = fg.SeqStates(w.fresh_states(), w.table_width)
    hb = fg.HostBatch(len(w.seqs), w.table_width)
    fg.fg_splitfuse_compose(h, ss, budget or w.budget, hb)
    return h, ss, hb


def decode_plan(info, work, hkv, head_dim=128):
    """The work list as one row per record: (s, h, tok0, ntok, klo, khi, mode, group, split,
    nsplit, poff of the group's slot 0); padding records have s = -1 and group = -1."""
    ni, IW = info.num_items, fg.FG_ITEM_INTS
    assert info.work_ints == len(work) == ni * IW + info.num_work
    items = work[:ni * IW].reshape(ni, IW)
    slot = {0: fg.FG_STREAM_ROWS * (head_dim + 2), 1: fg.FG_TILE_ROWS * (head_dim + 2)}
    recs = np.full((info.num_work, 11), -1, np.int64)
    for r, code in enumerate(work[ni * IW:]):
        code = int(code)
        if code == -1:
            continue
        assert 0 <= code < ni * hkv
        s, t0, nt, klo, khi, mode, g0, sp, nsp, poff0, r0, r1 = (int(x) for x in items[code // hkv])
        h = code % hkv
        assert r0 == 0 and r1 == 0
        grp = g0 + h if g0 >= 0 else -1
        poff = poff0 + h * nsp * slot[mode] if g0 >= 0 else 0
        recs[r] = (s, h, t0, nt, klo, khi, mode, grp, sp, nsp, poff)
    return recs


def check_plan(hb, info, work, hq, hkv, head_dim=128):
    G = hq // hkv
    S = hb.num_seqs
    work = decode_plan(info, work, hkv, head_dim)
    assert info.num_work == len(work) and 0 <= info.num_groups < max(info.num_work, 1)
    main, merges = work[:info.num_work - info.num_groups], work[info.num_work - info.num_groups:]
    slot = {0: fg.FG_STREAM_ROWS * (head_dim + 2), 1: fg.FG_TILE_ROWS * (head_dim + 2)}
    groups = {}
    cover = {}
    # the main list is laid out for the 8 XCDs (record i runs on XCD i % 8) and, within an
    # XCD's sequence, for its 4 shader engines (position j on engine j % 4); each engine's
    # list is padded with null records at its end only
    assert len(main) % 32 == 0
    for k in range(8):
        for r in range(4):
            sub = main[k::8][r::4]
            null = [int(x[0]) == -1 for x in sub]
            first = null.index(True) if True in null else len(null)
            assert all(null[first:]), "padding only at a list's end"
        # every engine of an XCD gets the same number of records of each kind, +-1
        for mode in (0, 1):
            n = [sum(1 for x in main[k::8][r::4] if int(x[0]) != -1 and int(x[6]) == mode)
                 for r in range(4)]
            assert max(n) - min(n) <= 1, ("records per shader engine", mode, n)
    xcd_of_tile_group = {}
    for i, rec in enumerate(main):
        if int(rec[0]) == -1:
            assert int(rec[7]) == -1
            continue
        s, h, t0, nt, klo, khi, mode, grp, sp, nsp, poff = (int(x) for x in rec)
        if mode == 1 and hkv % 8 == 0:  # tile records of one (sequence, head) share an XCD
            assert xcd_of_tile_group.setdefault((s, h), i % 8) == i % 8
    for rec in main:
        if int(rec[0]) == -1:
            continue
        s, h, t0, nt, klo, khi, mode, grp, sp, nsp, poff = (int(x) for x in rec)
        assert 0 <= s < S and 0 <= h < hkv and nt >= 1 and sp >= 0
        assert mode == (0 if nt * G <= fg.FG_STREAM_ROWS else 1) and nt * G <= fg.FG_TILE_ROWS
        c, n = int(hb.context_len[s]), int(hb.n_query[s])
        assert 0 <= t0 and t0 + nt <= n
        assert klo % 64 == 0 and klo < khi <= c + t0 + nt
        key = (s, h, t0, nt)
        cover.setdefault(key, []).append((klo, khi, grp, sp, nsp, poff, mode))
    # each sequence's tokens are covered exactly once per KV head
    for s in range(S):
        for h in range(hkv):
            toks = sorted((t0, nt) for (ss_, hh, t0, nt) in cover if ss_ == s and hh == h)
            pos = 0
            for t0, nt in toks:
                assert t0 == pos
                pos += nt
            assert pos == int(hb.n_query[s])
    # split groups partition the key range in split order; partial slots are disjoint
    spans = []
    for (s, h, t0, nt), recs in cover.items():
        c = int(hb.context_len[s])
        recs.sort(key=lambda r: r[3])
        if len(recs) == 1 and recs[0][2] == -1:
            assert recs[0][0] == 0 and recs[0][1] == c + t0 + nt
            continue
        grp, nsp, poff, mode = recs[0][2], recs[0][4], recs[0][5], recs[0][6]
        assert grp >= 0 and len(recs) == nsp > 1 and grp not in groups
        groups[grp] = (s, h, t0, nt, mode, nsp, poff)
        assert [r[3] for r in recs] == list(range(nsp))
        assert recs[0][0] == 0 and recs[-1][1] == c + t0 + nt
        for a, b in zip(recs, recs[1:]):
            assert a[1] == b[0]
        assert all(r[2] == grp and r[5] == poff for r in recs)
        spans.append((poff, poff + nsp * slot[mode]))
    assert sorted(groups) == list(range(info.num_groups))
    spans.sort()
    for a, b in zip(spans, spans[1:]):
        assert a[1] <= b[0]
    if spans:
        assert spans[0][0] >= 0 and spans[-1][1] * 4 <= info.workspace_bytes
    # one merge record per group, in group order, naming the group's rows and slots (the
    # record of its split 0)
    assert len(merges) == info.num_groups
    for g, rec in enumerate(merges):
        s, h, t0, nt, klo, khi, mode, grp, sp, nsp, poff = (int(x) for x in rec)
        assert grp == g and sp == 0
        assert groups[g] == (s, h, t0, nt, mode, nsp, poff)


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_plan_invariants_on_workloads(cfg):
    w = wl.make(cfg)
    h, ss, hb = _compose_c(w)
    info, work = fg.fg_attention_plan(h, hb, w.num_q_heads, 256)
    check_plan(hb, info, work, w.num_q_heads, w.num_kv_heads)
    fg.fg_blocked_cache_destroy(h)


def test_plan_invariants_chunked_prefill_passes():
    w = wl.make(4)
    h = fg.fg_blocked_cache_init(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                                 w.dtype, None, None, w.free_ids)
    ss = fg.SeqStates(w.fresh_states(), w.table_width)
    for k in range(w.passes):
        hb = fg.HostBatch(1, w.table_width)
        fg.fg_splitfuse_compose(h, ss, w.budget, hb)
        info, work = fg.fg_attention_plan(h, hb, 32, 256)
        check_plan(hb, info, work, 32, 32)
        fg.fg_splitfuse_commit(ss)
    fg.fg_blocked_cache_destroy(h)


@pytest.mark.parametrize("hq,hkv,num_cus", [(8, 8, 4), (12, 4, 16), (32, 1, 8), (16, 2, 1)])
def test_plan_invariants_random(hq, hkv, num_cus):
    rng = np.random.Generator(np.random.PCG64(hq * 100 + hkv))
    for trial in range(20):
        w = wl.custom(int(rng.integers(1 << 30)), hq=hq, hkv=hkv, budget=int(rng.integers(1, 700)),
                      n_decode=int(rng.integers(0, 6)), decode_ctx=(0, 3000),
                      prompts=((int(rng.integers(0, 900)), 1500), (0, 400)))
        h, ss, hb = _compose_c(w)
        info, work = fg.fg_attention_plan(h, hb, hq, num_cus)
        check_plan(hb, info, work, hq, hkv)
        fg.fg_blocked_cache_destroy(h)


def test_plan_errors():
    w = wl.make(2)
    h, ss, hb = _compose_c(w)
    assert _status(fg.fg_attention_plan, h, hb, 31, 256) == fg.FG_E_ARG       # Hq % Hkv
    assert _status(fg.fg_attention_plan, h, hb, 32, 0) == fg.FG_E_ARG        # no CUs
    info = fg.FgPlanInfo()
    work = np.zeros(12, np.int32)
    st = fg.lib().fg_attention_plan(h, ctypes.byref(hb.c), 32, 256, ctypes.byref(info),
                                    work.ctypes.data_as(fg.i32p), 12)
    assert st == fg.FG_E_ARG and info.work_ints > 12                          # capacity
    fg.fg_blocked_cache_destroy(h)


def test_plan_fp32_needs_no_records():
    w = wl.make(1)
    h, ss, hb = _compose_c(w)
    for buf in (None, np.zeros(96, np.int32)):
        info, work = fg.fg_attention_plan(h, hb, w.num_q_heads, 256, buf)
        assert info.num_work == 0 and info.work_ints == 0 and work.shape == (0,)
        assert info.num_tokens == hb.num_tokens and info.workspace_bytes == 0
    fg.fg_blocked_cache_destroy(h)


def test_plan_reuses_a_large_enough_buffer():
    w = wl.make(2)
    h, ss, hb = _compose_c(w)
    info0, work0 = fg.fg_attention_plan(h, hb, 32, 256)
    buf = np.zeros(info0.work_ints + 5, np.int32)
    info1, work1 = fg.fg_attention_plan(h, hb, 32, 256, buf)
    assert work1.base is buf and np.array_equal(work0, work1)
    small = np.zeros(36, np.int32)
    info2, work2 = fg.fg_attention_plan(h, hb, 32, 256, small)
    assert np.array_equal(work0, work2)
    fg.fg_blocked_cache_destroy(h)


# --------------------------------------------------------------------------------------
# work-list validation (the check FG_VALIDATE=1 runs on device copies) and workspace sizing
# --------------------------------------------------------------------------------------

def _planned(cfg=None, w=None, num_cus=256):
    w = w or wl.make(cfg)
    h, ss, hb = _compose_c(w)
    info, work = fg.fg_attention_plan(h, hb, w.num_q_heads, num_cus)
    return w, h, hb, info, np.array(work)


def test_validate_work_accepts_every_planned_list():
    for cfg in (2, 3, 5):
        w, h, hb, info, work = _planned(cfg)
        fg.fg_validate_work(h, hb, info, work, info.workspace_bytes)
        fg.fg_blocked_cache_destroy(h)
    # split groups present (a huge CU count forces the finest key splits)
    w, h, hb, info, work = _planned(2, num_cus=100000)
    assert info.num_groups > 0
    fg.fg_validate_work(h, hb, info, work, info.workspace_bytes)
    assert _status(fg.fg_validate_work, h, hb, info, work, info.workspace_bytes - 4) == fg.FG_E_DESC
    fg.fg_blocked_cache_destroy(h)


def test_validate_work_rejects_corrupted_lists():
    """Each plausible corruption of a valid list is caught (FG_E_DESC, a named violation)."""
    IW = fg.FG_ITEM_INTS
    w, h, hb, info, work = _planned(2, num_cus=100000)
    ni, hkv = info.num_items, w.num_kv_heads
    items = lambda a: a[:ni * IW].reshape(ni, IW)
    codes = lambda a: a[ni * IW:]
    split_item = next(i for i in range(ni) if items(work)[i][6] >= 0 and items(work)[i][7] == 1)
    plain_item = next(i for i in range(ni) if items(work)[i][6] < 0)
    main = info.num_work - info.num_groups
    first_real = next(r for r in range(main) if codes(work)[r] >= 0)
    muts = {
        "sequence out of range": lambda a: items(a).__setitem__((0, 0), hb.num_seqs),
        "tokens past the sequence": lambda a: items(a).__setitem__((plain_item, 2), 10**6),
        "unaligned key start": lambda a: items(a).__setitem__((split_item, 3), items(a)[split_item][3] + 1),
        "keys past the row's limit": lambda a: items(a).__setitem__((plain_item, 4), items(a)[plain_item][4] + 1),
        "keys short of the row's limit": lambda a: items(a).__setitem__((plain_item, 4), items(a)[plain_item][4] - 1),
        "bad mode": lambda a: items(a).__setitem__((0, 5), 7),
        "split gap": lambda a: items(a).__setitem__((split_item, 3), items(a)[split_item][3] + 64),
        "partials outside the workspace": lambda a: items(a).__setitem__((split_item, 9), 1 << 30),
        "record repeated": lambda a: codes(a).__setitem__(first_real + 1, codes(a)[first_real]),
        "record out of range": lambda a: codes(a).__setitem__(first_real, ni * hkv),
        "merge record names a plain item": lambda a: codes(a).__setitem__(main, plain_item * hkv),
    }
    for name, mut in muts.items():
        bad = work.copy()
        mut(bad)
        assert _status(fg.fg_validate_work, h, hb, info, bad, info.workspace_bytes) == fg.FG_E_DESC, name
        assert fg.fg_last_error(), name
    # a plan made for another token count
    other = fg.FgPlanInfo.from_buffer_copy(info)
    other.num_tokens += 1
    assert _status(fg.fg_validate_work, h, hb, other, work, info.workspace_bytes) == fg.FG_E_DESC
    fg.fg_blocked_cache_destroy(h)


def test_workspace_size_matches_the_plan():
    for cfg, cus in ((2, 256), (2, 100000), (3, 256), (4, 256), (5, 256), (5, 7)):
        w = wl.make(cfg)
        h, ss, hb = _compose_c(w)
        info, _ = fg.fg_attention_plan(h, hb, w.num_q_heads, cus)
        assert fg.fg_ragged_attention_workspace_size(h, hb, w.num_q_heads, cus) == info.workspace_bytes
        fg.fg_blocked_cache_destroy(h)
    w = wl.make(2)
    h, ss, hb = _compose_c(w)
    assert _status(fg.fg_ragged_attention_workspace_size, h, hb, 31, 256) == fg.FG_E_ARG
    n = ctypes.c_size_t(0)
    assert fg.lib().fg_ragged_attention_workspace_size(h, ctypes.byref(hb.c), 32, 256, None) == fg.FG_E_ARG
    fg.fg_blocked_cache_destroy(h)


def test_noalloc_rejects_plans_beyond_its_scratch():
    """The fixed-scratch attention refuses a plan whose split partials exceed the scratch,
    before any device call (so this runs without a GPU)."""
    h = fg.fg_blocked_cache_init(8, 64, 1, 128, "bf16", 0x1000, 0x2000)
    dev = fg.FgRaggedBatch()
    dev.num_seqs, dev.num_tokens = 1, 4
    info = fg.FgPlanInfo()
    info.workspace_bytes = fg.FG_NOALLOC_WORKSPACE_BYTES + 1
    info.num_q_heads, info.num_tokens = 1, 4
    assert _status(fg.fg_ragged_attention_noalloc, h, dev, info, 0x7000, 0x4000, 1, 1.0, 0x5000,
                   None) == fg.FG_E_WORKSPACE
    assert "scratch" in fg.fg_last_error()
    fg.fg_blocked_cache_destroy(h)


def test_linear_argument_errors():
    """Both projection entry points reject bad arguments before launching anything (so this
    runs without a GPU): T = 0 is a no-op, null or unaligned pointers and negative sizes are
    FG_E_ARG, widths off the tile grid are FG_E_UNSUPPORTED."""
    L = fg.lib()
    a = 4096  # an aligned stand-in address: never dereferenced on these paths
    qkv = L.fg_linear_qkv_bf16
    assert qkv(None, None, None, None, None, 0, 64, 128, 128, None) == fg.FG_OK
    assert qkv(None, None, None, None, None, 4, 64, 128, 128, None) == fg.FG_E_ARG
    assert qkv(a, a, a, a, a + 8, 4, 64, 128, 128, None) == fg.FG_E_ARG
    assert qkv(a, a, a, a, a, -1, 64, 128, 128, None) == fg.FG_E_ARG
    assert qkv(a, a, a, a, a, 4, 64, 0, 128, None) == fg.FG_E_ARG
    assert qkv(a, a, a, a, a, 4, 64, 128, 100, None) == fg.FG_E_UNSUPPORTED
    assert qkv(a, a, a, a, a, 4, 96, 128, 128, None) == fg.FG_E_UNSUPPORTED
    lin = L.fg_linear_bf16
    assert lin(None, None, None, 0, 64, 128, None) == fg.FG_OK
    assert lin(None, a, a, 4, 64, 128, None) == fg.FG_E_ARG
    assert lin(a, a, a + 4, 4, 64, 128, None) == fg.FG_E_ARG
    assert lin(a, a, a, 4, 64, 192, None) == fg.FG_E_UNSUPPORTED
    assert lin(a, a, a, 4, 100, 128, None) == fg.FG_E_UNSUPPORTED
