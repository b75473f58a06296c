"""Host side of the profiling sweeps: every sweep point composes to the pass it names
(S sequences of n new tokens each over c cached ones, T = S*n), and the composed batch
matches the oracle's composition."""
import numpy as np
import pytest

import bench
import harness
import oracle
from ragged_blocked_kv_splitfuse_amd import fg, workloads as wl

POINTS = bench.SWEEP_S + bench.SWEEP_T_CHUNK + bench.SWEEP_T_DECODE


@pytest.mark.parametrize("S,n,c", POINTS)
def test_sweep_point_composes_to_its_shape(S, n, c):
    w = wl.uniform_pass(S, n, c)
    h = fg.fg_blocked_cache_init(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                                 w.dtype, 0, 0, np.asarray(w.free_ids, np.int32))
    try:
        ss = fg.SeqStates(w.fresh_states(), w.table_width)
        hb = fg.HostBatch(ss.n, w.table_width)
        assert fg.fg_splitfuse_compose(h, ss, w.budget, hb) == fg.FG_OK
        assert hb.num_seqs == S and hb.num_tokens == S * n
        assert (hb.n_query[:S] == n).all() and (hb.context_len[:S] == c).all()
        fg.fg_validate_batch(h, hb)
        info, work = fg.fg_attention_plan(h, hb, w.num_q_heads, 256)
        assert info.num_work > 0
    finally:
        fg.fg_blocked_cache_destroy(h)
    if S * (c + n) <= 4096:
        ob, st = oracle.splitfuse_compose(harness.oracle_states(w), w.budget,
                                          oracle.FreeList(w.free_ids), w.block_size,
                                          w.table_width)
        assert st == "ok"
        assert np.array_equal(ob.block_table, hb.block_table[:S])
