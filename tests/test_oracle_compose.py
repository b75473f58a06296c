"""The oracle's composition policy: hand fixture, exhaustive tiny queues, multi-pass coverage."""
import numpy as np
import pytest

import oracle
import oracle.compose as oc
import oracle_pins as pins
import harness
from ragged_blocked_kv_splitfuse_amd import workloads as wl


def test_golden_queue():
    assert pins.check_golden_compose(oc)


def test_exhaustive_tiny_queues():
    assert pins.check_compose_exhaustive(oc) is None


def test_multipass_every_prompt_token_once():
    assert pins.check_multipass_coverage(oc, oc.commit_pass) is None


def test_no_blocks_status():
    seqs = [oc.SeqState(1, 4, 4, [0], 4)]     # decode at a block boundary, empty pool
    batch, status = oc.splitfuse_compose(seqs, 8, oc.FreeList([]), 4, 4)
    assert status == "no_blocks" and batch.num_seqs == 0


def test_budget_must_be_positive():
    with pytest.raises(ValueError):
        oc.splitfuse_compose([], 0, oc.FreeList([]), 4, 4)


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_workload_composition_shapes(cfg):
    """The generated workloads compose into the passes their descriptions promise."""
    w = wl.make(cfg)
    states = harness.oracle_states(w)
    batch, status = oc.splitfuse_compose(states, w.budget, oc.FreeList(w.free_ids),
                                         w.block_size, w.table_width)
    assert status == "ok"
    assert batch.num_tokens == w.budget
    dec = [k for k in range(batch.num_seqs)
           if states[batch.seq_index[k]].prompt_len <= batch.context_len[k]]
    if cfg == 1:
        assert batch.num_seqs == 4 and len(dec) == 2
        assert all(batch.n_query[k] == 1 for k in dec)
    if cfg == 2:
        assert len(dec) == 24
    if cfg == 3:
        assert len(dec) == 256 and batch.num_seqs == 256
    if cfg == 5:
        assert len(dec) == 64


def test_chunked_prefill_passes():
    w = wl.make(4)
    states = harness.oracle_states(w)
    free = oc.FreeList(w.free_ids)
    for k in range(w.passes):
        batch, status = oc.splitfuse_compose(states, w.budget, free, w.block_size, w.table_width)
        assert batch.num_seqs == 1
        assert int(batch.context_len[0]) == 512 * k and int(batch.n_query[0]) == 512
        oc.commit_pass(states)
    assert states[0].n_cached == 16384
