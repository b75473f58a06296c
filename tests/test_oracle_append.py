"""The oracle's scatter append: hand-derived slots, sentinel preservation, bit copy."""
import numpy as np

import oracle
import oracle_pins as pins
import harness
from ragged_blocked_kv_splitfuse_amd import workloads as wl


def test_golden_slots_and_sentinels():
    # the golden check also verifies every untouched slot kept its sentinel bits
    assert pins.check_golden_attention(oracle.ragged_attention, oracle.kv_append) < 1e-6


def test_append_is_bit_copy_and_touches_only_new_slots():
    w = wl.custom(12, dtype="bf16", hq=4, hkv=2, d=8, bs=4, budget=15, n_decode=3,
                  decode_ctx=(0, 13), prompts=((3, 30),), extra_blocks=3)
    states = harness.oracle_states(w)
    kp, vp = harness.empty_pools(w)
    harness.fill_history(w, kp, vp, states)
    k0, v0 = kp.copy(), vp.copy()
    batch, st = oracle.splitfuse_compose(states, w.budget, oracle.FreeList(w.free_ids),
                                         w.block_size, w.table_width)
    q, kn, vn = harness.new_rows(w, batch, states)
    oracle.kv_append(kp, vp, kn, vn, batch, w.block_size)
    # count changed elements: exactly T * Hkv * D in each pool (sentinels differ from data)
    T = batch.num_tokens
    assert int(np.sum(kp != k0)) == T * w.num_kv_heads * w.head_dim
    assert int(np.sum(vp != v0)) == T * w.num_kv_heads * w.head_dim
    # and the written bit patterns are exactly the new rows' bit patterns (as multisets)
    assert np.array_equal(np.sort(kp[kp != k0]), np.sort(kn.reshape(-1)))
    assert np.array_equal(np.sort(vp[vp != v0]), np.sort(vn.reshape(-1)))
