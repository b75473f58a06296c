"""The oracle against brute force, hand-derived values, closed forms and invariants."""
import numpy as np

import oracle
import oracle.compose as oc
import oracle_pins as pins


def test_bruteforce_tiny():
    assert pins.check_bruteforce(oracle.ragged_attention, oracle.kv_append, oc) < 1e-12


def test_golden_hand_example():
    assert pins.check_golden_attention(oracle.ragged_attention, oracle.kv_append) < 1e-6


def test_closed_forms():
    assert pins.check_closed_forms(oracle.ragged_attention) < 1e-12


def test_block_permutation_invariance_bit_identical():
    assert pins.check_permutation_invariance(oracle.ragged_attention, oracle.kv_append, oc)


def test_splitfuse_chunk_invariance():
    assert pins.check_chunk_invariance(oracle.ragged_attention, oracle.kv_append, oc) < 1e-13


def test_gqa_equals_repeated_kv_heads():
    """Hq/Hkv = G with contiguous groups equals MHA with each KV head repeated G times."""
    from ragged_blocked_kv_splitfuse_amd import workloads as wl
    import harness
    w = wl.custom(41, dtype="f32", hq=6, hkv=2, d=8, bs=4, budget=12, n_decode=2,
                  decode_ctx=(3, 10), prompts=((2, 20),))
    res = harness.oracle_pass(w)
    G = 3
    kp = np.repeat(res["k_pool"], G, axis=1)
    vp = np.repeat(res["v_pool"], G, axis=1)
    mha = oracle.ragged_attention(res["q"], kp, vp, res["batch"], 6, 6, w.scale,
                                  w.block_size, w.dtype)
    assert np.array_equal(mha, res["out"])


def test_empty_pass():
    from oracle.compose import OracleBatch
    b = OracleBatch(np.zeros(1, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32),
                    np.zeros((0, 4), np.int32), np.zeros(0, np.int32), np.zeros(0, np.int64))
    out = oracle.ragged_attention(np.zeros((0, 2, 8), np.float32), np.zeros((4, 2, 4, 8), np.float32),
                                  np.zeros((4, 2, 8, 4), np.float32), b, 2, 2, 1.0, 4, "f32")
    assert out.shape == (0, 2, 8)
