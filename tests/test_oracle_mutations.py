"""Planted mistakes in copies of the oracle must be caught by at least one pin.

Each mutation rewrites one line of an oracle module's source, executes the
copy as a throwaway module (the oracle package itself is left untouched) and
runs the pins against it.  This shows the pins would notice a dropped term, a
wrong sign, index or offset, or a transposed operand.
"""
import os
import sys
import types

import pytest

import oracle
import oracle.compose as real_compose
import oracle_pins as pins

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def mutant(fname, old, new):
    path = os.path.join(ORACLE, fname)
    with open(path) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found in {fname}: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle._mutant_" + fname[:-3])
    mod.__package__ = "oracle"
    mod.__file__ = path
    sys.modules[mod.__name__] = mod          # dataclasses look the module up
    try:
        exec(compile(src, path, "exec"), mod.__dict__)
    finally:
        sys.modules.pop(mod.__name__, None)
    return mod


def caught_attention(attn, append=oracle.kv_append, compose=real_compose):
    checks = [
        lambda: pins.check_bruteforce(attn, append, compose) < 1e-12,
        lambda: pins.check_golden_attention(attn, append) < 1e-6,
        lambda: pins.check_closed_forms(attn) < 1e-12,
        lambda: pins.check_permutation_invariance(attn, append, compose),
        lambda: pins.check_chunk_invariance(attn, append, compose) < 1e-13,
    ]
    for chk in checks:
        try:
            if not chk():
                return True
        except Exception:  # noqa: BLE001  (a crash is a detection too)
            return True
    return False


ATTN_MUTATIONS = [
    ("keys <= c + rows", "keys < c + rows"),                 # diagonal excluded
    ("keys <= c + rows", "keys <= c + rows + 1"),            # one future key leaks in
    ("keys <= c + rows", "keys <= rows"),                    # causal offset ignores the context
    (") * scale", ")"),                                      # scale dropped
    ("h = g // group", "h = g % num_kv_heads"),              # interleaved GQA groups
    ("V.transpose(1, 0, 2, 4, 3)", "V.transpose(1, 0, 2, 3, 4)"),  # V group read key-major
    ("w.sum(axis=1, keepdims=True)", "w.sum()"),             # wrong normaliser
    ("visible = c + i1", "visible = c + i1 - 1"),            # last key dropped
    ("blocks = np.asarray(table_row[:nb]", "blocks = np.asarray(table_row[1:nb + 1]"),
    ("np.exp(logits - m)", "np.exp(logits - m) + 1e-9"),   # stray additive term
]


@pytest.mark.parametrize("old,new", ATTN_MUTATIONS)
def test_attention_mutation_caught(old, new):
    m = mutant("attention.py", old, new)
    assert caught_attention(m.ragged_attention)


APPEND_MUTATIONS = [
    ("slot = p % block_size", "slot = (p + 1) % block_size"),
    ("p = c + i", "p = i"),
    ("v_pool[blk, :, grp, :, j]", "v_pool[blk, :, j % v_pool.shape[2], :, grp % v_pool.shape[4]]"),
    ("grp, j = v_slot(block_size, slot)", "grp, j = v_slot(block_size, slot)[::-1]"),
    ("block_table[s, p // block_size]", "block_table[s, p % block_size]"),
]


@pytest.mark.parametrize("old,new", APPEND_MUTATIONS)
def test_append_mutation_caught(old, new):
    m = mutant("append.py", old, new)
    assert caught_attention(oracle.ragged_attention, append=m.kv_append)


COMPOSE_MUTATIONS = [
    ("if s.n_cached >= s.prompt_len:\n            n = _grant(s, 1",
     "if False:\n            n = _grant(s, 1"),                             # decodes never served
    ("            left -= n\n    # then", "            left -= 0\n    # then"),  # budget ignored
    ("min(s.prompt_len - s.n_cached, left)", "s.prompt_len - s.n_cached"),  # prompt never cut
    ("need_blocks = -(-(c + want) // block_size)", "need_blocks = (c + want) // block_size"),
    ("[int(b) for b in reversed(list(ids))]", "[int(b) for b in list(ids)]"),
    ("for s in seqs:\n        if left == 0:\n            break\n        if s.n_cached < s.prompt_len",
     "for s in reversed(seqs):\n        if left == 0:\n            break\n        if s.n_cached < s.prompt_len"),
]


@pytest.mark.parametrize("old,new", COMPOSE_MUTATIONS)
def test_compose_mutation_caught(old, new):
    m = mutant("compose.py", old, new)
    checks = [
        lambda: pins.check_golden_compose(m),
        lambda: pins.check_compose_exhaustive(m) is None,
        lambda: pins.check_multipass_coverage(m, m.commit_pass) is None,
    ]
    caught = False
    for chk in checks:
        try:
            if not chk():
                caught = True
                break
        except Exception:  # noqa: BLE001
            caught = True
            break
    assert caught
