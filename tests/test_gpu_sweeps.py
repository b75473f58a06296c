"""Parity of the profiling sweeps' pass shapes (uniform passes: S sequences of n new tokens
over c cached ones), each whole against the oracle, at reduced cached lengths."""
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import gpu_harness as G
from ragged_blocked_kv_splitfuse_amd import workloads as wl
from ragged_blocked_kv_splitfuse_amd.runtime import num_cus


@pytest.mark.parametrize("S,n,c", [(1, 2048, 512), (16, 128, 512), (64, 32, 512),
                                   (2048, 1, 64), (256, 1, 1024)])
def test_uniform_pass(S, n, c):
    w = wl.uniform_pass(S, n, c)
    r = G.full_pass(w, num_cus=num_cus())
    G.assert_close(G.out_to_f64(r["out"]), r["ref"], "bf16", w.name)
