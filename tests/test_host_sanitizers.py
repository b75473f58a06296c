"""The host library built with AddressSanitizer + UBSan (g++, host code only), driven
through the same ABI calls in a child process.  Catches out-of-bounds and undefined
behaviour in composition, allocation, validation and planning."""
import os
import subprocess
import sys

import pytest

from ragged_blocked_kv_splitfuse_amd import build as B

DRIVER = r'''
import sys, numpy as np
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + "/tests")
from ragged_blocked_kv_splitfuse_amd import fg, workloads as wl
fg.load(sys.argv[2])
import test_host_abi as T
for cfg in (1, 2, 3, 5):
    w = wl.make(cfg)
    h, ss, hb = T._compose_c(w)
    fg.fg_validate_batch(h, hb)
    if w.dtype == "bf16":
        info, work = fg.fg_attention_plan(h, hb, w.num_q_heads, 256)
        T.check_plan(hb, info, work, w.num_q_heads, w.num_kv_heads)
    fg.fg_splitfuse_commit(ss)
    for i in range(ss.n):
        fg.fg_blocked_cache_release(h, ss.owned(i))
    fg.fg_blocked_cache_destroy(h)
T.test_compose_matches_oracle_random_queues()
T.test_compose_errors_and_no_state_change()
T.test_release_errors_and_reuse_order()
T.test_validate_batch()
T.test_plan_errors()
T.test_plan_invariants_chunked_prefill_passes()
print("SANITIZED-OK")
'''


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], stdout=subprocess.PIPE, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_host_library_under_asan_ubsan():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("libasan not available")
    B.build_host_asan()
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", DRIVER, B.ROOT, B.HOST_ASAN_LIB], env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0 and "SANITIZED-OK" in r.stdout, r.stdout[-4000:]
