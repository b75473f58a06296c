"""bench.main() assembles its one JSON line from the timed passes without touching anything it
has already released: the GPU-side pieces (pool setup, the timed passes, the practical-rate
references) are replaced by stand-ins with the same fields, and the default invocation (the
per-config block included) and the headline-only one must both print a complete line."""
import json
import sys
import types

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import bench


def _fake_pass(T=2048, nseq=26):
    info = types.SimpleNamespace(num_work=1056, num_groups=0)
    return {"info": info, "T": T, "nseq": nseq, "nq": np.ones(nseq, np.int64),
            "ctx": np.full(nseq, 1000, np.int64), "kv_tokens": 60000,
            "attn_bytes": 1.126e9, "attn_flops": 4.6e10, "append_bytes": 6.7e7,
            "t_attn": 200e-6, "t_app": 20e-6, "elapsed": 50 * 230e-6,
            "q": None, "k_new": None, "v_new": None,
            "host_s": [55e-6] * 50, "wait_s": [150e-6] * 50}


@pytest.mark.parametrize("per_config", ["1", "0"])
def test_main_prints_one_complete_line(monkeypatch, capsys, per_config):
    w = types.SimpleNamespace(name="llama2_7b_mixed", num_q_heads=32, num_kv_heads=32, head_dim=128,
                              block_size=64, budget=2048, dtype="bf16")
    monkeypatch.setattr(torch.cuda, "set_device", lambda *a: None)
    monkeypatch.setattr(torch.cuda, "empty_cache", lambda: None)
    monkeypatch.setattr(bench, "setup", lambda args, name=None: {"w": w, "cache": None, "hb": None})
    monkeypatch.setattr(bench, "time_pass", lambda S, steps, warmup: _fake_pass())
    monkeypatch.setattr(bench, "hbm_reference", lambda **kw: {"copy_GBps": 1.0})
    monkeypatch.setattr(bench, "mfma_reference", lambda **kw: {"gemm_8192_TFLOPs": 1.0})
    monkeypatch.setattr(sys, "argv", ["bench.py", "--cpu-seconds", "0", "--per-config", per_config])
    bench.main()
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "kernels", "cpu_baseline"):
        assert k in d, k
    assert d["value"] == pytest.approx(2048 * d["steps"] / (50 * 230e-6))
    assert d["kernels"]["host_us_per_step"] == pytest.approx(55.0)
    assert d["kernels"]["host_wait_us_per_step"] == pytest.approx(150.0)
    assert d["roofline"]["bound"] == "hbm"
    assert d["roofline"]["frac"] == pytest.approx(1.126e9 / 200e-6 / 8e12)
    if per_config == "1":
        assert set(d["per_config"]) == {"llama2", "decode", "chunked", "mistral"}
        assert d["hbm_reference"] and d["mfma_reference"]
    else:
        assert d["per_config"] is None and d["mfma_reference"] is None
