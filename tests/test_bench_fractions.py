"""The bench line's roofline arithmetic, checked against hand-computed values: the two
combinations of the HBM and MFMA bounds (the larger of the two roofline times, and their sum),
and the fraction each per-config entry reports for its bound."""
import types

import pytest

import bench


def test_bound_fractions_by_hand():
    # 8 GB at 8 TB/s is 1 ms of HBM time; 2.5 TFLOP at 2.5 PFLOP/s is 1 ms of MFMA time
    f = bench.bound_fracs(8e9, 2.5e12, 4e-3)
    assert f["max_bound_frac"] == pytest.approx(0.25)
    assert f["additive_bound_frac"] == pytest.approx(0.5)
    # an HBM-bound pass: the MFMA time (0.1 ms) only enters the additive bound
    f = bench.bound_fracs(8e9, 2.5e11, 2e-3)
    assert f["max_bound_frac"] == pytest.approx(0.5)
    assert f["additive_bound_frac"] == pytest.approx(0.55)


def _timed(B, F, t_attn, t_app=1e-5):
    info = types.SimpleNamespace(num_groups=0, num_work=1)
    return {"t_attn": t_attn, "t_app": t_app, "attn_bytes": B, "attn_flops": F, "T": 2048,
            "nseq": 1, "append_bytes": 1e6, "host_s": [0.0] * 4, "elapsed": 1e-3, "info": info}


@pytest.mark.parametrize("bound,expect", [("hbm", 0.5), ("mfma", 0.2), ("hbm+mfma", 0.5)])
def test_config_entry_fraction_follows_its_bound(bound, expect):
    w = types.SimpleNamespace(name="x")
    # 4 GB in 1 ms is 4 TB/s = 0.5 of HBM; 0.5 TFLOP in 1 ms is 500 TFLOP/s = 0.2 of MFMA
    e = bench.config_entry(w, _timed(4e9, 5e11, 1e-3), bound)
    assert e["frac"] == pytest.approx(expect)
    assert e["hbm_frac"] == pytest.approx(0.5) and e["mfma_frac"] == pytest.approx(0.2)
    assert e["max_bound_frac"] == pytest.approx(0.5)
    assert e["additive_bound_frac"] == pytest.approx(0.7)
