"""Randomised parity of the HIP path with the oracle: seeded draws of head grouping (MHA, GQA,
MQA), block size, budget, decode contexts, prompt chunks (fresh and continued), logit spread and
planner granularity (the device's compute units, or a huge count that forces the finest key
splits).  kv_append must be bit-exact on both pools and attention within the bf16 tolerance
(max-abs 2e-2, mean-abs 2e-3).  Sizes are kept small enough for the oracle to finish in
seconds while still spanning several key tiles, ragged tails and both record kinds."""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import gpu_harness as G
from ragged_blocked_kv_splitfuse_amd import workloads as wl

# Seeds per draw family; FG_RANDOM_SEEDS=n widens the sweep to n bf16 draws at head dim 128,
# n/2 at head dim 64 and n/4 in fp32 (the defaults keep the suite to seconds).
N_SEEDS = int(os.environ.get("FG_RANDOM_SEEDS", "24"))


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def draw_case(seed):
    """One seeded random pass shape; returns (custom kwargs, planner compute units)."""
    rng = np.random.Generator(np.random.PCG64(90000 + seed))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 8]))
    while hkv * g > 32:
        g //= 2
    bs = int(rng.choice([8, 16, 32, 64, 128]))
    n_decode = int(rng.integers(0, 7))
    lo = int(rng.integers(0, 200))
    hi = lo + int(rng.integers(0, 1800))
    prompts = []
    for _ in range(int(rng.integers(1, 3))):
        L = int(rng.integers(1, 1200))
        c = int(rng.integers(0, L)) if rng.random() < 0.5 else 0
        prompts.append((c, L))
    demand = n_decode + sum(L - c for c, L in prompts)
    budget = int(rng.integers(max(1, n_decode), min(demand, 320) + 1))
    # One case in three has steep logits (spread ~8): the softmax is then nearly one-hot, so O
    # is close to single V rows.  Values are halved there (value_scale 0.5, a narrowing of the
    # inputs, not of the bound): rounding to bf16 (unit roundoff 2^-8) carries an error of up
    # to 2^-8 |O| by itself, which alone reaches the 2e-2 bound once |O| > 5.12, and N(0, 1)
    # rows drawn by the thousand reach |v| ~ 4-5.
    steep = rng.random() < 1 / 3
    q_scale, value_scale = (32.0, 0.5) if steep else (1.0, 1.0)
    cus = int(rng.choice([256, 100000]))
    kw = dict(hq=hkv * g, hkv=hkv, bs=bs, budget=budget, n_decode=n_decode, decode_ctx=(lo, hi),
              prompts=tuple(prompts), q_scale=q_scale, value_scale=value_scale)
    return kw, cus


@pytest.mark.parametrize("seed", range(N_SEEDS))
def test_random_pass(seed):
    kw, cus = draw_case(seed)
    G.say(f"random case {seed}: {kw}, num_cus {cus}")
    w = wl.custom(70000 + seed, **kw)
    r = G.full_pass(w, num_cus=cus)
    dt = np.uint16
    assert np.array_equal(G.to_host_bits(r["gp"].cache.k_pool, "bf16").view(dt), r["k_pool"].view(dt))
    assert np.array_equal(G.to_host_bits(r["gp"].cache.v_pool, "bf16").view(dt), r["v_pool"].view(dt))
    G.assert_close(G.out_to_f64(r["out"]), r["ref"], "bf16", f"random[{seed}]")


def draw_case_f32(seed):
    """A seeded random fp32 pass shape (the accuracy path): head dims 64 and 128, small blocks."""
    rng = np.random.Generator(np.random.PCG64(95000 + seed))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([2, 8, 16, 64]))
    n_decode = int(rng.integers(0, 5))
    lo = int(rng.integers(0, 100))
    hi = lo + int(rng.integers(0, 600))
    prompts = []
    for _ in range(int(rng.integers(1, 3))):
        L = int(rng.integers(1, 400))
        c = int(rng.integers(0, L)) if rng.random() < 0.5 else 0
        prompts.append((c, L))
    demand = n_decode + sum(L - c for c, L in prompts)
    budget = int(rng.integers(max(1, n_decode), min(demand, 160) + 1))
    # fp32 rounding of the logits is amplified by the exponential: with a logit spread of 8
    # plain fp32 arithmetic already lands ~1e-5 from the float64 result at head_dim 128, so
    # the steeper draws here stop at a spread of 3.
    q_scale = float(rng.choice([1.0, 3.0]))
    return dict(dtype="f32", hq=hkv * g, hkv=hkv, d=d, bs=bs, budget=budget, n_decode=n_decode,
                decode_ctx=(lo, hi), prompts=tuple(prompts), q_scale=q_scale)


@pytest.mark.parametrize("seed", range(max(8, N_SEEDS // 4)))
def test_random_pass_f32(seed):
    kw = draw_case_f32(seed)
    G.say(f"random fp32 case {seed}: {kw}")
    w = wl.custom(80000 + seed, **kw)
    r = G.full_pass(w)
    dt = np.uint32
    assert np.array_equal(G.to_host_bits(r["gp"].cache.k_pool, "f32").view(dt), r["k_pool"].view(dt))
    assert np.array_equal(G.to_host_bits(r["gp"].cache.v_pool, "f32").view(dt), r["v_pool"].view(dt))
    G.assert_close(G.out_to_f64(r["out"]), r["ref"], "f32", f"random_f32[{seed}]")


@pytest.mark.parametrize("seed", range(max(12, N_SEEDS // 2)))
def test_random_pass_head_dim_64(seed):
    """The same random draws at head dim 64 (the bf16 kernels' other head size): stream and
    tile records, every block size, forced splits, steep logits."""
    kw, cus = draw_case(100 + seed)
    kw["d"] = 64
    G.say(f"random head-dim-64 case {seed}: {kw}, num_cus {cus}")
    w = wl.custom(71000 + seed, **kw)
    r = G.full_pass(w, num_cus=cus)
    dt = np.uint16
    assert np.array_equal(G.to_host_bits(r["gp"].cache.k_pool, "bf16").view(dt), r["k_pool"].view(dt))
    assert np.array_equal(G.to_host_bits(r["gp"].cache.v_pool, "bf16").view(dt), r["v_pool"].view(dt))
    G.assert_close(G.out_to_f64(r["out"]), r["ref"], "bf16", f"random_hd64[{seed}]")


@pytest.mark.parametrize("hq,hkv,bs", [(32, 32, 64), (32, 8, 64), (16, 2, 16)])
def test_head_dim_64_mixed_pass(hq, hkv, bs):
    """A mixed pass at head dim 64 large enough for long decode histories and several query
    tiles per chunk, planned for the device's compute units."""
    from ragged_blocked_kv_splitfuse_amd.runtime import num_cus
    w = wl.custom(72000 + hq + hkv + bs, hq=hq, hkv=hkv, d=64, bs=bs, budget=1024, n_decode=12,
                  decode_ctx=(64, 3000), prompts=((700, 1500), (0, 900)))
    r = G.full_pass(w, num_cus=num_cus())
    dt = np.uint16
    assert np.array_equal(G.to_host_bits(r["gp"].cache.k_pool, "bf16").view(dt), r["k_pool"].view(dt))
    assert np.array_equal(G.to_host_bits(r["gp"].cache.v_pool, "bf16").view(dt), r["v_pool"].view(dt))
    G.assert_close(G.out_to_f64(r["out"]), r["ref"], "bf16", f"hd64 mixed {hq}/{hkv} bs {bs}")
