"""Dense projections (QKV and output) through the C ABI against the oracle, at the
LLaMA-2-7B and Mistral-7B layer shapes over ragged token counts.

Bound (derived, any summation order): bf16 x bf16 products are exact in fp32, so the fp32
sum of K terms is within gamma_K * sum|x_i w_i| of the exact value (gamma_K ~ K * 2^-24), and
the final rounding to bf16 (8-bit significand, unit roundoff 2^-8) adds at most 2^-8 of the
accumulated value:
    |y_gpu - y| <= 1.01 * K * 2^-24 * sum_i |x_i w_i| * (1 + 2^-8) + 2^-8 * |y|."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle
from gpu_harness import say, to_dev
from ragged_blocked_kv_splitfuse_amd import fg
from ragged_blocked_kv_splitfuse_amd.runtime import stream_handle
from ragged_blocked_kv_splitfuse_amd.workloads import f32_to_bf16_bits

SHAPES = [  # (T, K, N): LLaMA-2-7B q/k/v/o (4096 -> 4096), Mistral-7B k/v (4096 -> 1024), a
    # fused QKV width (12288); the token counts reach each kernel the GEMM picks (the
    # weight-streaming kernel with 1 to 4 16-token tiles up to 64 rows; 64, 128 and 256-row
    # tiles above, 256 x 256 at T = 1174, N = 12288), with ragged tails, and N = 1536 the tile
    # placement without the per-XCD split
    (1, 4096, 4096), (17, 4096, 4096), (22, 4096, 1024), (37, 4096, 4096), (64, 4096, 1024),
    (512, 4096, 1024), (2048, 4096, 4096), (3000, 4096, 1024), (4100, 4096, 4096),
    (1174, 4096, 12288), (300, 512, 1536),
]


@pytest.mark.parametrize("T,K,N", SHAPES)
def test_linear_matches_oracle(T, K, N):
    rng = np.random.default_rng(T * 7 + N)
    x = f32_to_bf16_bits(rng.standard_normal((T, K), dtype=np.float32))
    w = f32_to_bf16_bits(rng.standard_normal((N, K), dtype=np.float32) / np.float32(np.sqrt(K)))
    xd, wd = to_dev(x, "bf16"), to_dev(w, "bf16")
    yd = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    fg.fg_linear_bf16(xd.data_ptr(), wd.data_ptr(), yd.data_ptr(), T, K, N, stream_handle())
    got = yd.float().cpu().numpy().astype(np.float64)
    ref = oracle.linear(x, w)
    absum = np.abs(oracle.bf16_bits_to_f64(x)) @ np.abs(oracle.bf16_bits_to_f64(w)).T
    bound = 1.01 * K * 2.0 ** -24 * absum * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref)
    err = np.abs(got - ref)
    say(f"linear T={T} K={K} N={N}: max err {err.max():.3e}, max err/bound {(err / bound).max():.3f}")
    assert np.isfinite(got).all()
    assert (err <= bound).all()


def test_linear_repeated_calls_and_shapes_share_state():
    rng = np.random.default_rng(5)
    K, N = 256, 128
    w = f32_to_bf16_bits(rng.standard_normal((N, K), dtype=np.float32))
    wd = to_dev(w, "bf16")
    for T in (3, 64, 3, 1000):
        x = f32_to_bf16_bits(rng.standard_normal((T, K), dtype=np.float32))
        yd = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        fg.fg_linear_bf16(to_dev(x, "bf16").data_ptr(), wd.data_ptr(), yd.data_ptr(), T, K, N,
                          stream_handle())
        ref = oracle.linear(x, w)
        absum = np.abs(oracle.bf16_bits_to_f64(x)) @ np.abs(oracle.bf16_bits_to_f64(w)).T
        bound = 1.01 * K * 2.0 ** -24 * absum * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref)
        assert (np.abs(yd.float().cpu().numpy() - ref) <= bound).all()
