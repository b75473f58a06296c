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
    # weight-streaming kernel with 1 to 4 16-token tiles up to 64 rows; above, 128 x 64 tiles
    # (T = 512, 3000 at N = 1024), 128 x 128 (T = 2048, 4100 at N = 4096; T = 640 at
    # N = 12288, where 128 x 128 needs one round as 256 x 256 does) and the eight-wave
    # 256 x 256 tile (T = 1174 and 700 at N = 12288, T = 3000 at N = 4096)), with ragged
    # tails, and N = 1536 the tile placement without the per-XCD split
    (1, 4096, 4096), (17, 4096, 4096), (22, 4096, 1024), (37, 4096, 4096), (64, 4096, 1024),
    (512, 4096, 1024), (2048, 4096, 4096), (3000, 4096, 1024), (4100, 4096, 4096),
    (1174, 4096, 12288), (700, 4096, 12288), (640, 4096, 12288), (3000, 4096, 4096),
    (300, 512, 1536),
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


QKV_SHAPES = [  # (T, K, Nq, Nkv): LLaMA-2-7B (4096 / 4096) and Mistral-7B (4096 / 1024) widths at
    # token counts that reach the weight-streaming kernel (T <= 64), the eight-wave 256 x 256
    # tile (T = 700 and 1174 at N = 12288, 2048 at N = 6144) and the 128 x 128 tile (T = 2048
    # at N = 12288, fewer rounds; T = 1174 at N = 6144); and widths that are
    # multiples of 128 but not 256 (the column boundaries then fall inside a 256-wide span)
    (17, 4096, 4096, 4096), (700, 4096, 4096, 4096), (1174, 4096, 4096, 4096),
    (2048, 4096, 4096, 4096), (40, 4096, 4096, 1024), (1174, 4096, 4096, 1024),
    (2048, 4096, 4096, 1024), (300, 512, 512, 384), (33, 512, 384, 128),
]


@pytest.mark.parametrize("T,K,Nq,Nkv", QKV_SHAPES)
def test_linear_qkv_matches_oracle_and_separate_calls(T, K, Nq, Nkv):
    rng = np.random.default_rng(T * 11 + Nq + 3 * Nkv)
    x = f32_to_bf16_bits(rng.standard_normal((T, K), dtype=np.float32))
    blocks = [f32_to_bf16_bits(rng.standard_normal((n, K), dtype=np.float32) /
                               np.float32(np.sqrt(K))) for n in (Nq, Nkv, Nkv)]
    xd = to_dev(x, "bf16")
    wd = to_dev(np.concatenate(blocks, axis=0), "bf16")
    outs = [torch.empty((T, n), dtype=torch.bfloat16, device="cuda") for n in (Nq, Nkv, Nkv)]
    fg.fg_linear_qkv_bf16(xd.data_ptr(), wd.data_ptr(), *(o.data_ptr() for o in outs), T, K, Nq,
                          Nkv, stream_handle())
    xa = np.abs(oracle.bf16_bits_to_f64(x))
    for name, w, o in zip("qkv", blocks, outs):
        # the same block through the plain entry point: identical bits
        sep = torch.empty_like(o)
        fg.fg_linear_bf16(xd.data_ptr(), to_dev(w, "bf16").data_ptr(), sep.data_ptr(), T, K,
                          w.shape[0], stream_handle())
        assert torch.equal(o, sep), name
        got = o.float().cpu().numpy().astype(np.float64)
        ref = oracle.linear(x, w)
        absum = xa @ np.abs(oracle.bf16_bits_to_f64(w)).T
        bound = 1.01 * K * 2.0 ** -24 * absum * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref)
        err = np.abs(got - ref)
        say(f"qkv {name} T={T} K={K} Nq={Nq} Nkv={Nkv}: max err/bound {(err / bound).max():.3f}")
        assert np.isfinite(got).all()
        assert (err <= bound).all(), name
