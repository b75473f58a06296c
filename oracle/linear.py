"""Dense projection of a pass's token rows, float64 (test infrastructure).

The layer ops either side of attention -- the QKV projection that produces the rows
kv_append stores and attention reads, and the output projection of attention's rows -- are
plain matrix products (DeepSpeed-FastGen paper card by Holmes et al. 2024, "Key points": the
kernels around attention come from FasterTransformer).  With w in the [out][in] layout of a
linear layer:

    y[t][o] = sum_i x[t][i] * w[o][i]

Inputs are bf16 bit patterns (or float32), widened exactly to float64; the product is numpy's
float64 matmul, the only step.
"""
import numpy as np

from .bf16 import to_f64


def linear(x, w, dtype: str = "bf16") -> np.ndarray:
    """x [T][K], w [N][K] -> y [T][N] float64."""
    X = to_f64(np.asarray(x), dtype)
    W = to_f64(np.asarray(w), dtype)
    if X.shape[-1] != W.shape[-1]:
        raise ValueError("inner sizes differ")
    return X @ W.T
