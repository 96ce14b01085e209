"""Explicit W-hat, fp64 products and the error metric.  TEST INFRASTRUCTURE.

The product is exact by definition: y[b][i] = sum_j W_hat[i][j] x[b][j],
with W_hat rebuilt explicitly from codes and group constants (group RTN) or
from the +-1 factors and channel scales (binary low-rank), and x decoded
exactly from the bf16/fp32 bits actually passed.  Prefill is the same
product for M token rows, Y = X W_hat^T.

Error metric (per output element, with the decoded weights):
    err = max_{b,i} |y - y_ref| / sum_j |W_hat[i][j]| |x[b][j]|
Where that denominator is 0 the output must be exactly 0.
"""
from __future__ import annotations

import numpy as np

from . import rtn, fmt


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bits (uint16): the bits are the top half of an fp32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def what_group(codes_words: np.ndarray, meta: np.ndarray, N: int, K: int,
               bits: int, group: int) -> np.ndarray:
    """W_hat [N][K] fp64 from packed codes and meta words."""
    q = fmt.unpack_codes(codes_words, N, K, bits)
    s, o = fmt.unpack_meta(np.asarray(meta).reshape(N, K // group))
    return rtn.dequantize(q, s, o, group)


def matmul_ref(W_hat: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Y[m][i] = sum_j W_hat[i][j] X[m][j] in fp64."""
    return np.asarray(X, dtype=np.float64) @ np.asarray(W_hat, dtype=np.float64).T


def abs_denominator(W_hat: np.ndarray, X: np.ndarray) -> np.ndarray:
    """D[m][i] = sum_j |W_hat[i][j]| |X[m][j]|."""
    return np.abs(np.asarray(X, dtype=np.float64)) @ np.abs(np.asarray(W_hat, dtype=np.float64)).T


def binlr_abs_denominator(U, V, s1_bits, s2_bits, X) -> np.ndarray:
    """Error denominator of the binary low-rank product.

    The plain D = sum_j |W_hat_ij| |x_j| with W_hat = s1 (U V^T) s2 ("70B en
    4GB de VRAM...", section 1).  Where a row of the sign product U V^T is
    identically zero, D = 0 while the method, evaluated in its two factored
    stages (t = V^T (s2 x), y = s1 U t), still adds r * K nonzero terms that
    cancel only in exact arithmetic; such elements are measured against the
    magnitude of those terms, |s1_i| * sum_l sum_j |U_il V_jl s2_j x_j| =
    |s1_i| * r * sum_j |s2_j x_j|, which bounds D everywhere (|C_ij| <= r).
    """
    U = np.asarray(U, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    s1 = f16_to_f64(s1_bits)
    s2 = f16_to_f64(s2_bits)
    X = np.asarray(X, dtype=np.float64)
    W_hat = s1[:, None] * (U @ V.T) * s2[None, :]
    D = abs_denominator(W_hat, X)
    r = U.shape[1]
    D_fact = np.abs(X) @ np.abs(s2)[:, None] * r * np.abs(s1)[None, :]
    return np.where(D > 0, D, D_fact)


def normalized_error(Y: np.ndarray, Y_ref: np.ndarray, D: np.ndarray) -> float:
    """max |Y - Y_ref| / D over elements with D > 0; inf if an element with D == 0 is nonzero."""
    Y = np.asarray(Y, dtype=np.float64)
    diff = np.abs(Y - Y_ref)
    zero = D == 0
    if np.any(zero & (Y != 0)):
        return float("inf")
    if np.all(zero):
        return 0.0
    return float(np.max(diff[~zero] / D[~zero]))


def gemv_binlr_stages(U, V, s1_bits, s2_bits, X):
    """The two-stage form t = V^T (s2 (.) x), y = s1 (.) (U t) in fp64.

    Used to pin the stage order: it must agree with the explicit product.
    """
    s1 = f16_to_f64(s1_bits)
    s2 = f16_to_f64(s2_bits)
    Xp = np.asarray(X, dtype=np.float64) * s2[None, :]
    T = Xp @ V.astype(np.float64)          # [B][r]
    return (T @ U.astype(np.float64).T) * s1[None, :]
