"""Outlier-aware mixed decomposition.  TEST INFRASTRUCTURE.

Source: "Métodos de cuantización de LLM para ejecutar un modelo de 70B en una
sola GPU".  Its opening notes that about 0.1 % of the hidden dimensions carry
values up to 20x larger than the rest of the tensor and spoil the
quantization grid for every other parameter; its LLM.int8() paragraph runs
the outlier dimensions in FP16, the remaining 99.9 % at low precision, and
adds the two results.

Readings (the pages give no selection rule, storage or low-bit format here):
  * The split is over W's input channels (columns k).  Weights only, no
    calibration data: channel k scores max_n |W[n][k]|; the n_out channels
    with the largest scores are the outliers, ties to the lower k; idx lists
    them in increasing k.
  * The low-bit part is the group RTN of rtn.py applied to W with the
    outlier columns set to 0; the packed codes keep all K columns.
  * The outlier columns are kept in fp16 as the difference between the true
    column and what the low-bit codes reconstruct there:
    side[n][j] = fp16(W[n][idx_j] - w_rest[n][idx_j]), one fp64 subtraction
    and one rounding to nearest even.  The two products then add up to the
    fp16-rounded true column on the outlier dimensions and to the RTN weight
    everywhere else: y = W_rest_hat x + side x[idx], one GEMV plus a rank-
    n_out term.  A difference beyond the fp16 range is a range error.
"""
from __future__ import annotations

import numpy as np

from . import rtn


def outlier_channels(W: np.ndarray, n_out: int) -> np.ndarray:
    """Indices (increasing) of the n_out input channels with the largest
    max |W[n][k]|; among equal scores the lower k is taken first."""
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    if not 0 <= n_out <= K:
        raise ValueError("n_out out of range")
    score = np.abs(W.astype(np.float64)).max(axis=0)
    if not np.all(np.isfinite(score)):
        raise rtn.RangeError("non-finite weight")
    # primary key: larger score first; secondary key: smaller k first
    order = np.lexsort((np.arange(K), -score))
    return np.sort(order[:n_out]).astype(np.int64)


def encode(W: np.ndarray, bits: int, group: int, n_out: int):
    """(q, s, o, side, idx): group RTN of W with the outlier columns zeroed,
    and the fp16 residual columns side[N][n_out] (float16)."""
    idx = outlier_channels(W, n_out)
    return encode_with(W, bits, group, idx) + (idx,)


def encode_with(W: np.ndarray, bits: int, group: int, idx: np.ndarray):
    """(q, s, o, side) for a given channel list idx.  Every step after the
    channel choice is row-local, so a subset of W's rows gives those rows'
    codes, constants and side values."""
    W = np.asarray(W, dtype=np.float32)
    idx = np.asarray(idx, dtype=np.int64)
    W_rest = W.copy()
    W_rest[:, idx] = 0.0
    q, s, o = rtn.quantize(W_rest, bits, group)
    w_rest = rtn.dequantize(q, s, o, group)
    diff = W[:, idx].astype(np.float64) - w_rest[:, idx]
    with np.errstate(over="ignore", invalid="ignore"):
        side = diff.astype(np.float16)
    if not np.all(np.isfinite(side)):
        raise rtn.RangeError("outlier residual leaves the fp16 range")
    return q, s, o, side


def reconstruct(q: np.ndarray, s: np.ndarray, o: np.ndarray, group: int,
                side: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Effective weights in fp64: the RTN reconstruction plus the fp16 side
    columns added on the outlier channels."""
    W_hat = rtn.dequantize(q, s, o, group)
    W_hat[:, np.asarray(idx, dtype=np.int64)] += np.asarray(side, dtype=np.float16).astype(np.float64)
    return W_hat
