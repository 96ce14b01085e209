"""Pins of the outlier-aware decomposition (oracle/outlier.py): channel choice
by brute force over index subsets, planted outliers with a known answer, the
reduction to plain RTN at n_out = 0, the fp16 rounding bound on the outlier
columns, and the gain the pages attribute to isolating outliers ("Métodos de
cuantización de LLM...", opening and LLM.int8() paragraph)."""
import itertools

import numpy as np
import pytest

from oracle import outlier, product, rtn
from workloads import rng_for


def _planted(N, K, cols, rng, sigma=0.02, scale=20.0):
    W = (rng.standard_normal((N, K)) * sigma).astype(np.float32)
    W[:, cols] *= np.float32(scale)
    return W


@pytest.mark.parametrize("seed", range(6))
def test_selection_matches_subset_brute_force(seed):
    """The chosen set maximizes the summed channel score; among such sets it
    is the lexicographically smallest index tuple (ties go to the lower k).
    Small integer weights make ties frequent and sums exact."""
    rng = np.random.default_rng(300 + seed)
    N, K = 4, 10
    W = rng.integers(-3, 4, size=(N, K)).astype(np.float32)
    score = [max(abs(float(W[n, k])) for n in range(N)) for k in range(K)]
    for n_out in range(K + 1):
        best = None
        for sub in itertools.combinations(range(K), n_out):
            key = (-sum(score[k] for k in sub), sub)
            if best is None or key < best:
                best = key
        assert tuple(outlier.outlier_channels(W, n_out)) == best[1], (seed, n_out)


def test_selection_edges():
    W = np.zeros((3, 6), np.float32)
    assert outlier.outlier_channels(W, 0).size == 0
    assert list(outlier.outlier_channels(W, 6)) == list(range(6))
    assert list(outlier.outlier_channels(W, 2)) == [0, 1]          # all tied
    W[1, 4] = -5.0
    W[2, 2] = 5.0                                                   # tie in |w|
    assert list(outlier.outlier_channels(W, 1)) == [2]
    assert list(outlier.outlier_channels(W, 2)) == [2, 4]
    with pytest.raises(ValueError):
        outlier.outlier_channels(W, 7)
    W[0, 0] = np.inf
    with pytest.raises(rtn.RangeError):
        outlier.outlier_channels(W, 1)


def test_planted_outliers_are_found():
    rng = rng_for(310, 0)
    K = 2048
    cols = np.array([5, 700, 701, 2047])
    W = _planted(48, K, cols, rng)
    assert list(outlier.outlier_channels(W, 4)) == list(cols)


@pytest.mark.parametrize("bits,group", [(4, 64), (3, 32), (2, 32), (6, 32)])
def test_zero_outliers_is_plain_rtn(bits, group):
    W = _planted(20, 256, [3, 99], rng_for(311, bits))
    q, s, o, side, idx = outlier.encode(W, bits, group, 0)
    q0, s0, o0 = rtn.quantize(W, bits, group)
    assert np.array_equal(q, q0) and np.array_equal(s.view(np.uint16), s0.view(np.uint16))
    assert np.array_equal(o.view(np.uint16), o0.view(np.uint16))
    assert side.shape == (20, 0) and idx.size == 0


@pytest.mark.parametrize("bits,group", [(4, 64), (3, 32), (5, 64)])
def test_outlier_columns_within_fp16_rounding(bits, group):
    """On an outlier channel the effective weight is the true column to within
    one fp16 rounding of the stored difference (half an fp16 ulp of it);
    every other channel carries the RTN weight of W with those columns
    zeroed, inside that group's s/2 bound."""
    rng = rng_for(312, bits)
    cols = np.array([1, 130, 131])
    W = _planted(32, 512, cols, rng)
    q, s, o, side, idx = outlier.encode(W, bits, group, 3)
    assert list(idx) == list(cols)
    W_hat = outlier.reconstruct(q, s, o, group, side, idx)
    w_rest = rtn.dequantize(q, s, o, group)
    diff = W[:, idx].astype(np.float64) - w_rest[:, idx]
    half_ulp = np.spacing(np.abs(diff).astype(np.float16)).astype(np.float64) / 2
    assert np.all(np.abs(W_hat[:, idx] - W[:, idx]) <= half_ulp)
    assert np.all(np.abs(side.astype(np.float64) - diff) <= half_ulp)
    rest = np.setdiff1d(np.arange(512), idx)
    s_full = np.repeat(s.astype(np.float64), group, axis=1)
    assert np.all(np.abs(W_hat[:, rest] - W[:, rest]) <= s_full[:, rest] / 2)
    # the zeroed columns were encoded as 0: their RTN value is within s/2 of 0
    assert np.all(np.abs(w_rest[:, idx]) <= s_full[:, idx] / 2)


@pytest.mark.parametrize("bits,group", [(4, 64), (3, 32)])
@pytest.mark.parametrize("seed", range(3))
def test_isolating_outliers_restores_the_grid(bits, group, seed):
    """0.1 % of channels 20x larger widen the grid of every group they fall
    in.  With them kept aside, no group's scale exceeds what the groups free
    of outliers already had, the worst weight error drops several-fold, and
    the product error decreases.  (With groups of 32 or 64 only the groups
    holding an outlier are affected, so the product gain is modest.)"""
    rng = rng_for(313, 10 * bits + seed)
    N, K = 64, 4096
    cols = np.sort(rng.choice(K, size=4, replace=False))
    W = _planted(N, K, cols, rng)
    q0, s0, o0 = rtn.quantize(W, bits, group)
    q, s, o, side, idx = outlier.encode(W, bits, group, 4)
    assert list(idx) == list(cols)
    hit = np.zeros(K // group, bool)
    hit[cols // group] = True
    s0 = s0.astype(np.float64)
    assert np.median(s0[:, hit]) > 2.5 * np.median(s0[:, ~hit])  # the spoiled grid
    assert s.astype(np.float64).max() <= 1.25 * s0[:, ~hit].max()  # restored
    W64 = W.astype(np.float64)
    W_rtn = rtn.dequantize(q0, s0.astype(np.float16), o0, group)
    W_out = outlier.reconstruct(q, s, o, group, side, idx)
    assert np.abs(W_out - W64).max() * 5 < np.abs(W_rtn - W64).max()
    x = rng.standard_normal((3, K))
    y_true = x @ W64.T
    D = np.abs(x) @ np.abs(W64).T
    err_rtn = product.normalized_error(product.matmul_ref(W_rtn, x), y_true, D)
    err_out = product.normalized_error(product.matmul_ref(W_out, x), y_true, D)
    assert err_out < err_rtn, (err_out, err_rtn)


def test_encode_with_is_row_local():
    """Rows encoded on their own, with the channel list of the whole matrix,
    give exactly the whole matrix's rows."""
    W = _planted(40, 256, [7, 200], rng_for(314, 0))
    q, s, o, side, idx = outlier.encode(W, 3, 32, 2)
    rows = [0, 5, 39]
    q2, s2, o2, side2 = outlier.encode_with(W[rows], 3, 32, idx)
    assert np.array_equal(q2, q[rows]) and np.array_equal(s2.view(np.uint16), s[rows].view(np.uint16))
    assert np.array_equal(o2.view(np.uint16), o[rows].view(np.uint16))
    assert np.array_equal(side2.view(np.uint16), side[rows].view(np.uint16))


def test_residual_range_error():
    W = np.zeros((2, 64), np.float32)
    W[0, 7] = 1e6          # survives as a channel score, but fp16 cannot hold it
    with pytest.raises(rtn.RangeError):
        outlier.encode(W, 4, 32, 1)
