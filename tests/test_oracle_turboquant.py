"""Pins of the key-cache quantizer (oracle/turboquant.py; "70B en 4GB de
VRAM: la compresión neural de 2026, ¿es real?", section 3): the coordinate
law, Lloyd-Max centroids against closed forms and the Gaussian limit, the
page's distortion factors, the rotation, the bias of the MSE estimate and the
unbiasedness of the QJL-corrected one."""
import math

import numpy as np
import pytest
from scipy import integrate

from oracle import turboquant as tq
from workloads import rng_for


def test_coordinate_law_is_a_density_with_variance_1_over_d():
    for d in (3, 16, 128):
        tot = integrate.quad(lambda t: tq.coord_density(d, t), -1, 1)[0]
        var = integrate.quad(lambda t: t * t * tq.coord_density(d, t), -1, 1)[0]
        assert abs(tot - 1) < 1e-9 and abs(var - 1.0 / d) < 1e-9


def test_coordinate_law_matches_sampled_unit_vectors():
    rng = rng_for(400, 0)
    d = 128
    x = rng.standard_normal((200000, d))
    t = (x / np.linalg.norm(x, axis=1, keepdims=True))[:, 0]
    for a in (0.05, 0.1, 0.2):
        p = integrate.quad(lambda s: tq.coord_density(d, s), -a, a)[0]
        assert abs(np.mean(np.abs(t) <= a) - p) < 0.004


def test_one_bit_centroid_closed_form():
    """At one bit the centroids are -+E|t| = Gamma(d/2)/(sqrt(pi) Gamma((d+1)/2))."""
    for d in (16, 64, 128):
        c = tq.lloyd_max(d, 1)
        e = math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
        assert np.allclose(c, [-e, e], rtol=1e-12, atol=0)


def test_gaussian_limit():
    """For large d, sqrt(d) c tends to the Lloyd-Max levels of N(0, 1)
    (Max, 1960): 0.7979; 0.4528, 1.510; 0.2451, 0.7560, 1.344, 2.152."""
    d = 200000
    ref = {1: [0.7979], 2: [0.4528, 1.510], 3: [0.2451, 0.7560, 1.344, 2.152]}
    for m, pos in ref.items():
        c = tq.lloyd_max(d, m) * math.sqrt(d)
        assert np.allclose(c[len(c) // 2:], pos, atol=2e-3), (m, c)
        assert np.allclose(c, -c[::-1], atol=1e-12)                   # symmetric


def test_lloyd_conditions_hold():
    """Every centroid is the conditional mean of its cell (cells bounded by
    midpoints), checked by direct quadrature."""
    d = 128
    for m in (2, 3):
        c = tq.lloyd_max(d, m)
        edges = np.concatenate([[-1.0], (c[1:] + c[:-1]) / 2, [1.0]])
        for k in range(len(c)):
            num = integrate.quad(lambda t: t * tq.coord_density(d, t), edges[k], edges[k + 1], epsabs=1e-14)[0]
            den = integrate.quad(lambda t: tq.coord_density(d, t), edges[k], edges[k + 1], epsabs=1e-14)[0]
            assert abs(num / den - c[k]) < 1e-9


def test_page_distortion_factors():
    """The page: MSE distortion within a factor ~2.7 of the bound 4^-b at
    every width, ~1.45 at one bit.  Distortion of a unit vector =
    d x the per-coordinate distortion."""
    d = 128
    ratios = []
    for m in (1, 2, 3, 4):
        D = d * tq.distortion(d, tq.lloyd_max(d, m))
        ratios.append(D / 4.0 ** -m)
    assert abs(ratios[0] - 1.45) < 0.02
    assert all(r <= 2.72 for r in ratios), ratios
    assert all(a < b for a, b in zip(ratios, ratios[1:]))            # grows with the width


def test_distortion_by_sampling():
    """E |x - x_hat|^2 for random unit vectors matches d x the closed-form
    per-coordinate distortion (stored 7-bit table included)."""
    rng = rng_for(401, 0)
    d = 128
    Pi = tq.rotation(rng.standard_normal((d, d)))
    X = rng.standard_normal((4000, d)).astype(np.float32)
    for m in (2, 3):
        delta, e = tq.stored_table(tq.lloyd_max(d, m))
        cv = tq.table_values(delta, e)
        codes, norm, y = tq.quantize_mse(X, Pi, cv)
        Xh = tq.dequantize_mse(codes, norm, Pi, cv)
        Xn = X.astype(np.float64) / norm[:, None]
        err = np.mean(np.sum((Xn - Xh / norm[:, None]) ** 2, axis=1))
        assert abs(err / (d * tq.distortion(d, cv)) - 1) < 0.03, (m, err)


def test_stored_table():
    d = 128
    for m in (2, 3):
        c = tq.lloyd_max(d, m)
        delta, e = tq.stored_table(c)
        cv = tq.table_values(delta, e)
        assert e.min() >= 1 and e.max() <= 127 and delta.dtype == np.float32
        assert np.all(np.abs(cv - c) <= float(delta) / 2 * (1 + 1e-12))
        assert np.all(np.diff(cv) > 0)
        assert e[0] + e[-1] == 128                                    # symmetric grid


def test_rotation_is_orthogonal_haar_qr():
    rng = rng_for(402, 0)
    G = rng.standard_normal((128, 128))
    Pi = tq.rotation(G)
    assert np.allclose(Pi.T @ Pi, np.eye(128), atol=1e-12)
    R = Pi.T @ G                                                      # G = Pi R
    assert np.allclose(np.tril(R, -1), 0, atol=1e-10) and np.all(np.diag(R) > 0)


def test_nearest_centroid_brute_force():
    rng = rng_for(403, 0)
    cv = tq.table_values(*tq.stored_table(tq.lloyd_max(128, 3)))
    y = rng.standard_normal(5000) * 0.1
    mids = (cv[1:] + cv[:-1]) / 2
    y = np.concatenate([y, mids])                                     # exact ties go to the lower index
    k = tq.nearest(y, cv)
    for yi, ki in zip(y, k):
        dist = [abs(yi - c) for c in cv]
        assert ki == min(range(len(cv)), key=lambda j: (dist[j], j))


def test_sequential_sums_equal_plain_products_closely():
    rng = rng_for(404, 0)
    A = rng.standard_normal((128, 128))
    X = rng.standard_normal((5, 128))
    assert np.allclose(tq._seq_dot(A, X), X @ A.T, rtol=1e-12, atol=1e-12)
    assert np.allclose(tq._seq_norm(X), np.linalg.norm(X, axis=1), rtol=1e-14)


def test_mse_estimate_is_biased_and_qjl_removes_it():
    """The page: the MSE-optimal quantizer biases inner products; one QJL bit
    on the residual makes the estimate unbiased.  At m = 1 the MSE estimate
    shrinks <q, x> by d (E|t|)^2 (~2/pi) on average over rotations; averaged
    over independent (Pi, S), the QJL-corrected estimate has mean <q, x>."""
    rng = rng_for(405, 0)
    d = 128
    x = rng.standard_normal(d)
    q = x + 0.5 * rng.standard_normal(d)
    X = x[None, :].astype(np.float32)
    true = float(q @ X[0].astype(np.float64))
    for m, shrink in ((1, d * (math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)) ** 2),
                      (2, None)):
        cv = tq.lloyd_max(d, m)          # unrounded levels for the statistics
        mse_est, prod_est = [], []
        for t in range(600):
            Pi = tq.rotation(rng.standard_normal((d, d)))
            S = rng.standard_normal((d, d))
            codes, norm, y = tq.quantize_mse(X, Pi, cv)
            mse_est.append(float(q @ tq.dequantize_mse(codes, norm, Pi, cv)[0]))
            c2, sg, n16, g16 = tq.quantize_prod(X, Pi, S, cv)
            prod_est.append(float(tq.logits_prod(q[None, :], c2, sg, n16, g16, Pi, S, cv)[0, 0]))
        mse_est, prod_est = np.array(mse_est), np.array(prod_est)
        se = prod_est.std() / math.sqrt(len(prod_est))
        assert abs(prod_est.mean() - true) < 4 * se + 1e-3 * abs(true), (m, prod_est.mean(), true, se)
        if shrink is not None:
            assert abs(mse_est.mean() / true - shrink) < 0.02, (mse_est.mean() / true, shrink)
        assert mse_est.mean() < true                                   # shrunk toward 0


def test_prod_estimate_error_shrinks_with_bits():
    """More MSE bits leave a smaller residual, so the spread of the
    unbiased estimate falls with the width."""
    rng = rng_for(406, 0)
    d = 128
    X = rng.standard_normal((400, d)).astype(np.float32)
    q = rng.standard_normal((1, d))
    true = q @ X.astype(np.float64).T
    Pi = tq.rotation(rng.standard_normal((d, d)))
    S = rng.standard_normal((d, d))
    spread = []
    for m in (1, 2, 3):
        cv = tq.table_values(*tq.stored_table(tq.lloyd_max(d, m))) if m > 1 else tq.lloyd_max(d, m)
        c, sg, n16, g16 = tq.quantize_prod(X, Pi, S, cv)
        est = tq.logits_prod(q, c, sg, n16, g16, Pi, S, cv)
        spread.append(np.std(est - true) / np.std(true))
    assert spread[0] > spread[1] > spread[2]


def test_value_path():
    """Values: one-hot weights return the dequantized value; the output is
    linear in the weights; at 4 bits the weighted sum of reconstructions is
    within the distortion of the exact weighted sum."""
    rng = rng_for(407, 0)
    d, n = 128, 300
    Pi = tq.rotation(rng.standard_normal((d, d)))
    V = rng.standard_normal((n, d)).astype(np.float32)
    cv = tq.table_values(*tq.stored_table(tq.lloyd_max(d, 4)))
    codes, n16 = tq.quantize_values(V, Pi, cv)
    c2, nrm, _ = tq.quantize_mse(V, Pi, cv)
    assert np.array_equal(codes, c2) and np.array_equal(n16, nrm.astype(np.float16))
    Vh = tq.dequantize_mse(codes, n16.astype(np.float64), Pi, cv)
    P = np.zeros((2, n))
    P[0, 17] = 1.0
    P[1] = rng.random(n)
    P[1] /= P[1].sum()
    O = tq.attend_values(P, codes, n16, Pi, cv)
    assert np.allclose(O[0], Vh[17], rtol=0, atol=1e-15)
    O2 = tq.attend_values(2 * P, codes, n16, Pi, cv)
    assert np.allclose(O2, 2 * O, rtol=1e-14, atol=0)
    exact = P[1] @ V.astype(np.float64)
    # per-value squared error ~ d * distortion |v|^2 (4 bits: ~0.0095); the
    # average over 300 values with random weights is much smaller
    err = np.sum((O[1] - exact) ** 2)
    assert err < 0.0095 * np.mean(np.sum(V.astype(np.float64) ** 2, axis=1))
