"""Key-cache vector quantization with a random rotation, Lloyd-Max
coordinates and a 1-bit QJL residual.  TEST INFRASTRUCTURE.

Source: "70B en 4GB de VRAM: la compresión neural de 2026, ¿es real?",
section 3 (TurboQuant): a random orthogonal rotation (Q factor of a Gaussian
matrix) makes every coordinate of a rotated unit vector follow one known law
(a concentrated Beta, close to N(0, 1/d)) whatever the data, so one Lloyd-Max
codebook serves every vector with no per-block constants; the MSE-optimal
quantizer biases inner products, and spending one bit per coordinate on the
signs of a random projection of the residual (QJL) makes the inner-product
estimate unbiased.  Two variants: one for inner products (keys), one for
reconstruction (values).  Distortion within a factor ~2.7 of the bound 4^-b
at every width, ~1.45 at one bit.

Definitions used here (the page gives the outline only):
  * Coordinate law of a uniform unit vector in R^d: density
    f(t) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) (1 - t^2)^((d-3)/2) on
    [-1, 1]; (t + 1)/2 ~ Beta((d-1)/2, (d-1)/2).
  * lloyd_max(d, m): the 2^m centroids minimizing E (t - c(t))^2 under f,
    by Lloyd's iteration (boundaries at midpoints, centroids at conditional
    means, both in closed form through the regularized incomplete beta
    function and the antiderivative of t f(t)).
  * rotation(G): Q of the QR factorization of a Gaussian G with the signs
    fixed so diag(R) > 0 (a Haar-distributed orthogonal matrix).
  * MSE variant with m bits: y = Pi x / |x|, code = nearest centroid.
  * Inner-product variant with b = m + 1 bits per coordinate: the MSE
    variant with m bits, the residual r = y - c[code] of the rotated unit
    vector, gamma = |r|, and the signs of z = S r for a d x d matrix S of
    i.i.d. N(0, 1) entries (bit 1 <-> z >= 0).  For a query q:
      <q, x> ~ |x| (<Pi q, c[code]> + gamma sqrt(pi/2)/d <S Pi q, sign(z)>),
    unbiased over S because E[(s.a) sign(s.r)] = sqrt(2/pi) <a, r>/|r| for
    s ~ N(0, I).

Readings of this build (for the GPU format):
  * Stored centroids: the m-bit table is kept on a 7-bit grid,
    c_k = delta (e_k - 64) with delta = c_max / 63 (fp32) and integer
    e_k in 1..127; encoding picks the nearest *stored* centroid (ties to the
    lower index) and the estimate uses the same values.  The grid moves a
    centroid by at most c_max/126 (well below the m-bit distortion).
  * |x| and gamma are stored as fp16 (round to nearest even); the estimate
    uses the stored values.
  * Every sum over coordinates (norms, Pi x, S r) is taken in fp64 in
    increasing index order with no fused multiply-add, so a GPU encoder can
    reproduce the codes and signs bit for bit.
"""
from __future__ import annotations

import math

import numpy as np
from scipy import special


def coord_density(d: int, t: np.ndarray) -> np.ndarray:
    t = np.asarray(t, dtype=np.float64)
    c = math.exp(math.lgamma(d / 2) - math.lgamma((d - 1) / 2)) / math.sqrt(math.pi)
    return c * np.clip(1.0 - t * t, 0.0, None) ** ((d - 3) / 2)


def _cdf(d: int, t):
    a = (d - 1) / 2
    return special.betainc(a, a, (np.asarray(t, dtype=np.float64) + 1.0) / 2.0)


def _first_moment(d: int, t):
    """Antiderivative of t f(t): -C (1 - t^2)^((d-1)/2) / (d - 1)."""
    c = math.exp(math.lgamma(d / 2) - math.lgamma((d - 1) / 2)) / math.sqrt(math.pi)
    t = np.asarray(t, dtype=np.float64)
    return -c * np.clip(1.0 - t * t, 0.0, None) ** ((d - 1) / 2) / (d - 1)


def lloyd_max(d: int, m: int, iters: int = 2000) -> np.ndarray:
    """Increasing centroids (fp64, 2^m of them) of the coordinate law."""
    L = 1 << m
    # start at the conditional means of equal-probability cells
    qs = special.betaincinv((d - 1) / 2, (d - 1) / 2, np.arange(1, L) / L) * 2.0 - 1.0
    edges = np.concatenate([[-1.0], qs, [1.0]])
    c = None
    for _ in range(iters):
        mass = _cdf(d, edges[1:]) - _cdf(d, edges[:-1])
        mom = _first_moment(d, edges[1:]) - _first_moment(d, edges[:-1])
        c_new = mom / mass
        if c is not None and np.max(np.abs(c_new - c)) < 1e-16:
            c = c_new
            break
        c = c_new
        edges = np.concatenate([[-1.0], (c[1:] + c[:-1]) / 2.0, [1.0]])
    return c


def distortion(d: int, c: np.ndarray) -> float:
    """E (t - c(t))^2 per coordinate for centroids c (nearest-centroid
    cells), by the same closed forms plus the second moment."""
    edges = np.concatenate([[-1.0], (c[1:] + c[:-1]) / 2.0, [1.0]])
    mass = _cdf(d, edges[1:]) - _cdf(d, edges[:-1])
    mom = _first_moment(d, edges[1:]) - _first_moment(d, edges[:-1])
    # E t^2 = 1/d for a coordinate of a unit vector; per cell second moment
    # by quadrature on a fine grid (smooth integrand)
    sec = np.empty_like(mass)
    for k in range(len(c)):
        tt = np.linspace(edges[k], edges[k + 1], 20001)
        sec[k] = np.trapezoid(tt * tt * coord_density(d, tt), tt)
    return float(np.sum(sec - 2 * c * mom + c * c * mass))


def stored_table(c: np.ndarray):
    """(delta fp32, e uint8[L]) with c_k ~ delta (e_k - 64), e in 1..127."""
    delta = np.float32(np.max(np.abs(c)) / 63.0)
    e = np.rint(c / np.float64(delta)).astype(np.int64) + 64
    if e.min() < 1 or e.max() > 127:
        raise ValueError("centroid outside the 7-bit grid")
    return delta, e.astype(np.uint8)


def table_values(delta, e) -> np.ndarray:
    return np.float64(np.float32(delta)) * (np.asarray(e, dtype=np.float64) - 64.0)


def rotation(G: np.ndarray) -> np.ndarray:
    """Q of G = QR with diag(R) > 0 (fp64)."""
    Q, R = np.linalg.qr(np.asarray(G, dtype=np.float64))
    return Q * np.where(np.diag(R) < 0, -1.0, 1.0)[None, :]


def _seq_dot(A: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Rows of X times A^T, each output summed in increasing index order
    without fused multiply-add: out[n][i] = sum_j A[i][j] X[n][j]."""
    A = np.asarray(A, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    acc = np.zeros((X.shape[0], A.shape[0]))
    for j in range(A.shape[1]):
        acc = acc + X[:, j:j + 1] * A[None, :, j]
    return acc


def _seq_norm(X: np.ndarray) -> np.ndarray:
    X = np.asarray(X, dtype=np.float64)
    acc = np.zeros(X.shape[0])
    for j in range(X.shape[1]):
        acc = acc + X[:, j] * X[:, j]
    return np.sqrt(acc)


def nearest(y: np.ndarray, cv: np.ndarray) -> np.ndarray:
    """Index of the nearest centroid (ties to the lower index)."""
    return np.abs(y[..., None] - cv).argmin(axis=-1)


def quantize_mse(X: np.ndarray, Pi: np.ndarray, cv: np.ndarray):
    """(codes int [n][d], norm fp64 [n], y fp64 [n][d]) for rows of X (fp32)
    with the stored centroid values cv."""
    X = np.asarray(X, dtype=np.float32).astype(np.float64)
    norm = _seq_norm(X)
    safe = np.where(norm > 0, norm, 1.0)
    y = _seq_dot(Pi, X) / safe[:, None]
    return nearest(y, cv), norm, y


def quantize_prod(X: np.ndarray, Pi: np.ndarray, S: np.ndarray, cv: np.ndarray):
    """Inner-product variant: (codes [n][d], signs uint8 [n][d], norm16
    float16 [n], gamma16 float16 [n])."""
    codes, norm, y = quantize_mse(X, Pi, cv)
    r = y - cv[codes]
    gamma = _seq_norm(r)
    z = _seq_dot(S, r)
    signs = (z >= 0).astype(np.uint8)
    return codes, signs, norm.astype(np.float16), gamma.astype(np.float16)


def dequantize_mse(codes, norm, Pi, cv) -> np.ndarray:
    """|x| Pi^T c[code] (fp64)."""
    return np.asarray(norm, dtype=np.float64)[:, None] * (cv[codes] @ np.asarray(Pi, dtype=np.float64))


def logits_prod(Q: np.ndarray, codes, signs, norm16, gamma16, Pi, S, cv) -> np.ndarray:
    """Estimated <q, x> for every query row of Q and every stored key: fp64."""
    Q = np.asarray(Q, dtype=np.float64)
    d = Q.shape[1]
    qr = Q @ np.asarray(Pi, dtype=np.float64).T              # Pi q
    u = qr @ np.asarray(S, dtype=np.float64).T               # S Pi q
    mse = qr @ cv[codes].T                                   # [nq][n]
    pm = 2.0 * np.asarray(signs, dtype=np.float64) - 1.0
    qjl = u @ pm.T
    g = np.asarray(gamma16, dtype=np.float64) * math.sqrt(math.pi / 2) / d
    return np.asarray(norm16, dtype=np.float64)[None, :] * (mse + g[None, :] * qjl)


def quantize_values(X: np.ndarray, Pi: np.ndarray, cv: np.ndarray):
    """Reconstruction variant for values: (codes [n][d], norm16 float16 [n]),
    the MSE codes of y = Pi x / |x| with |x| stored in fp16."""
    codes, norm, _ = quantize_mse(X, Pi, cv)
    return codes, norm.astype(np.float16)


def attend_values(P: np.ndarray, codes, norm16, Pi, cv) -> np.ndarray:
    """Attention output over quantized values: o[q] = sum_i P[q][i] v_hat_i
    with v_hat_i = |v_i| Pi^T c[code_i] (fp64); P [nq][n]."""
    Vh = dequantize_mse(codes, np.asarray(norm16, dtype=np.float64), Pi, cv)
    return np.asarray(P, dtype=np.float64) @ Vh
