"""Pins of the group-RTN encoding (oracle/rtn.py) against facts that do not
depend on the oracle itself: the fp16 number line enumerated by brute force,
the |w - w_hat| <= s/2 bound, nearest-level brute force, exact rational
arithmetic, and hand-built special cases."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import rtn
from workloads import gen_weights, rng_for

ALL_F16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
FINITE_F16 = np.unique(ALL_F16[np.isfinite(ALL_F16)].astype(np.float64))  # sorted, -0 merged


def brute_down(v):
    i = np.searchsorted(FINITE_F16, v, side="right") - 1
    return FINITE_F16[i] if i >= 0 else -np.inf


def brute_up(v):
    i = np.searchsorted(FINITE_F16, v, side="left")
    return FINITE_F16[i] if i < len(FINITE_F16) else np.inf


def test_fp16_directed_rounding_matches_number_line():
    rng = np.random.default_rng(1)
    vals = list(FINITE_F16[::37])                       # exact fp16 values
    mids = (FINITE_F16[1:] + FINITE_F16[:-1]) / 2        # ties of RNE
    vals += list(mids[::41])
    vals += list(rng.standard_normal(2000) * 0.05)
    vals += list(rng.standard_normal(500) * 1e-6)       # subnormal range
    vals += [0.0, -0.0, 65504.0, -65504.0, 65519.0, 1e-9, -1e-9, 6.1e-5]
    vals = np.array(vals, dtype=np.float64)
    d = rtn.fp16_round_down(vals).astype(np.float64)
    u = rtn.fp16_round_up(vals).astype(np.float64)
    for v, dv, uv in zip(vals, d, u):
        assert dv == brute_down(v), v
        assert uv == brute_up(v), v
    # +0, never -0
    assert not np.signbit(rtn.fp16_round_down(np.array([-0.0, 0.0, 1e-12]))).any()
    assert not np.signbit(rtn.fp16_round_up(np.array([-1e-12, -0.0]))).any()


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6])
@pytest.mark.parametrize("group", [32, 64])
def test_rtn_bound_and_range(bits, group):
    W = gen_weights(64, 1024, rng_for(99, bits * 100 + group), outliers=True)
    q, s, o = rtn.quantize(W, bits, group)
    L = (1 << bits) - 1
    assert q.dtype == np.uint8 and q.max() <= L
    w_hat = rtn.dequantize(q, s, o, group)
    s_full = np.repeat(s.astype(np.float64), group, axis=1)
    err = np.abs(W.astype(np.float64) - w_hat)
    assert np.all(err <= s_full / 2 * (1 + 2.0 ** -40))
    # outward rounding of the constants
    Wg = W.astype(np.float64).reshape(64, -1, group)
    mn, mx = Wg.min(2), Wg.max(2)
    o64, s64 = o.astype(np.float64), s.astype(np.float64)
    assert np.all(o64 <= mn)
    assert np.all(o64 + L * s64 >= mx * (1 - 2.0 ** -40) - 1e-30)
    # endpoints: min -> 0 and max -> L where the offset rounding gap is < s/2
    ok = (mn - o64) < s64 / 2
    qg = q.reshape(64, -1, group)
    amin = Wg.argmin(2)
    amax = Wg.argmax(2)
    rows, cols = np.nonzero(ok)
    assert np.all(qg[rows, cols, amin[rows, cols]] == 0)
    assert np.all(qg[rows, cols, amax[rows, cols]] == L)


@pytest.mark.parametrize("bits", [2, 4, 6])
def test_rtn_nearest_level_brute_force(bits):
    W = gen_weights(8, 128, rng_for(98, bits), outliers=True)
    q, s, o = rtn.quantize(W, bits, 32)
    L = (1 << bits) - 1
    s64 = np.repeat(s.astype(np.float64), 32, axis=1)
    o64 = np.repeat(o.astype(np.float64), 32, axis=1)
    levels = o64[:, :, None] + s64[:, :, None] * np.arange(L + 1)[None, None, :]
    dist = np.abs(W.astype(np.float64)[:, :, None] - levels)
    chosen = np.take_along_axis(dist, q[:, :, None].astype(np.int64), 2)[:, :, 0]
    assert np.all(chosen <= dist.min(2) * (1 + 1e-12) + 1e-300)


def test_rtn_codes_match_exact_rational_arithmetic():
    W = gen_weights(4, 256, rng_for(97, 0), outliers=True)
    q, s, o = rtn.quantize(W, 4, 64)
    for n in range(4):
        for j in range(256 // 64):
            sf = Fraction(float(s[n, j])); of = Fraction(float(o[n, j]))
            for k in range(64):
                w = Fraction(float(W[n, j * 64 + k]))
                t = (w - of) / sf
                fl = t.numerator // t.denominator
                rem = t - fl
                r = fl + (1 if rem > Fraction(1, 2) else 0 if rem < Fraction(1, 2) else fl % 2)
                assert q[n, j * 64 + k] == min(max(r, 0), 15)


def test_rtn_ties_go_to_even():
    g = np.zeros(32, dtype=np.float32)
    g[1] = 15.0                    # min 0 -> o = 0, max 15 -> s = 1 at 4 bits
    g[2], g[3], g[4], g[5] = 2.5, 3.5, 0.5, 14.5
    q, s, o = rtn.quantize(g[None, :], 4, 32)
    assert float(s[0, 0]) == 1.0 and float(o[0, 0]) == 0.0
    assert list(q[0, 2:6]) == [2, 4, 0, 14]


def test_rtn_constant_groups():
    g = np.full((1, 64), 0.25, dtype=np.float32)          # fp16-exact constant
    q, s, o = rtn.quantize(g, 3, 32)
    assert np.all(q == 0) and np.all(s.astype(np.float64) == 0) and np.all(o.astype(np.float64) == 0.25)
    g = np.full((1, 32), 0.1, dtype=np.float32)           # not fp16-exact
    q, s, o = rtn.quantize(g, 3, 32)
    assert float(s[0, 0]) > 0
    w_hat = rtn.dequantize(q, s, o, 32)
    assert np.all(np.abs(w_hat - np.float64(np.float32(0.1))) <= float(s[0, 0]) / 2)


def test_rtn_integer_special_case():
    """Integer weights in [0, L] with 0 and L in every group: s = 1, o = 0, q = w."""
    rng = np.random.default_rng(5)
    for bits in (2, 3, 4, 5, 6):
        L = (1 << bits) - 1
        W = rng.integers(0, L + 1, size=(3, 128)).astype(np.float32)
        W[:, ::32] = 0
        W[:, 1::32] = L
        q, s, o = rtn.quantize(W, bits, 32)
        assert np.all(s.astype(np.float64) == 1) and np.all(o.astype(np.float64) == 0)
        assert np.array_equal(q.astype(np.float32), W)


def test_rtn_errors():
    W = np.zeros((1, 32), dtype=np.float32)
    W[0, 3] = np.nan
    with pytest.raises(rtn.RangeError):
        rtn.quantize(W, 4, 32)
    W = np.zeros((1, 32), dtype=np.float32)
    W[0, 0] = -1e6
    with pytest.raises(rtn.RangeError):
        rtn.quantize(W, 4, 32)
    W = np.zeros((1, 32), dtype=np.float32)
    W[0, 0] = 3e6                                 # (max - o)/L above 65504
    with pytest.raises(rtn.RangeError):
        rtn.quantize(W, 4, 32)
    with pytest.raises(ValueError):
        rtn.quantize(np.zeros((1, 48), np.float32), 4, 32)
    with pytest.raises(ValueError):
        rtn.quantize(np.zeros((1, 64), np.float32), 7, 32)
