"""GPU parity of the key-cache quantizer and its attention logits ("70B en
4GB de VRAM: la compresión neural de 2026, ¿es real?", section 3,
TurboQuant) against the CPU oracle: codes, signs and fp16 norms bit-exact;
logits within the bound of one bf16 rounding of the rotated query operands.

Logit error bound: Pi q and S Pi q are formed in fp32 and rounded once to
bf16, which has 8 significant bits, so each element moves by at most 2^-8
of itself (round to nearest even, unit roundoff 2^-8); codebook values and
signs are exact and the products accumulate in fp32.  Against
D = |x| (sum |c||Pi q| + gamma sqrt(pi/2)/128 sum |S Pi q|) the error is
therefore <= 2^-8 D, plus the fp32 formation and accumulation of 128-term
sums (below 2^-16 D): the tests hold every logit to 2^-8 + 2^-14."""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev, host, say
from workloads import rng_for

pytestmark = pytest.mark.gpu
tq = oracle.turboquant
TOL = 2.0 ** -8 + 2.0 ** -14


def _setup(bits, seed):
    rng = rng_for(410, seed)
    Pi = tq.rotation(rng.standard_normal((128, 128)))
    S = rng.standard_normal((128, 128))
    delta, table = tq.stored_table(tq.lloyd_max(128, bits - 1))
    return Pi, S, delta, table, tq.table_values(delta, table)


def _keys(n, seed, outliers=True):
    rng = rng_for(411, seed)
    K = rng.standard_normal((n, 128)).astype(np.float32)
    if outliers:
        K[:, [3, 77]] *= 10.0          # a few heavy channels, as keys have
    return K


def _oracle_packed(K, bits, Pi, S, cv):
    codes, signs, n16, g16 = tq.quantize_prod(K, Pi, S, cv)
    words = oracle.fmt.pack_codes(codes.astype(np.uint8), bits - 1)            # [n][4 units][m words]
    sw = np.zeros((K.shape[0], 4), dtype=np.uint64)
    for j in range(128):
        sw[:, j // 32] |= signs[:, j].astype(np.uint64) << np.uint64(j % 32)
    nw = n16.view(np.uint16).astype(np.uint32) | (g16.view(np.uint16).astype(np.uint32) << 16)
    return (codes, signs, n16, g16), words, sw.astype(np.uint32), nw


@pytest.mark.parametrize("bits", [3, 4])
def test_encoder_bit_exact(gpu, bits):
    Pi, S, delta, table, cv = _setup(bits, bits)
    K = _keys(300, bits)
    K[5] = 0.0                          # zero key: norm 0, codes of y = 0
    K[6] = 0.0
    K[6, 17] = 1.0                      # one-hot
    K[7] = np.float32(1e-3) * K[8]      # tiny norm
    (_, _, _, _), words, sw, nw = _oracle_packed(K, bits, Pi, S, cv)
    c, s, nm = gpu.qtq_quant_keys(dev(K), bits, dev(Pi), dev(S), delta, table)
    assert np.array_equal(host(c).view(np.uint32), words.reshape(-1))
    assert np.array_equal(host(s).view(np.uint32), sw)
    assert np.array_equal(host(nm).view(np.uint32), nw)


def test_encoder_range_errors(gpu):
    Pi, S, delta, table, cv = _setup(4, 0)
    K = _keys(4, 0)
    K[2, 0] = 1e6                       # |x| beyond fp16
    with pytest.raises(gpu.QError) as e:
        gpu.qtq_quant_keys(dev(K), 4, dev(Pi), dev(S), delta, table)
    assert e.value.status == gpu.Q_ERANGE
    K[2, 0] = np.nan
    with pytest.raises(gpu.QError) as e:
        gpu.qtq_quant_keys(dev(K), 4, dev(Pi), dev(S), delta, table)
    assert e.value.status == gpu.Q_ERANGE


def _check_logits(out, Qv, parts, Pi, S, cv, keys_idx=None):
    codes, signs, n16, g16 = parts
    H, nq, _ = Qv.shape
    worst = 0.0
    for h in range(H):
        sel = slice(None) if keys_idx is None else keys_idx
        ref = tq.logits_prod(Qv[h], codes[h][sel], signs[h][sel], n16[h][sel], g16[h][sel], Pi, S, cv)
        qr = Qv[h].astype(np.float64) @ Pi.T
        u = qr @ S.T
        D = n16[h][sel].astype(np.float64)[None, :] * (
            np.abs(qr) @ np.abs(cv[codes[h][sel]]).T
            + (g16[h][sel].astype(np.float64) * math.sqrt(math.pi / 2) / 128)[None, :] * np.abs(u).sum(axis=1)[:, None])
        got = out[h][:, sel]
        err = np.max(np.abs(got - ref) / np.where(D > 0, D, 1.0))
        worst = max(worst, err)
    assert worst <= TOL, worst
    return worst


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("nq", [1, 3, 4, 8, 16, 18])
def test_logits(gpu, bits, nq):
    """Three heads of 1000 keys (a ragged last wave step), 1..18 queries per
    head (18: two chunks of the 16 matrix-core columns)."""
    Pi, S, delta, table, cv = _setup(bits, 10 + bits)
    H, n = 3, 1000
    K = _keys(H * n, 20 + bits)
    K[7] = 0.0
    parts, _, _, _ = _oracle_packed(K, bits, Pi, S, cv)
    parts = tuple(p.reshape((H, n) + p.shape[1:]) for p in parts)
    c, s, nm = gpu.qtq_quant_keys(dev(K), bits, dev(Pi), dev(S), delta, table)
    Qv = rng_for(412, nq).standard_normal((H, nq, 128)).astype(np.float32)
    out = host(gpu.qtq_logits(c, s, nm, n, H, bits, delta, table, dev(Pi), gpu.qtq_project(dev(S), dev(Pi)), dev(Qv)))
    err = _check_logits(out, Qv, parts, Pi, S, cv)
    say(f"  tq logits bits={bits} nq={nq}: err={err:.2e}")


@pytest.mark.parametrize("n", [1003, 17, 3, 1])
def test_logits_ragged_key_count(gpu, n):
    """Key counts that are not a multiple of 4 (the last group of four keys
    is partial) and fewer keys than one wave step."""
    bits = 4
    Pi, S, delta, table, cv = _setup(bits, 60)
    H = 2
    K = _keys(H * n, 61)
    parts, _, _, _ = _oracle_packed(K, bits, Pi, S, cv)
    parts = tuple(p.reshape((H, n) + p.shape[1:]) for p in parts)
    c, s, nm = gpu.qtq_quant_keys(dev(K), bits, dev(Pi), dev(S), delta, table)
    Qv = rng_for(415, n).standard_normal((H, 3, 128)).astype(np.float32)
    out = host(gpu.qtq_logits(c, s, nm, n, H, bits, delta, table, dev(Pi), gpu.qtq_project(dev(S), dev(Pi)), dev(Qv)))
    _check_logits(out, Qv, parts, Pi, S, cv)


def test_logits_long_context_sampled(gpu):
    """Two heads of 131072 keys (a 128K context), 4 grouped queries: every
    logit computed on the GPU, a sample of keys checked against the oracle
    (each estimate depends on its own key only)."""
    bits = 4
    Pi, S, delta, table, cv = _setup(bits, 30)
    H, n = 2, 131072
    say(f"tq long context H={H} n={n}")
    K = _keys(H * n, 31)
    c, s, nm = gpu.qtq_quant_keys(dev(K), bits, dev(Pi), dev(S), delta, table)
    Qv = rng_for(413, 0).standard_normal((H, 4, 128)).astype(np.float32)
    out = host(gpu.qtq_logits(c, s, nm, n, H, bits, delta, table, dev(Pi), gpu.qtq_project(dev(S), dev(Pi)), dev(Qv)))
    idx = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(19).choice(n, 200, replace=False)]))
    rows = np.concatenate([h * n + idx for h in range(H)])
    parts, words, sw, nw = _oracle_packed(K[rows], bits, Pi, S, cv)
    cw = host(c).view(np.uint32).reshape(H * n, -1)[rows]
    assert np.array_equal(cw, words.reshape(len(rows), -1))
    assert np.array_equal(host(s).view(np.uint32)[rows], sw)
    assert np.array_equal(host(nm).view(np.uint32)[rows], nw)
    parts = tuple(p.reshape((H, len(idx)) + p.shape[1:]) for p in parts)
    out_s = out[:, :, idx]
    _check_logits(out_s, Qv, parts, Pi, S, cv)


def test_logits_estimate_inner_products(gpu):
    """End to end on the GPU: over many keys the logits track the exact
    inner products with no systematic shrink (slope of the fit ~1).  The
    sign term's spread is gamma |q| sqrt(pi/2) / sqrt(d) per unit |x|; with 3
    codebook bits (gamma ~ 0.18) that is ~0.23 of the spread |q|/sqrt(d) of
    the true products, so the correlation is ~1/sqrt(1 + 0.23^2) = 0.975."""
    bits = 4
    Pi, S, delta, table, cv = _setup(bits, 40)
    n = 20000
    K = _keys(n, 41, outliers=False)
    c, s, nm = gpu.qtq_quant_keys(dev(K), bits, dev(Pi), dev(S), delta, table)
    Qv = rng_for(414, 0).standard_normal((1, 1, 128)).astype(np.float32)
    est = host(gpu.qtq_logits(c, s, nm, n, 1, bits, delta, table, dev(Pi), gpu.qtq_project(dev(S), dev(Pi)), dev(Qv)))[0, 0]
    true = K.astype(np.float64) @ Qv[0, 0].astype(np.float64)
    slope = float(est @ true / (true @ true))
    assert abs(slope - 1.0) < 0.02, slope
    assert np.corrcoef(est, true)[0, 1] > 0.96


# ------------------------------------------------------------------ values
def _value_setup(bits, seed):
    rng = rng_for(420, seed)
    Pi = tq.rotation(rng.standard_normal((128, 128)))
    delta, table = tq.stored_table(tq.lloyd_max(128, bits))
    return Pi, delta, table, tq.table_values(delta, table)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_value_encoder_bit_exact(gpu, bits):
    Pi, delta, table, cv = _value_setup(bits, bits)
    V = _keys(300, 30 + bits)
    V[9] = 0.0
    codes, n16 = tq.quantize_values(V, Pi, cv)
    words = oracle.fmt.pack_codes(codes.astype(np.uint8), bits)
    c, nm = gpu.qtq_quant_values(dev(V), bits, dev(Pi), delta, table)
    assert np.array_equal(host(c).view(np.uint32), words.reshape(-1))
    assert np.array_equal(host(nm).view(np.uint32), n16.view(np.uint16).astype(np.uint32))


@pytest.mark.parametrize("bits,nq,n", [(3, 1, 1000), (3, 4, 1000), (4, 2, 1000), (2, 5, 1000), (3, 18, 777), (4, 4, 20000),
                                       (3, 2, 1), (2, 1, 5)])
def test_attend(gpu, bits, nq, n):
    """Attention output over quantized values against the oracle's fp64
    sum, element by element.  The kernel sums over the values in the rotated
    domain (weights p |v| as bf16 hi + lo, 2^-16 relative; fp32 sums) and
    then applies Pi^T, so the error of output coordinate c is bounded by the
    relative error of the rotated sums times
    D[c] = sum_d |Pi[d][c]| sum_j |p_j| |v_j| |c_j[d]|; tested at 1e-4."""
    Pi, delta, table, cv = _value_setup(bits, 40 + nq)
    H = 3
    V = _keys(H * n, 50 + bits)
    say(f"tq attend bits={bits} nq={nq} n={n}")
    codes, n16 = tq.quantize_values(V, Pi, cv)
    c, nm = gpu.qtq_quant_values(dev(V), bits, dev(Pi), delta, table)
    rng = rng_for(421, nq)
    P = rng.random((H, nq, n)).astype(np.float32)
    P /= P.sum(axis=2, keepdims=True)
    out = host(gpu.qtq_attend(c, nm, n, H, bits, delta, table, dev(Pi), dev(P)))
    for h in range(H):
        sl = slice(h * n, (h + 1) * n)
        ref = tq.attend_values(P[h], codes[sl], n16[sl], Pi, cv)
        # rotated-domain magnitudes |p_j| |v_j| |c_j[d]|, mapped through |Pi|
        rot = np.abs(cv[codes[sl]]) * n16[sl].astype(np.float64)[:, None]
        D = (np.abs(P[h]).astype(np.float64) @ rot) @ np.abs(Pi)
        assert np.all(D > 0)
        err = np.max(np.abs(out[h] - ref) / D)
        assert err <= 1e-4, (h, err)
