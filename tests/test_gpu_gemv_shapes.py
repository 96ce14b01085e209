"""GPU parity of the decode GEMVs on seeded random shapes: group RTN (batch
1 with fp32 or bf16 x, batch 2..16 with bf16 x), binary low-rank and
codebook codes, against the CPU oracle on sampled outputs.

Each launcher derives its geometry from the shape (how far a row's units
are split over waves, rows per stream or row tiles per workgroup, one bf16
weight operand or hi + lo below 512 inputs, the binary stages' steps per
wave and their full or general variants); random N, K, r and batch sizes
with ragged tails reach those branches without naming them.  The shapes are
drawn once from a fixed seed.
"""
import numpy as np
import pytest

import oracle
from gpu_util import check_err, dev, dev_bf16, host, say
from workloads import gen_binlr, gen_weights, gen_x_bf16, gen_x_f32, rng_for

pytestmark = pytest.mark.gpu

_R = np.random.default_rng(31337)


def _dim(lo, hi, i):
    # even cases log-uniform, odd cases uniform
    if i % 2 == 0:
        return int(np.exp(_R.uniform(np.log(lo), np.log(hi))))
    return int(_R.integers(lo, hi + 1))


GROUP_CASES = []
for i in range(12):
    bits, group = int(_R.integers(2, 7)), int(_R.choice([32, 64]))
    B = 1 if i % 3 == 0 else int(_R.integers(1, 17))
    xkind = "f32" if (B == 1 and i % 2 == 0) else "bf16"
    GROUP_CASES.append((bits, group, B, xkind, _dim(1, 30000, i), group * _dim(1, 12000 // group, i)))
BIN_CASES = [(int(_R.integers(1, 17)) if i % 2 else 1, _dim(1, 30000, i), _dim(1, 9000, i), _dim(1, 3000, i))
             for i in range(8)]
CB_CASES = []
for i in range(6):
    bits, group = int(_R.integers(2, 5)), int(_R.choice([32, 64]))
    B = 1 if i % 2 == 0 else int(_R.integers(2, 17))
    CB_CASES.append((bits, group, B, _dim(1, 30000, i), group * _dim(1, 12000 // group, i)))


def _x(B, K, xkind, rng):
    if xkind == "f32":
        xh = gen_x_f32(B, K, rng)
        return xh.astype(np.float64), dev(xh)
    xb = gen_x_bf16(B, K, rng)
    return oracle.product.bf16_to_f64(xb), dev_bf16(xb)


def _cols(N, seed):
    r = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, N - 1], r.choice(N, min(N, 48), replace=False)]))


@pytest.mark.parametrize("bits,group,B,xkind,N,K", GROUP_CASES)
def test_group_random_shape(gpu, bits, group, B, xkind, N, K):
    say(f"gemv group b={bits} g={group} B={B} x={xkind} N={N} K={K}")
    seed = N * 7 + K * 3 + B
    W = gen_weights(N, K, rng_for(610, seed), outliers=True)
    codes, meta = gpu.qpack_group(dev(W), bits, group)
    xv, xd = _x(B, K, xkind, rng_for(611, seed))
    y = host(gpu.qgemv_group(codes, meta, N, K, bits, group, xd)).reshape(B, N)
    cols = _cols(N, seed)
    q, s, o = oracle.rtn.quantize(W[cols], bits, group)
    W_hat = oracle.rtn.dequantize(q, s, o, group)
    err = check_err(y[:, cols], oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv))
    say(f"  err={err:.2e}")


@pytest.mark.parametrize("B,N,K,r", BIN_CASES)
def test_binlr_random_shape(gpu, B, N, K, r):
    say(f"gemv binlr B={B} N={N} K={K} r={r}")
    seed = N * 7 + K * 3 + r + B
    U, V, s1, s2 = gen_binlr(N, K, r, rng_for(612, seed))
    ubd, vbd = gpu.qpack_binlr(dev(U), dev(V))
    xv, xd = _x(B, K, "bf16", rng_for(613, seed))
    y = host(gpu.qgemv_binlr(ubd, vbd, dev(s1.view(np.int16)), dev(s2.view(np.int16)), N, K, r, xd)).reshape(B, N)
    cols = _cols(N, seed)
    W = oracle.binlr.reconstruct(U[cols], V, s1[cols], s2)
    err = check_err(y[:, cols], oracle.product.matmul_ref(W, xv),
                    oracle.product.binlr_abs_denominator(U[cols], V, s1[cols], s2, xv))
    say(f"  err={err:.2e}")


@pytest.mark.parametrize("bits,group,B,N,K", CB_CASES)
def test_codebook_random_shape(gpu, bits, group, B, N, K):
    say(f"gemv codebook b={bits} g={group} B={B} N={N} K={K}")
    seed = N * 7 + K * 3 + B
    books = rng_for(614, seed).integers(0, 128, size=(8, 1 << bits)).astype(np.uint8)
    W = gen_weights(N, K, rng_for(615, seed), outliers=True)
    bd = dev(books)
    c, m, k = gpu.qpack_group_cb(dev(W), bits, group, bd)
    xv, xd = _x(B, K, "bf16", rng_for(616, seed))
    y = host(gpu.qgemv_group_cb(c, m, k, bd, N, K, bits, group, xd)).reshape(B, N)
    cols = _cols(N, seed)
    q, s, o, ids = oracle.codebook.quantize(W[cols], bits, group, books)
    assert np.array_equal(host(k)[cols], ids)
    W_hat = oracle.codebook.dequantize(q, s, o, ids, books, bits, group)
    err = check_err(y[:, cols], oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv))
    say(f"  err={err:.2e}")


# Tall matrices whose batched launch takes seven 16-row tiles per workgroup
# (N of about 20000 and more; 3-bit codes take four), with a ragged last
# workgroup: plain codes with one bf16 weight operand (K >= 512) and with the
# hi + lo split (K < 512), outlier columns and codebooks.
RT7_CASES = [
    ("plain", 4, 64, 16, 28632, 1024),
    ("plain", 3, 32, 8, 27000, 576),
    ("plain", 2, 32, 5, 28672, 448),
    ("plain", 5, 64, 3, 25000, 640),
    ("plain", 6, 32, 2, 25001, 512),
    ("outlier", 4, 64, 16, 28600, 1024),
    ("outlier", 3, 32, 9, 25003, 448),
    ("codebook", 4, 64, 16, 28600, 512),
    ("codebook", 3, 32, 7, 25001, 448),
]


@pytest.mark.parametrize("kind,bits,group,B,N,K", RT7_CASES)
def test_batched_seven_tile_workgroups(gpu, kind, bits, group, B, N, K):
    say(f"gemv {kind} b={bits} g={group} B={B} N={N} K={K} (seven-tile workgroups)")
    seed = N * 5 + K + B
    W = gen_weights(N, K, rng_for(617, seed), outliers=True)
    xv, xd = _x(B, K, "bf16", rng_for(618, seed))
    cols = _cols(N, seed)
    if kind == "plain":
        codes, meta = gpu.qpack_group(dev(W), bits, group)
        y = gpu.qgemv_group(codes, meta, N, K, bits, group, xd)
        q, s, o = oracle.rtn.quantize(W[cols], bits, group)
        W_hat = oracle.rtn.dequantize(q, s, o, group)
    elif kind == "outlier":
        c, m, sd, ix = gpu.qpack_group_outlier(dev(W), bits, group, 6)
        y = gpu.qgemv_group_outlier(c, m, sd, ix, N, K, bits, group, xd)
        idx = oracle.outlier.outlier_channels(W, 6)
        assert np.array_equal(host(ix), idx.astype(np.int32))
        q, s, o, side = oracle.outlier.encode_with(W[cols], bits, group, idx)
        W_hat = oracle.outlier.reconstruct(q, s, o, group, side, idx)
    else:
        books = rng_for(619, seed).integers(0, 128, size=(8, 1 << bits)).astype(np.uint8)
        bd = dev(books)
        c, m, k = gpu.qpack_group_cb(dev(W), bits, group, bd)
        y = gpu.qgemv_group_cb(c, m, k, bd, N, K, bits, group, xd)
        q, s, o, ids = oracle.codebook.quantize(W[cols], bits, group, books)
        W_hat = oracle.codebook.dequantize(q, s, o, ids, books, bits, group)
    y = host(y).reshape(B, N)
    err = check_err(y[:, cols], oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv))
    say(f"  err={err:.2e}")


# Binary GEMV shapes with tall second stages (N of 16000 to 28672) and
# ragged last workgroups, one or several K-steps per table chunk, full and
# general kernels, batch 1 and more.
BIN_RT_CASES = [
    (1, 28600, 1024, 512),
    (3, 25001, 640, 4100),
    (4, 28672, 512, 1024),
    (2, 16384, 512, 2048),
    (1, 16000, 1000, 3000),
    (5, 20003, 448, 700),
]


@pytest.mark.parametrize("B,N,K,r", BIN_RT_CASES)
def test_binlr_tall_stage2(gpu, B, N, K, r):
    say(f"gemv binlr B={B} N={N} K={K} r={r} (tall second stage)")
    seed = N * 11 + K * 5 + r + B
    U, V, s1, s2 = gen_binlr(N, K, r, rng_for(620, seed))
    ubd, vbd = gpu.qpack_binlr(dev(U), dev(V))
    xv, xd = _x(B, K, "bf16", rng_for(621, seed))
    y = host(gpu.qgemv_binlr(ubd, vbd, dev(s1.view(np.int16)), dev(s2.view(np.int16)), N, K, r, xd)).reshape(B, N)
    cols = _cols(N, seed)
    W = oracle.binlr.reconstruct(U[cols], V, s1[cols], s2)
    err = check_err(y[:, cols], oracle.product.matmul_ref(W, xv),
                    oracle.product.binlr_abs_denominator(U[cols], V, s1[cols], s2, xv))
    say(f"  err={err:.2e}")
