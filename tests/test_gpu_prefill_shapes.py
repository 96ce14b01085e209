"""GPU parity of the prefill GEMM on seeded random shapes, all three weight
formats, against the CPU oracle on sampled rows and columns.

The launcher picks the tile (256 x 256, 128 x 256 or 64 x 128, or the
split-precision kernel below K = 512) from the shape, and plain bf16 X tiles
take a different staging path from scaled or split ones; random M, N and K
(with ragged tails in every dimension) reach each combination without
naming it.  The shapes are drawn once from a fixed seed, so every run checks
the same cases.
"""
import numpy as np
import pytest

import oracle
from gpu_util import check_err, dev, dev_bf16, host, say
from workloads import gen_binlr, gen_weights, gen_x_bf16, rng_for

pytestmark = pytest.mark.gpu

_R = np.random.default_rng(20260)


def _dim(lo, hi, i):
    # even cases log-uniform (short dimensions common), odd cases uniform
    # (large ones common, so the big tiles are reached too)
    if i % 2 == 0:
        return int(np.exp(_R.uniform(np.log(lo), np.log(hi))))
    return int(_R.integers(lo, hi + 1))


RTN_CASES = []
for i in range(8):
    bits, group = int(_R.integers(2, 7)), int(_R.choice([32, 64]))
    RTN_CASES.append((bits, group, _dim(1, 2600, i), _dim(1, 9000, i), group * _dim(1, 3200 // group, i)))
BIN_CASES = [(_dim(1, 2600, i), _dim(1, 9000, i), 8 * _dim(1, 400, i), _dim(1, 1500, i)) for i in range(8)]
CB_CASES = []
for i in range(6):
    bits, group = int(_R.integers(2, 5)), int(_R.choice([32, 64]))
    CB_CASES.append((bits, group, _dim(1, 2600, i), _dim(1, 9000, i), group * _dim(1, 3200 // group, i)))


def _rows_cols(M, N, seed):
    r = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, M - 1], r.choice(M, min(M, 12), replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], r.choice(N, min(N, 40), replace=False)]))
    return rows, cols


@pytest.mark.parametrize("bits,group,M,N,K", RTN_CASES)
def test_rtn_random_shape(gpu, bits, group, M, N, K):
    say(f"prefill rtn b={bits} g={group} M={M} N={N} K={K}")
    seed = M * 7 + N * 13 + K
    W = gen_weights(N, K, rng_for(600, seed), outliers=True)
    codes, meta = gpu.qpack_group(dev(W), bits, group)
    X = gen_x_bf16(M, K, rng_for(601, seed))
    Y = host(gpu.qgemm_prefill(gpu.make_qweight_group(codes, meta, N, K, bits, group), dev_bf16(X)))
    rows, cols = _rows_cols(M, N, seed)
    q, s, o = oracle.rtn.quantize(W[cols], bits, group)
    W_hat = oracle.rtn.dequantize(q, s, o, group)
    Xv = oracle.product.bf16_to_f64(X[rows])
    err = check_err(Y[np.ix_(rows, cols)], oracle.product.matmul_ref(W_hat, Xv),
                    oracle.product.abs_denominator(W_hat, Xv))
    say(f"  err={err:.2e}")


@pytest.mark.parametrize("M,N,K,r", BIN_CASES)
def test_binlr_random_shape(gpu, M, N, K, r):
    say(f"prefill binlr M={M} N={N} K={K} r={r}")
    seed = M * 7 + N * 13 + K * 3 + r
    U, V, s1, s2 = gen_binlr(N, K, r, rng_for(602, seed))
    ubd, vbd = gpu.qpack_binlr(dev(U), dev(V))
    X = gen_x_bf16(M, K, rng_for(603, seed))
    w = gpu.make_qweight_binlr(ubd, vbd, dev(s1.view(np.int16)), dev(s2.view(np.int16)), N, K, r)
    Y = host(gpu.qgemm_prefill(w, dev_bf16(X)))
    rows, cols = _rows_cols(M, N, seed)
    W = oracle.binlr.reconstruct(U[cols], V, s1[cols], s2)
    Xv = oracle.product.bf16_to_f64(X[rows])
    err = check_err(Y[np.ix_(rows, cols)], oracle.product.matmul_ref(W, Xv),
                    oracle.product.binlr_abs_denominator(U[cols], V, s1[cols], s2, Xv))
    say(f"  err={err:.2e}")


@pytest.mark.parametrize("bits,group,M,N,K", CB_CASES)
def test_codebook_random_shape(gpu, bits, group, M, N, K):
    say(f"prefill codebook b={bits} g={group} M={M} N={N} K={K}")
    seed = M * 7 + N * 13 + K
    books = rng_for(604, seed).integers(0, 128, size=(8, 1 << bits)).astype(np.uint8)
    W = gen_weights(N, K, rng_for(605, seed), outliers=True)
    bd = dev(books)
    c, m, k = gpu.qpack_group_cb(dev(W), bits, group, bd)
    X = gen_x_bf16(M, K, rng_for(606, seed))
    w = gpu.make_qweight_group(c, m, N, K, bits, group, book_ids=k, books=bd)
    Y = host(gpu.qgemm_prefill(w, dev_bf16(X)))
    rows, cols = _rows_cols(M, N, seed)
    q, s, o, ids = oracle.codebook.quantize(W[cols], bits, group, books)
    assert np.array_equal(host(k)[cols], ids)
    W_hat = oracle.codebook.dequantize(q, s, o, ids, books, bits, group)
    Xv = oracle.product.bf16_to_f64(X[rows])
    err = check_err(Y[np.ix_(rows, cols)], oracle.product.matmul_ref(W_hat, Xv),
                    oracle.product.abs_denominator(W_hat, Xv))
    say(f"  err={err:.2e}")
