"""GPU parity of the prefill GEMM (both formats) against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, check_err, dev, dev_bf16, group_reference, host, say
from workloads import binlr_factors, gen_binlr, gen_weights, gen_x_bf16, layer_weights, layer_x, rng_for

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits,group", [(4, 64), (4, 32), (2, 32), (3, 32), (5, 64), (6, 32)])
def test_rtn_small(gpu, bits, group):
    M, N, K = 40, 200, 384
    W = gen_weights(N, K, rng_for(70, bits * 100 + group), outliers=True)
    _, _, _, words, meta, W_hat = group_reference(W, bits, group)
    X = gen_x_bf16(M, K, rng_for(71, bits))
    w = gpu.make_qweight_group(cd := dev(words.view(np.uint8).reshape(-1)), md := dev(meta.view(np.int32).reshape(-1)),
                               N, K, bits, group)
    Y = host(gpu.qgemm_prefill(w, dev_bf16(X)))
    Xv = oracle.product.bf16_to_f64(X)
    check_err(Y, oracle.product.matmul_ref(W_hat, Xv), oracle.product.abs_denominator(W_hat, Xv))
    # each prefill row equals the GEMV of that row within the bound
    y8 = host(gpu.qgemv_group(cd, md, N, K, bits, group, dev_bf16(X[:8])))
    check_err(Y[:8], y8.astype(np.float64), oracle.product.abs_denominator(W_hat, Xv[:8]))


def test_rtn_integer_exact(gpu):
    rng = np.random.default_rng(72)
    M, N, K, g = 130, 140, 256, 32
    W = rng.integers(0, 16, size=(N, K)).astype(np.float32)
    W[:, ::g] = 0
    W[:, 1::g] = 15
    codes, meta = gpu.qpack_group(dev(W), 4, g)
    Xi = rng.integers(-3, 4, size=(M, K)).astype(np.float32)
    Xb = (Xi.view(np.uint32) >> 16).astype(np.uint16)
    Y = host(gpu.qgemm_prefill(gpu.make_qweight_group(codes, meta, N, K, 4, g), dev_bf16(Xb)))
    assert np.array_equal(Y, (Xi.astype(np.int64) @ W.astype(np.int64).T).astype(np.float64))


@pytest.mark.parametrize("M,N,K,r", [(40, 200, 136, 45), (130, 70, 256, 300)])
def test_binlr_small(gpu, M, N, K, r):
    U, V, s1, s2 = gen_binlr(N, K, r, rng_for(73, M + r))
    W = oracle.binlr.reconstruct(U, V, s1, s2)
    ubd, vbd = gpu.qpack_binlr(dev(U), dev(V))
    X = gen_x_bf16(M, K, rng_for(74, M))
    s1d, s2d = dev(s1.view(np.int16)), dev(s2.view(np.int16))
    Y = host(gpu.qgemm_prefill(gpu.make_qweight_binlr(ubd, vbd, s1d, s2d, N, K, r), dev_bf16(X)))
    Xv = oracle.product.bf16_to_f64(X)
    check_err(Y, oracle.product.matmul_ref(W, Xv), oracle.product.abs_denominator(W, Xv))


def test_binlr_integer_exact(gpu):
    """s1 = s2 = 1, X in {-1, 0, 1}, small K so every T entry is bf16-exact."""
    rng = np.random.default_rng(75)
    M, N, K, r = 64, 96, 128, 40
    U, V, _, _ = gen_binlr(N, K, r, rng)
    one = dev(np.full(max(N, K), 0x3C00, np.uint16).view(np.int16))
    ubd, vbd = gpu.qpack_binlr(dev(U), dev(V))
    Xi = rng.integers(-1, 2, size=(M, K)).astype(np.float32)
    Xb = (Xi.view(np.uint32) >> 16).astype(np.uint16)
    Y = host(gpu.qgemm_prefill(gpu.make_qweight_binlr(ubd, vbd, one, one, N, K, r), dev_bf16(Xb)))
    C = oracle.binlr.sign_product(U, V)
    assert np.array_equal(Y, (Xi.astype(np.int64) @ C.T).astype(np.float64))


def _sample_cols(N, n, seed):
    """The first and last output and n more, sorted."""
    return np.unique(np.concatenate([[0, N - 1], np.random.default_rng(seed).choice(N, n, replace=False)]))


@pytest.mark.parametrize("M", [512, 4096])
def test_full_rtn(gpu, M):
    """Config 5, group RTN: the 8192 x 28672 gate matrix (4-bit g64, with its
    outlier channels) against M = 512 and 4096 tokens, in the launch the
    benchmark times.  Every token row is checked on 64 sampled outputs."""
    say(f"prefill full RTN M={M}")
    W = layer_weights("gate")
    N, K = W.shape
    codes, meta = gpu.qpack_group(dev(W), 4, 64)
    X = layer_x(K, M, config=5)
    Y = gpu.qgemm_prefill(gpu.make_qweight_group(codes, meta, N, K, 4, 64), dev_bf16(X))
    cols = _sample_cols(N, 62, 6 + M)
    Ys = host(Y)[:, cols]
    _, _, _, _, _, W_hat = group_reference(W[cols], 4, 64)
    Xv = oracle.product.bf16_to_f64(X)
    err = check_err(Ys, oracle.product.matmul_ref(W_hat, Xv), oracle.product.abs_denominator(W_hat, Xv))
    say(f"  err={err:.3e}")


@pytest.fixture(scope="module")
def binlr_full(gpu):
    K, N, r = 8192, 28672, 4096
    U, V, s1, s2 = binlr_factors(K, N, r)
    ubd, vbd = gpu.qpack_binlr(dev(U), dev(V))
    w = gpu.make_qweight_binlr(ubd, vbd, dev(s1.view(np.int16)), dev(s2.view(np.int16)), N, K, r)
    return U, V, s1, s2, w


@pytest.mark.parametrize("M", [512, 4096])
def test_full_binlr(gpu, binlr_full, M):
    """Config 5, binary: the r = 4096 factors of 8192 x 28672 against M = 512
    and 4096 tokens; every token row checked on 42 sampled outputs."""
    K, N, r = 8192, 28672, 4096
    say(f"prefill full binary M={M}")
    U, V, s1, s2, w = binlr_full
    X = layer_x(K, M, config=5)
    Y = gpu.qgemm_prefill(w, dev_bf16(X))
    cols = _sample_cols(N, 40, 8 + M)
    Ys = host(Y)[:, cols]
    W = oracle.binlr.reconstruct(U[cols], V, s1[cols], s2)
    Xv = oracle.product.bf16_to_f64(X)
    err = check_err(Ys, oracle.product.matmul_ref(W, Xv),
                    oracle.product.binlr_abs_denominator(U[cols], V, s1[cols], s2, Xv))
    say(f"  err={err:.3e}")


def test_big_tile_rtn_ragged(gpu):
    """With 256 CUs this shape takes the 256 x 256 tile (496 tiles, two
    rounds, against four rounds of 128 x 256 tiles), with ragged M and N and
    an odd number of 64-wide K steps."""
    M, N, K = 4000, 7900, 4032
    say(f"prefill big-tile RTN M={M} N={N} K={K}")
    W = gen_weights(N, K, rng_for(76, 0), outliers=True)
    codes, meta = gpu.qpack_group(dev(W), 3, 32)
    X = gen_x_bf16(M, K, rng_for(77, 0))
    Y = host(gpu.qgemm_prefill(gpu.make_qweight_group(codes, meta, N, K, 3, 32), dev_bf16(X)))
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(9).choice(M, 12, replace=False)]))
    cols = np.unique(np.concatenate([[0, 255, 256, N - 1], np.random.default_rng(10).choice(N, 40, replace=False)]))
    _, _, _, _, _, W_hat = group_reference(W[cols], 3, 32)
    Xv = oracle.product.bf16_to_f64(X[rows])
    err = check_err(Y[np.ix_(rows, cols)], oracle.product.matmul_ref(W_hat, Xv),
                    oracle.product.abs_denominator(W_hat, Xv))
    say(f"  err={err:.3e}")


@pytest.mark.parametrize("r", [1001, 1000])
def test_big_tile_binlr_ragged(gpu, r):
    """The second pass (M x N) takes the 256 x 256 tile: with r % 8 != 0 its
    masked K tail (T staged through registers), with r = 1000 the X tile
    loaded straight into LDS, K ending mid-step; the first (M x r) takes the
    64 x 128 one."""
    M, N, K = 4000, 7900, 3000
    say(f"prefill big-tile binary M={M} N={N} K={K} r={r}")
    U, V, s1, s2 = gen_binlr(N, K, r, rng_for(78, 0))
    ubd, vbd = gpu.qpack_binlr(dev(U), dev(V))
    X = gen_x_bf16(M, K, rng_for(79, 0))
    Y = host(gpu.qgemm_prefill(gpu.make_qweight_binlr(ubd, vbd, dev(s1.view(np.int16)), dev(s2.view(np.int16)),
                                                      N, K, r), dev_bf16(X)))
    rows = np.unique(np.concatenate([[0, 256, M - 1], np.random.default_rng(11).choice(M, 10, replace=False)]))
    cols = np.unique(np.concatenate([[0, 256, N - 1], np.random.default_rng(12).choice(N, 40, replace=False)]))
    W = oracle.binlr.reconstruct(U[cols], V, s1[cols], s2)
    Xv = oracle.product.bf16_to_f64(X[rows])
    err = check_err(Y[np.ix_(rows, cols)], oracle.product.matmul_ref(W, Xv),
                    oracle.product.binlr_abs_denominator(U[cols], V, s1[cols], s2, Xv))
    say(f"  err={err:.3e}")


def test_small_tile_rtn_ragged(gpu):
    """With 256 CUs this shape takes the 128 x 256 tile (218 tiles in one
    round, against 109 slower 256 x 256 tiles or four rounds of 64 x 128
    ones), with ragged M and N."""
    M, N, K = 250, 27900, 1024
    say(f"prefill small-tile RTN M={M} N={N} K={K}")
    W = gen_weights(N, K, rng_for(80, 0), outliers=True)
    codes, meta = gpu.qpack_group(dev(W), 4, 64)
    X = gen_x_bf16(M, K, rng_for(81, 0))
    Y = host(gpu.qgemm_prefill(gpu.make_qweight_group(codes, meta, N, K, 4, 64), dev_bf16(X)))
    rows = np.unique(np.concatenate([[0, 127, 128, M - 1], np.random.default_rng(13).choice(M, 12, replace=False)]))
    cols = np.unique(np.concatenate([[0, 255, 256, N - 1], np.random.default_rng(14).choice(N, 40, replace=False)]))
    _, _, _, _, _, W_hat = group_reference(W[cols], 4, 64)
    Xv = oracle.product.bf16_to_f64(X[rows])
    err = check_err(Y[np.ix_(rows, cols)], oracle.product.matmul_ref(W_hat, Xv),
                    oracle.product.abs_denominator(W_hat, Xv))
    say(f"  err={err:.3e}")


def test_tiny_tile_rtn_half_step(gpu):
    """Short M and narrow N take the 64 x 128 tile; K = 1056 (single bf16
    weights) ends on half a 64-wide step, one 32-code unit per row.  Every
    output is checked."""
    M, N, K = 100, 1000, 1056
    say(f"prefill tiny-tile RTN M={M} N={N} K={K}")
    W = gen_weights(N, K, rng_for(82, 0), outliers=True)
    codes, meta = gpu.qpack_group(dev(W), 5, 32)
    X = gen_x_bf16(M, K, rng_for(83, 0))
    Y = host(gpu.qgemm_prefill(gpu.make_qweight_group(codes, meta, N, K, 5, 32), dev_bf16(X)))
    _, _, _, _, _, W_hat = group_reference(W, 5, 32)
    Xv = oracle.product.bf16_to_f64(X)
    err = check_err(Y, oracle.product.matmul_ref(W_hat, Xv), oracle.product.abs_denominator(W_hat, Xv))
    say(f"  err={err:.3e}")
