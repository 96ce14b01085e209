"""GPU parity of the outlier-aware decomposition (group RTN + fp16 outlier
columns; "Métodos de cuantización de LLM...", opening and LLM.int8()
paragraph) against the CPU oracle: packing bit-exact, products within the
normalized bound."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_bf16_out, check_err, dev, dev_bf16, host, say
from workloads import gen_x_bf16, gen_x_f32, layer_weights, layer_x, rng_for

pytestmark = pytest.mark.gpu


def _planted(N, K, cols, seed, scale=20.0):
    rng = rng_for(320, seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, cols] *= np.float32(scale)
    return W


def _oracle(W, bits, group, n_out):
    q, s, o, side, idx = oracle.outlier.encode(W, bits, group, n_out)
    words = oracle.fmt.pack_codes(q, bits)
    meta = oracle.fmt.pack_meta(s, o)
    W_hat = oracle.outlier.reconstruct(q, s, o, group, side, idx)
    return words, meta, side, idx, W_hat


@pytest.mark.parametrize("bits,group", [(4, 64), (3, 32), (2, 32), (5, 64), (6, 32), (4, 32)])
def test_pack_bit_exact(gpu, bits, group):
    N, K = 45, 1024
    cols = [0, 77, 78, 640, 1023]
    W = _planted(N, K, cols, bits * 10 + group)
    words, meta, side, idx, _ = _oracle(W, bits, group, 5)
    c, m, sd, ix = gpu.qpack_group_outlier(dev(W), bits, group, 5)
    assert list(idx) == cols and np.array_equal(host(ix), idx.astype(np.int32))
    assert np.array_equal(host(c), words.view(np.uint8).reshape(-1))
    assert np.array_equal(host(m), meta.view(np.int32).reshape(-1))
    assert np.array_equal(host(sd).view(np.uint16), side.view(np.uint16))


def test_pack_ties_and_zero_count(gpu):
    """Equal channel scores go to the lower k; n_out = 0 is qpack_group."""
    rng = rng_for(321, 0)
    N, K = 30, 256
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    for k in (9, 40, 41, 200):
        W[3, k] = 1.5
    W[7, 100] = -1.5
    words, meta, side, idx, _ = _oracle(W, 4, 32, 3)
    c, m, sd, ix = gpu.qpack_group_outlier(dev(W), 4, 32, 3)
    assert list(host(ix)) == list(idx) == [9, 40, 41]
    assert np.array_equal(host(sd).view(np.uint16), side.view(np.uint16))
    assert np.array_equal(host(c), words.view(np.uint8).reshape(-1))
    c0, m0, sd0, ix0 = gpu.qpack_group_outlier(dev(W), 3, 64, 0)
    c1, m1 = gpu.qpack_group(dev(W), 3, 64)
    assert sd0.numel() == 0 and ix0.numel() == 0
    assert torch.equal(c0, c1) and torch.equal(m0, m1)


def test_pack_range_error(gpu):
    W = np.zeros((4, 128), np.float32)
    W[1, 5] = 1e6
    with pytest.raises(gpu.QError) as e:
        gpu.qpack_group_outlier(dev(W), 4, 32, 1)
    assert e.value.status == gpu.Q_ERANGE


@pytest.mark.parametrize("B,xkind", [(1, "bf16"), (1, "f32"), (2, "bf16"), (16, "bf16")])
@pytest.mark.parametrize("bits,group", [(4, 64), (3, 32)])
def test_gemv(gpu, bits, group, B, xkind):
    N, K = 300, 2048
    cols = [3, 500, 1999, 2000]
    W = _planted(N, K, cols, 7 * bits + B)
    words, meta, side, idx, W_hat = _oracle(W, bits, group, 4)
    rng = rng_for(322, B)
    if xkind == "f32":
        xh = gen_x_f32(B, K, rng)
        xv, xd = xh.astype(np.float64), dev(xh)
    else:
        xb = gen_x_bf16(B, K, rng)
        xv, xd = oracle.product.bf16_to_f64(xb), dev_bf16(xb)
    c, m, sd, ix = gpu.qpack_group_outlier(dev(W), bits, group, 4)
    y = host(gpu.qgemv_group_outlier(c, m, sd, ix, N, K, bits, group, xd))
    err = check_err(y, oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv))
    say(f"  outlier gemv b={bits} B={B} {xkind}: err={err:.2e}")


def test_gemv_long_rows_split_k(gpu):
    """K = 65536 splits each row over 8 waves; only one of them adds the
    side term."""
    N, K = 40, 65536
    W = _planted(N, K, [10, 30000, 65535], 5)
    words, meta, side, idx, W_hat = _oracle(W, 4, 64, 3)
    xb = gen_x_bf16(1, K, rng_for(323, 0))
    xv = oracle.product.bf16_to_f64(xb)
    c, m, sd, ix = gpu.qpack_group_outlier(dev(W), 4, 64, 3)
    y = host(gpu.qgemv_group_outlier(c, m, sd, ix, N, K, 4, 64, dev_bf16(xb)))
    check_err(y, oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv))


@pytest.mark.parametrize("M,N,K", [(40, 257, 512), (4000, 7900, 1024), (70, 200, 384)])
def test_prefill(gpu, M, N, K):
    """Every tile shape: 128 x 256, 256 x 256 (M = 4000) and the
    split-precision kernel of short reductions (K = 384), whose outlier step
    carries the side columns as bf16 hi + lo too."""
    say(f"outlier prefill M={M} N={N} K={K}")
    W = _planted(N, K, [1, K // 2 - 1, K // 2], 11)
    words, meta, side, idx, W_hat = _oracle(W, 4, 64, 3)
    X = gen_x_bf16(M, K, rng_for(324, M))
    c, m, sd, ix = gpu.qpack_group_outlier(dev(W), 4, 64, 3)
    w = gpu.make_qweight_group(c, m, N, K, 4, 64, side=sd, idx=ix)
    Y = host(gpu.qgemm_prefill(w, dev_bf16(X)))
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(13).choice(M, min(M, 24), replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(14).choice(N, 48, replace=False)]))
    Xv = oracle.product.bf16_to_f64(X[rows])
    check_err(Y[np.ix_(rows, cols)], oracle.product.matmul_ref(W_hat[cols], Xv),
              oracle.product.abs_denominator(W_hat[cols], Xv))


def test_prefill_bf16_output(gpu):
    M, N, K = 64, 300, 1024
    W = _planted(N, K, [100, 101], 12)
    words, meta, side, idx, W_hat = _oracle(W, 3, 32, 2)
    X = gen_x_bf16(M, K, rng_for(325, 0))
    c, m, sd, ix = gpu.qpack_group_outlier(dev(W), 3, 32, 2)
    w = gpu.make_qweight_group(c, m, N, K, 3, 32, side=sd, idx=ix)
    Y16 = host(gpu.qgemm_prefill(w, dev_bf16(X), y_dtype=torch.bfloat16))
    Y32 = host(gpu.qgemm_prefill(w, dev_bf16(X)))
    Xv = oracle.product.bf16_to_f64(X)
    check_bf16_out(Y16, Y32, oracle.product.matmul_ref(W_hat, Xv), oracle.product.abs_denominator(W_hat, Xv))


def test_full_gate_shape(gpu):
    """The gate matrix of the layer set with its 8 outlier channels kept
    aside: packing sampled bit-exact, GEMV B = 1 and 16 on sampled rows."""
    W = layer_weights("gate")
    N, K = W.shape
    say(f"outlier full gate {N}x{K}")
    c, m, sd, ix = gpu.qpack_group_outlier(dev(W), 4, 64, 8)
    idx = oracle.outlier.outlier_channels(W, 8)
    assert np.array_equal(host(ix), idx.astype(np.int32))
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(15).choice(N, 64, replace=False)]))
    # once the channels are fixed every step is row-local: the oracle on the sampled rows
    q, s, o, side = oracle.outlier.encode_with(W[rows], 4, 64, idx)
    assert np.array_equal(host(sd)[rows].view(np.uint16), side.view(np.uint16))
    W_hat = oracle.outlier.reconstruct(q, s, o, 64, side, idx)
    for B in (1, 16):
        X = layer_x(K, B)
        y = host(gpu.qgemv_group_outlier(c, m, sd, ix, N, K, 4, 64, dev_bf16(X)))
        Xv = oracle.product.bf16_to_f64(X)
        err = check_err(y[:, rows], oracle.product.matmul_ref(W_hat, Xv), oracle.product.abs_denominator(W_hat, Xv))
        say(f"  B={B} err={err:.2e}")
