"""GPU parity of group codes read through per-group books ("TurboQuant:
cuantizar modelos grandes para que quepan en local", introduction and
"Compresión por bloques") against the CPU oracle: codes, meta words and
book ids bit-exact; products within the normalized bound."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_bf16_out, check_err, dev, dev_bf16, host, say
from workloads import gen_weights, gen_x_bf16, gen_x_f32, layer_weights, layer_x, rng_for

pytestmark = pytest.mark.gpu


def _random_books(bits, seed, D=16):
    """Unsorted entries over the whole 0..127 range with repeated levels, so
    every table byte and every lookup path is exercised."""
    rng = rng_for(370, seed)
    books = rng.integers(0, 128, size=(D, 1 << bits)).astype(np.uint8)
    books[1, 1] = books[1, 2]
    return books


def _oracle(W, bits, group, books):
    q, s, o, ids = oracle.codebook.quantize(W, bits, group, books)
    return (oracle.fmt.pack_codes(q, bits), oracle.fmt.pack_meta(s, o), ids,
            oracle.codebook.dequantize(q, s, o, ids, books, bits, group))


def _check_pack(gpu, W, bits, group, books):
    words, meta, ids, W_hat = _oracle(W, bits, group, books)
    c, m, k = gpu.qpack_group_cb(dev(W), bits, group, dev(books))
    assert np.array_equal(host(k), ids)
    assert np.array_equal(host(m), meta.view(np.int32).reshape(-1))
    assert np.array_equal(host(c), words.view(np.uint8).reshape(-1))
    return c, m, k, W_hat


@pytest.mark.parametrize("bits,group", [(2, 32), (2, 64), (3, 32), (3, 64), (4, 32), (4, 64)])
def test_pack_bit_exact(gpu, bits, group):
    W = gen_weights(45, 1024, rng_for(371, bits * 100 + group), outliers=True)
    _check_pack(gpu, W, bits, group, oracle.codebook.default_dictionary(bits))
    _check_pack(gpu, W, bits, group, _random_books(bits, bits + group))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_ties_and_constant_groups(gpu, bits):
    """Weights half-way between uniform levels (exact ties, s = 2^-4, o = 0),
    a one-book uniform dictionary (= plain RTN, codes equal to qpack_group's)
    and constant groups."""
    L = (1 << bits) - 1
    u = np.resize(np.concatenate([[0.0, L], np.arange(2 * L + 1) / 2.0]), 64)
    W = np.stack([u * 2.0 ** -4, np.full(64, 0.375), -u * 2.0 ** -3]).astype(np.float32)
    uni = (np.arange(L + 1) * (1 << (7 - bits))).astype(np.uint8)[None, :]
    c, m, k, _ = _check_pack(gpu, W, bits, 32, uni)
    c0, m0 = gpu.qpack_group(dev(W), bits, 32)
    assert torch.equal(c, c0) and torch.equal(m, m0)
    _check_pack(gpu, W, bits, 64, oracle.codebook.default_dictionary(bits))


def test_pack_errors(gpu):
    W = gen_weights(4, 128, rng_for(372, 0), outliers=False)
    bad = oracle.codebook.default_dictionary(3).copy()
    bad[5, 2] = 128
    with pytest.raises(gpu.QError) as e:
        gpu.qpack_group_cb(dev(W), 3, 32, dev(bad))
    assert e.value.status == gpu.Q_EINVAL
    W[2, 7] = np.inf
    with pytest.raises(gpu.QError) as e:
        gpu.qpack_group_cb(dev(W), 3, 32, dev(oracle.codebook.default_dictionary(3)))
    assert e.value.status == gpu.Q_ERANGE


@pytest.mark.parametrize("B,xkind", [(1, "bf16"), (1, "f32"), (2, "bf16"), (16, "bf16")])
@pytest.mark.parametrize("bits,group", [(2, 64), (3, 32), (4, 64), (4, 32)])
def test_gemv(gpu, bits, group, B, xkind):
    """Random 16-book dictionaries (every code of every book), three
    ragged N, K spanning several K-slices."""
    books = _random_books(bits, 10 * bits + B)
    rng = rng_for(373, bits * 100 + B)
    K = 2048
    if xkind == "f32":
        xh = gen_x_f32(B, K, rng)
        xv, xd = xh.astype(np.float64), dev(xh)
    else:
        xb = gen_x_bf16(B, K, rng)
        xv, xd = oracle.product.bf16_to_f64(xb), dev_bf16(xb)
    for N in (1, 37, 300):
        W = gen_weights(N, K, rng_for(374, N + bits), outliers=True)
        c, m, k, W_hat = _check_pack(gpu, W, bits, group, books)
        y = host(gpu.qgemv_group_cb(c, m, k, dev(books), N, K, bits, group, xd))
        err = check_err(y, oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv))
        say(f"  codebook gemv b={bits} g={group} B={B} {xkind} N={N}: err={err:.2e}")


def test_gemv_bf16_output_and_long_rows(gpu):
    """bf16 output rounds once; K = 65536 splits rows over 8 waves."""
    books = oracle.codebook.default_dictionary(4)
    for K, B, y_dtype in [(1024, 1, torch.bfloat16), (65536, 1, torch.float32), (4096, 8, torch.bfloat16)]:
        say(f"codebook gemv K={K} B={B}")
        W = gen_weights(40, K, rng_for(375, K), outliers=True)
        c, m, k, W_hat = _check_pack(gpu, W, 4, 64, books)
        xb = gen_x_bf16(B, K, rng_for(376, K))
        xv = oracle.product.bf16_to_f64(xb)
        y = host(gpu.qgemv_group_cb(c, m, k, dev(books), 40, K, 4, 64, dev_bf16(xb)))
        y_ref, D = oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv)
        if y_dtype == torch.bfloat16:
            y16 = host(gpu.qgemv_group_cb(c, m, k, dev(books), 40, K, 4, 64, dev_bf16(xb), y_dtype=y_dtype))
            check_bf16_out(y16, y, y_ref, D)
        else:
            check_err(y, y_ref, D)


@pytest.mark.parametrize("bits", [2, 4])
def test_full_gate_shape(gpu, bits):
    """The gate matrix of the layer set (28672 x 8192, groups of 64) with the
    default dictionary: packing bit-exact on sampled rows (every step is
    row-local), GEMV B = 1 and 16 on sampled rows."""
    W = layer_weights("gate")
    N, K = W.shape
    say(f"codebook full gate {N}x{K} b={bits}")
    books = oracle.codebook.default_dictionary(bits)
    c, m, k = gpu.qpack_group_cb(dev(W), bits, 64, dev(books))
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(16).choice(N, 64, replace=False)]))
    q, s, o, ids = oracle.codebook.quantize(W[rows], bits, 64, books)
    assert np.array_equal(host(k)[rows], ids)
    words = oracle.fmt.pack_codes(q, bits).view(np.uint8).reshape(len(rows), -1)
    assert np.array_equal(host(c).reshape(N, -1)[rows], words)
    W_hat = oracle.codebook.dequantize(q, s, o, ids, books, bits, 64)
    for B in (1, 16):
        X = layer_x(K, B)
        y = host(gpu.qgemv_group_cb(c, m, k, dev(books), N, K, bits, 64, dev_bf16(X)))
        Xv = oracle.product.bf16_to_f64(X)
        err = check_err(y[:, rows], oracle.product.matmul_ref(W_hat, Xv), oracle.product.abs_denominator(W_hat, Xv))
        say(f"  B={B} err={err:.2e}")


@pytest.mark.parametrize("bits,M,N,K", [(4, 40, 257, 512), (3, 64, 300, 1024), (2, 40, 257, 512),
                                        (4, 4000, 7900, 1024), (4, 250, 27900, 1024), (4, 70, 200, 256),
                                        (3, 33, 65, 128)])
def test_prefill(gpu, bits, M, N, K):
    """Every tile shape (with 256 CUs): the 256 x 256 tile (M = 4000), the
    128 x 256 one (M = 250, N = 27900), the 64 x 128 one (the short and
    narrow shapes) and the split-precision kernel of short reductions
    (K < 512); sampled rows and columns."""
    say(f"codebook prefill b={bits} M={M} N={N} K={K}")
    books = _random_books(bits, 40 + bits)
    W = gen_weights(N, K, rng_for(377, M + bits), outliers=True)
    c, m, k = gpu.qpack_group_cb(dev(W), bits, 64, dev(books))
    bd = dev(books)
    X = gen_x_bf16(M, K, rng_for(378, M))
    w = gpu.make_qweight_group(c, m, N, K, bits, 64, book_ids=k, books=bd)
    Y = host(gpu.qgemm_prefill(w, dev_bf16(X)))
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(17).choice(M, min(M, 24), replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(18).choice(N, 48, replace=False)]))
    q, s, o, ids = oracle.codebook.quantize(W[cols], bits, 64, books)
    assert np.array_equal(host(k)[cols], ids)
    W_hat = oracle.codebook.dequantize(q, s, o, ids, books, bits, 64)
    Xv = oracle.product.bf16_to_f64(X[rows])
    err = check_err(Y[np.ix_(rows, cols)], oracle.product.matmul_ref(W_hat, Xv),
                    oracle.product.abs_denominator(W_hat, Xv))
    say(f"  err={err:.2e}")


def test_prefill_bf16_output(gpu):
    M, N, K = 64, 300, 1024
    books = oracle.codebook.default_dictionary(4)
    W = gen_weights(N, K, rng_for(379, 0), outliers=True)
    c, m, k, W_hat = _check_pack(gpu, W, 4, 32, books)
    X = gen_x_bf16(M, K, rng_for(380, 0))
    w = gpu.make_qweight_group(c, m, N, K, 4, 32, book_ids=k, books=dev(books))
    Y16 = host(gpu.qgemm_prefill(w, dev_bf16(X), y_dtype=torch.bfloat16))
    Y32 = host(gpu.qgemm_prefill(w, dev_bf16(X)))
    Xv = oracle.product.bf16_to_f64(X)
    check_bf16_out(Y16, Y32, oracle.product.matmul_ref(W_hat, Xv), oracle.product.abs_denominator(W_hat, Xv))


@pytest.mark.parametrize("bits,group,K", [(4, 64, 64), (2, 32, 32), (3, 32, 96)])
def test_gemv_single_group_rows(gpu, bits, group, K):
    """The smallest rows: one or a few groups (K = 32..96), N = 1 and 5,
    B = 1 and 3."""
    books = _random_books(bits, 90 + K)
    for N in (1, 5):
        W = gen_weights(N, K, rng_for(380, N + K), outliers=False)
        c, m, k, W_hat = _check_pack(gpu, W, bits, group, books)
        for B in (1, 3):
            xb = gen_x_bf16(B, K, rng_for(381, B))
            xv = oracle.product.bf16_to_f64(xb)
            y = host(gpu.qgemv_group_cb(c, m, k, dev(books), N, K, bits, group, dev_bf16(xb)))
            check_err(y, oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv))
