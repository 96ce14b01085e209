"""Edge cases of every GPU entry point against the CPU oracle: the largest
supported K, the smallest shapes (one row, one unit, one token), zero
weights, batch 16 on the binary path and bf16 outputs."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_bf16_out, check_err, dev, dev_bf16, group_reference, host, say
from workloads import gen_binlr, gen_weights, gen_x_bf16, gen_x_f32, rng_for

pytestmark = pytest.mark.gpu


def _group(gpu, N, K, bits, group, B, xkind, seed, y_dtype=torch.float32):
    W = gen_weights(N, K, rng_for(90, seed), outliers=True)
    _, _, _, words, meta, W_hat = group_reference(W, bits, group)
    rng = rng_for(91, seed)
    if xkind == "f32":
        xh = gen_x_f32(B, K, rng)
        xv, xd = xh.astype(np.float64), dev(xh)
    else:
        xb = gen_x_bf16(B, K, rng)
        xv, xd = oracle.product.bf16_to_f64(xb), dev_bf16(xb)
    cd, md = dev(words.view(np.uint8).reshape(-1)), dev(meta.view(np.int32).reshape(-1))
    y = gpu.qgemv_group(cd, md, N, K, bits, group, xd)
    y_ref, D = oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv)
    if y_dtype == torch.bfloat16:
        y16 = gpu.qgemv_group(cd, md, N, K, bits, group, xd, y_dtype=torch.bfloat16)
        return check_bf16_out(host(y16), host(y), y_ref, D)
    return check_err(host(y), y_ref, D)


@pytest.mark.parametrize("xkind,K", [("bf16", 65536), ("f32", 32768)])
def test_gemv_b1_largest_k(gpu, xkind, K):
    """The batch-1 kernel holds a row slice of at most 8 x 64 lanes x UI units."""
    say(f"gemv b1 largest K={K} {xkind}")
    _group(gpu, 24, K, 4, 64, 1, xkind, K + (xkind == "f32"))


def test_gemv_b1_just_past_largest_k(gpu):
    """Argument validation on the host: status before any buffer is read."""
    import ctypes
    lib = gpu.load()
    good = torch.zeros(16, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(good.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.qgemv_group(p, p, 8, 65536 + 128, 4, 64, p, gpu.Q_BF16, 1, p, gpu.Q_F32, s) == gpu.Q_EUNSUPPORTED
    assert lib.qgemv_group(p, p, 8, 32768 + 128, 4, 64, p, gpu.Q_F32, 1, p, gpu.Q_F32, s) == gpu.Q_EUNSUPPORTED
    assert lib.qgemv_group(p, p, 8, 256, 4, 64, p, gpu.Q_F32, 2, p, gpu.Q_F32, s) == gpu.Q_EUNSUPPORTED


def test_gemv_batched_long_rows(gpu):
    say("gemv B=16 K=65536")
    _group(gpu, 40, 65536, 3, 32, 16, "bf16", 5)


@pytest.mark.parametrize("B", [1, 2, 16])
@pytest.mark.parametrize("N", [1, 15])
def test_gemv_single_rows_and_unit(gpu, B, N):
    """One output row, and rows of a single 32-code unit."""
    say(f"gemv tiny N={N} B={B}")
    _group(gpu, N, 32, 5, 32, B, "bf16", 10 * N + B)
    _group(gpu, N, 256, 6, 64, B, "bf16", 10 * N + B + 1)


@pytest.mark.parametrize("B", [1, 16])
def test_gemv_zero_weights_give_zero(gpu, B):
    """All-zero groups: s = 0, codes 0, o = +0; y must be +0 exactly."""
    N, K = 70, 512
    codes, meta = gpu.qpack_group(torch.zeros(N, K, device="cuda"), 4, 32)
    assert int(codes.count_nonzero()) == 0 and int(meta.count_nonzero()) == 0
    x = dev_bf16(gen_x_bf16(B, K, rng_for(92, B)))
    y = host(gpu.qgemv_group(codes, meta, N, K, 4, 32, x))
    assert np.array_equal(y, np.zeros((B, N)))


@pytest.mark.parametrize("B", [2, 16])
def test_gemv_batched_bf16_output(gpu, B):
    _group(gpu, 300, 1024, 4, 64, B, "bf16", 20 + B, y_dtype=torch.bfloat16)


@pytest.mark.parametrize("N,K,r,B", [(1, 32, 1, 1), (1, 1, 1, 3), (3, 5, 2, 16), (600, 700, 130, 16)])
def test_binlr_small_and_batched(gpu, N, K, r, B):
    say(f"binlr N={N} K={K} r={r} B={B}")
    U, V, s1, s2 = gen_binlr(N, K, r, rng_for(93, N + K + r + B))
    W = oracle.binlr.reconstruct(U, V, s1, s2)
    x = gen_x_bf16(B, K, rng_for(94, B))
    ubd, vbd = gpu.qpack_binlr(dev(U), dev(V))
    y = gpu.qgemv_binlr(ubd, vbd, dev(s1.view(np.int16)), dev(s2.view(np.int16)), N, K, r, dev_bf16(x))
    xv = oracle.product.bf16_to_f64(x)
    # r = 2 makes all-zero rows of U V^T likely: see binlr_abs_denominator
    check_err(host(y), oracle.product.matmul_ref(W, xv), oracle.product.binlr_abs_denominator(U, V, s1, s2, xv))


def test_binlr_bf16_output(gpu):
    N, K, r = 257, 1000, 300
    U, V, s1, s2 = gen_binlr(N, K, r, rng_for(95, 0))
    W = oracle.binlr.reconstruct(U, V, s1, s2)
    x = gen_x_bf16(1, K, rng_for(96, 0))
    ubd, vbd = gpu.qpack_binlr(dev(U), dev(V))
    s1d, s2d = dev(s1.view(np.int16)), dev(s2.view(np.int16))
    y16 = gpu.qgemv_binlr(ubd, vbd, s1d, s2d, N, K, r, dev_bf16(x), y_dtype=torch.bfloat16)
    y32 = gpu.qgemv_binlr(ubd, vbd, s1d, s2d, N, K, r, dev_bf16(x))
    xv = oracle.product.bf16_to_f64(x)
    check_bf16_out(host(y16), host(y32), oracle.product.matmul_ref(W, xv), oracle.product.abs_denominator(W, xv))


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (1, 300, 512), (129, 257, 96), (70, 130, 480), (65, 129, 448)])
def test_prefill_rtn_small_shapes(gpu, M, N, K):
    """Short reductions (K < 512) take the split-precision kernel (weights as
    bf16 hi + lo) and meet the same bound as long ones; K = 512 is the first
    single-bf16 shape."""
    say(f"prefill rtn M={M} N={N} K={K}")
    W = gen_weights(N, K, rng_for(97, M + N + K), outliers=True)
    _, _, _, words, meta, W_hat = group_reference(W, 3, 32)
    X = gen_x_bf16(M, K, rng_for(98, M))
    w = gpu.make_qweight_group(dev(words.view(np.uint8).reshape(-1)), dev(meta.view(np.int32).reshape(-1)),
                               N, K, 3, 32)
    Y = host(gpu.qgemm_prefill(w, dev_bf16(X)))
    Xv = oracle.product.bf16_to_f64(X)
    check_err(Y, oracle.product.matmul_ref(W_hat, Xv), oracle.product.abs_denominator(W_hat, Xv))


@pytest.mark.parametrize("M,N,K,r", [(1, 1, 8, 1), (3, 500, 64, 7), (257, 33, 520, 515), (66, 140, 256, 100),
                                     (130, 300, 504, 1000)])
def test_prefill_binlr_small_shapes(gpu, M, N, K, r):
    """r % 8 != 0 exercises the masked K tail of the second pass; K < 512
    takes the split-precision passes (X s2 as bf16 hi + lo, T in fp32 split
    again for the second pass)."""
    say(f"prefill binlr M={M} N={N} K={K} r={r}")
    U, V, s1, s2 = gen_binlr(N, K, r, rng_for(99, M + r))
    W = oracle.binlr.reconstruct(U, V, s1, s2)
    X = gen_x_bf16(M, K, rng_for(100, M))
    ubd, vbd = gpu.qpack_binlr(dev(U), dev(V))
    w = gpu.make_qweight_binlr(ubd, vbd, dev(s1.view(np.int16)), dev(s2.view(np.int16)), N, K, r)
    Y = host(gpu.qgemm_prefill(w, dev_bf16(X)))
    Xv = oracle.product.bf16_to_f64(X)
    check_err(Y, oracle.product.matmul_ref(W, Xv), oracle.product.binlr_abs_denominator(U, V, s1, s2, Xv))


@pytest.mark.parametrize("K", [256, 1024])
def test_prefill_bf16_output(gpu, K):
    """Split-precision (K = 256) and plain tiles: the bf16 output is the fp32
    result rounded once."""
    M, N = 64, 300
    W = gen_weights(N, K, rng_for(101, K), outliers=True)
    _, _, _, words, meta, W_hat = group_reference(W, 4, 64)
    X = gen_x_bf16(M, K, rng_for(102, K))
    w = gpu.make_qweight_group(dev(words.view(np.uint8).reshape(-1)), dev(meta.view(np.int32).reshape(-1)),
                               N, K, 4, 64)
    Y16 = host(gpu.qgemm_prefill(w, dev_bf16(X), y_dtype=torch.bfloat16))
    Y32 = host(gpu.qgemm_prefill(w, dev_bf16(X)))
    Xv = oracle.product.bf16_to_f64(X)
    check_bf16_out(Y16, Y32, oracle.product.matmul_ref(W_hat, Xv), oracle.product.abs_denominator(W_hat, Xv))
