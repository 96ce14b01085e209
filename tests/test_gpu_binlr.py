"""GPU parity of the binary low-rank path against the CPU oracle: bit
packing exact, brute-force tiny ranks through unit probes, the integer
special case, random cases within the bound, and the full-size shapes."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, check_err, dev, dev_bf16, host, say
from workloads import BINLR_SHAPES, binlr_factors, gen_binlr, gen_x_bf16, gen_x_f32, layer_x, rng_for

pytestmark = pytest.mark.gpu


def test_pack_bit_exact_and_unpack(gpu):
    U, V, s1, s2 = gen_binlr(37, 70, 45, rng_for(60, 0))
    ub, vb = oracle.binlr.pack(U, V)
    ubd, vbd = gpu.qpack_binlr(dev(U), dev(V))
    assert np.array_equal(ubd.cpu().numpy().view(np.uint32), ub.reshape(-1))
    assert np.array_equal(vbd.cpu().numpy().view(np.uint32), vb.reshape(-1))
    Ud, Vd = gpu.qunpack_binlr(dev(ub.view(np.int32).reshape(-1)), dev(vb.view(np.int32).reshape(-1)), 37, 70, 45)
    assert np.array_equal(Ud.cpu().numpy(), U) and np.array_equal(Vd.cpu().numpy(), V)


def test_pack_rejects_non_sign_entries(gpu):
    U, V, _, _ = gen_binlr(8, 40, 5, rng_for(60, 1))
    U[3, 2] = 0
    with pytest.raises(gpu.QError) as e:
        gpu.qpack_binlr(dev(U), dev(V))
    assert e.value.status == -4


def _run(gpu, U, V, s1, s2, x, xkind="bf16", y_dtype=torch.float32):
    N, r = U.shape
    K = V.shape[0]
    ubd, vbd = gpu.qpack_binlr(dev(U), dev(V))
    xd = dev_bf16(x) if xkind == "bf16" else dev(x)
    y = gpu.qgemv_binlr(ubd, vbd, dev(s1.view(np.int16)), dev(s2.view(np.int16)), N, K, r, xd, y_dtype=y_dtype)
    return host(y)


@pytest.mark.parametrize("r", [1, 2, 3, 4])
def test_tiny_ranks_by_probes(gpu, r):
    """x = e_k returns column k of W_hat = s1 (U V^T) s2 (brute force on tiny ranks)."""
    U, V, s1, s2 = gen_binlr(16, 16, r, rng_for(61, r))
    W = oracle.binlr.reconstruct(U, V, s1, s2)
    assert np.array_equal(oracle.binlr.sign_product(U, V), oracle.binlr.sign_product_loops(U, V))
    for k in range(16):
        e = np.zeros((1, 16), np.uint16)
        e[0, k] = 0x3F80
        y = _run(gpu, U, V, s1, s2, e)[0]
        assert np.all(np.abs(y - W[:, k]) <= np.abs(W[:, k]) * 2.0 ** -23 + 1e-30), (k, y, W[:, k])


def test_integer_case_exact(gpu):
    rng = np.random.default_rng(62)
    U, V, _, _ = gen_binlr(70, 300, 37, rng)
    one = np.full(70, 0x3C00, np.uint16), np.full(300, 0x3C00, np.uint16)   # fp16 1.0
    xi = rng.integers(-1, 2, size=(1, 300)).astype(np.float32)
    xb = (xi.view(np.uint32) >> 16).astype(np.uint16)
    y = _run(gpu, U, V, one[0], one[1], xb)
    C = oracle.binlr.sign_product(U, V)
    assert np.array_equal(y, (xi.astype(np.int64) @ C.T).astype(np.float64))


@pytest.mark.parametrize("N,K,r", [(257, 1000, 300), (64, 8192, 2048), (33, 96, 129), (40, 20000, 9000),
                                   (16421, 300, 129), (16400, 96, 1100), (48, 1024, 8200)])
@pytest.mark.parametrize("xkind", ["bf16", "f32"])
def test_random_within_bound(gpu, N, K, r, xkind):
    say(f"binlr N={N} K={K} r={r} {xkind}")
    U, V, s1, s2 = gen_binlr(N, K, r, rng_for(63, N + K + r))
    W = oracle.binlr.reconstruct(U, V, s1, s2)
    rng = rng_for(64, N)
    if xkind == "bf16":
        x = gen_x_bf16(2, K, rng)
        xv = oracle.product.bf16_to_f64(x)
    else:
        x = gen_x_f32(2, K, rng)
        xv = x.astype(np.float64)
    y = _run(gpu, U, V, s1, s2, x, xkind)
    check_err(y, oracle.product.matmul_ref(W, xv), oracle.product.abs_denominator(W, xv))


@pytest.mark.parametrize("K,N,r", BINLR_SHAPES)
def test_full_size(gpu, K, N, r):
    say(f"binlr full K={K} N={N} r={r}")
    U, V, s1, s2 = binlr_factors(K, N, r)
    ubd, vbd = gpu.qpack_binlr(dev(U), dev(V))
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(1).choice(N, 40, replace=False)]))
    ub_ref = oracle.binlr.pack_rows(U[rows])
    rw = ub_ref.shape[1]
    got = ubd.view(torch.int32).reshape(N, rw)[torch.from_numpy(rows).to(DEV)].cpu().numpy().view(np.uint32)
    assert np.array_equal(got, ub_ref)
    vt_ref = oracle.binlr.pack_rows(V.T[:64])
    kw = vt_ref.shape[1]
    assert np.array_equal(vbd.view(torch.int32).reshape(r, kw)[:64].cpu().numpy().view(np.uint32), vt_ref)
    x = layer_x(K, 1, config=4)
    y = gpu.qgemv_binlr(ubd, vbd, dev(s1.view(np.int16)), dev(s2.view(np.int16)), N, K, r, dev_bf16(x))
    y = host(y)[:, rows]
    W = oracle.binlr.reconstruct(U[rows], V, s1[rows], s2)
    xv = oracle.product.bf16_to_f64(x)
    err = check_err(y, oracle.product.matmul_ref(W, xv), oracle.product.abs_denominator(W, xv))
    say(f"  err={err:.3e}")


@pytest.mark.parametrize("xkind", ["bf16", "f32"])
@pytest.mark.parametrize("shift_s2", [False, True])
def test_unaligned_vector_and_scale(gpu, xkind, shift_s2):
    """x starting 4 bytes into its buffer (the alignment the entry point
    requires) and optionally s2 one element in, so neither is 16-byte
    aligned: stage 1 reads every vector entry one by one; K = 1003 also
    leaves a ragged last group."""
    N, K, r = 300, 1003, 200
    U, V, s1, s2 = gen_binlr(N, K, r, rng_for(65, K))
    W = oracle.binlr.reconstruct(U, V, s1, s2)
    rng = rng_for(66, int(shift_s2))
    if xkind == "bf16":
        xf = gen_x_bf16(1, K + 2, rng)
        xd = dev_bf16(xf)[:, 2:]
        xv = oracle.product.bf16_to_f64(xf[:, 2:])
    else:
        xf = gen_x_f32(1, K + 1, rng)
        xd = dev(xf)[:, 1:]
        xv = xf[:, 1:].astype(np.float64)
    s2d = dev(s2.view(np.int16))
    if shift_s2:
        s2d = dev(np.concatenate([[0], s2]).astype(np.uint16).view(np.int16))[1:]
    assert xd.data_ptr() % 16 != 0
    ubd, vbd = gpu.qpack_binlr(dev(U), dev(V))
    y = host(gpu.qgemv_binlr(ubd, vbd, dev(s1.view(np.int16)), s2d, N, K, r, xd))
    check_err(y, oracle.product.matmul_ref(W, xv), oracle.product.abs_denominator(W, xv))
