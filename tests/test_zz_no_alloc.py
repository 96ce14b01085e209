"""qgemv_binlr_noalloc (the binary GEMV with the library's per-device scratch
array as its workspace, for callers that cannot allocate) against
qgemv_binlr with a caller workspace, and both against the CPU oracle: two
calls in a row, the second on a smaller input, so the second call runs on
whatever the first left in the shared array."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_err, dev, dev_bf16, host, say
from workloads import gen_binlr, gen_x_bf16, rng_for

pytestmark = pytest.mark.gpu


def _case(gpu, N, K, r, B, seed):
    U, V, s1, s2 = gen_binlr(N, K, r, rng_for(500, seed))
    x = gen_x_bf16(B, K, rng_for(501, seed))
    ubd, vbd = gpu.qpack_binlr(dev(U), dev(V))
    return U, V, s1, s2, x, ubd, vbd, dev(s1.view(np.int16)), dev(s2.view(np.int16)), dev_bf16(x)


def test_noalloc_matches_workspace_entry_point(gpu):
    lib = gpu.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for N, K, r, B, seed in [(3000, 2048, 1024, 4, 0), (500, 700, 130, 1, 1)]:
        say(f"noalloc binary GEMV N={N} K={K} r={r} B={B}")
        U, V, s1, s2, x, ubd, vbd, s1d, s2d, xd = _case(gpu, N, K, r, B, seed)
        y_ws = gpu.qgemv_binlr(ubd, vbd, s1d, s2d, N, K, r, xd)
        # straight through the C ABI: no workspace argument
        y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
        st = lib.qgemv_binlr_noalloc(ctypes.c_void_p(ubd.data_ptr()), ctypes.c_void_p(vbd.data_ptr()),
                                     ctypes.c_void_p(s1d.data_ptr()), ctypes.c_void_p(s2d.data_ptr()), N, K, r,
                                     ctypes.c_void_p(xd.data_ptr()), gpu.Q_BF16, B, ctypes.c_void_p(y.data_ptr()),
                                     gpu.Q_F32, stream)
        assert st == gpu.Q_OK, st
        yn, yw = host(y), host(y_ws)
        # the same kernels on the same inputs: the same bits
        assert np.array_equal(yn, yw)
        xv = oracle.product.bf16_to_f64(x)
        W = oracle.binlr.reconstruct(U, V, s1, s2)
        check_err(yn, oracle.product.matmul_ref(W, xv), oracle.product.binlr_abs_denominator(U, V, s1, s2, xv))
        # and through the binding, into a caller-owned output
        y2 = torch.empty_like(y)
        gpu.qgemv_binlr_noalloc(ubd, vbd, s1d, s2d, N, K, r, xd, y=y2)
        assert np.array_equal(host(y2), yw)


def test_noalloc_rejects_sizes_beyond_the_scratch_array(gpu):
    N, K, r, B = 64, 128, 65536, 16
    _, _, ws = gpu.qbinlr_sizes(N, K, r, B)
    assert ws > (2 << 20)
    ub, vb, _ = gpu.qbinlr_sizes(N, K, r, B)
    z = lambda n: torch.zeros(n, dtype=torch.uint8, device="cuda")   # noqa: E731
    with pytest.raises(gpu.QError) as e:
        gpu.qgemv_binlr_noalloc(z(ub), z(vb), torch.zeros(N, dtype=torch.int16, device="cuda"),
                                torch.zeros(K, dtype=torch.int16, device="cuda"), N, K, r,
                                torch.zeros(B, K, dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == gpu.Q_EUNSUPPORTED
