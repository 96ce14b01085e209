"""Every entry point writes inside its output and workspace buffers only,
writes every element of its outputs, and gives the same bytes when called
twice on the same inputs.

Each output and workspace is carved out of a larger device buffer: 4 KiB
guard bands of 0xA5 on both sides (checked after the calls) and the buffer
itself filled with 0xFF first (a NaN in fp32 and bf16, a code word no packer
writes for these inputs), so an element a kernel skipped shows up either as
a NaN or as a difference from the oracle.  No kernel on these paths
combines partial results with atomics (the packers' atomics only raise
status bits), so two calls must agree bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, check_err, dev, dev_bf16, group_reference, host, say
from workloads import gen_binlr, gen_weights, gen_x_bf16, rng_for

pytestmark = pytest.mark.gpu

GUARD = 4096
GUARD_BYTE = 0xA5
POISON = 0xFF


class Guarded:
    """A device tensor with guard bands of GUARD bytes on either side."""

    def __init__(self, nbytes, dtype, shape=None):
        self.nbytes = int(nbytes)
        self.buf = torch.full((2 * GUARD + self.nbytes,), GUARD_BYTE, dtype=torch.uint8, device=DEV)
        self.buf[GUARD:GUARD + self.nbytes] = POISON
        t = self.buf[GUARD:GUARD + self.nbytes].view(dtype)
        self.t = t.view(shape) if shape is not None else t

    def check(self, what):
        torch.cuda.synchronize()
        b = self.buf.cpu().numpy()
        lo, hi = b[:GUARD], b[GUARD + self.nbytes:]
        assert np.all(lo == GUARD_BYTE), f"{what}: write below the buffer at {np.nonzero(lo != GUARD_BYTE)[0][:4]}"
        assert np.all(hi == GUARD_BYTE), f"{what}: write past the buffer at {np.nonzero(hi != GUARD_BYTE)[0][:4]}"

    def bytes(self):
        torch.cuda.synchronize()
        return self.buf[GUARD:GUARD + self.nbytes].cpu().numpy().copy()


def _out(shape, dtype):
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    return Guarded(n, dtype, shape)


def _ws(nbytes):
    return Guarded(max(int(nbytes), 16), torch.uint8)


def _twice(call, outs, what):
    """Run call(outs_a) and call(outs_b) into two sets of guarded buffers;
    check the guards and that the outputs agree byte for byte."""
    a, b = outs(), outs()
    call(*[g.t for g in a])
    call(*[g.t for g in b])
    for i, (ga, gb) in enumerate(zip(a, b)):
        ga.check(f"{what} buffer {i}")
        gb.check(f"{what} buffer {i} (second call)")
    return a, b


def _same(ga, gb, what):
    assert np.array_equal(ga.bytes(), gb.bytes()), f"{what}: two calls differ"


def _finite(g, what):
    v = host(g.t)
    assert np.all(np.isfinite(v)), f"{what}: element left unwritten (NaN poison) or non-finite"
    return v


@pytest.mark.parametrize("bits,group", [(3, 64), (5, 32), (4, 64)])
def test_pack_group(gpu, bits, group):
    N, K = 70, 448
    W = gen_weights(N, K, rng_for(900, bits), outliers=True)
    _, _, _, words, meta, _ = group_reference(W, bits, group)
    cb, mb = gpu.qgroup_sizes(N, K, bits, group)
    Wd = dev(W)
    a, b = _twice(lambda c, m: gpu.qpack_group(Wd, bits, group, codes=c, meta=m),
                  lambda: (_ws(cb), Guarded(mb, torch.int32)), "qpack_group")
    assert np.array_equal(a[0].bytes(), words.view(np.uint8).reshape(-1))
    assert np.array_equal(a[1].bytes().view(np.uint32), meta.reshape(-1))
    _same(a[0], b[0], "codes")
    _same(a[1], b[1], "meta")


@pytest.mark.parametrize("B", [1, 5, 16])
@pytest.mark.parametrize("y_dtype", [torch.float32, torch.bfloat16])
def test_gemv_group(gpu, B, y_dtype):
    N, K, bits, group = 70, 448, 4, 64
    W = gen_weights(N, K, rng_for(901, B), outliers=True)
    _, _, _, words, meta, W_hat = group_reference(W, bits, group)
    cd, md = dev(words.view(np.uint8).reshape(-1)), dev(meta.view(np.int32).reshape(-1))
    X = gen_x_bf16(B, K, rng_for(902, B))
    xd = dev_bf16(X)
    a, b = _twice(lambda y: gpu.qgemv_group(cd, md, N, K, bits, group, xd, y=y),
                  lambda: (_out((B, N), y_dtype),), "qgemv_group")
    _same(a[0], b[0], "y")
    y = _finite(a[0], "y")
    Xv = oracle.product.bf16_to_f64(X)
    tol_extra = 0.0 if y_dtype == torch.float32 else 2.0 ** -8
    ref = oracle.product.matmul_ref(W_hat, Xv)
    D = oracle.product.abs_denominator(W_hat, Xv)
    err = np.max((np.abs(y - ref) - tol_extra * np.abs(y)) / D)
    assert err <= 2e-3, err


@pytest.mark.parametrize("B,K", [(1, 448), (6, 448), (6, 576)])
def test_gemv_group_multi(gpu, B, K):
    bits, group = 4, 64
    shapes = [70, 33]
    mats, refs = [], []
    for i, N in enumerate(shapes):
        W = gen_weights(N, K, rng_for(903, i), outliers=True)
        _, _, _, words, meta, W_hat = group_reference(W, bits, group)
        mats.append((dev(words.view(np.uint8).reshape(-1)), dev(meta.view(np.int32).reshape(-1)), N))
        refs.append(W_hat)
    X = gen_x_bf16(B, K, rng_for(904, B))
    xd = dev_bf16(X)
    a, b = _twice(lambda y0, y1: gpu.qgemv_group_multi(mats, K, bits, group, xd, ys=[y0, y1]),
                  lambda: (_out((B, 70), torch.float32), _out((B, 33), torch.float32)), "qgemv_group_multi")
    Xv = oracle.product.bf16_to_f64(X)
    for i in range(2):
        _same(a[i], b[i], f"y{i}")
        check_err(_finite(a[i], f"y{i}"), oracle.product.matmul_ref(refs[i], Xv),
                  oracle.product.abs_denominator(refs[i], Xv))


@pytest.mark.parametrize("B", [1, 4])
def test_gemv_outlier_and_codebook(gpu, B):
    N, K, bits, group = 70, 448, 4, 64
    W = gen_weights(N, K, rng_for(905, B), outliers=True)
    Wd = dev(W)
    X = gen_x_bf16(B, K, rng_for(906, B))
    xd = dev_bf16(X)
    c, m, sd, ix = gpu.qpack_group_outlier(Wd, bits, group, 5)
    a, b = _twice(lambda y: gpu.qgemv_group_outlier(c, m, sd, ix, N, K, bits, group, xd, y=y),
                  lambda: (_out((B, N), torch.float32),), "qgemv_group_outlier")
    _same(a[0], b[0], "outlier y")
    _finite(a[0], "outlier y")
    books = gpu.qcodebook_default(bits).to(DEV)
    c2, m2, ids = gpu.qpack_group_cb(Wd, bits, group, books)
    a, b = _twice(lambda y: gpu.qgemv_group_cb(c2, m2, ids, books, N, K, bits, group, xd, y=y),
                  lambda: (_out((B, N), torch.float32),), "qgemv_group_cb")
    _same(a[0], b[0], "codebook y")
    _finite(a[0], "codebook y")


@pytest.mark.parametrize("B", [1, 3, 16])
def test_binlr(gpu, B):
    N, K, r = 70, 300, 37
    U, V, s1, s2 = gen_binlr(N, K, r, rng_for(907, B))
    ub, vb, wsb = gpu.qbinlr_sizes(N, K, r, B)
    Ud, Vd = dev(U), dev(V)
    a, b = _twice(lambda u, v: gpu.qpack_binlr(Ud, Vd, ubits=u, vtbits=v),
                  lambda: (Guarded(ub, torch.int32), Guarded(vb, torch.int32)), "qpack_binlr")
    pu, pv = oracle.binlr.pack(U, V)
    assert np.array_equal(a[0].bytes().view(np.uint32), pu.reshape(-1))
    assert np.array_equal(a[1].bytes().view(np.uint32), pv.reshape(-1))
    _same(a[0], b[0], "ubits")
    _same(a[1], b[1], "vtbits")
    ubd, vbd = a[0].t, a[1].t
    s1d, s2d = dev(s1.view(np.int16)), dev(s2.view(np.int16))
    X = gen_x_bf16(B, K, rng_for(908, B))
    xd = dev_bf16(X)
    a, b = _twice(lambda y, ws: gpu.qgemv_binlr(ubd, vbd, s1d, s2d, N, K, r, xd, y=y, ws=ws),
                  lambda: (_out((B, N), torch.float32), _ws(wsb)), "qgemv_binlr")
    _same(a[0], b[0], "binlr y")
    y = _finite(a[0], "binlr y")
    Wr = oracle.binlr.reconstruct(U, V, s1, s2)
    Xv = oracle.product.bf16_to_f64(X)
    check_err(y, oracle.product.matmul_ref(Wr, Xv), oracle.product.binlr_abs_denominator(U, V, s1, s2, Xv))
    if B <= 8:
        c, d = _twice(lambda y: gpu.qgemv_binlr_noalloc(ubd, vbd, s1d, s2d, N, K, r, xd, y=y),
                      lambda: (_out((B, N), torch.float32),), "qgemv_binlr_noalloc")
        _same(c[0], a[0], "noalloc vs workspace y")
        _same(c[0], d[0], "noalloc y")


@pytest.mark.parametrize("K", [448, 576])
def test_prefill(gpu, K):
    """Both formats, M and N ragged against the tiles; K = 448 takes the
    split-precision tiles, K = 576 the plain ones."""
    M, N, bits, group, r = 70, 130, 4, 64, 100
    W = gen_weights(N, K, rng_for(909, K), outliers=True)
    _, _, _, words, meta, W_hat = group_reference(W, bits, group)
    w = gpu.make_qweight_group(dev(words.view(np.uint8).reshape(-1)), dev(meta.view(np.int32).reshape(-1)),
                               N, K, bits, group)
    X = gen_x_bf16(M, K, rng_for(910, K))
    xd = dev_bf16(X)
    Xv = oracle.product.bf16_to_f64(X)
    need = gpu.qgemm_prefill_ws(w, M)
    a, b = _twice(lambda Y, ws: gpu.qgemm_prefill(w, xd, Y=Y, ws=ws if need else None),
                  lambda: (_out((M, N), torch.float32), _ws(need)), "prefill group")
    _same(a[0], b[0], "prefill group Y")
    check_err(_finite(a[0], "prefill group Y"), oracle.product.matmul_ref(W_hat, Xv),
              oracle.product.abs_denominator(W_hat, Xv))
    U, V, s1, s2 = gen_binlr(N, K, r, rng_for(911, K))
    wb = gpu.make_qweight_binlr(*gpu.qpack_binlr(dev(U), dev(V)), dev(s1.view(np.int16)), dev(s2.view(np.int16)),
                                N, K, r)
    need = gpu.qgemm_prefill_ws(wb, M)
    a, b = _twice(lambda Y, ws: gpu.qgemm_prefill(wb, xd, Y=Y, ws=ws),
                  lambda: (_out((M, N), torch.float32), _ws(need)), "prefill binlr")
    _same(a[0], b[0], "prefill binlr Y")
    Wr = oracle.binlr.reconstruct(U, V, s1, s2)
    check_err(_finite(a[0], "prefill binlr Y"), oracle.product.matmul_ref(Wr, Xv),
              oracle.product.binlr_abs_denominator(U, V, s1, s2, Xv))
    say(f"  prefill K={K}: guards intact, repeatable")


def test_key_cache(gpu):
    tq = oracle.turboquant
    bits, H, n, nq = 4, 2, 1003, 3
    rng = rng_for(912, 0)
    Pi = tq.rotation(rng.standard_normal((128, 128)))
    S = rng.standard_normal((128, 128))
    delta, table = tq.stored_table(tq.lloyd_max(128, bits - 1))
    Kc = rng.standard_normal((H * n, 128)).astype(np.float32)
    Pid, Sd = dev(Pi), dev(S)
    c, s, nm = gpu.qtq_quant_keys(dev(Kc), bits, Pid, Sd, delta, table)
    c2, s2, nm2 = gpu.qtq_quant_keys(dev(Kc), bits, Pid, Sd, delta, table)
    assert torch.equal(c, c2) and torch.equal(s, s2) and torch.equal(nm, nm2)
    SPi = gpu.qtq_project(Sd, Pid)
    Qv = dev(rng.standard_normal((H, nq, 128)).astype(np.float32))
    need = ctypes.c_size_t()
    assert gpu.load().qtq_logits_ws(H, nq, ctypes.byref(need)) == 0
    a, b = _twice(lambda out, ws: gpu.qtq_logits(c, s, nm, n, H, bits, delta, table, Pid, SPi, Qv, out=out, ws=ws),
                  lambda: (_out((H, nq, n), torch.float32), _ws(need.value)), "qtq_logits")
    _same(a[0], b[0], "logits")
    _finite(a[0], "logits")
    vbits = 3
    vdelta, vtable = tq.stored_table(tq.lloyd_max(128, vbits))
    Vc = rng.standard_normal((H * n, 128)).astype(np.float32)
    vc, vn = gpu.qtq_quant_values(dev(Vc), vbits, Pid, vdelta, vtable)
    P = dev(rng.random((H, nq, n)).astype(np.float32))
    need = gpu.qtq_attend_ws(n, H, nq)
    a, b = _twice(lambda out, ws: gpu.qtq_attend(vc, vn, n, H, vbits, vdelta, vtable, Pid, P, out=out, ws=ws),
                  lambda: (_out((H, nq, 128), torch.float32), _ws(need)), "qtq_attend")
    _same(a[0], b[0], "attend")
    _finite(a[0], "attend")
