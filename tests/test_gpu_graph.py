"""The hot-path entry points captured in a HIP graph give, on every replay,
the same bits as eager calls (the benchmark times graph replays).  Between
replays the program does its own eager work and synchronizes; the inputs are
changed in place so each replay must read the current data."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, say
from workloads import gen_binlr, gen_weights, gen_x_bf16, rng_for

pytestmark = pytest.mark.gpu


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def _check_replays(g, out, eager, xs, x_dev):
    for i, xnew in enumerate(xs):
        x_dev.copy_(xnew)                   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = eager()
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay {i} differs from the eager call"


@pytest.mark.parametrize("B", [1, 16])
def test_graph_gemv_group(gpu, B):
    say(f"graph gemv_group B={B}")
    N, K = 1000, 4096
    W = gen_weights(N, K, rng_for(80, B), outliers=True)
    codes, meta = gpu.qpack_group(dev(W), 4, 64)
    x = dev_bf16(gen_x_bf16(B, K, rng_for(81, 0)))
    y = torch.empty((B, N), dtype=torch.float32, device=x.device)
    g = _capture(lambda: gpu.qgemv_group(codes, meta, N, K, 4, 64, x, y=y))
    xs = [dev_bf16(gen_x_bf16(B, K, rng_for(82, i))) for i in range(3)]
    _check_replays(g, y, lambda: gpu.qgemv_group(codes, meta, N, K, 4, 64, x), xs, x)


def test_graph_gemv_binlr(gpu):
    say("graph gemv_binlr")
    N, K, r = 700, 2048, 300
    U, V, s1, s2 = gen_binlr(N, K, r, rng_for(83, 0))
    ub, vb = gpu.qpack_binlr(dev(U), dev(V))
    s1d, s2d = dev(s1.view(np.int16)), dev(s2.view(np.int16))
    x = dev_bf16(gen_x_bf16(1, K, rng_for(84, 0)))
    y = torch.empty((1, N), dtype=torch.float32, device=x.device)
    ws = torch.empty(gpu.qbinlr_sizes(N, K, r, 1)[2], dtype=torch.uint8, device=x.device)
    g = _capture(lambda: gpu.qgemv_binlr(ub, vb, s1d, s2d, N, K, r, x, y=y, ws=ws))
    xs = [dev_bf16(gen_x_bf16(1, K, rng_for(85, i))) for i in range(3)]
    _check_replays(g, y, lambda: gpu.qgemv_binlr(ub, vb, s1d, s2d, N, K, r, x), xs, x)


def test_graph_prefill(gpu):
    say("graph prefill")
    M, N, K = 96, 300, 512
    W = gen_weights(N, K, rng_for(86, 0), outliers=True)
    codes, meta = gpu.qpack_group(dev(W), 4, 64)
    w = gpu.make_qweight_group(codes, meta, N, K, 4, 64)
    X = dev_bf16(gen_x_bf16(M, K, rng_for(87, 0)))
    Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    g = _capture(lambda: gpu.qgemm_prefill(w, X, Y=Y))
    xs = [dev_bf16(gen_x_bf16(M, K, rng_for(88, i))) for i in range(3)]
    _check_replays(g, Y, lambda: gpu.qgemm_prefill(w, X), xs, X)


@pytest.mark.parametrize("B", [1, 4])
def test_graph_gemv_outlier(gpu, B):
    say(f"graph gemv_group_outlier B={B}")
    N, K = 600, 2048
    W = gen_weights(N, K, rng_for(89, B), outliers=True)
    codes, meta, side, idx = gpu.qpack_group_outlier(dev(W), 4, 64, 4)
    x = dev_bf16(gen_x_bf16(B, K, rng_for(90, 0)))
    y = torch.empty((B, N), dtype=torch.float32, device=x.device)
    g = _capture(lambda: gpu.qgemv_group_outlier(codes, meta, side, idx, N, K, 4, 64, x, y=y))
    xs = [dev_bf16(gen_x_bf16(B, K, rng_for(91, i))) for i in range(3)]
    _check_replays(g, y, lambda: gpu.qgemv_group_outlier(codes, meta, side, idx, N, K, 4, 64, x), xs, x)


def test_graph_gemv_multi(gpu):
    say("graph gemv_group_multi")
    K = 2048
    mats = []
    for i, N in enumerate([500, 64, 64]):
        c, m = gpu.qpack_group(dev(gen_weights(N, K, rng_for(92, i), outliers=True)), 3, 32)
        mats.append((c, m, N))
    x = dev_bf16(gen_x_bf16(1, K, rng_for(93, 0)))
    ys = [torch.empty((1, n), dtype=torch.float32, device=x.device) for _, _, n in mats]
    out = torch.empty(sum(n for _, _, n in mats), dtype=torch.float32, device=x.device)

    def run(dst):
        gpu.qgemv_group_multi(mats, K, 3, 32, x, ys=ys)
        torch.cat([y.reshape(-1) for y in ys], out=dst)
    g = _capture(lambda: run(out))
    xs = [dev_bf16(gen_x_bf16(1, K, rng_for(94, i))) for i in range(3)]

    def eager():
        ref = torch.empty_like(out)
        run(ref)
        return ref
    _check_replays(g, out, eager, xs, x)


@pytest.mark.parametrize("B", [1, 16])
def test_graph_gemv_codebook(gpu, B):
    say(f"graph gemv_group_cb B={B}")
    N, K = 1000, 4096
    W = gen_weights(N, K, rng_for(95, B), outliers=True)
    books = dev(np.asarray(gpu.qcodebook_default(4)))
    codes, meta, ids = gpu.qpack_group_cb(dev(W), 4, 64, books)
    x = dev_bf16(gen_x_bf16(B, K, rng_for(96, 0)))
    y = torch.empty((B, N), dtype=torch.float32, device=x.device)
    g = _capture(lambda: gpu.qgemv_group_cb(codes, meta, ids, books, N, K, 4, 64, x, y=y))
    xs = [dev_bf16(gen_x_bf16(B, K, rng_for(97, i))) for i in range(3)]
    _check_replays(g, y, lambda: gpu.qgemv_group_cb(codes, meta, ids, books, N, K, 4, 64, x), xs, x)


def test_graph_key_logits(gpu):
    """Query prep and logits (two launches) replayed with new queries."""
    say("graph qtq_logits")
    rng = rng_for(98, 0)
    Pi = dev(gpu.qtq_rotation(rng.standard_normal((128, 128))))
    S = dev(rng.standard_normal((128, 128)))
    delta, table = gpu.qtq_centroids(128, 3)
    H, n, nq = 2, 3000, 4
    K = dev(rng.standard_normal((H * n, 128)).astype(np.float32))
    c, sg, nm = gpu.qtq_quant_keys(K, 4, Pi, S, delta, table)
    Qv = dev(rng.standard_normal((H, nq, 128)).astype(np.float32))
    out = torch.empty((H, nq, n), dtype=torch.float32, device=Qv.device)
    ws = torch.empty(H * nq * 132 * 4, dtype=torch.uint8, device=Qv.device)
    SPi = gpu.qtq_project(S, Pi)
    g = _capture(lambda: gpu.qtq_logits(c, sg, nm, n, H, 4, delta, table, Pi, SPi, Qv, out=out, ws=ws))
    qs = [dev(rng_for(99, i).standard_normal((H, nq, 128)).astype(np.float32)) for i in range(3)]
    _check_replays(g, out, lambda: gpu.qtq_logits(c, sg, nm, n, H, 4, delta, table, Pi, SPi, Qv), qs, Qv)


def test_graph_value_attend(gpu):
    """Value output (the streaming pass and its finishing pass) replayed with
    new weights."""
    say("graph qtq_attend")
    rng = rng_for(100, 0)
    Pi = dev(gpu.qtq_rotation(rng.standard_normal((128, 128))))
    delta, table = gpu.qtq_centroids(128, 3)
    H, n, nq = 2, 3000, 4
    V = dev(rng.standard_normal((H * n, 128)).astype(np.float32))
    c, nm = gpu.qtq_quant_values(V, 3, Pi, delta, table)
    P = dev(rng.random((H, nq, n)).astype(np.float32))
    out = torch.empty((H, nq, 128), dtype=torch.float32, device=P.device)
    ws = torch.empty(gpu.qtq_attend_ws(n, H, nq), dtype=torch.uint8, device=P.device)
    g = _capture(lambda: gpu.qtq_attend(c, nm, n, H, 3, delta, table, Pi, P, out=out, ws=ws))
    ps = [dev(rng_for(101, i).random((H, nq, n)).astype(np.float32)) for i in range(3)]
    _check_replays(g, out, lambda: gpu.qtq_attend(c, nm, n, H, 3, delta, table, Pi, P), ps, P)
