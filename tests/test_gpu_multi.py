"""Grouped decode GEMV (several group-RTN matrices sharing x in one launch):
equal to separate calls, and to the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_bf16_out, check_err, dev, dev_bf16, group_reference, host, say
from workloads import gen_weights, gen_x_bf16, gen_x_f32, layer_weights, rng_for

pytestmark = pytest.mark.gpu


def _mats(gpu, shapes, K, bits, group, seed):
    out = []
    for i, N in enumerate(shapes):
        W = gen_weights(N, K, rng_for(330 + seed, i), outliers=True)
        _, _, _, words, meta, W_hat = group_reference(W, bits, group)
        out.append((dev(words.view(np.uint8).reshape(-1)), dev(meta.view(np.int32).reshape(-1)), N, W_hat))
    return out


def test_fused_equals_separate_calls(gpu):
    """Shapes where every call keeps whole rows per wave (no K split): the
    fused launch runs the same per-row arithmetic, so the results are equal
    bit for bit."""
    K, bits, group = 4096, 4, 64
    mats = _mats(gpu, [1536, 1024, 1100], K, bits, group, 0)
    x = dev_bf16(gen_x_bf16(1, K, rng_for(331, 0)))
    ys = gpu.qgemv_group_multi([(c, m, n) for c, m, n, _ in mats], K, bits, group, x)
    for (c, m, n, W_hat), y in zip(mats, ys):
        y1 = gpu.qgemv_group(c, m, n, K, bits, group, x)
        assert torch.equal(y, y1)


@pytest.mark.parametrize("bits,group,xkind", [(4, 64, "bf16"), (3, 32, "bf16"), (6, 32, "f32"), (2, 64, "bf16"),
                                              (6, 32, "bf16"), (5, 32, "bf16"), (2, 32, "bf16")])
@pytest.mark.parametrize("shapes", [[45, 7, 300], [100], [64, 1, 33, 17]])
def test_against_oracle(gpu, bits, group, xkind, shapes):
    K = 512
    mats = _mats(gpu, shapes, K, bits, group, bits + len(shapes))
    rng = rng_for(332, bits)
    if xkind == "f32":
        xh = gen_x_f32(1, K, rng)
        xv, xd = xh.astype(np.float64), dev(xh)
    else:
        xb = gen_x_bf16(1, K, rng)
        xv, xd = oracle.product.bf16_to_f64(xb), dev_bf16(xb)
    ys = gpu.qgemv_group_multi([(c, m, n) for c, m, n, _ in mats], K, bits, group, xd)
    for (c, m, n, W_hat), y in zip(mats, ys):
        check_err(host(y), oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv))


def test_batched_and_bf16_output(gpu):
    """B > 1 runs one matrix-core launch over all the matrices' tiles; bf16
    outputs round once."""
    K, bits, group = 1024, 5, 32
    mats = _mats(gpu, [200, 40], K, bits, group, 7)
    for B in (2, 1):
        xb = gen_x_bf16(B, K, rng_for(333, B))
        xv = oracle.product.bf16_to_f64(xb)
        ys = gpu.qgemv_group_multi([(c, m, n) for c, m, n, _ in mats], K, bits, group, dev_bf16(xb))
        for (c, m, n, W_hat), y in zip(mats, ys):
            check_err(host(y), oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv))
        if B == 1:
            y16 = gpu.qgemv_group_multi([(c, m, n) for c, m, n, _ in mats], K, bits, group, dev_bf16(xb),
                                        y_dtype=torch.bfloat16)
            for (c, m, n, W_hat), a, y in zip(mats, y16, ys):
                check_bf16_out(host(a), host(y), oracle.product.matmul_ref(W_hat, xv),
                               oracle.product.abs_denominator(W_hat, xv))


def test_long_rows_split_k(gpu):
    """K = 65536: rows are split over several waves that meet in LDS before
    the store picks the matrix of each row."""
    K, bits, group = 65536, 4, 64
    mats = _mats(gpu, [24, 9], K, bits, group, 9)
    say("grouped gemv K=65536")
    xb = gen_x_bf16(1, K, rng_for(334, 0))
    xv = oracle.product.bf16_to_f64(xb)
    ys = gpu.qgemv_group_multi([(c, m, n) for c, m, n, _ in mats], K, bits, group, dev_bf16(xb))
    for (c, m, n, W_hat), y in zip(mats, ys):
        check_err(host(y), oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv))


@pytest.mark.parametrize("bits,group", [(6, 32), (5, 32), (3, 32), (2, 32)])
def test_mixed_width_layer_shapes(gpu, bits, group):
    """The grouped launches of the mixed-width layer sets at their real shapes
    (q/k/v 8192 x 8192, 1024, 1024 with attention widths; gate/up 28672 x 2
    with MLP widths), each matrix on sampled rows against the oracle."""
    K = 8192
    names = ("q", "k", "v") if bits >= 5 else ("gate", "up")
    if bits >= 5:
        Ws = [layer_weights(n) for n in names]
    else:
        Wg = layer_weights("gate")      # gate and up share the shape (and here the weights)
        Ws = [Wg, Wg]
    packed = [gpu.qpack_group(dev(W), bits, group) for W in Ws]
    xb = gen_x_bf16(1, K, rng_for(333, bits))
    xv = oracle.product.bf16_to_f64(xb)
    say(f"grouped {'/'.join(names)} b={bits} g={group}")
    ys = gpu.qgemv_group_multi([(c, m, W.shape[0]) for (c, m), W in zip(packed, Ws)], K, bits, group, dev_bf16(xb))
    for W, y in zip(Ws, ys):
        N = W.shape[0]
        rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(N + bits).choice(N, 48, replace=False)]))
        q, s, o = oracle.rtn.quantize(W[rows], bits, group)
        W_hat = oracle.rtn.dequantize(q, s, o, group)
        check_err(host(y)[0, rows], oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv))


# Batched grouped launches: ragged matrices (tiles that end inside the
# matrix, one-row matrices), K below 512 (weights as hi + lo) and at or
# above it (pair loads, g64 blocks and g32), batch 2..16, and matrix counts
# 1..4; every output equals a separate qgemv_group call bit for bit and
# meets the oracle's bound.
BATCHED_CASES = [
    (4, 64, 16, 1024, [45, 7, 300]),
    (4, 64, 5, 448, [100]),
    (3, 32, 8, 576, [64, 1, 33, 17]),
    (6, 32, 2, 512, [200, 16, 16]),
    (2, 32, 9, 1024, [513, 511]),
    (5, 64, 16, 320, [31, 64, 97]),
]


@pytest.mark.parametrize("bits,group,B,K,shapes", BATCHED_CASES)
def test_batched_grouped_launch(gpu, bits, group, B, K, shapes):
    say(f"grouped batched b={bits} g={group} B={B} K={K} N={shapes}")
    mats = _mats(gpu, shapes, K, bits, group, 40 + bits + B)
    xb = gen_x_bf16(B, K, rng_for(334, B * 100 + bits))
    xv = oracle.product.bf16_to_f64(xb)
    xd = dev_bf16(xb)
    ys = gpu.qgemv_group_multi([(c, m, n) for c, m, n, _ in mats], K, bits, group, xd)
    for (c, m, n, W_hat), y in zip(mats, ys):
        y1 = gpu.qgemv_group(c, m, n, K, bits, group, xd)
        assert torch.equal(y, y1), "grouped launch differs from a separate call"
        check_err(host(y).reshape(B, n), oracle.product.matmul_ref(W_hat, xv),
                  oracle.product.abs_denominator(W_hat, xv))


def test_batched_grouped_layer_shapes(gpu):
    """q/k/v of the 4-bit layer set at batch 16 in one launch: sampled rows
    against the oracle, every output equal to a separate call."""
    K = 8192
    Ws = [layer_weights(n) for n in ("q", "k", "v")]
    packed = [gpu.qpack_group(dev(W), 4, 64) for W in Ws]
    xb = gen_x_bf16(16, K, rng_for(335, 16))
    xv = oracle.product.bf16_to_f64(xb)
    xd = dev_bf16(xb)
    ys = gpu.qgemv_group_multi([(c, m, W.shape[0]) for (c, m), W in zip(packed, Ws)], K, 4, 64, xd)
    for (c, m), W, y in zip(packed, Ws, ys):
        N = W.shape[0]
        assert torch.equal(y, gpu.qgemv_group(c, m, N, K, 4, 64, xd))
        rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(N).choice(N, 32, replace=False)]))
        q, s, o = oracle.rtn.quantize(W[rows], 4, 64)
        W_hat = oracle.rtn.dequantize(q, s, o, 64)
        check_err(host(y)[:, rows], oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv))
