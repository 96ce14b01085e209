"""Grouped decode GEMV (several group-RTN matrices sharing x in one launch):
equal to separate calls, and to the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_err, dev, dev_bf16, group_reference, host, say
from workloads import gen_weights, gen_x_bf16, gen_x_f32, rng_for

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


@pytest.mark.parametrize("bits,group,xkind", [(4, 64, "bf16"), (3, 32, "bf16"), (6, 32, "f32"), (2, 64, "bf16")])
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
    """B > 1 runs one launch per matrix through the same entry point; bf16
    outputs round once."""
    K, bits, group = 1024, 5, 32
    mats = _mats(gpu, [200, 40], K, bits, group, 7)
    for B, y_dtype, tol in [(2, torch.float32, 2e-3), (1, torch.bfloat16, 2e-3 + 2.0 ** -8)]:
        xb = gen_x_bf16(B, K, rng_for(333, B))
        xv = oracle.product.bf16_to_f64(xb)
        ys = gpu.qgemv_group_multi([(c, m, n) for c, m, n, _ in mats], K, bits, group, dev_bf16(xb), y_dtype=y_dtype)
        for (c, m, n, W_hat), y in zip(mats, ys):
            check_err(host(y), oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv), tol)


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
