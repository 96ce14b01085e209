"""GPU parity of the group-RTN path against the CPU oracle: packing and
unpacking bit-exact, GEMV within the normalized-error bound, exact integer
cases, unit probes, linearity, and the full-size layer shapes (sampled rows)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, TOL, check_bf16_out, check_err, dev, dev_bf16, group_reference, host, say
from workloads import (LAYER_SHAPES, config1_inputs, f32_to_bf16_bits, gen_weights, gen_x_bf16, gen_x_f32, layer_weights,
                       layer_x, rng_for)

pytestmark = pytest.mark.gpu
WIDTHS = [2, 3, 4, 5, 6]
GROUPS = [32, 64]


@pytest.mark.parametrize("bits", WIDTHS)
@pytest.mark.parametrize("group", GROUPS)
def test_pack_and_unpack_bit_exact(gpu, bits, group):
    say(f"pack b={bits} g={group}")
    W = gen_weights(37, 320 if group == 32 else 384, rng_for(50, bits * 100 + group), outliers=True)
    N, K = W.shape
    q, s, o, words, meta, W_hat = group_reference(W, bits, group)
    codes_d, meta_d = gpu.qpack_group(dev(W), bits, group)
    assert np.array_equal(codes_d.cpu().numpy(), words.view(np.uint8).reshape(-1))
    assert np.array_equal(meta_d.cpu().numpy().view(np.uint32), meta.reshape(-1))
    # unpack of the oracle's bytes
    qd, wd = gpu.qunpack_group(dev(words.view(np.uint8).reshape(-1)), dev(meta.view(np.int32).reshape(-1)),
                               N, K, bits, group, want_w=True)
    assert np.array_equal(qd.cpu().numpy(), q)
    w32 = wd.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(w32 - W_hat) <= np.abs(W_hat) * 2.0 ** -24)


def test_pack_config1(gpu):
    W, _ = config1_inputs()
    q, s, o, words, meta, _ = group_reference(W, 4, 32)
    codes_d, meta_d = gpu.qpack_group(dev(W), 4, 32)
    assert np.array_equal(codes_d.cpu().numpy(), words.view(np.uint8).reshape(-1))
    assert np.array_equal(meta_d.cpu().numpy().view(np.uint32), meta.reshape(-1))


def test_pack_special_groups(gpu):
    """Constant groups, exact fp16 values, negative zero, ties."""
    W = np.zeros((4, 128), dtype=np.float32)
    W[0, :32] = 0.25
    W[0, 32:64] = np.float32(0.1)
    W[1, :32] = -0.0
    W[1, 32:64] = np.linspace(-1, 1, 32, dtype=np.float32)
    W[2, :32] = np.arange(32, dtype=np.float32) % 16
    W[2, 32] = 2.5
    W[3, :] = np.float32(1e-7) * np.arange(128, dtype=np.float32)
    for bits in (3, 4, 6):
        _, _, _, words, meta, _ = group_reference(W, bits, 32)
        codes_d, meta_d = gpu.qpack_group(dev(W), bits, 32)
        assert np.array_equal(codes_d.cpu().numpy(), words.view(np.uint8).reshape(-1))
        assert np.array_equal(meta_d.cpu().numpy().view(np.uint32), meta.reshape(-1))


def test_pack_range_errors(gpu):
    W = np.zeros((2, 64), dtype=np.float32)
    W[1, 5] = np.nan
    with pytest.raises(gpu.QError) as e:
        gpu.qpack_group(dev(W), 4, 32)
    assert e.value.status == -4
    W = np.zeros((2, 64), dtype=np.float32)
    W[0, 0] = -1e6
    with pytest.raises(gpu.QError):
        gpu.qpack_group(dev(W), 4, 32)


def _gemv_case(gpu, bits, group, N, K, B, xkind, seed):
    W = gen_weights(N, K, rng_for(51, seed), outliers=True)
    _, _, _, words, meta, W_hat = group_reference(W, bits, group)
    rng = rng_for(52, seed)
    if xkind == "f32":
        xh = gen_x_f32(B, K, rng)
        xv = xh.astype(np.float64)
        xd = dev(xh)
    else:
        xb = gen_x_bf16(B, K, rng)
        xv = oracle.product.bf16_to_f64(xb)
        xd = dev_bf16(xb)
    y = gpu.qgemv_group(dev(words.view(np.uint8).reshape(-1)), dev(meta.view(np.int32).reshape(-1)),
                        N, K, bits, group, xd)
    y_ref = oracle.product.matmul_ref(W_hat, xv)
    D = oracle.product.abs_denominator(W_hat, xv)
    return check_err(host(y), y_ref, D)


@pytest.mark.parametrize("bits", WIDTHS)
@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("K", [320 * 2, 10240])
def test_gemv_b1_bf16(gpu, bits, group, K):
    say(f"gemv b1 bf16 b={bits} g={group} K={K}")
    _gemv_case(gpu, bits, group, 203, K, 1, "bf16", bits * 1000 + group + K)


@pytest.mark.parametrize("bits", [2, 4, 6])
@pytest.mark.parametrize("K", [512, 10240])
def test_gemv_b1_f32(gpu, bits, K):
    say(f"gemv b1 f32 b={bits} K={K}")
    err = _gemv_case(gpu, bits, 32, 131, K, 1, "f32", bits + K)
    assert err < 1e-5     # hi/lo split keeps ~16 bits of the fp32 activations


@pytest.mark.parametrize("bits", WIDTHS)
@pytest.mark.parametrize("B", [2, 8, 16])
def test_gemv_batched(gpu, bits, B):
    say(f"gemv B={B} b={bits}")
    _gemv_case(gpu, bits, 32 if bits != 4 else 64, 77, 1088, B, "bf16", bits * 10 + B)


@pytest.mark.parametrize("bits", WIDTHS)
@pytest.mark.parametrize("B", [3, 16])
def test_gemv_batched_other_group(gpu, bits, B):
    """The group size not covered above (groups of 64 hold two units each)."""
    say(f"gemv B={B} b={bits} other group")
    _gemv_case(gpu, bits, 64 if bits != 4 else 32, 45, 1216, B, "bf16", bits * 10 + B + 1)


@pytest.mark.parametrize("bits", WIDTHS)
@pytest.mark.parametrize("B", [1, 2, 16])
def test_gemv_integer_case_exact(gpu, bits, B):
    """Integer weights with both ends in every group (s = 1, o = 0, q = w) and
    small-integer activations: every partial sum is an exact fp32 integer."""
    rng = np.random.default_rng(bits * 7 + B)
    L = (1 << bits) - 1
    N, K, g = 45, 640, 32
    W = rng.integers(0, L + 1, size=(N, K)).astype(np.float32)
    W[:, ::g] = 0
    W[:, 1::g] = L
    xi = rng.integers(-4, 5, size=(B, K)).astype(np.float32)
    codes, meta = gpu.qpack_group(dev(W), bits, g)
    xb = (xi.view(np.uint32) >> 16).astype(np.uint16)
    y = gpu.qgemv_group(codes, meta, N, K, bits, g, dev_bf16(xb))
    assert np.array_equal(host(y), (xi.astype(np.int64) @ W.astype(np.int64).T).astype(np.float64))
    if B == 1:
        y = gpu.qgemv_group(codes, meta, N, K, bits, g, dev(xi))
        assert np.array_equal(host(y), (xi.astype(np.int64) @ W.astype(np.int64).T).astype(np.float64))


@pytest.mark.parametrize("bits", [2, 3, 5])
def test_gemv_unit_probes_and_linearity(gpu, bits):
    N, K, g = 29, 256, 32
    W = gen_weights(N, K, rng_for(53, bits), outliers=True)
    q, s, o, words, meta, W_hat = group_reference(W, bits, g)
    cd, md = dev(words.view(np.uint8).reshape(-1)), dev(meta.view(np.int32).reshape(-1))
    for k in (0, 1, 31, 32, 100, 255):
        e = np.zeros((1, K), np.uint16)
        e[0, k] = 0x3F80                                   # bf16 1.0
        y = host(gpu.qgemv_group(cd, md, N, K, bits, g, dev_bf16(e)))[0]
        col = W_hat[:, k]
        assert np.all(np.abs(y - col) <= np.abs(col) * 2.0 ** -24 + 1e-300)
        sg, og = s[:, k // g].astype(np.float64), o[:, k // g].astype(np.float64)
        ok = sg > 0
        assert np.array_equal(np.rint((y[ok] - og[ok]) / sg[ok]).astype(np.int64), q[ok, k].astype(np.int64))
    z = host(gpu.qgemv_group(cd, md, N, K, bits, g, dev_bf16(np.zeros((1, K), np.uint16))))
    assert np.all(z == 0)
    xb = gen_x_bf16(1, K, rng_for(54, bits))
    x2 = f32_to_bf16_bits((2 * oracle.product.bf16_to_f64(xb)).astype(np.float32))  # exactly 2x
    y1 = host(gpu.qgemv_group(cd, md, N, K, bits, g, dev_bf16(xb)))
    y2 = host(gpu.qgemv_group(cd, md, N, K, bits, g, dev_bf16(x2)))
    assert np.array_equal(y2, 2 * y1)


def test_gemv_bf16_output(gpu):
    N, K = 64, 512
    W = gen_weights(N, K, rng_for(55, 0), outliers=False)
    _, _, _, words, meta, W_hat = group_reference(W, 4, 64)
    xb = gen_x_bf16(1, K, rng_for(55, 1))
    cd, md = dev(words.view(np.uint8).reshape(-1)), dev(meta.view(np.int32).reshape(-1))
    y16 = gpu.qgemv_group(cd, md, N, K, 4, 64, dev_bf16(xb), y_dtype=torch.bfloat16)
    y32 = gpu.qgemv_group(cd, md, N, K, 4, 64, dev_bf16(xb))
    xv = oracle.product.bf16_to_f64(xb)
    check_bf16_out(host(y16), host(y32), oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv))


def test_config1_end_to_end(gpu):
    W, x = config1_inputs()
    _, _, _, words, meta, W_hat = group_reference(W, 4, 32)
    codes, metad = gpu.qpack_group(dev(W), 4, 32)
    y = gpu.qgemv_group(codes, metad, 512, 512, 4, 32, dev(x))
    xv = x.astype(np.float64)
    err = check_err(host(y), oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv))
    say(f"config 1 normalized error {err:.3e}")


# ------------------------------------------------------------ full sizes
_W_CACHE = {}


def _full(name):
    if name not in _W_CACHE:
        _W_CACHE.clear()
        _W_CACHE[name] = layer_weights(name)
    return _W_CACHE[name]


def _sample_rows(N, n=48):
    rows = np.unique(np.concatenate([[0, 1, N - 1], np.random.default_rng(N).choice(N, n, replace=False)]))
    return rows


def _full_case(gpu, name, bits, group, batches):
    K, N = LAYER_SHAPES[name]
    say(f"full {name} K={K} N={N} b={bits} g={group} B={batches}")
    W = _full(name)
    codes, meta = gpu.qpack_group(dev(W), bits, group)
    rows = _sample_rows(N)
    q, s, o, words, metaw, W_hat = group_reference(W[rows], bits, group)
    rb = K * bits // 8
    cbytes = codes.view(torch.uint8).reshape(N, rb)[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    assert np.array_equal(cbytes, words.view(np.uint8).reshape(len(rows), rb))
    mw = meta.view(torch.int32).reshape(N, K // group)[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    assert np.array_equal(mw.view(np.uint32), metaw)
    for B in batches:
        xb = layer_x(K, B)
        y = host(gpu.qgemv_group(codes, meta, N, K, bits, group, dev_bf16(xb)))[:, rows]
        xv = oracle.product.bf16_to_f64(xb)
        err = check_err(y, oracle.product.matmul_ref(W_hat, xv), oracle.product.abs_denominator(W_hat, xv))
        say(f"  B={B} err={err:.3e}")
    del codes, meta
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["gate", "down", "k", "q"])
def test_full_config2_4bit_g64(gpu, name):
    _full_case(gpu, name, 4, 64, [1, 16])


@pytest.mark.parametrize("name,bits", [("q", 6), ("q", 5), ("v", 6), ("gate", 3), ("gate", 2), ("down", 3), ("down", 2)])
def test_full_config3_mixed(gpu, name, bits):
    _full_case(gpu, name, bits, 32, [1, 8])
