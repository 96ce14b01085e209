"""Pins of the product, the metric and the size arithmetic."""
import json
import os

import numpy as np

from oracle import fmt, product, rtn, sizes
from workloads import LAYER_SHAPES, f32_to_bf16_bits, gen_weights, rng_for

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def test_bf16_decode():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F], dtype=np.uint16)
    v = product.bf16_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 2.0 ** -133
    assert v[3] == (2 - 2.0 ** -7) * 2.0 ** 127
    # round trip through the generator's rounding
    x = np.array([1.0, 1.00390625, 1.01171875, -3.5], dtype=np.float32)
    assert np.array_equal(product.bf16_to_f64(f32_to_bf16_bits(x)), [1.0, 1.0, 1.015625, -3.5])


def test_integer_case_full_path_is_exact():
    """Integer weights in [0, L] with both ends in every group, small-integer
    activations: quantize -> pack -> unpack -> product equals the int64 matvec."""
    rng = np.random.default_rng(21)
    for bits, g in [(4, 64), (2, 32), (6, 32), (3, 32), (5, 64)]:
        L = (1 << bits) - 1
        W = rng.integers(0, L + 1, size=(6, 256)).astype(np.float32)
        W[:, ::g] = 0
        W[:, 1::g] = L
        q, s, o = rtn.quantize(W, bits, g)
        words = fmt.pack_codes(q, bits)
        meta = fmt.pack_meta(s, o)
        W_hat = product.what_group(words, meta, 6, 256, bits, g)
        x = rng.integers(-3, 4, size=(3, 256))
        y = product.matmul_ref(W_hat, x)
        assert np.array_equal(y, (x.astype(np.int64) @ W.astype(np.int64).T).astype(np.float64))


def test_linearity_and_probes():
    W = gen_weights(16, 128, rng_for(90, 1), outliers=True)
    q, s, o = rtn.quantize(W, 4, 32)
    W_hat = rtn.dequantize(q, s, o, 32)
    assert np.all(product.matmul_ref(W_hat, np.zeros((1, 128))) == 0)
    x = np.random.default_rng(0).standard_normal((2, 128))
    assert np.array_equal(product.matmul_ref(W_hat, 4 * x), 4 * product.matmul_ref(W_hat, x))
    assert np.array_equal(product.matmul_ref(W_hat, np.eye(128)).T, W_hat)


def test_normalized_error_by_hand():
    W = np.array([[1.0, -2.0], [0.0, 0.0]])
    x = np.array([[3.0, 1.0]])
    D = product.abs_denominator(W, x)
    assert D.tolist() == [[5.0, 0.0]]
    y_ref = product.matmul_ref(W, x)
    assert y_ref.tolist() == [[1.0, 0.0]]
    assert abs(product.normalized_error(np.array([[1.01, 0.0]]), y_ref, D) - 0.002) < 1e-12
    assert product.normalized_error(np.array([[1.0, 1e-30]]), y_ref, D) == float("inf")


def test_oracle_summation_error_is_negligible():
    """fp64 product vs exact rational sum on a small case: error << 2e-3."""
    from fractions import Fraction
    W = gen_weights(3, 256, rng_for(91, 0), outliers=True)
    q, s, o = rtn.quantize(W, 3, 32)
    W_hat = rtn.dequantize(q, s, o, 32)
    x = product.bf16_to_f64(f32_to_bf16_bits(np.random.default_rng(2).standard_normal((1, 256)).astype(np.float32)))
    y = product.matmul_ref(W_hat, x)
    D = product.abs_denominator(W_hat, x)
    for i in range(3):
        exact = sum(Fraction(W_hat[i, j]) * Fraction(x[0, j]) for j in range(256))
        assert abs(Fraction(y[0, i]) - exact) / Fraction(D[0, i]) < Fraction(1, 10 ** 12)


def _llama70b_params():
    per_layer = sum(K * N for K, N in LAYER_SHAPES.values())
    return per_layer, 80 * per_layer + 2 * 32000 * 8192   # decoder + embeddings/lm_head


def test_sizes_against_page_figures():
    gold = json.load(open(GOLDEN))
    per_layer, total = _llama70b_params()
    assert gold["n_layers"]["value"] == 80

    def close(key, v):
        g = gold[key]
        assert abs(v - g["value"]) <= g["rel_tol"] * g["value"], (key, v)

    close("fp16_70b_GB", total * 2 / 1e9)
    close("nanoquant_fp16_GB", total * 2 / 1e9)
    close("nanoquant_v3_fp16_GB", total * 2 / 1e9)
    close("int4_70b_GB", total * 4 / 8 / 1e9)
    close("fp16_per_layer_GB", per_layer * 2 / 1e9)
    assert sizes.group_bpw(4, 64) == gold["q4km_bpw"]["value"]
    close("q4km_70b_GB", total * sizes.group_bpw(4, 64) / 8 / 1e9)
    lo, hi = gold["block_constant_overhead_bits"]["value"]
    assert lo <= sizes.group_bpw(4, 32) - 4 <= hi
    for gbytes, bw, sec in gold["disk_seconds_per_token"]["value"]:
        assert sizes.seconds_per_token(gbytes, bw) == sec
    a, b, ratio = gold["nanoquant_compression"]["value"]
    assert round(a / b, 1) == ratio
    a, b, ratio = gold["nanoquant_v3_compression"]["value"]
    assert round(a / b) == ratio


def test_layer_set_bytes():
    """A layer's compressed bytes: with one width and group for all seven
    matrices it is the layer's parameter count times b + 32/g bits; mixed
    widths split the count into the attention and MLP parts; 80 layers at
    4.5 bits (4-bit codes, groups of 64) plus 4.5-bit embeddings reproduce
    the page's ~40 GB for a dense 70B at about 4.5 bpw."""
    gold = json.load(open(GOLDEN))
    per_layer, total = _llama70b_params()
    uni = sizes.layer_set_bytes(LAYER_SHAPES, lambda n: 4, lambda n: 64)
    assert uni * 8 == per_layer * 4.5
    assert uni == 481_296_384
    attn = sum(K * N for n, (K, N) in LAYER_SHAPES.items() if n in ("q", "k", "v", "o"))
    mlp = per_layer - attn
    hi = sizes.layer_set_bytes(LAYER_SHAPES, lambda n: 6 if n in ("q", "k", "v", "o") else 3, lambda n: 32)
    assert hi * 8 == attn * (6 + 1) + mlp * (3 + 1)
    lo = sizes.layer_set_bytes(LAYER_SHAPES, lambda n: 5 if n in ("q", "k", "v", "o") else 2, lambda n: 32)
    assert lo * 8 == attn * (5 + 1) + mlp * (2 + 1)
    g = gold["q4km_70b_GB"]
    model = (80 * uni + (total - 80 * per_layer) * sizes.group_bpw(4, 64) / 8) / 1e9
    assert abs(model - g["value"]) <= g["rel_tol"] * g["value"], model


def test_sizes_formulas():
    assert sizes.group_bytes(28672, 8192, 4, 64) == 132_120_576
    assert sizes.group_bytes(512, 512, 4, 32) == 163_840
    assert sizes.binlr_bytes(28672, 8192, 4096) == 18_948_096
    assert sizes.binlr_bytes(8192, 8192, 2048) == 4_227_072
    assert abs(sizes.binlr_bpw(28672, 8192, 4096) - 0.6454) < 1e-4
    assert abs(sizes.binlr_bpw(8192, 8192, 2048) - 0.5039) < 1e-4
    assert abs(sizes.binlr_core_bpw(28672, 8192, 4096) - 0.6429) < 1e-4
    assert sizes.binlr_core_bpw(8192, 8192, 2048) == 0.5
    # codes + meta byte counts agree with the packed buffers
    q = np.zeros((4, 256), np.uint8)
    assert fmt.pack_codes(q, 5).nbytes + 4 * (256 // 64) * 4 == sizes.group_bytes(4, 256, 5, 64)


def test_binlr_denominator_degenerate_rows():
    """A sign-product row that is identically zero (U_i orthogonal to every
    V_j) has D = 0; the binary denominator then falls back to the factored
    terms' magnitude |s1_i| r sum_j |s2_j x_j|, and it never undercuts D."""
    U = np.array([[1, -1], [1, 1]], np.int8)            # row 0: (1,-1) . (1,1) = 0
    V = np.array([[1, 1], [1, 1], [-1, -1]], np.int8)
    s1 = np.array([0x3C00, 0x4000], np.uint16)           # fp16 1.0, 2.0
    s2 = np.array([0x3C00, 0x3800, 0x4000], np.uint16)   # 1.0, 0.5, 2.0
    x = np.array([[1.0, -4.0, 0.25]])
    D = product.binlr_abs_denominator(U, V, s1, s2, x)
    # row 0: C = 0 -> 1 * 2 * (1 + 2 + 0.5) = 7 ; row 1: C = (2, 2, -2) -> 2 * (2*1 + 2*0.5*4 + 2*2*0.25) = 14
    assert np.array_equal(D, np.array([[7.0, 14.0]]))
    rng = np.random.default_rng(3)
    for r in (1, 2, 3, 8):
        U = np.where(rng.integers(0, 2, (9, r)) == 1, 1, -1).astype(np.int8)
        V = np.where(rng.integers(0, 2, (7, r)) == 1, 1, -1).astype(np.int8)
        s1 = (np.abs(rng.standard_normal(9)) + 0.1).astype(np.float16).view(np.uint16)
        s2 = (np.abs(rng.standard_normal(7)) + 0.1).astype(np.float16).view(np.uint16)
        x = rng.standard_normal((2, 7))
        W = product.f16_to_f64(s1)[:, None] * (U.astype(np.int64) @ V.T.astype(np.int64)) * product.f16_to_f64(s2)
        D0 = product.abs_denominator(W, x)
        D1 = product.binlr_abs_denominator(U, V, s1, s2, x)
        assert np.all(D1 >= D0) and np.array_equal(D1[D0 > 0], D0[D0 > 0]) and np.all(D1 > 0)
