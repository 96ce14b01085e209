"""Pins of the binary low-rank oracle (oracle/binlr.py, oracle/product.py):
bit order worked by hand, brute-force U V^T on tiny ranks, exact rational
reconstruction, the rank-1 closed form and the two-stage order."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import binlr, product
from workloads import gen_binlr


def test_bit_order_by_hand():
    row = -np.ones((1, 40), dtype=np.int8)
    row[0, 0] = 1
    row[0, 33] = 1
    row[0, 31] = 1
    w = binlr.pack_rows(row)
    assert w.shape == (1, 4)                   # 2 words rounded up to 4
    assert int(w[0, 0]) == 0x80000001 and int(w[0, 1]) == 0x2 and int(w[0, 2]) == 0 and int(w[0, 3]) == 0
    assert np.array_equal(binlr.unpack_rows(w, 1, 40), row)


def test_pack_roundtrip_and_padding():
    rng = np.random.default_rng(3)
    U, V, s1, s2 = gen_binlr(37, 70, 45, rng)
    ub, vtb = binlr.pack(U, V)
    assert ub.shape == (37, binlr.padded_words(45)) and vtb.shape == (45, binlr.padded_words(70))
    assert np.array_equal(binlr.unpack_rows(ub, 37, 45), U)
    assert np.array_equal(binlr.unpack_rows(vtb, 45, 70), V.T)
    # padding bits are zero
    assert np.all(ub[:, 1] >> np.uint32(45 - 32) == 0) and np.all(ub[:, 2:] == 0)


@pytest.mark.parametrize("r", [1, 2, 3, 4])
def test_sign_product_brute_force(r):
    rng = np.random.default_rng(r)
    U, V, _, _ = gen_binlr(11, 16, r, rng)
    C = binlr.sign_product(U, V)
    assert np.array_equal(C, binlr.sign_product_loops(U, V))
    assert np.all(np.abs(C) <= r) and np.all((C + r) % 2 == 0)


def test_reconstruct_exact_rationals():
    rng = np.random.default_rng(7)
    U, V, s1, s2 = gen_binlr(5, 6, 9, rng)
    W = binlr.reconstruct(U, V, s1, s2)
    s1f = s1.view(np.float16)
    s2f = s2.view(np.float16)
    for i in range(5):
        for j in range(6):
            c = sum(int(U[i, l]) * int(V[j, l]) for l in range(9))
            assert Fraction(W[i, j]) == Fraction(float(s1f[i])) * Fraction(float(s2f[j])) * c


def test_rank1_closed_form_and_stage_order():
    rng = np.random.default_rng(11)
    U, V, s1, s2 = gen_binlr(13, 17, 1, rng)
    x = rng.standard_normal((2, 17))
    W = binlr.reconstruct(U, V, s1, s2)
    y = product.matmul_ref(W, x)
    s1d = s1.view(np.float16).astype(np.float64)
    s2d = s2.view(np.float16).astype(np.float64)
    closed = (s1d * U[:, 0])[None, :] * (x @ (s2d * V[:, 0]))[:, None]
    assert np.allclose(y, closed, rtol=1e-13, atol=0)
    U, V, s1, s2 = gen_binlr(13, 17, 6, rng)
    W = binlr.reconstruct(U, V, s1, s2)
    assert np.allclose(product.matmul_ref(W, x), product.gemv_binlr_stages(U, V, s1, s2, x), rtol=1e-12, atol=1e-12)


def test_probe_columns():
    rng = np.random.default_rng(12)
    U, V, s1, s2 = gen_binlr(9, 10, 5, rng)
    W = binlr.reconstruct(U, V, s1, s2)
    E = np.eye(10)
    Y = product.matmul_ref(W, E)
    assert np.array_equal(Y.T, W)              # x = e_k returns column k exactly
