"""Pins of the per-group codebook encoding (oracle/codebook.py; "TurboQuant:
cuantizar modelos grandes para que quepan en local", "Compresión por
bloques"): the reduction to group RTN when the dictionary holds only the
uniform grid (with RTN's ties to even), an exact rational brute force over
books and levels on inputs where every fp64 step is exact, the nearest-level
invariant, planted skewed groups, and the default dictionary's structure."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import codebook, rtn
from workloads import gen_weights, rng_for


def _uniform(bits):
    L = 1 << bits
    return (np.arange(L) * (1 << (7 - bits))).astype(np.uint8)[None, :]


@pytest.mark.parametrize("bits,group", [(2, 32), (2, 64), (3, 32), (3, 64), (4, 32), (4, 64)])
def test_uniform_book_is_group_rtn(bits, group):
    W = gen_weights(24, 512, rng_for(340, bits * 100 + group), outliers=True)
    q, s, o, book = codebook.quantize(W, bits, group, _uniform(bits))
    q0, s0, o0 = rtn.quantize(W, bits, group)
    assert np.array_equal(q, q0)
    assert np.array_equal(s.view(np.uint16), s0.view(np.uint16))
    assert np.array_equal(o.view(np.uint16), o0.view(np.uint16))
    assert not book.any()
    assert np.array_equal(codebook.dequantize(q, s, o, book, _uniform(bits), bits, group),
                          rtn.dequantize(q0, s0, o0, group))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_uniform_book_ties_go_to_even(bits):
    """Weights exactly half-way between two grid points: RTN rounds to the
    even code and so must the nearest-level rule.  s = 2^-4 and o = 0 make
    every u = w/s exact."""
    L = (1 << bits) - 1
    u = np.concatenate([[0.0, L], np.arange(2 * L + 1) / 2.0])
    u = np.resize(u, 64)
    W = (u * 2.0 ** -4).astype(np.float32)[None, :]
    q, s, o, book = codebook.quantize(W, bits, 64, _uniform(bits))
    q0, _, _ = rtn.quantize(W, bits, 64)
    assert float(s[0, 0]) == 2.0 ** -4 and float(o[0, 0]) == 0.0
    assert np.array_equal(q, q0)
    assert list(q[0, 2:2 + 2 * L + 1]) == [int(np.rint(v)) for v in np.arange(2 * L + 1) / 2.0]


def _brute(u_group, books, bits):
    """Exact rational brute force: (book, codes) of least squared error,
    nearest level per weight with ties to the even and then lower index,
    books tied in error to the lower index."""
    den = 1 << (7 - bits)
    best = None
    for d, row in enumerate(books):
        lv = [Fraction(int(e), den) for e in row]
        codes, err = [], Fraction(0)
        for u in u_group:
            dist = [abs(u - c) for c in lv]
            m = min(dist)
            j = min((j for j in range(len(lv)) if dist[j] == m), key=lambda j: (j % 2, j))
            codes.append(j)
            err += dist[j] ** 2
        if best is None or err < best[0]:
            best = (err, d, codes)
    return best[1], best[2]


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("seed", range(3))
def test_exact_brute_force(bits, seed):
    """Groups whose min is 0 and max is (2^b - 1)/8, so s = 1/8 and o = 0
    exactly, with values on a 1/128 grid: u has at most 11 significant bits,
    every distance, square and sum is exact in fp64, and the oracle must
    reproduce the rational brute force decision for decision (ties included:
    the 1/16 grid of u meets level midpoints)."""
    rng = np.random.default_rng(350 + 10 * bits + seed)
    L = (1 << bits) - 1
    G = 32
    n_groups = 12
    u16 = rng.integers(0, 16 * L + 1, size=(n_groups, G))
    u16[:, 0], u16[:, 1] = 0, 16 * L
    W = (u16 / 16.0 * 0.125).astype(np.float32).reshape(1, n_groups * G)
    rng_b = np.random.default_rng(360 + seed)
    books = np.sort(rng_b.integers(0, 128, size=(5, 1 << bits)), axis=1)
    books[0] = _uniform(bits)[0]
    books[3] = books[2]                         # an exact book tie
    q, s, o, book = codebook.quantize(W, bits, G, books)
    assert np.all(s.astype(np.float64) == 0.125) and np.all(o.astype(np.float64) == 0.0)
    for g in range(n_groups):
        d, codes = _brute([Fraction(int(v), 16) for v in u16[g]], books, bits)
        assert book[0, g] == d, g
        assert list(q[0, g * G:(g + 1) * G]) == codes, g


@pytest.mark.parametrize("bits,group", [(2, 64), (3, 32), (4, 64)])
def test_codes_are_nearest_levels_and_book_is_best(bits, group):
    """Invariants on the outlier workload: every code is a nearest level of
    its group's book, and no other book gives a smaller group error."""
    W = gen_weights(16, 1024, rng_for(341, bits), outliers=True)
    books = codebook.default_dictionary(bits)
    q, s, o, book = codebook.quantize(W, bits, group, books)
    lv = codebook.levels(books, bits)
    N, K = W.shape
    Gn = K // group
    s64 = np.repeat(s.astype(np.float64), group, axis=1)
    o64 = np.repeat(o.astype(np.float64), group, axis=1)
    u = (W.astype(np.float64) - o64) / s64
    bk = np.repeat(book.astype(np.int64), group, axis=1)
    c = lv[bk, q]
    all_d = np.abs(u[:, :, None] - lv[bk])            # distance to every level of the book
    assert np.all(np.abs(u - c) <= all_d.min(axis=2))
    for d in range(books.shape[0]):
        e_d = (np.abs(u[:, :, None] - lv[d][None, None, :]).min(axis=2) ** 2).reshape(N, Gn, group).sum(axis=2)
        e_b = ((u - c) ** 2).reshape(N, Gn, group).sum(axis=2)
        assert np.all(e_b <= e_d * (1 + 1e-12))


def test_skewed_groups_take_one_sided_books():
    """A group of small values with one large positive weight has most of
    its range empty above the bulk: a book dense near the minimum (4 or 5)
    wins; the mirrored group takes a book dense near the maximum (6 or 7).
    A group drawn from a bell-shaped law takes the uniform or a centre-dense
    book (0..3)."""
    rng = rng_for(342, 0)
    books = codebook.default_dictionary(3)
    base = rng.standard_normal((64, 64)) * 0.02
    skew = base.copy()
    skew[:, 5] = 0.5
    q, s, o, book = codebook.quantize(skew.astype(np.float32), 3, 64, books)
    assert np.all(np.isin(book, [4, 5]))
    q, s, o, book = codebook.quantize((-skew).astype(np.float32), 3, 64, books)
    assert np.all(np.isin(book, [6, 7]))
    q, s, o, book = codebook.quantize(base.astype(np.float32), 3, 64, books)
    assert np.all(book <= 3)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_default_dictionary_structure(bits):
    D = codebook.default_dictionary(bits)
    L = 1 << bits
    top = (L - 1) << (7 - bits)
    assert D.shape == (8, L) and D.dtype == np.uint8 and D.max() <= 127
    assert np.array_equal(D[0], _uniform(bits)[0])
    assert np.all(D[:, 0] == 0) and np.all(D[:, -1] == top)   # the group's min and max
    assert np.all(np.diff(D.astype(int), axis=1) >= 0)
    for b in (1, 2, 3):                                        # symmetric about the middle
        assert np.all(D[b].astype(int) + D[b][::-1] == top)
        assert np.all(D[b, 1:L // 2] > D[0, 1:L // 2])         # pulled toward the centre
    for b in (4, 5):                                           # mirrors
        assert np.all(D[b + 2].astype(int) == top - D[b][::-1])
        assert np.all(D[b, 1:-1] < D[0, 1:-1])                 # pulled toward the minimum


@pytest.mark.parametrize("bits,group", [(2, 64), (3, 32), (4, 64)])
def test_dictionary_lowers_the_error(bits, group):
    """Choosing among the books never raises a group's error over plain RTN
    (book 0 is the RTN grid); on the layer workload the mean squared weight
    error drops by more than a quarter."""
    W = gen_weights(64, 2048, rng_for(343, bits), outliers=True)
    books = codebook.default_dictionary(bits)
    q, s, o, book = codebook.quantize(W, bits, group, books)
    Wc = codebook.dequantize(q, s, o, book, books, bits, group)
    q0, s0, o0 = rtn.quantize(W, bits, group)
    Wr = rtn.dequantize(q0, s0, o0, group)
    W64 = W.astype(np.float64)
    N, K = W.shape
    ec = ((Wc - W64) ** 2).reshape(N, K // group, group).sum(axis=2)
    er = ((Wr - W64) ** 2).reshape(N, K // group, group).sum(axis=2)
    assert np.all(ec <= er * (1 + 1e-9))
    assert ec.sum() < 0.75 * er.sum()


def test_constant_group_and_errors():
    W = np.full((2, 64), 0.375, np.float32)
    W[1, 32:] = -1.5
    books = codebook.default_dictionary(2)
    q, s, o, book = codebook.quantize(W, 2, 32, books)
    assert not q.any() and not book.any() and not s.view(np.uint16).any()
    assert np.array_equal(codebook.dequantize(q, s, o, book, books, 2, 32), W.astype(np.float64))
    with pytest.raises(ValueError):
        codebook.quantize(W, 5, 32, books)
    with pytest.raises(ValueError):
        codebook.quantize(W, 2, 32, np.full((1, 4), 128))
    with pytest.raises(ValueError):
        codebook.quantize(W, 2, 32, np.zeros((17, 4), np.uint8))
    with pytest.raises(ValueError):
        codebook.quantize(W, 2, 32, np.zeros((2, 8), np.uint8))
    Wb = W.copy()
    Wb[0, 3] = np.inf
    with pytest.raises(rtn.RangeError):
        codebook.quantize(Wb, 2, 32, books)
