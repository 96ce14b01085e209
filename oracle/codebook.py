"""Group codes with a per-group codebook drawn from a shared dictionary.
TEST INFRASTRUCTURE.

Source: "TurboQuant: cuantizar modelos grandes para que quepan en local".
Its "Compresión por bloques" paragraph gives each block of 32 or 64 weights
a shared scale and offset plus a compressed codebook of its own; its
introduction calls the scheme block compression with a shared dictionary.

Readings (the page gives no level set, selection rule or storage):
  * A dictionary of D <= 16 books is shared by every group of a matrix.  A
    book is a list of L = 2^b levels on a grid 2^(7-b) times finer than the
    code grid: entry e (an integer 0..127) stands for the level
    c = e / 2^(7-b) in code units.  A group's "compressed codebook" is the
    index of one book (one byte per group).
  * s and o are the group-RTN constants of rtn.py (o = largest fp16 <= min,
    s = smallest fp16 >= (max - o)/(2^b - 1)), so the code range [0, 2^b-1]
    spans the group, and w_hat = s*c + o.
  * Encoding a group: u = (w - o)/s (fp64 subtraction and division, as
    RTN).  For each book, every weight takes its nearest level; among
    equally near levels the even index, then the lower index.  The book's
    error is sum_k (u_k - c_k)^2 summed in increasing k in fp64 (no fused
    multiply-add).  The group keeps the book with the least error, ties to
    the lower book.  s == 0 (a constant group that is an fp16 value) gives
    book 0 and codes 0, and w_hat = o.
  * The even-index rule makes the uniform book (e_j = j * 2^(7-b)) the RTN
    grid with RTN's ties to even: a dictionary holding only that book is
    plain group RTN, code for code.
  * Widths b = 2, 3, 4 (at most 16 levels per book).

default_dictionary(b) is one dictionary of 8 books, a fixed family of
monotone warps of the uniform grid chosen here (the page names none): the
uniform book, three books denser near the middle of the range (bell-shaped
groups), two denser near the minimum and their two mirrors denser near the
maximum (groups skewed by a large value on one side).
"""
from __future__ import annotations

import numpy as np

from . import rtn

MAX_BOOKS = 16
BITS = (2, 3, 4)


def levels(books: np.ndarray, bits: int) -> np.ndarray:
    """Levels c = e / 2^(7-b) in code units, fp64, shape [D][L]."""
    return np.asarray(books, dtype=np.float64) / float(1 << (7 - bits))


def check_books(books: np.ndarray, bits: int) -> np.ndarray:
    if bits not in BITS:
        raise ValueError("codebook widths are 2, 3 and 4 bits")
    books = np.asarray(books)
    L = 1 << bits
    if books.ndim != 2 or books.shape[1] != L or not 1 <= books.shape[0] <= MAX_BOOKS:
        raise ValueError("books must be [D][2^b] with 1 <= D <= 16")
    if books.min() < 0 or books.max() > 127:
        raise ValueError("book entries must lie in 0..127")
    return books.astype(np.uint8)


def default_dictionary(bits: int) -> np.ndarray:
    """The 8-book dictionary described in the module docstring, uint8 [8][2^b]:
    book 0 uniform; books 1-3 c = m(1 + sign(t)|t|^g), t = 2j/(L-1) - 1,
    m = (L-1)/2, g = 1.5, 2, 3; books 4-5 c = (L-1) a^g, a = j/(L-1),
    g = 1.5, 2.5; books 6-7 their mirrors (L-1)(1 - (1-a)^g).  Entries are
    c * 2^(7-b) rounded to the nearest integer, ties to even."""
    if bits not in BITS:
        raise ValueError("codebook widths are 2, 3 and 4 bits")
    L = 1 << bits
    top = float(L - 1)
    j = np.arange(L, dtype=np.float64)
    t = 2.0 * j / top - 1.0
    a = j / top
    m = top / 2.0
    rows = [j.copy()]
    for g in (1.5, 2.0, 3.0):
        rows.append(m * (1.0 + np.sign(t) * np.abs(t) ** g))
    for g in (1.5, 2.5):
        rows.append(top * a ** g)
    for g in (1.5, 2.5):
        rows.append(top * (1.0 - (1.0 - a) ** g))
    c = np.stack(rows)
    return np.rint(c * float(1 << (7 - bits))).astype(np.uint8)


def nearest(u: np.ndarray, lv: np.ndarray):
    """Index of the nearest level of lv (1-D) for every u, with the tie rule
    of the module docstring, and the distance |u - c|.  u is fp64 of any
    shape."""
    d = np.abs(u[..., None] - lv)                      # [..., L]
    best = d.min(axis=-1, keepdims=True)
    L = lv.shape[0]
    j = np.arange(L)
    # among the minima: even indices first, then the lower index
    key = np.where(d == best, (j % 2) * L + j, 2 * L)
    q = key.argmin(axis=-1)
    return q, np.take_along_axis(d, q[..., None], axis=-1)[..., 0]


def quantize(W: np.ndarray, bits: int, group: int, books: np.ndarray):
    """Encode W[N][K] (fp32).  Returns (q uint8 [N][K], s float16 [N][K/g],
    o float16 [N][K/g], book uint8 [N][K/g]).  Steps, per row and group:
      1. s, o as group RTN;
      2. u = (w - o)/s in fp64;
      3. per book: nearest levels, error summed in increasing k;
      4. the book of least error (lower index on ties) and its codes."""
    books = check_books(books, bits)
    _, s, o = rtn.quantize(W, bits, group)          # s, o of the group RTN
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    G = K // group
    lv = levels(books, bits)
    Wg = W.astype(np.float64).reshape(N, G, group)
    s64 = s.astype(np.float64)[:, :, None]
    o64 = o.astype(np.float64)[:, :, None]
    zero = s64 == 0.0
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(zero, 0.0, (Wg - o64) / np.where(zero, 1.0, s64))
    D = books.shape[0]
    q_all = np.empty((D, N, G, group), dtype=np.int64)
    err = np.empty((D, N, G), dtype=np.float64)
    for d in range(D):
        q, dist = nearest(u, lv[d])
        q_all[d] = q
        e = np.zeros((N, G), dtype=np.float64)
        for k in range(group):                       # sequential sum
            e = e + dist[:, :, k] * dist[:, :, k]
        err[d] = e
    book = err.argmin(axis=0)                        # first minimum: lower book
    book = np.where(zero[:, :, 0], 0, book)
    q = np.take_along_axis(q_all, book[None, :, :, None], axis=0)[0]
    q = np.where(zero, 0, q)
    return q.reshape(N, K).astype(np.uint8), s, o, book.astype(np.uint8)


def dequantize(q: np.ndarray, s: np.ndarray, o: np.ndarray, book: np.ndarray,
               books: np.ndarray, bits: int, group: int) -> np.ndarray:
    """w_hat = s * c[book][q] + o in fp64 (exact: an 11-bit times a 7-bit
    significand plus an fp16 offset)."""
    lv = levels(check_books(books, bits), bits)
    N, K = q.shape
    qg = q.astype(np.int64).reshape(N, K // group, group)
    c = lv[book.astype(np.int64)[:, :, None], qg]
    w = c * s.astype(np.float64)[:, :, None] + o.astype(np.float64)[:, :, None]
    return w.reshape(N, K)
