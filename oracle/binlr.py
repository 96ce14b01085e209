"""Binary low-rank format: bit packing and explicit reconstruction.  TEST INFRASTRUCTURE.

Definition ("70B en 4GB de VRAM...", section 1, NanoQuant, the formulation
bullet): W ~ s1 (.) (U+-1 . V+-1^T) (.) s2^T, with U, V binary (+-1) of low
rank r and channel scales s1, s2.

Readings:
  * U is N x r (output side), V is K x r (input side); s1 has length N and
    scales outputs, s2 has length K and scales inputs, so the product runs
    in two stages t = V^T (s2 (.) x), y = s1 (.) (U t).
  * No extra normalization of U V^T: the magnitude lives in s1, s2.
  * Bits: +1 -> 1, -1 -> 0, least significant bit first inside
    little-endian 32-bit words.
  * Storage: Ubits[N][rw] with U[n][l] at bit l % 32 of word l // 32, and
    VTbits[r][Kw] with V[k][l] at bit k % 32 of word k // 32 of row l (the
    reduction dimension is contiguous in both).  rw = ceil(r/32) and
    Kw = ceil(K/32) are rounded up to multiples of 4 words (16 bytes);
    padding bits are 0 and contribute nothing to a product.
  * s1, s2 are fp16.
"""
from __future__ import annotations

import numpy as np


def padded_words(n: int) -> int:
    w = (n + 31) // 32
    return (w + 3) // 4 * 4


def pack_rows(M: np.ndarray) -> np.ndarray:
    """Pack a +-1 matrix row by row: M[R][C] -> uint32 [R][padded_words(C)].

    Bit l of a row (l = 0..C-1) is 1 for +1; bytes are filled least
    significant bit first and read as little-endian 32-bit words.
    """
    M = np.asarray(M)
    R, C = M.shape
    if not np.all((M == 1) | (M == -1)):
        raise ValueError("entries must be +-1")
    Wn = padded_words(C)
    bits = np.zeros((R, Wn * 32), dtype=np.uint8)
    bits[:, :C] = (M == 1)
    by = np.packbits(bits, axis=1, bitorder="little")
    return np.ascontiguousarray(by).view("<u4").astype(np.uint32).reshape(R, Wn)


def unpack_rows(words: np.ndarray, R: int, C: int) -> np.ndarray:
    """Inverse of pack_rows -> int8 +-1 [R][C]."""
    w = np.ascontiguousarray(np.asarray(words, dtype=np.uint32).reshape(R, -1))
    by = w.astype("<u4").view(np.uint8).reshape(R, -1)
    bits = np.unpackbits(by, axis=1, bitorder="little")[:, :C]
    return np.where(bits == 1, 1, -1).astype(np.int8)


def pack(U: np.ndarray, V: np.ndarray):
    """(U[N][r], V[K][r]) -> (Ubits[N][rw], VTbits[r][Kw])."""
    U = np.asarray(U)
    V = np.asarray(V)
    if U.shape[1] != V.shape[1]:
        raise ValueError("rank mismatch")
    return pack_rows(U), pack_rows(V.T)


def sign_product(U: np.ndarray, V: np.ndarray) -> np.ndarray:
    """C = U V^T in int64 (exact)."""
    return U.astype(np.int64) @ V.astype(np.int64).T


def sign_product_loops(U: np.ndarray, V: np.ndarray) -> np.ndarray:
    """The same C = U V^T by an explicit triple loop (tiny shapes only)."""
    N, r = U.shape
    K = V.shape[0]
    C = np.zeros((N, K), dtype=np.int64)
    for i in range(N):
        for j in range(K):
            acc = 0
            for l in range(r):
                acc += int(U[i, l]) * int(V[j, l])
            C[i, j] = acc
    return C


def reconstruct(U, V, s1_bits, s2_bits) -> np.ndarray:
    """W_hat[i][j] = s1[i] * s2[j] * C[i][j] in fp64.

    Exact: s1, s2 carry 11 significant bits each and |C| <= r needs at most
    log2(r)+1 more, well inside fp64's 53.
    """
    s1 = np.asarray(s1_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    s2 = np.asarray(s2_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    C = sign_product(U, V).astype(np.float64)
    return s1[:, None] * C * s2[None, :]
