"""Packed layout of group-RTN codes and group constants.  TEST INFRASTRUCTURE.

The pages fix what a block holds (32 or 64 codes plus one scale and one
offset, "TurboQuant: cuantizar modelos grandes...", "Compresión por
bloques") but not a byte layout.  This module is the layout's definition,
written out bit by bit; the GPU packer must produce the same bytes.

Layout, version 1
-----------------
codes: each row of K codes is cut into K/32 *units* of 32 consecutive codes
(code c of unit u is the code of input k = 32u + c).  A unit of b-bit codes
is b little-endian 32-bit words, stored contiguously; units follow each other
along K, rows follow each other along N.  Row n, unit u starts at word
(n*K/32 + u)*b, so a row holds K*b/8 bytes and no bit is padding.

Inside a unit, every 16-bit half of every word holds F = floor(16/b) b-bit
fields from its bit 0 up; the R = 16 - F*b bits above them ("spare" bits)
hold the codes that do not fit in fields.  For each code c (0..31) and each
code bit i (0 = least significant) the position is:

  regular codes (2F per word, b words: c < 2*F*b, which is all 32 codes
  for b = 2 and 4, 30 codes for b = 3 and 5, 24 codes for b = 6):
      word = c // (2F),  half h = (c % (2F)) // F,  field j = c % F,
      bit position 16*h + b*j + i
  b = 3 or 5 (one spare bit per half), codes 30 and 31, h = c - 30:
      word = i, bit position 16*h + 15
  b = 6 (four spare bits per half), codes 24..31, c = 24 + 4*h + p:
      bits i = 0..3:  word = p,          bit position 16*h + 12 + i
      bits i = 4, 5:  word = 4 + p // 2, bit position 16*h + 12 + 2*(p % 2) + (i - 4)

For b = 2 and 4 this is plain LSB-first packing of the unit (code c at bit
b*c of the 32*b-bit unit).  Same-index fields of the two halves of a word
form the code pairs a kernel turns into two bf16 lanes with one shift and
one masked OR.

meta: one 32-bit word per group, row-major [N][K/g]: bits 0..15 are the fp16
scale s, bits 16..31 the fp16 offset o.
"""
from __future__ import annotations

import numpy as np

FORMAT_VERSION = 1


def fields_per_half(b: int) -> int:
    return 16 // b


def unit_positions(b: int) -> np.ndarray:
    """pos[c, i] = (word, bit) of bit i of code c in a b-bit unit.

    Returned as an int array of shape (32, b, 2).
    """
    if b not in (2, 3, 4, 5, 6):
        raise ValueError("bits must be 2..6")
    F = fields_per_half(b)
    pos = np.full((32, b, 2), -1, dtype=np.int64)
    n_regular = 2 * F * b  # 2F codes per word, b words
    n_regular = min(n_regular, 32)
    for c in range(32):
        for i in range(b):
            if c < n_regular:
                word = c // (2 * F)
                h = (c % (2 * F)) // F
                j = c % F
                pos[c, i] = (word, 16 * h + b * j + i)
            elif b in (3, 5):
                h = c - 30
                pos[c, i] = (i, 16 * h + 15)
            else:  # b == 6
                h, p = divmod(c - 24, 4)
                if i < 4:
                    pos[c, i] = (p, 16 * h + 12 + i)
                else:
                    pos[c, i] = (4 + p // 2, 16 * h + 12 + 2 * (p % 2) + (i - 4))
    return pos


def pack_codes(q: np.ndarray, b: int) -> np.ndarray:
    """Codes q[N][K] (uint8, < 2^b) -> uint32 words [N][K/32*b]."""
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    if q.size and int(q.max()) >= (1 << b):
        raise ValueError("code out of range")
    pos = unit_positions(b)
    units = q.reshape(N, K // 32, 32).astype(np.uint64)
    words = np.zeros((N, K // 32, b), dtype=np.uint64)
    for c in range(32):
        for i in range(b):
            w, bit = pos[c, i]
            words[:, :, w] |= ((units[:, :, c] >> np.uint64(i)) & np.uint64(1)) << np.uint64(bit)
    return words.astype(np.uint32).reshape(N, (K // 32) * b)


def unpack_codes(words: np.ndarray, N: int, K: int, b: int) -> np.ndarray:
    """Inverse of pack_codes: uint32 words -> uint8 codes [N][K]."""
    words = np.asarray(words, dtype=np.uint32).reshape(N, K // 32, b).astype(np.uint64)
    pos = unit_positions(b)
    q = np.zeros((N, K // 32, 32), dtype=np.uint64)
    for c in range(32):
        for i in range(b):
            w, bit = pos[c, i]
            q[:, :, c] |= ((words[:, :, w] >> np.uint64(bit)) & np.uint64(1)) << np.uint64(i)
    return q.astype(np.uint8).reshape(N, K)


def pack_meta(s: np.ndarray, o: np.ndarray) -> np.ndarray:
    """fp16 s, o [N][K/g] -> uint32 meta words (s low half, o high half)."""
    sb = np.asarray(s, dtype=np.float16).view(np.uint16).astype(np.uint32)
    ob = np.asarray(o, dtype=np.float16).view(np.uint16).astype(np.uint32)
    return (sb | (ob << np.uint32(16))).astype(np.uint32)


def unpack_meta(meta: np.ndarray):
    m = np.asarray(meta, dtype=np.uint32)
    s = (m & np.uint32(0xFFFF)).astype(np.uint16).view(np.float16)
    o = (m >> np.uint32(16)).astype(np.uint16).view(np.float16)
    return s, o


def codes_bytes(N: int, K: int, b: int) -> int:
    return N * K * b // 8


def meta_bytes(N: int, K: int, g: int) -> int:
    return N * (K // g) * 4
