"""Group-wise asymmetric round-to-nearest (RTN) encoding.  TEST INFRASTRUCTURE.

Definition ("Métodos de cuantización de LLM...", RTN paragraph; "TurboQuant:
cuantizar modelos grandes...", "Compresión por bloques"): the K inputs of each
output row are cut into consecutive groups of g in {32, 64} weights; a group
shares one fp16 scale s and one fp16 offset o; each weight w is replaced by
the nearest of the 2^b levels o + s*q, q in [0, 2^b - 1], without calibration.

Readings where the pages are silent (plain min-max RTN, no clipping search):
  * o is the largest fp16 value <= min(group); s is the smallest fp16 value
    >= (max - o) / (2^b - 1) computed in IEEE fp64.  Rounding o down and s up
    keeps every weight inside the grid, so |w - w_hat| <= s/2 for all w.
  * A zero o or s is stored as +0 (never -0).
  * q = rint((w - o) / s), fp64 subtraction and IEEE division, ties to even,
    clamped to [0, 2^b - 1] (the clamp is a guard; it never fires).
  * s == 0 only for a constant group whose value is an fp16 number; then all
    codes are 0 and w_hat = o exactly.
  * Non-finite weights, an offset below -65504 or a scale above 65504 are
    errors (the GPU entry point reports them as a range error).
"""
from __future__ import annotations

import numpy as np

F16_MAX = 65504.0


class RangeError(ValueError):
    pass


def fp16_round_down(v: np.ndarray) -> np.ndarray:
    """Largest fp16 value <= v (elementwise, v in fp64).  Returns float16.

    numpy's float64 -> float16 conversion rounds to nearest even; when that
    lands above v we step one fp16 value toward -inf.
    """
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        h = v.astype(np.float16)
    up = h.astype(np.float64) > v
    with np.errstate(over="ignore"):
        h = np.where(up, np.nextafter(h, np.float16(-np.inf)), h)
    h = np.where(h == 0, np.float16(0.0), h)  # canonical +0
    return h.astype(np.float16)


def fp16_round_up(v: np.ndarray) -> np.ndarray:
    """Smallest fp16 value >= v (elementwise, v in fp64).  Returns float16."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        h = v.astype(np.float16)
    down = h.astype(np.float64) < v
    with np.errstate(over="ignore"):
        h = np.where(down, np.nextafter(h, np.float16(np.inf)), h)
    h = np.where(h == 0, np.float16(0.0), h)
    return h.astype(np.float16)


def quantize(W: np.ndarray, bits: int, group: int):
    """Encode W[N][K] (fp32) with b-bit codes in groups of `group` along K.

    Returns (q uint8 [N][K], s float16 [N][K/g], o float16 [N][K/g]).
    Steps, per row and group, in the order of the definition above:
      1. mn, mx = min, max of the group (exact);
      2. o = largest fp16 <= mn;
      3. v = (mx - o) / L in fp64, s = smallest fp16 >= v;
      4. q = clamp(rint((w - o) / s), 0, L), or 0 where s == 0.
    """
    if bits not in (2, 3, 4, 5, 6):
        raise ValueError("bits must be 2..6")
    if group not in (32, 64):
        raise ValueError("group must be 32 or 64")
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    if not np.all(np.isfinite(W)):
        raise RangeError("non-finite weight")
    L = (1 << bits) - 1
    Wg = W.astype(np.float64).reshape(N, K // group, group)
    mn = Wg.min(axis=2)
    mx = Wg.max(axis=2)
    o = fp16_round_down(mn)
    if np.any(~np.isfinite(o.astype(np.float64))):
        raise RangeError("group minimum below the fp16 range")
    o64 = o.astype(np.float64)
    v = (mx - o64) / float(L)
    s = fp16_round_up(v)
    if np.any(~np.isfinite(s.astype(np.float64))):
        raise RangeError("group scale above the fp16 range")
    s64 = s.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (Wg - o64[:, :, None]) / s64[:, :, None]
    q = np.rint(t)
    q = np.where(s64[:, :, None] == 0.0, 0.0, q)
    q = np.clip(q, 0, L).astype(np.uint8)
    return q.reshape(N, K), s, o


def dequantize(q: np.ndarray, s: np.ndarray, o: np.ndarray, group: int) -> np.ndarray:
    """w_hat = s*q + o per group, in fp64 (exact: at most 46 significant bits)."""
    N, K = q.shape
    qg = q.astype(np.float64).reshape(N, K // group, group)
    w = qg * s.astype(np.float64)[:, :, None] + o.astype(np.float64)[:, :, None]
    return w.reshape(N, K)
