"""Byte counts and bits per weight.  TEST INFRASTRUCTURE.

Group RTN: b bits per code plus one 32-bit (s, o) word per group of g, so
b + 32/g bits per weight ("70B en 4GB de VRAM...", section 3, notes that
per-block constants cost 1-2 extra bits per number).

Binary low-rank: r*(N+K) sign bits plus 16*(N+K) bits of fp16 channel
scales, over N*K weights; padding of the stored rows is not counted.
"""
from __future__ import annotations


def group_bytes(N: int, K: int, bits: int, group: int) -> int:
    """Compressed bytes of one group-RTN matrix: codes + meta."""
    return N * K * bits // 8 + N * (K // group) * 4


def group_bpw(bits: int, group: int) -> float:
    return bits + 32.0 / group


def binlr_bytes(N: int, K: int, r: int) -> int:
    """Compressed bytes of one binary matrix: sign bits + fp16 scales."""
    return (r * (N + K)) // 8 + 2 * (N + K)


def binlr_bpw(N: int, K: int, r: int) -> float:
    return 8.0 * binlr_bytes(N, K, r) / (N * K)


def binlr_core_bpw(N: int, K: int, r: int) -> float:
    return r * (N + K) / (N * K)


def layer_set_bytes(shapes, bits_of, group_of) -> int:
    """Sum of compressed bytes over a layer's matrices.

    shapes: dict name -> (K, N); bits_of/group_of: name -> int.
    """
    return sum(group_bytes(N, K, bits_of(n), group_of(n)) for n, (K, N) in shapes.items())


def seconds_per_token(model_bytes: float, bytes_per_second: float) -> float:
    """Decode time per token when every weight byte is read once per token
    ("AirLLM corre un modelo 70B", "Por qué es lento": size / read speed)."""
    return model_bytes / bytes_per_second
