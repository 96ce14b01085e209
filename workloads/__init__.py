"""Seeded synthetic inputs for the compressed-weight product.

This module only draws random numbers and stores them in the dtypes the
inputs are defined in (fp32 weights, bf16 activations, fp16 channel scales,
+-1 factors).  It holds none of the method's arithmetic: no quantization, no
packing, no product.  Both the CPU oracle and the GPU path take their inputs
from here, so the two sides always see the same bits.

Workload shapes follow the Llama-70B decode layer (hidden 8192, MLP 28672,
8 KV heads x 128, 80 layers) that the pages use as their running example
("70B en 4GB de VRAM", section 4; "AirLLM corre un modelo 70B", section
"El truco"; "Nvidia comprime un modelo de 74B", the KV formula paragraph).
A shape written K x N means K inputs and N outputs; weights are stored
output-major, W[N][K].

Outlier columns: about 0.1 % of the input channels are scaled by 20 before
quantization, the outlier statistic of "Métodos de cuantización de LLM",
introduction.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "LAYER_SHAPES", "ATTN", "MLP", "rng_for", "f32_to_bf16_bits",
    "f32_to_f16_bits", "gen_weights", "gen_x_bf16", "gen_x_f32", "gen_binlr",
    "outlier_columns", "config1_inputs",
]

# name -> (K, N): K inputs, N outputs
LAYER_SHAPES = {
    "q": (8192, 8192),
    "k": (8192, 1024),
    "v": (8192, 1024),
    "o": (8192, 8192),
    "gate": (8192, 28672),
    "up": (8192, 28672),
    "down": (28672, 8192),
}
LAYER_ORDER = ["q", "k", "v", "o", "gate", "up", "down"]
ATTN = ("q", "k", "v", "o")
MLP = ("gate", "up", "down")
N_LAYERS = 80

# Mixed-width layer sets: attention at 6 or 5 bits, MLP at 3 or 2 bits,
# groups of 32 ("TurboQuant: cuantizar modelos grandes", "Asignación de bits
# por capa" and "Compresión por bloques").
MIXED_SETS = {
    "hi": {"attn_bits": 6, "mlp_bits": 3, "group": 32},
    "lo": {"attn_bits": 5, "mlp_bits": 2, "group": 32},
}

BINLR_SHAPES = [  # (K, N, r)
    (8192, 28672, 4096),
    (8192, 8192, 2048),
]


def rng_for(config: int, tensor_id: int) -> np.random.Generator:
    """Independent stream per (config, tensor).  Config 1 uses plain seed 0."""
    return np.random.default_rng(np.random.SeedSequence([0, int(config), int(tensor_id)]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits.

    This only fixes the dtype the activations are delivered in; the rounded
    values *are* the inputs.  NaN/Inf are not produced by the generators.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """Round to fp16 (numpy's conversion is round to nearest even)."""
    return np.asarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def outlier_columns(K: int, rng: np.random.Generator) -> np.ndarray:
    """round(0.001*K) distinct input channels, drawn without replacement."""
    n = int(round(0.001 * K))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng.choice(K, size=n, replace=False))


def gen_weights(N: int, K: int, rng: np.random.Generator, outliers: bool,
                sigma: float = 0.02, scale: float = 20.0) -> np.ndarray:
    """fp32 W[N][K] ~ N(0, sigma); optionally 0.1 % of columns scaled 20x."""
    W = rng.standard_normal((N, K), dtype=np.float32)
    W *= np.float32(sigma)
    if outliers:
        cols = outlier_columns(K, rng)
        W[:, cols] *= np.float32(scale)
    return W


def gen_x_bf16(B: int, K: int, rng: np.random.Generator) -> np.ndarray:
    """Activations x[B][K] ~ N(0,1) delivered as bf16 bits (uint16)."""
    x = rng.standard_normal((B, K), dtype=np.float32)
    return f32_to_bf16_bits(x)


def gen_x_f32(B: int, K: int, rng: np.random.Generator) -> np.ndarray:
    return rng.standard_normal((B, K), dtype=np.float32)


def gen_binlr(N: int, K: int, r: int, rng: np.random.Generator):
    """Random +-1 factors U[N][r], V[K][r] (int8) and fp16 channel scales.

    s1 (length N, output side) and s2 (length K, input side) ~ |N(1, 0.1)|,
    rounded to fp16.  Returned as (U, V, s1_bits, s2_bits).
    """
    U = np.where(rng.integers(0, 2, size=(N, r), dtype=np.int8) == 1, 1, -1).astype(np.int8)
    V = np.where(rng.integers(0, 2, size=(K, r), dtype=np.int8) == 1, 1, -1).astype(np.int8)
    s1 = np.abs(1.0 + 0.1 * rng.standard_normal(N)).astype(np.float32)
    s2 = np.abs(1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    return U, V, f32_to_f16_bits(s1), f32_to_f16_bits(s2)


def config1_inputs():
    """512x512 layer, fp32 W ~ N(0,0.02), fp32 x ~ N(0,1), seed 0 (W first)."""
    rng = np.random.default_rng(0)
    W = rng.standard_normal((512, 512), dtype=np.float32) * np.float32(0.02)
    x = rng.standard_normal((1, 512), dtype=np.float32)
    return W, x


def layer_weights(name: str, config: int = 2, outliers: bool = True) -> np.ndarray:
    """Full-size fp32 weights of one layer matrix (deterministic per name)."""
    K, N = LAYER_SHAPES[name]
    return gen_weights(N, K, rng_for(config, LAYER_ORDER.index(name)), outliers)


def layer_x(K: int, B: int, config: int = 2) -> np.ndarray:
    return gen_x_bf16(B, K, rng_for(config, 1_000_000 + 100 * K + B))


def binlr_factors(K: int, N: int, r: int, config: int = 4):
    return gen_binlr(N, K, r, rng_for(config, 2_000_000 + r))
