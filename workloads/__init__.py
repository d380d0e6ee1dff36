"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

This module only draws random numbers and places them at the byte offsets of the
block formats. It holds none of the method's arithmetic (no decoding, no dot
products, no scale unpacking), so neither side of a parity check can inherit a
mistake from it.

Formats (byte offsets, little-endian):
  Q4_K super-block, 144 B per 256 weights: [0:2] fp16 d, [2:4] fp16 dmin,
      [4:16] twelve bytes holding sixteen 6-bit fields (8 sub-scales, 8 mins),
      [16:144] 128 bytes of 4-bit quants.
  Q8_0 block, 34 B per 32 weights: [0:2] fp16 d, [2:34] 32 x int8.

Distributions (the synthetic workloads of the decode GEMV, the LM head and the
verify GEMM described by "Why Local LLMs Don't Need C++ or Python" sections 2 and
4 and the dotLLM README's quantized-inference feature):
  * d, dmin ~ U(0.001, 0.02), drawn in float64 and rounded to binary16
    (numpy's round-to-nearest-even cast).
  * the twelve scale bytes are uniform random bytes. The 6-bit packing maps the 96
    bits one-to-one onto the sixteen 6-bit fields, so uniform bytes are exactly
    sixteen independent U{0..63} fields.
  * the 128 quant bytes are uniform random bytes, i.e. 256 independent U{0..15}
    nibbles.
  * Q8_0 quants ~ U{-127..127} (the value -128 is never drawn).
  * activations x ~ N(0, 1) in float32.

Every stream is keyed: numpy PCG64 seeded from SeedSequence([BASE_SEED, *key]).
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 20261202

Q4K_BLOCK_BYTES = 144
Q4K_BLOCK_WEIGHTS = 256
Q8_0_BLOCK_BYTES = 34
Q8_0_BLOCK_WEIGHTS = 32

# role tags inside a key
ROLE_W = 1
ROLE_X = 2

# 7B-shaped decode layer (hidden 3584): name, rows M, cols K. Stages are the
# dependency groups of one transformer layer: {q,k,v} -> {o} -> {gate,up} -> {down}.
LAYER_MATRICES = (
    ("wq", 3584, 3584),
    ("wk", 512, 3584),
    ("wv", 512, 3584),
    ("wo", 3584, 3584),
    ("gate", 18944, 3584),
    ("up", 18944, 3584),
    ("down", 3584, 18944),
)
LAYER_STAGES = ((0, 1, 2), (3,), (4, 5), (6,))
N_LAYERS = 28
VOCAB = 152064
HIDDEN = 3584
FFN = 18944


def rng_for(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, *[int(k) for k in key]])))


def _fp16_bits(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.uniform(0.001, 0.02, size=n).astype(np.float16).view(np.uint16)


def q4k_blocks(M: int, K: int, key=(0,)) -> np.ndarray:
    """Random canonical Q4_K matrix: uint8 array of shape (M, K // 256 * 144), row-major."""
    if K % Q4K_BLOCK_WEIGHTS:
        raise ValueError("K must be a multiple of 256 for Q4_K")
    nb = K // Q4K_BLOCK_WEIGHTS
    rng = rng_for(*key, ROLE_W)
    out = rng.integers(0, 256, size=(M, nb, Q4K_BLOCK_BYTES), dtype=np.uint8)
    d = _fp16_bits(rng, M * nb).reshape(M, nb)
    dmin = _fp16_bits(rng, M * nb).reshape(M, nb)
    hdr = out[:, :, 0:4].view(np.uint16)  # (M, nb, 2) little-endian halves
    hdr[:, :, 0] = d
    hdr[:, :, 1] = dmin
    return out.reshape(M, nb * Q4K_BLOCK_BYTES)


def q6k_blocks(M: int, K: int, key=(0,)) -> np.ndarray:
    """Random canonical Q6_K matrix: uint8 array of shape (M, K // 256 * 210), row-major.
    The 128 + 64 quant bytes and the 16 scale bytes are uniform random bytes (so the
    6-bit quants are i.i.d. U{0..63} and the int8 scales U{-128..127}); d is fp16
    ~U(0.001, 0.02), stored in the block's last two bytes."""
    if K % Q4K_BLOCK_WEIGHTS:
        raise ValueError("K must be a multiple of 256 for Q6_K")
    nb = K // Q4K_BLOCK_WEIGHTS
    rng = rng_for(*key, ROLE_W)
    out = rng.integers(0, 256, size=(M, nb, 210), dtype=np.uint8)
    d = _fp16_bits(rng, M * nb).reshape(M, nb)
    out[:, :, 208:210] = d.astype(np.uint16)[..., None].view(np.uint8)
    return out.reshape(M, nb * 210)


def q8_0_blocks(M: int, K: int, key=(0,)) -> np.ndarray:
    """Random canonical Q8_0 matrix: uint8 array of shape (M, K // 32 * 34), row-major."""
    if K % Q8_0_BLOCK_WEIGHTS:
        raise ValueError("K must be a multiple of 32 for Q8_0")
    nb = K // Q8_0_BLOCK_WEIGHTS
    rng = rng_for(*key, ROLE_W)
    out = np.empty((M, nb, Q8_0_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 2:] = rng.integers(-127, 128, size=(M, nb, 32), dtype=np.int8).view(np.uint8)
    out[:, :, 0:2] = _fp16_bits(rng, M * nb).reshape(M, nb, 1).view(np.uint8)
    return out.reshape(M, nb * Q8_0_BLOCK_BYTES)


def x_vector(K: int, key=(0,)) -> np.ndarray:
    """Activation vector x ~ N(0,1), float32[K]."""
    return rng_for(*key, ROLE_X).standard_normal(K, dtype=np.float32)


def x_columns(K: int, N: int, key=(0,)) -> np.ndarray:
    """N activation columns, returned as float32 (N, K): column n is contiguous, so the
    buffer is the column-major K x N matrix with leading dimension K."""
    return rng_for(*key, ROLE_X).standard_normal((N, K), dtype=np.float32)


def layer_key(config: int, layer: int, matrix: int, extra: int = 0):
    return (config, layer, matrix, extra)


def q4k_bytes(M: int, K: int) -> int:
    return M * (K // Q4K_BLOCK_WEIGHTS) * Q4K_BLOCK_BYTES


def q8_0_bytes(M: int, K: int) -> int:
    return M * (K // Q8_0_BLOCK_WEIGHTS) * Q8_0_BLOCK_BYTES
