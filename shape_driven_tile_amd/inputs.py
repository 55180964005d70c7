"""Seeded synthetic inputs for the fp16 GEMM and the M=1 decode GEMV.

This module is shared by the GPU path's tests/benchmark and by the CPU oracle's
tests.  It holds no arithmetic of the method: it only draws numbers and lays
them out in memory.  Every array is a host numpy array of float16; callers copy
it to the device themselves.

bfloat16 arrays are handed around as uint16 bit patterns (numpy has no
bfloat16 type): the fp64 draw is cast to float32 by numpy and then to
bfloat16 by torch, both rounding to nearest even.

Distributions (the pages state the shapes, not the generator):
  * square GEMM operands: uniform in [-1, 1], drawn in fp64 with numpy's PCG64
    ``default_rng(seed).uniform``, then cast to float16 (round to nearest even);
  * decode weights: normal with mean 0 and standard deviation 0.02, same cast;
  * exact-arithmetic suites: small integers drawn uniformly from [lo, hi].

Seeds: A operand 1000 + c, B operand 2000 + c (c = workload index), decode
activations 3000, rotating decode weight buffer r: 4000 + r.
"""
from __future__ import annotations

import numpy as np

SEED_A = 1000
SEED_B = 2000
SEED_X = 3000
SEED_W = 4000

# Square shapes of "Beating hipBLASLt on a Gaming GPU" (The result) carried to
# MI355X sizes, the K sweep of the FlyDSL pull request (Motivation), and the
# decode shape of the mojo-baro page (Four rounds on the decode shape).
SQUARE_SMALL = (256,)
SQUARE_SWEEP = (512, 768, 1024, 1536, 2048)
SQUARE_LARGE = (4096, 8192)
K_SWEEP_MN = 2048
K_SWEEP_K = (1920, 1984, 2048, 2112, 2176, 2304)
DECODE_N = 12288
DECODE_K = 4096
DECODE_BUFFERS = 8


def uniform_f16(shape, seed: int) -> np.ndarray:
    """float16 array, values uniform in [-1, 1] (fp64 draw, RNE cast)."""
    return np.random.default_rng(seed).uniform(-1.0, 1.0, size=shape).astype(np.float16)


def normal_f16(shape, seed: int, std: float = 0.02) -> np.ndarray:
    """float16 array, values N(0, std^2) (fp64 draw, RNE cast)."""
    return np.random.default_rng(seed).normal(0.0, std, size=shape).astype(np.float16)


def integer_f16(shape, seed: int, lo: int = -2, hi: int = 2) -> np.ndarray:
    """float16 array of integers drawn uniformly from [lo, hi] (exact in fp16)."""
    return np.random.default_rng(seed).integers(lo, hi + 1, size=shape).astype(np.float16)


def padded(a: np.ndarray, ld: int, fill: float = np.nan) -> np.ndarray:
    """Copy a 2-D float16 array into a (rows, ld) buffer whose columns past the
    original width hold ``fill`` (NaN by default, so a kernel that reads the
    padding poisons its output)."""
    rows, cols = a.shape
    if ld < cols:
        raise ValueError("ld smaller than the row length")
    out = np.full((rows, ld), fill, dtype=np.float16)
    out[:, :cols] = a
    return out


def square_operands(n: int, c: int, k: int | None = None):
    """(A [n x k], B [n x k]) for workload index c; B is stored K-contiguous."""
    k = n if k is None else k
    return uniform_f16((n, k), SEED_A + c), uniform_f16((n, k), SEED_B + c)


def decode_activations(k: int = DECODE_K) -> np.ndarray:
    return uniform_f16((k,), SEED_X)


def decode_weights(r: int, n: int = DECODE_N, k: int = DECODE_K) -> np.ndarray:
    """Rotating weight buffer r, stored as [n][k] (K contiguous per column)."""
    return normal_f16((n, k), SEED_W + r)


def decode_weights_kn(r: int, n: int = DECODE_N, k: int = DECODE_K) -> np.ndarray:
    """The same matrix as decode_weights(r), stored the other way round:
    K rows of N contiguous values (a layout change only)."""
    return np.ascontiguousarray(decode_weights(r, n, k).T)


# ---- bfloat16 (uint16 bit patterns) --------------------------------------------

BF16_NAN_BITS = 0x7FC0


def to_bf16_bits(a) -> np.ndarray:
    """Cast an array of draws to bfloat16 bit patterns (float32 by numpy, then
    bfloat16 by torch; both round to nearest even)."""
    import torch
    f32 = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    return torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def uniform_bf16(shape, seed: int) -> np.ndarray:
    """bfloat16 bits, values uniform in [-1, 1]."""
    return to_bf16_bits(np.random.default_rng(seed).uniform(-1.0, 1.0, size=shape))


def normal_bf16(shape, seed: int, std: float = 0.02) -> np.ndarray:
    return to_bf16_bits(np.random.default_rng(seed).normal(0.0, std, size=shape))


def integer_bf16(shape, seed: int, lo: int = -2, hi: int = 2) -> np.ndarray:
    """bfloat16 bits of integers drawn uniformly from [lo, hi] (exact)."""
    return to_bf16_bits(np.random.default_rng(seed).integers(lo, hi + 1, size=shape))


def padded_bits(a: np.ndarray, ld: int, fill_bits: int = BF16_NAN_BITS) -> np.ndarray:
    """Copy a 2-D uint16 bit array into (rows, ld) with `fill_bits` (a
    bfloat16 NaN by default) in the columns past the original width."""
    rows, cols = a.shape
    if ld < cols:
        raise ValueError("ld smaller than the row length")
    out = np.full((rows, ld), fill_bits, dtype=np.uint16)
    out[:, :cols] = a
    return out


def square_operands_bf16(n: int, c: int, k: int | None = None):
    k = n if k is None else k
    return uniform_bf16((n, k), SEED_A + c), uniform_bf16((n, k), SEED_B + c)


def decode_activations_bf16(k: int = DECODE_K) -> np.ndarray:
    return uniform_bf16((k,), SEED_X)


def decode_weights_bf16(r: int, n: int = DECODE_N, k: int = DECODE_K) -> np.ndarray:
    return normal_bf16((n, k), SEED_W + r)
