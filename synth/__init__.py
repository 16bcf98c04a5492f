"""Seeded synthetic inputs for the GEMM workloads.

This module draws random numbers and lays logical matrices out in memory.  It
holds none of the GEMM arithmetic: both the CPU oracle's tests and the GPU
path's tests/bench take their inputs from here, and nothing here computes a
product.

Generator (counter based, version independent, no numpy RNG involved):
  * SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): word i of stream `seed` is
    mix64(seed + (i + 1) * 0x9E3779B97F4A7C15 mod 2^64).
  * uniform u in [0, 1): the top 53 bits of the word times 2^-53.
  * uniform[-1, 1): 2u - 1.
  * standard normal: Box-Muller on the word pair (2i, 2i+1):
    sqrt(-2 ln(1 - u0)) * cos(2 pi u1).

Stream order for one problem: the logical op(A) (M x K, row-major), then the
logical op(B) (K x N), then C0 (M x N), each continuing the word counter of
the previous one, so every transpose variant of a shape sees the same logical
operands.

Rounding: values are drawn in fp64, then rounded once (IEEE round to nearest
even) to the storage type (fp32, fp16 or bf16).  numpy has no bf16 type, so
bf16 matrices are held as their 16-bit patterns (uint16): the upper half of
the fp32 encoding, 8 significant bits.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Words start .. start+count-1 of the SplitMix64 stream of `seed` (uint64)."""
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform01(seed: int, start: int, count: int) -> np.ndarray:
    """fp64 uniforms in [0, 1) from the top 53 bits of each word."""
    w = splitmix64(seed, start, count)
    return (w >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


class Stream:
    """A cursor over one seed's word stream."""

    def __init__(self, seed: int):
        self.seed = int(seed)
        self.pos = 0

    def uniform(self, shape, lo=-1.0, hi=1.0) -> np.ndarray:
        n = int(np.prod(shape))
        u = uniform01(self.seed, self.pos, n)
        self.pos += n
        return (lo + (hi - lo) * u).reshape(shape)

    def normal(self, shape, std=1.0) -> np.ndarray:
        n = int(np.prod(shape))
        u = uniform01(self.seed, self.pos, 2 * n)
        self.pos += 2 * n
        u0, u1 = u[0::2], u[1::2]
        z = np.sqrt(-2.0 * np.log1p(-u0)) * np.cos(2.0 * np.pi * u1)
        return (std * z).reshape(shape)

    def integers(self, shape, lo: int, hi: int) -> np.ndarray:
        """Integers in [lo, hi] (inclusive) as fp64, for exact-arithmetic cases."""
        n = int(np.prod(shape))
        u = uniform01(self.seed, self.pos, n)
        self.pos += n
        return (lo + np.floor(u * (hi - lo + 1))).reshape(shape)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit patterns with one round-to-nearest-even.

    bf16 keeps 8 significant bits over fp32's exponent range: the quantum of
    a value in [2^(e-1), 2^e) is 2^(e-8), and 2^-133 below 2^-126
    (subnormals).  The significand in units of the quantum is rounded half to
    even (np.rint); the rounded value is then exactly an fp32 number whose low
    16 bits are zero (or an infinity past the largest finite bf16)."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)
    q = np.maximum(e - 8, -133)
    v = np.ldexp(np.rint(np.ldexp(ax, -q)), q)
    with np.errstate(over="ignore", invalid="ignore"):
        f = np.where(np.signbit(x), -v, v).astype(np.float32)
    bits = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """One IEEE round-to-nearest-even from fp64 to the storage type (bf16 as
    uint16 bit patterns)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float64).astype(np.float16)
    if dtype == "bf16":
        return _bf16_bits(x)
    raise ValueError(dtype)


BF16_NAN = np.uint16(0x7FC0)


def store(logical: np.ndarray, trans: bool, ld: int | None = None, pad_value=np.nan) -> tuple[np.ndarray, int]:
    """Lay a logical matrix out row-major as the library expects it.

    trans=False stores `logical` itself (rows x cols); trans=True stores its
    transpose.  The stored matrix gets row stride `ld` (defaults to its column
    count); padding columns are filled with `pad_value` (NaN canaries by
    default, so a kernel that reads them poisons its output).
    Returns (buffer with shape (stored_rows, ld), ld).
    """
    s = logical.T if trans else logical
    rows, cols = s.shape
    if ld is None:
        ld = cols
    if ld < cols:
        raise ValueError("ld below the stored column count")
    buf = np.empty((rows, ld), dtype=logical.dtype)
    if ld > cols:
        # bf16 bit patterns: the NaN canary is a bf16 quiet NaN
        buf[:, cols:] = BF16_NAN if logical.dtype == np.uint16 and pad_value is np.nan else pad_value
    buf[:, :cols] = s
    return buf, ld


# ---------------------------------------------------------------------------
# Workload recipes (shapes, distributions and seeds of the measured problems)
# ---------------------------------------------------------------------------

# Storage types of the operands and of C for each dtype name: the operand type
# itself, or (names ending in "o32") 16-bit operands with an fp32 C.
OPERAND_TYPE = {"f32": "f32", "f16": "f16", "bf16": "bf16", "f16o32": "f16", "bf16o32": "bf16"}
OUTPUT_TYPE = {"f32": "f32", "f16": "f16", "bf16": "bf16", "f16o32": "f32", "bf16o32": "f32"}


def problem(M: int, N: int, K: int, dtype: str, dist: str, seed: int, with_c0: bool = False,
            std: float = 1.0):
    """Logical op(A) [M,K], op(B) [K,N] rounded to the operand type of
    `dtype`, and optional C0 [M,N] rounded to its output type (the draws are
    the same for every dtype name, so "f16" and "f16o32" share operands).

    dist: "uniform" (iid uniform[-1,1)), "normal_sqrtk" (iid N(0,1)/sqrt(K)),
          "normal" (iid N(0, std^2)), "int2" (integers in [-2, 2]).
    """
    st = Stream(seed)

    def draw(shape):
        if dist == "uniform":
            return st.uniform(shape)
        if dist == "normal_sqrtk":
            return st.normal(shape) / np.sqrt(K)
        if dist == "normal":
            return st.normal(shape, std)
        if dist == "int2":
            return st.integers(shape, -2, 2)
        raise ValueError(dist)

    a = round_to(draw((M, K)), OPERAND_TYPE[dtype])
    b = round_to(draw((K, N)), OPERAND_TYPE[dtype])
    c0 = round_to(draw((M, N)), OUTPUT_TYPE[dtype]) if with_c0 else None
    return a, b, c0


# The LoRA MLP-block step over 512 tokens, d_model 2048, FFN 5632, rank 32:
# (name, M, N, K, transA, transB, beta, operand kinds) where the kinds say
# which operands are weights (N(0, 0.02)) and which are activations or
# gradients (N(0, 1)).
LORA_TOKENS, LORA_DMODEL, LORA_FFN, LORA_RANK = 512, 2048, 5632, 32
LORA_GEMMS = [
    # forward
    ("gate = X Wg^T",        512, 5632, 2048, False, True, 0.0, ("a", "w")),
    ("up = X Wu^T",          512, 5632, 2048, False, True, 0.0, ("a", "w")),
    ("down = S Wd^T",        512, 2048, 5632, False, True, 0.0, ("a", "w")),
    ("Tg = X Ag^T",          512, 32, 2048, False, True, 0.0, ("a", "w")),
    ("Tu = X Au^T",          512, 32, 2048, False, True, 0.0, ("a", "w")),
    ("gate += Tg Bg^T",      512, 5632, 32, False, True, 1.0, ("a", "w")),
    ("up += Tu Bu^T",        512, 5632, 32, False, True, 1.0, ("a", "w")),
    # backward
    ("dS = dY Wd",           512, 5632, 2048, False, False, 0.0, ("a", "w")),
    ("dH += dG Wg",          512, 2048, 5632, False, False, 1.0, ("a", "w")),
    ("dH += dU Wu",          512, 2048, 5632, False, False, 1.0, ("a", "w")),
    ("dGa = dG Bg",          512, 32, 5632, False, False, 0.0, ("a", "w")),
    ("dUa = dU Bu",          512, 32, 5632, False, False, 0.0, ("a", "w")),
    ("dBg = dG^T Tg",        5632, 32, 512, True, False, 0.0, ("a", "a")),
    ("dBu = dU^T Tu",        5632, 32, 512, True, False, 0.0, ("a", "a")),
    ("dAg = dGa^T X",        32, 2048, 512, True, False, 0.0, ("a", "a")),
    ("dAu = dUa^T X",        32, 2048, 512, True, False, 0.0, ("a", "a")),
    ("dX += dGa Ag",         512, 2048, 32, False, False, 1.0, ("a", "w")),
    ("dX += dUa Au",         512, 2048, 32, False, False, 1.0, ("a", "w")),
]


# The products of the step that come in pairs of one shape with separate
# outputs, by index into LORA_GEMMS: gate/up, the two rank-32 "+=" updates,
# dBg/dBu, dAg/dAu.  One strided-batch launch can run each pair (the two
# "dH +=" and "dX +=" products write one output per pair, so they cannot).
LORA_PAIRS = ((0, 1), (5, 6), (12, 13), (14, 15))


def lora_problem(index: int, seed: int = 3, out: str = "f16"):
    """Logical fp16 operands of one LoRA-step GEMM (and C0 when beta != 0,
    rounded to `out`, the type of C: "f16", or "f32" for the fp32-output
    form of the step).

    Each GEMM draws from its own stream (seed, then the GEMM's index in the
    list mixed into the seed), weights iid N(0, 0.02), activations and
    gradients iid N(0, 1).
    """
    name, M, N, K, ta, tb, beta, kinds = LORA_GEMMS[index]
    st = Stream((seed << 8) | index)
    std = {"w": 0.02, "a": 1.0}
    a = round_to(st.normal((M, K), std[kinds[0]]), "f16")
    b = round_to(st.normal((K, N), std[kinds[1]]), "f16")
    c0 = round_to(st.normal((M, N), 1.0), out) if beta != 0.0 else None
    return a, b, c0
