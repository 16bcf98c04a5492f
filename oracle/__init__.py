"""Python access to the CPU oracle (oracle_gemm.c).

TEST INFRASTRUCTURE ONLY: the plain fp64 reference that the GPU library is
checked against.  Only the test suite, the smoke check and the CPU-baseline leg
of the benchmark may import this package; the GPU library never does, and this
package imports nothing from it.

`build()` compiles oracle_gemm.c with gcc (no HIP, no BLAS, no fast-math, no
FMA contraction) into liboracle.so next to this file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

# element types of the C oracle; bf16 matrices are held as uint16 bit patterns
_TYPE = {np.dtype(np.float32): 0, np.dtype(np.float16): 1, np.dtype(np.float64): 2,
         np.dtype(np.uint16): 3}

ACT = {"none": 0, "relu": 1, "gelu": 2}


def build(force: bool = True) -> str:
    """Compile the oracle.  Called by the project's build step."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-pthread", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def bind(path: str):
    """Load an oracle shared library and declare its entry points."""
    lib = ctypes.CDLL(path)
    i64, dbl, vp, ci = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
    lib.oracle_gemm.argtypes = [ci, ci, i64, i64, i64, dbl, vp, i64, ci, vp, i64, ci,
                                dbl, vp, i64, ci, vp, vp, ci]
    lib.oracle_gemm.restype = ci
    lib.oracle_gemm_points.argtypes = [ci, ci, i64, i64, i64, dbl, vp, i64, ci, vp, i64, ci,
                                       dbl, vp, i64, ci, i64, vp, vp, vp, vp, ci]
    lib.oracle_gemm_points.restype = ci
    lib.oracle_gemm_ex.argtypes = [ci, ci, i64, i64, i64, dbl, vp, i64, i64, ci, vp, i64, i64, ci,
                                   dbl, vp, i64, i64, ci, vp, ci, ci, i64, vp, vp, vp, ci]
    lib.oracle_gemm_ex.restype = ci
    lib.oracle_gemm_points_ex.argtypes = [ci, ci, i64, i64, i64, dbl, vp, i64, i64, ci, vp, i64,
                                          i64, ci, dbl, vp, i64, i64, ci, vp, ci, ci, i64, vp, vp,
                                          vp, vp, vp, vp, ci]
    lib.oracle_gemm_points_ex.restype = ci
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = dbl
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = dbl
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = bind(_LIB)
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def default_threads() -> int:
    """Threads for a call that asks for none: the cores this process may run
    on, capped by OMP_NUM_THREADS when it is set (a container's CPU share can
    be far below the host's core count)."""
    n = len(os.sched_getaffinity(0))
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return min(n, cap) if cap > 0 else n


def _threads(n: int) -> int:
    return int(n) if n and n > 0 else default_threads()


def _check(a, name):
    if a is None:
        return
    if a.dtype not in _TYPE:
        raise TypeError(f"{name}: unsupported dtype {a.dtype}")
    if not a.flags.c_contiguous:
        raise ValueError(f"{name} must be C-contiguous (row stride is passed as ld)")


def gemm(transA: bool, transB: bool, M: int, N: int, K: int, alpha: float, A: np.ndarray, lda: int,
         B: np.ndarray, ldb: int, beta: float, C0: np.ndarray | None, ldc: int,
         nthreads: int = 0, want_abs: bool = True):
    """Full oracle result.  A, B, C0 are the *stored* buffers (fp32, fp16 or
    fp64, C-contiguous, row stride lda/ldb/ldc).  Returns (ref, absum) as fp64
    M x N arrays (absum is None when want_abs is False)."""
    lib = _load()
    for a, n in ((A, "A"), (B, "B"), (C0, "C0")):
        _check(a, n)
    ref = np.empty((M, N), dtype=np.float64)
    absum = np.empty((M, N), dtype=np.float64) if want_abs else None
    tc = _TYPE[C0.dtype] if C0 is not None else 2
    rc = lib.oracle_gemm(int(transA), int(transB), M, N, K, float(alpha), _ptr(A), lda,
                         _TYPE[A.dtype], _ptr(B), ldb, _TYPE[B.dtype], float(beta), _ptr(C0), ldc,
                         tc, ref.ctypes.data, _ptr(absum), _threads(nthreads))
    if rc < 0:
        raise RuntimeError(f"oracle_gemm failed ({rc})")
    return ref, absum


def gemm_points(transA: bool, transB: bool, M: int, N: int, K: int, alpha: float, A, lda, B, ldb,
                beta: float, C0, ldc, rows: np.ndarray, cols: np.ndarray, nthreads: int = 0):
    """Oracle value and absum at the elements (rows[p], cols[p])."""
    lib = _load()
    for a, n in ((A, "A"), (B, "B"), (C0, "C0")):
        _check(a, n)
    pi = np.ascontiguousarray(rows, dtype=np.int64)
    pj = np.ascontiguousarray(cols, dtype=np.int64)
    ref = np.empty(pi.shape[0], dtype=np.float64)
    absum = np.empty(pi.shape[0], dtype=np.float64)
    tc = _TYPE[C0.dtype] if C0 is not None else 2
    rc = lib.oracle_gemm_points(int(transA), int(transB), M, N, K, float(alpha), _ptr(A), lda,
                                _TYPE[A.dtype], _ptr(B), ldb, _TYPE[B.dtype], float(beta),
                                _ptr(C0), ldc, tc, pi.shape[0], pi.ctypes.data, pj.ctypes.data,
                                ref.ctypes.data, absum.ctypes.data, _threads(nthreads))
    if rc < 0:
        raise RuntimeError(f"oracle_gemm_points failed ({rc})")
    return ref, absum


def gemm_ex(transA: bool, transB: bool, M: int, N: int, K: int, alpha: float, A, lda: int,
            B, ldb: int, beta: float, C0, ldc: int, bias=None, act: str = "none", batch: int = 1,
            strideA: int = 0, strideB: int = 0, strideC: int = 0, nthreads: int = 0):
    """Oracle of act(alpha*op(A)op(B) + beta*C0 + bias) over a strided batch.
    A, B, C0 are flat or 2-D stored buffers holding every batch (batch b at
    element offset b*stride); bias has N elements.  bf16 buffers are uint16
    bit patterns.  Returns (ref, pre, absum), each batch x M x N fp64 (pre is
    the value before the activation)."""
    lib = _load()
    for a, n in ((A, "A"), (B, "B"), (C0, "C0"), (bias, "bias")):
        _check(a, n)
    ref = np.empty((batch, M, N), dtype=np.float64)
    pre = np.empty((batch, M, N), dtype=np.float64)
    absum = np.empty((batch, M, N), dtype=np.float64)
    tc = _TYPE[C0.dtype] if C0 is not None else 2
    tbias = _TYPE[bias.dtype] if bias is not None else 2
    rc = lib.oracle_gemm_ex(int(transA), int(transB), M, N, K, float(alpha), _ptr(A), lda,
                            strideA, _TYPE[A.dtype], _ptr(B), ldb, strideB, _TYPE[B.dtype],
                            float(beta), _ptr(C0), ldc, strideC, tc, _ptr(bias), tbias, ACT[act],
                            batch, ref.ctypes.data, pre.ctypes.data, absum.ctypes.data,
                            _threads(nthreads))
    if rc < 0:
        raise RuntimeError(f"oracle_gemm_ex failed ({rc})")
    return ref, pre, absum


def gemm_points_ex(transA: bool, transB: bool, M: int, N: int, K: int, alpha: float, A, lda, B,
                   ldb, beta: float, C0, ldc, batches, rows, cols, bias=None, act: str = "none",
                   strideA: int = 0, strideB: int = 0, strideC: int = 0, nthreads: int = 0):
    """Oracle (ref, pre, absum) at the elements (batches[p], rows[p], cols[p])."""
    lib = _load()
    for a, n in ((A, "A"), (B, "B"), (C0, "C0"), (bias, "bias")):
        _check(a, n)
    pb = np.ascontiguousarray(batches, dtype=np.int64)
    pi = np.ascontiguousarray(rows, dtype=np.int64)
    pj = np.ascontiguousarray(cols, dtype=np.int64)
    n = pi.shape[0]
    ref, pre, absum = (np.empty(n, dtype=np.float64) for _ in range(3))
    tc = _TYPE[C0.dtype] if C0 is not None else 2
    tbias = _TYPE[bias.dtype] if bias is not None else 2
    rc = lib.oracle_gemm_points_ex(int(transA), int(transB), M, N, K, float(alpha), _ptr(A), lda,
                                   strideA, _TYPE[A.dtype], _ptr(B), ldb, strideB, _TYPE[B.dtype],
                                   float(beta), _ptr(C0), ldc, strideC, tc, _ptr(bias), tbias,
                                   ACT[act], n, pb.ctypes.data, pi.ctypes.data, pj.ctypes.data,
                                   ref.ctypes.data, pre.ctypes.data, absum.ctypes.data,
                                   _threads(nthreads))
    if rc < 0:
        raise RuntimeError(f"oracle_gemm_points_ex failed ({rc})")
    return ref, pre, absum


def f16_to_f64(bits: int) -> float:
    return _load().oracle_f16_to_f64(bits)


def bf16_to_f64(bits: int) -> float:
    return _load().oracle_bf16_to_f64(bits)


def values(buf) -> np.ndarray:
    """fp64 values of a stored buffer (bf16 given as uint16 bit patterns): the
    magnitudes the error bound needs (|beta * C0|, |bias|).  bf16 is the upper
    half of an fp32 encoding, so its value is that fp32 number."""
    buf = np.asarray(buf)
    if buf.dtype == np.uint16:
        return (buf.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return buf.astype(np.float64)


# ---------------------------------------------------------------------------
# Error bound of the comparison
# ---------------------------------------------------------------------------
# Output types.  "f32": fp32 operands and output.  "f16" / "bf16": 16-bit
# operands, fp32 sums, 16-bit output.  "f16o32" / "bf16o32": 16-bit operands,
# fp32 sums, fp32 output (no 16-bit rounding at the end).
#
# fp32 and fp16-in/fp32-acc take the stated bounds; bf16 operands also
# multiply exactly in fp32 (8 x 8 significant bits) and accumulate in fp32, so
# they take the fp16 path's bound, with the output rounding of bf16.  An fp32
# output of 16-bit operands has the same sums, so the same rtol and atol,
# without the 16-bit output rounding.
RTOL = {"f32": 2e-5, "f16": 2e-3, "bf16": 2e-3, "f16o32": 2e-3, "bf16o32": 2e-3}
ATOL = {"f32": 1e-6, "f16": 1e-4, "bf16": 1e-4, "f16o32": 1e-4, "bf16o32": 1e-4}
# the storage type of C for each output type
OUT_TYPE = {"f32": "f32", "f16": "f16", "bf16": "bf16", "f16o32": "f32", "bf16o32": "f32"}
# largest slope of gelu(x) = x Phi(x): at x = sqrt(2), Phi(sqrt 2) + sqrt(2) phi(sqrt 2)
GELU_LIPSCHITZ = 1.129
# fp32 evaluation of gelu: erf to a few ulp of 1, times |x|/2
GELU_ABS = 1e-6

F16_MAX = 65504.0                  # (2 - 2^-10) * 2^15
BF16_MAX = 3.3895313892515355e38   # (2 - 2^-7) * 2^127
F32_MAX = 3.4028234663852886e38    # (2 - 2^-23) * 2^127
# Round-to-nearest-even gives an infinity from these magnitudes on: the
# largest finite value plus half the spacing of its binade (the tie rounds
# to the even neighbour, which is the infinity, since the largest finite
# value has an odd last significand bit).
OVERFLOW = {"f16": F16_MAX + 2.0 ** 4, "bf16": BF16_MAX + 2.0 ** 119, "f32": F32_MAX + 2.0 ** 103}
# half the spacing in the top finite binade: the largest rounding error of a
# value that rounds to a finite number
TOP_HALF_ULP = {"f16": 2.0 ** 4, "bf16": 2.0 ** 119, "f32": 2.0 ** 103}


def _half_ulp(x, mant_bits, emin):
    """Half the spacing of a binary format with `mant_bits` fraction bits and
    smallest normal exponent `emin`, in the binade that holds |x|: 2^(e-1-p)
    for |x| in [2^e, 2^(e+1)), e >= emin; the subnormal spacing's half below
    2^emin.  The rounding of any |x| in that binade moves it by at most this."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(ax)                       # ax = f * 2^e, f in [0.5, 1): binade 2^(e-1)
    return np.ldexp(1.0, np.maximum(e - 1, emin) - mant_bits - 1)


def half_ulp_f16(x: np.ndarray) -> np.ndarray:
    """Half the spacing of fp16 numbers in the binade of |x| (2^(e-11) for
    |x| in [2^e, 2^(e+1)), 2^-25 among subnormals); infinite from the
    overflow threshold 65520 on, where the output is an infinity."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    return np.where(ax >= OVERFLOW["f16"], np.inf, _half_ulp(ax, 10, -14))


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 numbers in the binade of |x|: 2^(e-8) for
    |x| in [2^e, 2^(e+1)), 2^-134 among subnormals; infinite past the
    overflow threshold (the output is then an infinity)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    return np.where(ax >= OVERFLOW["bf16"], np.inf, _half_ulp(ax, 7, -126))


def half_ulp_out(dtype: str, x) -> np.ndarray:
    """The output rounding allowed at magnitude |x|: half a 16-bit ulp for
    16-bit outputs; nothing for fp32 outputs (their rounding is part of the
    fp32 sums the rtol covers).  Infinite from the output type's overflow
    threshold on."""
    out = OUT_TYPE[dtype]
    ax = np.abs(np.asarray(x, dtype=np.float64))
    if out == "f16":
        return half_ulp_f16(ax)
    if out == "bf16":
        return half_ulp_bf16(ax)
    return np.where(ax >= OVERFLOW["f32"], np.inf, 0.0)


def bound_pre(dtype: str, absum, alpha: float, beta: float, c0_logical=None, bias_logical=None,
              act: str = "none", pre=None) -> np.ndarray:
    """The bound before the output rounding:
    rtol * (|alpha| * absum + |beta * C0| + |bias|) + atol, carried through
    the activation.

    The stated bound is rtol * sum_k |a_ik b_kj| + atol at alpha=1, beta=0;
    with general alpha and beta the sum is scaled by |alpha| and the C0 term
    |beta * C0| is added; a bias adds its magnitude the same way (one more
    fp32 addition).  An activation maps an input error e to at most L * e, L
    its largest slope (relu 1, gelu 1.129, rounded up); gelu's own fp32
    evaluation adds GELU_ABS * |x|."""
    extra = 0.0
    if beta != 0.0 and c0_logical is not None:
        extra = np.abs(beta * np.asarray(c0_logical, dtype=np.float64))
    if bias_logical is not None:
        extra = extra + np.abs(np.asarray(bias_logical, dtype=np.float64))
    b = RTOL[dtype] * (abs(alpha) * np.asarray(absum) + extra) + ATOL[dtype]
    if act == "gelu":
        b = GELU_LIPSCHITZ * b + GELU_ABS * np.abs(np.asarray(pre, dtype=np.float64))
    return b


def bound(dtype: str, ref, absum, alpha: float, beta: float, c0_logical=None, bias_logical=None,
          act: str = "none", pre=None) -> np.ndarray:
    """bound_pre plus the output rounding: half an ulp of a 16-bit output type
    in the binade of |ref| + bound_pre, the largest magnitude the unrounded
    result can have (so a result on the far side of a binade boundary is
    covered); infinite where that magnitude reaches the overflow threshold."""
    b = bound_pre(dtype, absum, alpha, beta, c0_logical, bias_logical, act, pre)
    reach = np.abs(np.asarray(ref, dtype=np.float64)) + b
    return b + half_ulp_out(dtype, reach)


def compare(dtype: str, got, ref, absum, alpha: float, beta: float, c0_logical=None,
            bias_logical=None, act: str = "none", pre=None):
    """Returns (max err/bound, number of violations).

    The unrounded result y lies within bound_pre of ref, and the output is y
    rounded to the output type.  So:
      - a finite output passes when |got - ref| <= bound_pre + h, h = half an
        output ulp in the binade of |ref| + bound_pre (for a reach at or past
        the overflow threshold, h is the top finite binade's half ulp: a
        finite output still came from a y below the threshold);
      - an infinite output passes only where |ref| + bound_pre reaches the
        threshold, with the sign of ref;
      - NaN never passes."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    b = bound_pre(dtype, absum, alpha, beta, c0_logical, bias_logical, act, pre)
    b = np.broadcast_to(b, np.broadcast_shapes(np.shape(b), ref.shape))
    reach = np.abs(ref) + b
    h = half_ulp_out(dtype, reach)
    can_overflow = np.isinf(h)
    h = np.where(can_overflow, TOP_HALF_ULP[OUT_TYPE[dtype]] if OUT_TYPE[dtype] != "f32" else 0.0, h)
    with np.errstate(invalid="ignore", over="ignore"):
        ratio = np.abs(got - ref) / (b + h)
        inf_ok = np.isinf(got) & can_overflow & (np.sign(got) == np.sign(ref))
        ratio = np.where(np.isinf(got), np.where(inf_ok, 0.0, np.inf), ratio)
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    bad = int(np.count_nonzero(ratio > 1.0))
    return (float(ratio.max()) if ratio.size else 0.0), bad
