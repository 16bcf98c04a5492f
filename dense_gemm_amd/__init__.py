"""Python binding of libdense_gemm_amd.so (MI355X / gfx950 dense GEMM).

The functions named like the C ABI (include/dense_gemm.h) only marshal
arguments: every step of the computation runs in the library's HIP kernels.
`gemm()` is a convenience over torch tensors (torch is used for device memory
and streams only).

The library must have been built (python dense_gemm_amd/build.py); importing
this package fails loudly when it is missing.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdense_gemm_amd.so")

DG_OP_N, DG_OP_T = 0, 1
DG_F32, DG_F16_F32ACC = 0, 1
DG_OK, DG_ERR_UNSUPPORTED, DG_ERR_HIP = 0, -100, -200
DG_KERNEL_AUTO = -1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python dense_gemm_amd/build.py`")

# torch (the owner of the device memory and streams handed to the library)
# ships its own HIP runtime.  Load it first so the library's libamdhip64.so.7
# dependency resolves to that same runtime: a second HIP/HSA runtime in the
# process would not see the device (hipErrorNoDevice), and torch's stream
# handles are only meaningful to the runtime that created them.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)
_i64, _f32, _vp, _ci = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int
_GEMM_ARGS = [_ci, _ci, _i64, _i64, _i64, _f32, _vp, _i64, _vp, _i64, _f32, _vp, _i64, _ci, _vp]
_lib.dg_gemm.argtypes = _GEMM_ARGS
_lib.dg_gemm.restype = _ci
_lib.dg_gemm_with_kernel.argtypes = _GEMM_ARGS + [_ci]
_lib.dg_gemm_with_kernel.restype = _ci
_lib.dg_gemm_splitk.argtypes = _GEMM_ARGS + [_ci, _vp, ctypes.c_size_t]
_lib.dg_gemm_splitk.restype = _ci
_lib.dg_gemm_splitk_choose.argtypes = [_ci, _ci, _i64, _i64, _i64, _ci]
_lib.dg_gemm_splitk_choose.restype = _ci
_lib.dg_gemm_splitk_workspace_size.argtypes = [_i64, _i64, _ci]
_lib.dg_gemm_splitk_workspace_size.restype = ctypes.c_size_t
_lib.dg_select_kernel.argtypes = [_ci, _ci, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _ci]
_lib.dg_select_kernel.restype = _ci
_lib.dg_kernel_count.argtypes = []
_lib.dg_kernel_count.restype = _ci
_lib.dg_kernel_name.argtypes = [_ci]
_lib.dg_kernel_name.restype = ctypes.c_char_p
_lib.dg_kernel_tile_m.argtypes = [_ci]
_lib.dg_kernel_tile_m.restype = _ci
_lib.dg_kernel_tile_n.argtypes = [_ci]
_lib.dg_kernel_tile_n.restype = _ci
_lib.dg_status_string.argtypes = [_ci]
_lib.dg_status_string.restype = ctypes.c_char_p
_lib.dg_last_hip_error.argtypes = []
_lib.dg_last_hip_error.restype = _ci
_lib.dg_version.argtypes = []
_lib.dg_version.restype = _ci

EXPORTED = ["dg_gemm", "dg_gemm_with_kernel", "dg_gemm_splitk", "dg_gemm_splitk_choose",
            "dg_gemm_splitk_workspace_size", "dg_select_kernel", "dg_kernel_count",
            "dg_kernel_name", "dg_kernel_tile_m", "dg_kernel_tile_n", "dg_status_string",
            "dg_last_hip_error", "dg_version"]


def hip_error_name(code: int) -> str:
    """Name of a hipError_t, from the HIP runtime the library is linked to."""
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipGetErrorName.restype = ctypes.c_char_p
        hip.hipGetErrorName.argtypes = [ctypes.c_int]
        return hip.hipGetErrorName(int(code)).decode()
    except OSError:
        return "?"


class GemmError(RuntimeError):
    def __init__(self, status: int):
        msg = dg_status_string(status)
        if status == DG_ERR_HIP:
            e = dg_last_hip_error()
            msg += f" (hipError_t {e} {hip_error_name(e)})"
        super().__init__(f"dg_gemm failed: {status} ({msg})")
        self.status = status


# ---- the C ABI, one to one ------------------------------------------------
def dg_gemm(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, stream) -> int:
    return _lib.dg_gemm(int(transA), int(transB), M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                        int(dtype), stream)


def dg_gemm_with_kernel(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype,
                        stream, kernel) -> int:
    return _lib.dg_gemm_with_kernel(int(transA), int(transB), M, N, K, alpha, A, lda, B, ldb, beta,
                                    C, ldc, int(dtype), stream, int(kernel))


def dg_gemm_splitk(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, stream,
                   splits, workspace, workspace_bytes) -> int:
    return _lib.dg_gemm_splitk(int(transA), int(transB), M, N, K, alpha, A, lda, B, ldb, beta, C,
                               ldc, int(dtype), stream, int(splits), workspace, int(workspace_bytes))


def dg_gemm_splitk_choose(transA, transB, M, N, K, dtype) -> int:
    return _lib.dg_gemm_splitk_choose(int(transA), int(transB), M, N, K, int(dtype))


def dg_gemm_splitk_workspace_size(M, N, splits) -> int:
    return _lib.dg_gemm_splitk_workspace_size(M, N, int(splits))


def dg_select_kernel(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, dtype) -> int:
    return _lib.dg_select_kernel(int(transA), int(transB), M, N, K, A, lda, B, ldb, C, ldc,
                                 int(dtype))


def dg_kernel_count() -> int:
    return _lib.dg_kernel_count()


def dg_kernel_name(kernel: int):
    n = _lib.dg_kernel_name(int(kernel))
    return None if n is None else n.decode()


def dg_kernel_tile_m(kernel: int) -> int:
    return _lib.dg_kernel_tile_m(int(kernel))


def dg_kernel_tile_n(kernel: int) -> int:
    return _lib.dg_kernel_tile_n(int(kernel))


def dg_status_string(status: int) -> str:
    return _lib.dg_status_string(int(status)).decode()


def dg_last_hip_error() -> int:
    return _lib.dg_last_hip_error()


def dg_version() -> int:
    return _lib.dg_version()


def kernel_names() -> list[str]:
    return [dg_kernel_name(i) for i in range(dg_kernel_count())]


# ---- torch convenience -------------------------------------------------------
def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return DG_F32
    if t.dtype == torch.float16:
        return DG_F16_F32ACC
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or float16)")


def _ld(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError(f"{name} must have unit column stride (row-major rows)")
    return max(t.stride(0), t.shape[1], 1)


def gemm(A, B, C=None, transA=False, transB=False, alpha=1.0, beta=0.0, kernel=DG_KERNEL_AUTO,
         stream=None):
    """C = alpha * op(A) @ op(B) + beta * C on torch CUDA (HIP) tensors.

    A is [M, K] (or [K, M] with transA), B is [K, N] (or [N, K] with transB);
    all row-major with unit column stride; ld comes from stride(0).  C is
    allocated (uninitialised, so beta must be 0) when None.  Runs on the
    current torch stream unless `stream` (a torch stream) is given."""
    import torch
    dt = _dtype_code(A)
    if B.dtype != A.dtype or (C is not None and C.dtype != A.dtype):
        raise TypeError("A, B and C must share one dtype")
    M, K = (A.shape[1], A.shape[0]) if transA else (A.shape[0], A.shape[1])
    Kb, N = (B.shape[1], B.shape[0]) if transB else (B.shape[0], B.shape[1])
    if Kb != K:
        raise ValueError(f"inner dimensions differ: {K} vs {Kb}")
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
        C = torch.empty((M, N), dtype=A.dtype, device=A.device)
    if tuple(C.shape) != (M, N):
        raise ValueError(f"C must be [{M}, {N}]")
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    rc = dg_gemm_with_kernel(transA, transB, M, N, K, float(alpha), A.data_ptr(), _ld(A, "A"),
                             B.data_ptr(), _ld(B, "B"), float(beta), C.data_ptr(), _ld(C, "C"), dt,
                             s.cuda_stream, kernel)
    if rc != DG_OK:
        raise GemmError(rc)
    return C
