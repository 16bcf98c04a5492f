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
DG_F32, DG_F16_F32ACC, DG_BF16_F32ACC, DG_F16_F32OUT, DG_BF16_F32OUT = 0, 1, 2, 3, 4
DG_EPI_NONE, DG_EPI_RELU, DG_EPI_GELU = 0, 1, 2
EPILOGUES = {"none": DG_EPI_NONE, "relu": DG_EPI_RELU, "gelu": DG_EPI_GELU}
DG_OK, DG_ERR_UNSUPPORTED, DG_ERR_SCRATCH, DG_ERR_HIP = 0, -100, -101, -200
DG_SCRATCH_BYTES = 16 * 1024 * 1024
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
_EX_ARGS = [_ci, _ci, _i64, _i64, _i64, _f32, _vp, _i64, _i64, _vp, _i64, _i64, _f32, _vp, _i64,
            _i64, _i64, _vp, _ci, _ci, _vp]
_lib.dg_gemm_ex.argtypes = _EX_ARGS
_lib.dg_gemm_ex.restype = _ci
_lib.dg_gemm_ex_with_kernel.argtypes = _EX_ARGS + [_ci]
_lib.dg_gemm_ex_with_kernel.restype = _ci
_lib.dg_gemm_splitk.argtypes = _GEMM_ARGS + [_ci, _vp, ctypes.c_size_t]
_lib.dg_gemm_splitk.restype = _ci
_lib.dg_gemm_splitk_noalloc.argtypes = _GEMM_ARGS + [_ci]
_lib.dg_gemm_splitk_noalloc.restype = _ci
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

EXPORTED = ["dg_gemm", "dg_gemm_with_kernel", "dg_gemm_ex", "dg_gemm_ex_with_kernel", "dg_gemm_splitk",
            "dg_gemm_splitk_noalloc", "dg_gemm_splitk_choose",
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


def dg_gemm_ex(transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
               strideC, batch, bias, epilogue, dtype, stream) -> int:
    return _lib.dg_gemm_ex(int(transA), int(transB), M, N, K, alpha, A, lda, strideA, B, ldb,
                           strideB, beta, C, ldc, strideC, batch, bias, int(epilogue), int(dtype),
                           stream)


def dg_gemm_ex_with_kernel(transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta,
                           C, ldc, strideC, batch, bias, epilogue, dtype, stream, kernel) -> int:
    return _lib.dg_gemm_ex_with_kernel(int(transA), int(transB), M, N, K, alpha, A, lda, strideA, B,
                                       ldb, strideB, beta, C, ldc, strideC, batch, bias,
                                       int(epilogue), int(dtype), stream, int(kernel))


def dg_gemm_splitk(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, stream,
                   splits, workspace, workspace_bytes) -> int:
    return _lib.dg_gemm_splitk(int(transA), int(transB), M, N, K, alpha, A, lda, B, ldb, beta, C,
                               ldc, int(dtype), stream, int(splits), workspace, int(workspace_bytes))


def dg_gemm_splitk_noalloc(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype,
                           stream, splits) -> int:
    return _lib.dg_gemm_splitk_noalloc(int(transA), int(transB), M, N, K, alpha, A, lda, B, ldb,
                                       beta, C, ldc, int(dtype), stream, int(splits))


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
def _dtype_code(ab, c):
    """The library's dtype for operands of torch dtype `ab` and an output of
    torch dtype `c`: the operand type itself, or fp32 for 16-bit operands."""
    import torch
    codes = {(torch.float32, torch.float32): DG_F32,
             (torch.float16, torch.float16): DG_F16_F32ACC,
             (torch.bfloat16, torch.bfloat16): DG_BF16_F32ACC,
             (torch.float16, torch.float32): DG_F16_F32OUT,
             (torch.bfloat16, torch.float32): DG_BF16_F32OUT}
    if (ab, c) not in codes:
        raise TypeError(f"unsupported operand/output dtypes {ab}/{c} (float32, float16 or "
                        "bfloat16 operands; an output of the operand dtype, or float32)")
    return codes[(ab, c)]


def _ld(t, name):
    if t.stride(-1) != 1 and t.shape[-1] > 1:
        raise ValueError(f"{name} must have unit column stride (row-major rows)")
    return max(t.stride(-2), t.shape[-1], 1)


def _batch_stride(t, batch, name):
    """Element stride between the matrices of a 3-D operand (0 for a 2-D one,
    which every batch then shares)."""
    if t.dim() == 2:
        return 0
    if t.dim() != 3 or t.shape[0] != batch:
        raise ValueError(f"{name} must be 2-D or [{batch}, rows, cols]")
    return t.stride(0) if batch > 1 else 0


def gemm(A, B, C=None, transA=False, transB=False, alpha=1.0, beta=0.0, bias=None,
         activation="none", kernel=DG_KERNEL_AUTO, stream=None, out_dtype=None):
    """C = act(alpha * op(A) @ op(B) + beta * C + bias) on torch CUDA (HIP)
    tensors, for one matrix or a strided batch.

    A is [M, K] (or [K, M] with transA), B is [K, N] (or [N, K] with transB);
    either may carry a leading batch dimension (a 2-D operand is shared by
    every batch); all row-major with unit column stride, ld from the row
    stride.  A and B share one dtype; C has that dtype or, for 16-bit
    operands, float32 (`out_dtype` picks it when C is allocated here).  bias
    (optional) has N elements of C's dtype; activation is "none", "relu" or
    "gelu".  C is allocated (uninitialised, so beta must be 0) when None.
    Runs on the current torch stream unless `stream` (a torch stream) is
    given."""
    import torch
    if B.dtype != A.dtype:
        raise TypeError("A and B must share one dtype")
    cdt = C.dtype if C is not None else (out_dtype if out_dtype is not None else A.dtype)
    dt = _dtype_code(A.dtype, cdt)
    if bias is not None and (bias.dtype != cdt or bias.dim() != 1 or bias.stride(0) != 1):
        raise TypeError("bias must be a contiguous 1-D tensor of C's dtype")
    batched = A.dim() == 3 or B.dim() == 3 or (C is not None and C.dim() == 3)
    batch = max(A.shape[0] if A.dim() == 3 else 1, B.shape[0] if B.dim() == 3 else 1,
                C.shape[0] if (C is not None and C.dim() == 3) else 1)
    M, K = (A.shape[-1], A.shape[-2]) if transA else (A.shape[-2], A.shape[-1])
    Kb, N = (B.shape[-1], B.shape[-2]) if transB else (B.shape[-2], B.shape[-1])
    if Kb != K:
        raise ValueError(f"inner dimensions differ: {K} vs {Kb}")
    if bias is not None and bias.shape[0] != N:
        raise ValueError(f"bias must have {N} elements")
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
        C = torch.empty((batch, M, N) if batched else (M, N), dtype=cdt, device=A.device)
    if tuple(C.shape[-2:]) != (M, N) or (batched and (C.dim() != 3 or C.shape[0] != batch)):
        raise ValueError(f"C must be [{batch}, {M}, {N}]" if batched else f"C must be [{M}, {N}]")
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    sa, sb = _batch_stride(A, batch, "A"), _batch_stride(B, batch, "B")
    sc = C.stride(0) if (batched and batch > 1) else 0
    rc = dg_gemm_ex_with_kernel(transA, transB, M, N, K, float(alpha), A.data_ptr(), _ld(A, "A"),
                                sa, B.data_ptr(), _ld(B, "B"), sb, float(beta), C.data_ptr(),
                                _ld(C, "C"), sc, batch, bias.data_ptr() if bias is not None else None,
                                EPILOGUES[activation], dt, s.cuda_stream, kernel)
    if rc != DG_OK:
        raise GemmError(rc)
    return C
