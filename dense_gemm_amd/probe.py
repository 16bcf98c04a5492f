"""Python binding of libdense_gemm_probe.so, the control probes of the
measurements (include/dense_gemm_probe.h): argument marshalling only."""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (torch's HIP runtime is the one the probe library binds to)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdense_gemm_probe.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python dense_gemm_amd/build.py`")

DGP_MFMA_F32, DGP_MFMA_F16, DGP_MFMA_F16_RANDOM = 0, 1, 2
DGP_SLAB_LOADS, DGP_SLAB_MFMA, DGP_SLAB_READS, DGP_SLAB_DEPTH1, DGP_SLAB_PANELS, DGP_SLAB_SWIZZLE = 1, 2, 4, 8, 16, 32

_lib = ctypes.CDLL(LIB_PATH)
_i64, _i32, _vp, _ci = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int
_lib.dgp_mfma_peak.argtypes = [_ci, _i64, _i32, _vp, _vp, _vp]
_lib.dgp_mfma_peak.restype = _ci
_lib.dgp_mfma_flops.argtypes = [_ci, _i64, _i32]
_lib.dgp_mfma_flops.restype = ctypes.c_double
_lib.dgp_copy.argtypes = [_vp, _vp, _i64, _vp]
_lib.dgp_copy.restype = _ci
_lib.dgp_slab_probe.argtypes = [_ci, _i64, _i32, _i32, _i32, _vp, _i64, _vp, _vp, _vp]
_lib.dgp_slab_probe.restype = _ci
_lib.dgp_wall_clock_khz.argtypes = []
_lib.dgp_wall_clock_khz.restype = _ci
_lib.dgp_last_hip_error.argtypes = []
_lib.dgp_last_hip_error.restype = _ci

EXPORTED = ["dgp_mfma_peak", "dgp_mfma_flops", "dgp_copy", "dgp_slab_probe", "dgp_wall_clock_khz",
            "dgp_last_hip_error"]


def dgp_mfma_peak(kind, workgroups, iters, sink, clocks, stream):
    return _lib.dgp_mfma_peak(kind, workgroups, iters, sink, clocks, stream)


def dgp_mfma_flops(kind, workgroups, iters):
    return _lib.dgp_mfma_flops(kind, workgroups, iters)


def dgp_copy(src, dst, nbytes, stream):
    return _lib.dgp_copy(src, dst, nbytes, stream)


def dgp_slab_probe(mode, workgroups, iters, windows, pitch, src, src_bytes, sink, clocks, stream):
    return _lib.dgp_slab_probe(mode, workgroups, iters, windows, pitch, src, src_bytes, sink, clocks, stream)


def dgp_wall_clock_khz():
    return _lib.dgp_wall_clock_khz()


def dgp_last_hip_error():
    return _lib.dgp_last_hip_error()
