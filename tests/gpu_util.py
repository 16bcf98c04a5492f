"""Helpers for the GPU parity tests: lay operands out (with NaN canaries in
the row padding), run the library through its C ABI on the current torch
stream, and compare with the CPU oracle."""
from __future__ import annotations

import numpy as np

import oracle
import synth

DTYPES = {"f32": 0, "f16": 1}


def torch_dtype(dtype):
    import torch
    return torch.float32 if dtype == "f32" else torch.float16


class Problem:
    """One GEMM: logical operands, their stored buffers, and the oracle."""

    def __init__(self, a, b, c0, ta, tb, alpha, beta, dtype, pad=(0, 0, 0)):
        self.a, self.b, self.c0 = a, b, c0
        self.ta, self.tb, self.alpha, self.beta, self.dtype = ta, tb, alpha, beta, dtype
        self.M, self.K = a.shape
        self.N = b.shape[1]
        M, N, K = self.M, self.N, self.K
        self.A, self.lda = synth.store(a, ta, (M if ta else K) + pad[0])
        self.B, self.ldb = synth.store(b, tb, (K if tb else N) + pad[1])
        self.ldc = N + pad[2]
        cinit = c0 if c0 is not None else np.full((M, N), np.nan, dtype=a.dtype)
        self.C0, _ = synth.store(cinit, False, self.ldc)

    def oracle_full(self):
        c0 = self.C0 if self.beta != 0.0 else None
        return oracle.gemm(self.ta, self.tb, self.M, self.N, self.K, self.alpha, self.A, self.lda,
                           self.B, self.ldb, self.beta, c0, self.ldc)

    def oracle_points(self, rows, cols):
        c0 = self.C0 if self.beta != 0.0 else None
        return oracle.gemm_points(self.ta, self.tb, self.M, self.N, self.K, self.alpha, self.A,
                                  self.lda, self.B, self.ldb, self.beta, c0, self.ldc, rows, cols)

    def run_gpu(self, kernel=-1, offset=(0, 0, 0), stream=None):
        """Runs on the GPU; returns the stored C (M x ldc) as a host array.
        `offset` shifts each buffer's start by that many elements (to test
        unaligned pointers)."""
        import torch

        import dense_gemm_amd as dg
        dev = torch.device("cuda:0")

        def up(x, off):
            flat = torch.empty(x.size + off + 8, dtype=torch_dtype(self.dtype), device=dev)
            flat.fill_(float("nan"))
            flat[off:off + x.size] = torch.from_numpy(np.ascontiguousarray(x).ravel()).to(dev)
            return flat, off

        At, oa = up(self.A, offset[0])
        Bt, ob = up(self.B, offset[1])
        Ct, oc = up(self.C0, offset[2])
        es = At.element_size()
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        rc = dg.dg_gemm_with_kernel(self.ta, self.tb, self.M, self.N, self.K, self.alpha,
                                    At.data_ptr() + oa * es, self.lda, Bt.data_ptr() + ob * es,
                                    self.ldb, self.beta, Ct.data_ptr() + oc * es, self.ldc,
                                    DTYPES[self.dtype], s.cuda_stream, kernel)
        if rc != 0:
            raise dg.GemmError(rc)
        s.synchronize()
        out = Ct[oc:oc + self.C0.size].cpu().numpy().reshape(self.C0.shape)
        # nothing outside the buffer view is touched
        assert torch.isnan(Ct[:oc]).all() and torch.isnan(Ct[oc + self.C0.size:]).all()
        return out

    def check_padding(self, out):
        if self.ldc > self.N:
            pad = out[:, self.N:]
            assert np.isnan(pad.astype(np.float64)).all(), "C padding was written"

    def logical_c0(self):
        return self.c0 if (self.beta != 0.0 and self.c0 is not None) else None


def check_full(p: Problem, kernel=-1, offset=(0, 0, 0), out=None):
    if out is None:
        out = p.run_gpu(kernel, offset)
    p.check_padding(out)
    got = out[:, :p.N].astype(np.float64)
    ref, ab = p.oracle_full()
    worst, bad = oracle.compare(p.dtype, got, ref, ab, p.alpha, p.beta, p.logical_c0())
    assert bad == 0, f"{bad} of {got.size} elements out of bound, max err/bound {worst:.3g}"
    return worst


def sample_points(M, N, n, seed, tile=(256, 128)):
    """n random elements plus the corners and elements on tile boundaries."""
    st = synth.Stream(seed)
    r = st.integers((n,), 0, M - 1).astype(np.int64)
    c = st.integers((n,), 0, N - 1).astype(np.int64)
    edge_r = sorted({0, M - 1, min(M - 1, tile[0] - 1), min(M - 1, tile[0]), M // 2,
                     max(0, M - 1 - (M - 1) % tile[0])})
    edge_c = sorted({0, N - 1, min(N - 1, tile[1] - 1), min(N - 1, tile[1]), N // 2,
                     max(0, N - 1 - (N - 1) % tile[1])})
    er, ec = np.meshgrid(edge_r, edge_c, indexing="ij")
    return np.concatenate([r, er.ravel()]), np.concatenate([c, ec.ravel()])


def check_sampled(p: Problem, n=2000, seed=0, kernel=-1, offset=(0, 0, 0), out=None):
    if out is None:
        out = p.run_gpu(kernel, offset)
    p.check_padding(out)
    rows, cols = sample_points(p.M, p.N, n, seed)
    got = out[rows, cols].astype(np.float64)
    ref, ab = p.oracle_points(rows, cols)
    c0 = None
    if p.logical_c0() is not None:
        c0 = p.c0[rows, cols]
    worst, bad = oracle.compare(p.dtype, got, ref, ab, p.alpha, p.beta, c0)
    assert bad == 0, f"{bad} of {got.size} sampled elements out of bound, max err/bound {worst:.3g}"
    # properties that hold at every element: finite everywhere, padding intact
    assert np.isfinite(out[:, :p.N].astype(np.float64)).all(), "non-finite output"
    return worst
