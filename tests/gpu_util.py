"""Helpers for the GPU parity tests: lay operands out (with NaN canaries in
the row padding), run the library through its C ABI on the current torch
stream, and compare with the CPU oracle."""
from __future__ import annotations

import numpy as np

import oracle
import synth

DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "f16o32": 3, "bf16o32": 4}
# storage types of the operands and of C per dtype name
OPND = synth.OPERAND_TYPE
OUTT = synth.OUTPUT_TYPE
EPI = {"none": 0, "relu": 1, "gelu": 2}


def torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_device(x, dtype, dev):
    """A host buffer as a flat device tensor of the storage type (bf16 from its
    uint16 bit patterns)."""
    import torch
    x = np.ascontiguousarray(x).ravel()
    if dtype == "bf16":
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    return torch.from_numpy(x).to(dev)


def to_host(t):
    """A device tensor's values as a float64 host array (bf16 widened exactly)."""
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


class Problem:
    """One GEMM (optionally with a bias and an activation): logical operands,
    their stored buffers, and the oracle.  Without an epilogue it runs through
    dg_gemm_with_kernel, with one through dg_gemm_ex_with_kernel (batch 1)."""

    def __init__(self, a, b, c0, ta, tb, alpha, beta, dtype, pad=(0, 0, 0), bias=None,
                 act="none"):
        self.a, self.b, self.c0 = a, b, c0
        self.ta, self.tb, self.alpha, self.beta, self.dtype = ta, tb, alpha, beta, dtype
        self.bias, self.act = bias, act
        self.M, self.K = a.shape
        self.N = b.shape[1]
        M, N, K = self.M, self.N, self.K
        self.A, self.lda = synth.store(a, ta, (M if ta else K) + pad[0])
        self.B, self.ldb = synth.store(b, tb, (K if tb else N) + pad[1])
        self.ldc = N + pad[2]
        if c0 is not None:
            cinit = c0
        elif OUTT[dtype] == "bf16":
            cinit = np.full((M, N), synth.BF16_NAN, dtype=np.uint16)
        else:
            cinit = np.full((M, N), np.nan, dtype=np.float32 if OUTT[dtype] == "f32" else a.dtype)
        self.C0, _ = synth.store(cinit, False, self.ldc)

    @property
    def extended(self):
        return self.bias is not None or self.act != "none"

    def oracle_full(self):
        """(ref, absum, pre) over the whole M x N output."""
        c0 = self.C0 if self.beta != 0.0 else None
        ref, pre, ab = oracle.gemm_ex(self.ta, self.tb, self.M, self.N, self.K, self.alpha, self.A,
                                      self.lda, self.B, self.ldb, self.beta, c0, self.ldc,
                                      bias=self.bias, act=self.act)
        return ref[0], ab[0], pre[0]

    def oracle_points(self, rows, cols):
        c0 = self.C0 if self.beta != 0.0 else None
        ref, pre, ab = oracle.gemm_points_ex(self.ta, self.tb, self.M, self.N, self.K, self.alpha,
                                             self.A, self.lda, self.B, self.ldb, self.beta, c0,
                                             self.ldc, np.zeros_like(rows), rows, cols,
                                             bias=self.bias, act=self.act)
        return ref, ab, pre

    def run_gpu(self, kernel=-1, offset=(0, 0, 0), stream=None):
        """Runs on the GPU; returns the stored C (M x ldc) as fp64 host values.
        `offset` shifts each buffer's start by that many elements (to test
        unaligned pointers)."""
        import torch

        import dense_gemm_amd as dg
        dev = torch.device("cuda:0")

        def up(x, off, st):
            flat = torch.empty(x.size + off + 8, dtype=torch_dtype(st), device=dev)
            flat.fill_(float("nan"))
            flat[off:off + x.size] = to_device(x, st, dev)
            return flat, off

        At, oa = up(self.A, offset[0], OPND[self.dtype])
        Bt, ob = up(self.B, offset[1], OPND[self.dtype])
        Ct, oc = up(self.C0, offset[2], OUTT[self.dtype])
        es = At.element_size()
        esc = Ct.element_size()
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        if self.extended:
            bias_t = to_device(self.bias, OUTT[self.dtype], dev) if self.bias is not None else None
            rc = dg.dg_gemm_ex_with_kernel(
                self.ta, self.tb, self.M, self.N, self.K, self.alpha, At.data_ptr() + oa * es,
                self.lda, 0, Bt.data_ptr() + ob * es, self.ldb, 0, self.beta,
                Ct.data_ptr() + oc * esc, self.ldc, 0, 1,
                bias_t.data_ptr() if bias_t is not None else None, EPI[self.act],
                DTYPES[self.dtype], s.cuda_stream, kernel)
        else:
            rc = dg.dg_gemm_with_kernel(self.ta, self.tb, self.M, self.N, self.K, self.alpha,
                                        At.data_ptr() + oa * es, self.lda, Bt.data_ptr() + ob * es,
                                        self.ldb, self.beta, Ct.data_ptr() + oc * esc, self.ldc,
                                        DTYPES[self.dtype], s.cuda_stream, kernel)
        if rc != 0:
            raise dg.GemmError(rc)
        s.synchronize()
        out = to_host(Ct[oc:oc + self.C0.size]).reshape(self.C0.shape)
        # nothing outside the buffer view is touched
        assert torch.isnan(Ct[:oc].float()).all() and torch.isnan(Ct[oc + self.C0.size:].float()).all()
        return out

    def check_padding(self, out):
        if self.ldc > self.N:
            pad = out[:, self.N:]
            assert np.isnan(pad.astype(np.float64)).all(), "C padding was written"

    def logical_c0(self):
        if self.beta == 0.0 or self.c0 is None:
            return None
        return oracle.values(self.c0)

    def logical_bias(self):
        return None if self.bias is None else oracle.values(self.bias)


def check_full(p: Problem, kernel=-1, offset=(0, 0, 0), out=None):
    if out is None:
        out = p.run_gpu(kernel, offset)
    p.check_padding(out)
    got = out[:, :p.N].astype(np.float64)
    ref, ab, pre = p.oracle_full()
    bias = p.logical_bias()
    worst, bad = oracle.compare(p.dtype, got, ref, ab, p.alpha, p.beta, p.logical_c0(),
                                None if bias is None else bias[None, :], p.act, pre)
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
    ref, ab, pre = p.oracle_points(rows, cols)
    c0 = p.logical_c0()
    c0 = None if c0 is None else c0[rows, cols]
    bias = p.logical_bias()
    worst, bad = oracle.compare(p.dtype, got, ref, ab, p.alpha, p.beta, c0,
                                None if bias is None else bias[cols], p.act, pre)
    assert bad == 0, f"{bad} of {got.size} sampled elements out of bound, max err/bound {worst:.3g}"
    # properties that hold at every element: finite everywhere, padding intact
    assert np.isfinite(out[:, :p.N].astype(np.float64)).all(), "non-finite output"
    return worst


class Batched:
    """A strided batch of GEMMs sharing M, N, K: batch q's stored operands sit
    at q * stride in one flat buffer per operand (stride 0: one matrix shared
    by every batch), with NaN canaries in the gaps between batches."""

    def __init__(self, M, N, K, dtype, nb, ta, tb, alpha, beta, seed, dist="uniform",
                 gap=(0, 0, 0), shared=(False, False), bias=None, act="none"):
        self.M, self.N, self.K, self.dtype, self.nb = M, N, K, dtype, nb
        self.ta, self.tb, self.alpha, self.beta = ta, tb, alpha, beta
        self.bias, self.act = bias, act
        probs = [synth.problem(M, N, K, dtype, dist, seed + q, with_c0=True) for q in range(nb)]
        ar, ac = (K, M) if ta else (M, K)
        br, bc = (N, K) if tb else (K, N)
        self.lda, self.ldb, self.ldc = ac, bc, N
        self.sA = 0 if shared[0] else ar * ac + gap[0]
        self.sB = 0 if shared[1] else br * bc + gap[1]
        self.sC = M * N + gap[2]
        def flat(stride, size, st, like):
            nanv = synth.BF16_NAN if st == "bf16" else np.nan
            return np.full(stride * (nb - 1) + size, nanv, dtype=like.dtype)

        self.A = flat(self.sA, ar * ac, OPND[dtype], probs[0][0])
        self.B = flat(self.sB, br * bc, OPND[dtype], probs[0][1])
        self.C0 = flat(self.sC, M * N, OUTT[dtype], probs[0][2])
        for q, (a, b, c0) in enumerate(probs):
            self.A[q * self.sA:q * self.sA + ar * ac] = (a.T if ta else a).ravel()
            self.B[q * self.sB:q * self.sB + br * bc] = (b.T if tb else b).ravel()
            self.C0[q * self.sC:q * self.sC + M * N] = c0.ravel()
        self.c0_values = oracle.values(self.C0)

    def run_gpu(self, kernel=-1):
        """Runs every batch in one call; returns the flat C buffer as fp64."""
        import torch

        import dense_gemm_amd as dg
        dev = torch.device("cuda:0")
        At, Bt = (to_device(x, OPND[self.dtype], dev) for x in (self.A, self.B))
        Ct = to_device(self.C0, OUTT[self.dtype], dev)
        bias_t = to_device(self.bias, OUTT[self.dtype], dev) if self.bias is not None else None
        s = torch.cuda.current_stream(dev)
        rc = dg.dg_gemm_ex_with_kernel(self.ta, self.tb, self.M, self.N, self.K, self.alpha,
                                       At.data_ptr(), self.lda, self.sA, Bt.data_ptr(), self.ldb,
                                       self.sB, self.beta, Ct.data_ptr(), self.ldc, self.sC,
                                       self.nb, bias_t.data_ptr() if bias_t is not None else None,
                                       EPI[self.act], DTYPES[self.dtype], s.cuda_stream, kernel)
        if rc != 0:
            raise dg.GemmError(rc)
        s.synchronize()
        return to_host(Ct)

    def check(self, out, full=True, n=500, seed=0):
        """Every batch against the oracle (whole outputs, or n sampled elements
        per batch); the gaps between the batches of C stay untouched."""
        M, N = self.M, self.N
        for q in range(self.nb - 1):
            gap = out[q * self.sC + M * N:(q + 1) * self.sC]
            assert np.isnan(gap).all(), f"gap after batch {q} was written"
        c0 = self.C0 if self.beta != 0.0 else None
        bias = None if self.bias is None else oracle.values(self.bias)
        if full:
            ref, pre, ab = oracle.gemm_ex(self.ta, self.tb, M, N, self.K, self.alpha, self.A,
                                          self.lda, self.B, self.ldb, self.beta, c0, self.ldc,
                                          bias=self.bias, act=self.act, batch=self.nb,
                                          strideA=self.sA, strideB=self.sB, strideC=self.sC)
            got = np.stack([out[q * self.sC:q * self.sC + M * N].reshape(M, N)
                            for q in range(self.nb)])
            c0v = None if c0 is None else np.stack(
                [self.c0_values[q * self.sC:q * self.sC + M * N].reshape(M, N) for q in range(self.nb)])
            worst, bad = oracle.compare(self.dtype, got, ref, ab, self.alpha, self.beta, c0v,
                                        None if bias is None else bias[None, None, :], self.act, pre)
        else:
            st = synth.Stream(seed)
            bs = st.integers((n * self.nb,), 0, self.nb - 1).astype(np.int64)
            rs = st.integers((n * self.nb,), 0, M - 1).astype(np.int64)
            cs = st.integers((n * self.nb,), 0, N - 1).astype(np.int64)
            ref, pre, ab = oracle.gemm_points_ex(self.ta, self.tb, M, N, self.K, self.alpha, self.A,
                                                 self.lda, self.B, self.ldb, self.beta, c0, self.ldc,
                                                 bs, rs, cs, bias=self.bias, act=self.act,
                                                 strideA=self.sA, strideB=self.sB, strideC=self.sC)
            idx = bs * self.sC + rs * self.ldc + cs
            got = out[idx]
            c0v = None if c0 is None else self.c0_values[idx]
            worst, bad = oracle.compare(self.dtype, got, ref, ab, self.alpha, self.beta, c0v,
                                        None if bias is None else bias[cs], self.act, pre)
        assert bad == 0, f"{bad} elements out of bound, max err/bound {worst:.3g}"
        return worst
