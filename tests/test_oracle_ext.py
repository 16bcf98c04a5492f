"""Pins of the oracle's extended form: bf16 operands, the fused bias +
activation epilogue, and strided batches.

Each part is pinned to something other than the oracle itself: torch's bf16
decoding and exact-erf gelu (library routines), closed forms (gelu(0),
gelu(1) = Phi(1), gelu(x) - gelu(-x) = x), numpy's integer matmul for exact
integer cases, and an independent Python triple loop for tiny shapes."""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import synth

TRANS = list(itertools.product([False, True], [False, True]))
PHI_1 = 0.8413447460685429   # standard normal distribution function at 1


def dec(x):
    """fp64 values of logical operands; bf16 bit patterns decoded by torch."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    return x.astype(np.float64)


def run_ex(ta, tb, a, b, alpha=1.0, beta=0.0, c0=None, bias=None, act="none", pad=(0, 0, 0)):
    M, K = a.shape
    N = b.shape[1]
    A, lda = synth.store(a, ta, (M if ta else K) + pad[0])
    B, ldb = synth.store(b, tb, (K if tb else N) + pad[1])
    C0, ldc = (None, N)
    if c0 is not None:
        C0, ldc = synth.store(c0, False, N + pad[2])
    ref, pre, ab = oracle.gemm_ex(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, bias=bias,
                                  act=act, nthreads=1)
    return ref[0], pre[0], ab[0]


def py_ijk_ex(a, b, alpha, beta, c0, bias, act):
    """Independent triple loop over logical fp64 values, k ascending, then the
    epilogue x = alpha*acc + beta*c0 + bias[j] and the activation."""
    av, bv = dec(a).tolist(), dec(b).tolist()
    cv = dec(c0) if c0 is not None else None
    bsv = dec(bias) if bias is not None else None
    M, K = len(av), len(av[0]) if av else 0
    N = len(bv[0]) if bv else 0
    out = np.zeros((M, N))
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                s += av[i][k] * bv[k][j]
            r = alpha * s if (alpha != 0.0 and K > 0) else 0.0
            if beta != 0.0:
                r += beta * cv[i, j]
            if bsv is not None:
                r += bsv[j]
            if act == "relu":
                r = r if r > 0 else 0.0
            elif act == "gelu":
                r = 0.5 * r * (1.0 + math.erf(r / math.sqrt(2.0)))
            out[i, j] = r
    return out


# ---------------------------------------------------------------------------
# bf16
# ---------------------------------------------------------------------------
def test_bf16_decode_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = dec(bits)
    got = np.array([oracle.bf16_to_f64(int(h)) for h in bits])
    both_nan = np.isnan(got) & np.isnan(want)
    assert np.array_equal(got[~both_nan], want[~both_nan])
    assert np.count_nonzero(np.isnan(got)) == np.count_nonzero(np.isnan(want)) == 254


def test_bf16_rounding_of_inputs_is_nearest_even():
    """One rounding straight from fp64: the chosen bf16 value is at least as
    close as both neighbouring bf16 values, and a tie goes to the even pattern.
    (torch's fp64 -> bf16 passes through fp32 and rounds twice, so it is not
    the reference here.)  The differences are exact in fp64 (Sterbenz)."""
    x = synth.Stream(77).normal((50000,), 4.0)
    mid = 1.0 + 2.0 ** -8 + np.arange(8) * 2.0 ** -6        # exact midpoints
    x = np.concatenate([x, mid, -mid, [1e-40, -2e-39, 3e38]])
    bits = synth.round_to(x, "bf16")
    v = dec(bits)
    up = dec((bits.astype(np.int32) + 1).astype(np.uint16))
    down = dec((bits.astype(np.int32) - 1).astype(np.uint16))
    dv, du, dd = np.abs(x - v), np.abs(x - up), np.abs(x - down)
    assert np.all(dv <= du) and np.all(dv <= dd)
    tie = (dv == du) | (dv == dd)
    assert np.count_nonzero(tie) >= 16
    assert np.all(bits[tie] % 2 == 0)


def test_bruteforce_bf16_tiny_shapes():
    for M, N, K in itertools.product(range(1, 6), repeat=3):
        a, b, c0 = synth.problem(M, N, K, "bf16", "uniform", 500 + M * 100 + N * 10 + K,
                                 with_c0=True)
        ta, tb = TRANS[(M + N + K) % 4]
        alpha, beta = (1.0, 0.0) if (M * N * K) % 2 else (1.5, -0.5)
        ref, pre, _ = run_ex(ta, tb, a, b, alpha, beta, c0 if beta else None, pad=(1, 2, 3))
        want = py_ijk_ex(a, b, alpha, beta, c0 if beta else None, None, "none")
        assert np.array_equal(ref, want), (M, N, K, ta, tb)
        assert np.array_equal(pre, want)


@pytest.mark.parametrize("ta,tb", TRANS)
def test_bf16_integer_inputs_exact(ta, tb):
    a, b, c0 = synth.problem(29, 33, 41, "bf16", "int2", 41, with_c0=True)
    ai, bi, ci = (dec(x).astype(np.int64) for x in (a, b, c0))
    ref, _, ab = run_ex(ta, tb, a, b, 2.0, -1.0, c0, pad=(3, 0, 5))
    assert np.array_equal(ref, (2 * (ai @ bi) - ci).astype(np.float64))
    assert np.array_equal(ab, (np.abs(ai) @ np.abs(bi)).astype(np.float64))


# ---------------------------------------------------------------------------
# bias and activation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("ta,tb", TRANS)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_relu_bias_integer_exact(ta, tb, dtype):
    M, N, K = 23, 31, 19
    a, b, c0 = synth.problem(M, N, K, dtype, "int2", 61, with_c0=True)
    bias = synth.round_to(synth.Stream(62).integers((N,), -6, 6), dtype)
    ai, bi, ci, bsi = (dec(x).astype(np.int64) for x in (a, b, c0, bias))
    x = (ai @ bi) - 2 * ci + bsi[None, :]
    ref, pre, _ = run_ex(ta, tb, a, b, 1.0, -2.0, c0, bias=bias, act="relu", pad=(2, 1, 3))
    assert np.array_equal(pre, x.astype(np.float64))
    assert np.array_equal(ref, np.maximum(x, 0).astype(np.float64))
    ref, _, _ = run_ex(ta, tb, a, b, 1.0, -2.0, c0, bias=bias, act="none")
    assert np.array_equal(ref, x.astype(np.float64))


@pytest.mark.parametrize("act", ["relu", "gelu"])
def test_activation_of_bias_alone(act):
    """alpha = 0, beta = 0: every row is act(bias), so the activation is seen on
    its own and the bias is seen to follow the column index."""
    M, N, K = 5, 401, 3
    xs = np.linspace(-8.0, 8.0, N)
    xs[N // 2] = 0.0
    bias = xs.copy()
    a, b, _ = synth.problem(M, N, K, "f32", "uniform", 63)
    ref, pre, ab = run_ex(False, False, a, b, 0.0, 0.0, None, bias=bias, act=act)
    assert np.array_equal(pre, np.broadcast_to(xs, (M, N)))
    assert np.array_equal(ab, np.zeros((M, N)))
    t = torch.tensor(xs, dtype=torch.float64)
    want = (torch.relu(t) if act == "relu" else torch.nn.functional.gelu(t, approximate="none")).numpy()
    # erf of C's libm vs torch's: within an ulp of 1 each, times |x|/2
    tol = 4e-16 * (np.abs(want) + np.abs(xs))
    assert np.all(np.abs(ref - want[None, :]) <= tol[None, :])


def test_gelu_closed_forms():
    xs = np.array([0.0, 1.0, -1.0, 2.5, -2.5, 0.125, -0.125, -7.0])
    a, b, _ = synth.problem(1, xs.size, 1, "f32", "uniform", 64)
    ref, _, _ = run_ex(False, False, a, b, 0.0, 0.0, None, bias=xs, act="gelu")
    g = dict(zip(xs.tolist(), ref[0].tolist()))
    assert g[0.0] == 0.0
    assert abs(g[1.0] - PHI_1) <= 2e-16
    for x in (1.0, 2.5, 0.125):
        assert abs((g[x] - g[-x]) - x) <= 4e-16 * (1 + x)     # Phi(-x) = 1 - Phi(x)
    assert 0.0 > g[-7.0] > -1e-10                              # x Phi(x) -> 0 from below
    assert abs(g[2.5] - 2.5 * 0.9937903346742238) <= 1e-15     # Phi(2.5)


@pytest.mark.parametrize("act", ["none", "relu", "gelu"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bruteforce_epilogue_tiny(act, dtype):
    for M, N, K in ((1, 1, 1), (3, 5, 4), (4, 3, 7), (6, 2, 5)):
        a, b, c0 = synth.problem(M, N, K, dtype, "uniform", 65 + M + N + K, with_c0=True)
        bias = synth.round_to(synth.Stream(66).uniform((N,)), dtype)
        for ta, tb in TRANS:
            ref, _, _ = run_ex(ta, tb, a, b, 0.75, 0.5, c0, bias=bias, act=act, pad=(1, 0, 2))
            want = py_ijk_ex(a, b, 0.75, 0.5, c0, bias, act)
            if act == "gelu":     # erf of C's libm vs Python's math.erf
                assert np.all(np.abs(ref - want) <= 1e-15 * (np.abs(want) + 1.0))
            else:
                assert np.array_equal(ref, want)


# ---------------------------------------------------------------------------
# strided batches
# ---------------------------------------------------------------------------
def batched(ta, tb, M, N, K, dtype, nb, seed, strides_pad=(5, 3, 7), b_shared=False, beta=-0.5):
    """nb logical problems stored back to back with padded batch strides."""
    probs = [synth.problem(M, N, K, dtype, "int2", seed + q, with_c0=True) for q in range(nb)]
    sa_rows, sa_cols = (K, M) if ta else (M, K)
    sb_rows, sb_cols = (N, K) if tb else (K, N)
    sA = sa_rows * sa_cols + strides_pad[0]
    sB = 0 if b_shared else sb_rows * sb_cols + strides_pad[1]
    sC = M * N + strides_pad[2]
    dt = probs[0][0].dtype
    A = np.zeros(sA * (nb - 1) + sa_rows * sa_cols, dtype=dt)
    B = np.zeros(sB * (nb - 1) + sb_rows * sb_cols, dtype=dt)
    C = np.zeros(sC * (nb - 1) + M * N, dtype=dt)
    for q, (a, b, c0) in enumerate(probs):
        A[q * sA:q * sA + sa_rows * sa_cols] = (a.T if ta else a).ravel()
        if not b_shared or q == 0:
            B[q * sB:q * sB + sb_rows * sb_cols] = (b.T if tb else b).ravel()
        C[q * sC:q * sC + M * N] = c0.ravel()
    ref, pre, ab = oracle.gemm_ex(ta, tb, M, N, K, 1.0, A, sa_cols, B, sb_cols, beta, C, N,
                                  batch=nb, strideA=sA, strideB=sB, strideC=sC, nthreads=2)
    want = []
    for q, (a, b, c0) in enumerate(probs):
        bb = probs[0][1] if b_shared else b
        ai, bi, ci = (dec(x).astype(np.int64) for x in (a, bb, c0))
        want.append((ai @ bi) + beta * ci)
    return ref, np.array(want, dtype=np.float64)


@pytest.mark.parametrize("ta,tb", TRANS)
def test_batched_integer_exact(ta, tb):
    ref, want = batched(ta, tb, 9, 11, 13, "f32", 4, 70)
    assert np.array_equal(ref, want)


def test_batched_shared_operand_stride_zero():
    ref, want = batched(False, True, 8, 6, 10, "f16", 3, 80, b_shared=True)
    assert np.array_equal(ref, want)


def test_batched_bf16():
    ref, want = batched(True, False, 7, 5, 9, "bf16", 3, 90)
    assert np.array_equal(ref, want)


def test_batched_points_match_full():
    M, N, K, nb = 6, 7, 5, 3
    a, b, c0 = synth.problem(M, N * nb, K, "f32", "uniform", 95, with_c0=True)
    # three problems sharing A (stride 0), B and C0 slices at column offsets
    B = np.ascontiguousarray(b)
    C0 = np.ascontiguousarray(c0)
    bias = synth.round_to(synth.Stream(96).uniform((N,)), "f32")
    ref, pre, ab = oracle.gemm_ex(False, False, M, N, K, 1.25, a, K, B, N * nb, -0.5, C0, N * nb,
                                  bias=bias, act="gelu", batch=nb, strideA=0, strideB=N,
                                  strideC=N, nthreads=1)
    bs, rs, cs = np.meshgrid(np.arange(nb), np.arange(M), np.arange(N), indexing="ij")
    r2, p2, a2 = oracle.gemm_points_ex(False, False, M, N, K, 1.25, a, K, B, N * nb, -0.5, C0,
                                       N * nb, bs.ravel(), rs.ravel(), cs.ravel(), bias=bias,
                                       act="gelu", strideA=0, strideB=N, strideC=N, nthreads=2)
    assert np.array_equal(r2, ref.ravel())
    assert np.array_equal(p2, pre.ravel())
    assert np.array_equal(a2, ab.ravel())


# ---------------------------------------------------------------------------
# the bound of the extended form
# ---------------------------------------------------------------------------
def test_bound_terms():
    ref = np.array([1.0, 3.0, 1000.0])
    ab = np.array([10.0, 0.0, 5.0])
    bias = np.array([0.0, -2.0, 0.0])
    b = oracle.bound("bf16", ref, ab, 1.0, 0.0, None, bias, "relu", ref)
    want = 2e-3 * (ab + np.abs(bias)) + 1e-4 + oracle.half_ulp_bf16(ref)
    assert np.allclose(b, want, rtol=1e-15)
    assert oracle.half_ulp_bf16(np.array([1.0]))[0] == 2.0 ** -8
    assert oracle.half_ulp_bf16(np.array([1000.0]))[0] == 2.0
    g = oracle.bound("f32", ref, ab, 1.0, 0.0, act="gelu", pre=ref)
    assert np.allclose(g, 1.129 * (2e-5 * ab + 1e-6) + 1e-6 * np.abs(ref), rtol=1e-15)


def test_gelu_lipschitz_constant():
    # slope of x Phi(x) is Phi(x) + x phi(x), largest at x = sqrt(2)
    x = np.linspace(-10, 10, 200001)
    t = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.gelu(t, approximate="none").sum().backward()
    assert abs(t.grad.max().item() - oracle.GELU_LIPSCHITZ) < 1e-4
    assert t.grad.max().item() <= oracle.GELU_LIPSCHITZ
