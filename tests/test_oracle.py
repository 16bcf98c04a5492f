"""Pins for the CPU oracle: each test ties it to something other than itself
(brute force, exact integer arithmetic, closed forms, the pages' worked index
facts, the exactly rounded sum, invariants of the definition)."""
import itertools
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TRANS = list(itertools.product([False, True], [False, True]))


def read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("="))
            out[k] = float(v) if "." in v else int(v)
    return out


def run(ta, tb, a, b, alpha=1.0, beta=0.0, c0=None, pad=(0, 0, 0), fill=np.nan, nthreads=1):
    """Store logical operands as the library expects them and call the oracle."""
    M, K = a.shape
    N = b.shape[1]
    A, lda = synth.store(a, ta, (M if ta else K) + pad[0], fill)
    B, ldb = synth.store(b, tb, (K if tb else N) + pad[1], fill)
    C0, ldc = (None, N)
    if c0 is not None:
        C0, ldc = synth.store(c0, False, N + pad[2], fill)
    return oracle.gemm(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, nthreads=nthreads)


def py_ijk(a, b, alpha, beta, c0):
    """Independent brute force over the logical matrices with Python floats:
    the plain triple loop of the pages, k ascending."""
    M, K = a.shape
    N = b.shape[1]
    al = a.astype(np.float64).tolist()
    bl = b.astype(np.float64).tolist()
    out = [[0.0] * N for _ in range(M)]
    ab = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = 0.0
            t = 0.0
            for k in range(K):
                p = al[i][k] * bl[k][j]
                s += p
                t += abs(p)
            r = alpha * s if (alpha != 0.0 and K > 0) else 0.0
            if beta != 0.0:
                r += beta * float(c0[i, j])
            out[i][j] = r
            ab[i][j] = t if (alpha != 0.0 and K > 0) else 0.0
    return np.array(out).reshape(M, N), np.array(ab).reshape(M, N)


# ---------------------------------------------------------------------------
# fp16 decoding (the oracle widens fp16 inputs from their bits itself)
# ---------------------------------------------------------------------------
def test_f16_decode_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(h)) for h in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero is kept
    assert math.copysign(1.0, oracle.f16_to_f64(0x8000)) == -1.0


# ---------------------------------------------------------------------------
# brute force on every tiny shape
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_bruteforce_all_tiny_shapes(dtype):
    seed = 11 if dtype == "f32" else 12
    n_checked = 0
    for M, N, K in itertools.product(range(1, 9), repeat=3):
        a, b, c0 = synth.problem(M, N, K, dtype, "uniform", seed + M * 100 + N * 10 + K,
                                 with_c0=True)
        ta, tb = TRANS[(M + N + K) % 4]
        alpha, beta = (1.0, 0.0) if (M * N * K) % 2 else (1.5, -0.5)
        ref, ab = run(ta, tb, a, b, alpha, beta, c0 if beta else None, pad=(1, 2, 3))
        want, want_ab = py_ijk(a, b, alpha, beta, c0)
        assert np.array_equal(ref, want), (M, N, K, ta, tb)
        assert np.array_equal(ab, want_ab), (M, N, K, ta, tb)
        n_checked += 1
    assert n_checked == 512


@pytest.mark.parametrize("ta,tb", TRANS)
def test_bruteforce_every_transpose_pair(ta, tb):
    a, b, c0 = synth.problem(7, 5, 8, "f32", "uniform", 21, with_c0=True)
    ref, ab = run(ta, tb, a, b, -0.75, 2.0, c0, pad=(3, 1, 2))
    want, want_ab = py_ijk(a, b, -0.75, 2.0, c0)
    assert np.array_equal(ref, want)
    assert np.array_equal(ab, want_ab)


# ---------------------------------------------------------------------------
# exact integer arithmetic against numpy's integer matmul
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("ta,tb", TRANS)
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_integer_inputs_exact(ta, tb, dtype):
    M, N, K = 37, 45, 29
    a, b, c0 = synth.problem(M, N, K, dtype, "int2", 31, with_c0=True)
    ai, bi, ci = (x.astype(np.int64) for x in (a, b, c0))
    ref, ab = run(ta, tb, a, b, 1.0, 0.0, None, pad=(5, 3, 0))
    assert np.array_equal(ref, (ai @ bi).astype(np.float64))
    assert np.array_equal(ab, (np.abs(ai) @ np.abs(bi)).astype(np.float64))
    ref, _ = run(ta, tb, a, b, 2.0, -3.0, c0, pad=(5, 3, 7))
    assert np.array_equal(ref, (2 * (ai @ bi) - 3 * ci).astype(np.float64))


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("ta,tb", TRANS)
def test_identity_gives_opB(ta, tb):
    _, b, _ = synth.problem(16, 24, 16, "f32", "uniform", 41)
    ref, _ = run(ta, tb, np.eye(16, dtype=np.float32), b, pad=(2, 2, 0))
    assert np.array_equal(ref, b.astype(np.float64))
    a, _, _ = synth.problem(20, 12, 12, "f32", "uniform", 42)
    ref, _ = run(ta, tb, a, np.eye(12, dtype=np.float32), pad=(1, 1, 0))
    assert np.array_equal(ref, a.astype(np.float64))


@pytest.mark.parametrize("ta,tb", TRANS)
def test_permutations_permute(ta, tb):
    # row permutation on the left: (P X)[i, :] = X[perm[i], :]
    _, x, _ = synth.problem(1, 11, 9, "f32", "uniform", 43)        # x is 9 x 11
    perm_r = np.array([3, 0, 8, 5, 1, 7, 2, 6, 4])
    P = np.zeros((9, 9), dtype=np.float32)
    P[np.arange(9), perm_r] = 1.0
    ref, _ = run(ta, tb, P, x, pad=(1, 1, 0))
    assert np.array_equal(ref, x[perm_r, :].astype(np.float64))
    # column permutation on the right: (Y Q)[:, j] = Y[:, perm[j]]
    y, _, _ = synth.problem(6, 1, 11, "f32", "uniform", 44)        # y is 6 x 11
    perm_c = np.array([10, 2, 4, 6, 8, 0, 1, 3, 5, 7, 9])
    Q = np.zeros((11, 11), dtype=np.float32)
    Q[perm_c, np.arange(11)] = 1.0
    ref, _ = run(ta, tb, y, Q, pad=(2, 3, 0))
    assert np.array_equal(ref, y[:, perm_c].astype(np.float64))


@pytest.mark.parametrize("ta,tb", TRANS)
def test_all_ones_gives_column_sums(ta, tb):
    M, N, K = 5, 17, 33
    _, b, _ = synth.problem(M, N, K, "f32", "int2", 51)
    ones = np.ones((M, K), dtype=np.float32)
    ref, _ = run(ta, tb, ones, b, pad=(2, 4, 0))
    colsum = b.astype(np.int64).sum(axis=0).astype(np.float64)
    assert np.array_equal(ref, np.broadcast_to(colsum, (M, N)))
    # with real-valued B: every row equals the exactly rounded column sum
    # up to the error of a K-term fp64 sum
    _, b, _ = synth.problem(M, N, K, "f32", "uniform", 52)
    ref, ab = run(ta, tb, ones, b)
    exact = np.array([math.fsum(b[:, j].astype(np.float64)) for j in range(N)])
    u = 2.0 ** -53
    assert np.all(np.abs(ref - exact) <= K * u * ab)


@pytest.mark.parametrize("ta,tb", TRANS)
def test_rank_one(ta, tb):
    # A = u v^T, B = x y^T  =>  C = (v . x) u y^T, exact with small integers
    st = synth.Stream(61)
    u_ = st.integers((12, 1), -3, 3)
    v_ = st.integers((1, 19), -3, 3)
    x_ = st.integers((19, 1), -3, 3)
    y_ = st.integers((1, 14), -3, 3)
    a = (u_ @ v_).astype(np.float32)
    b = (x_ @ y_).astype(np.float32)
    ref, _ = run(ta, tb, a, b, pad=(1, 1, 0))
    vx = float((v_ @ x_)[0, 0])
    assert np.array_equal(ref, vx * (u_ @ y_))


# ---------------------------------------------------------------------------
# alpha / beta and what is (not) read
# ---------------------------------------------------------------------------
def test_alpha_zero_reads_neither_A_nor_B():
    M, N, K = 6, 7, 8
    a = np.full((M, K), np.nan, dtype=np.float32)
    b = np.full((K, N), np.inf, dtype=np.float32)
    _, _, c0 = synth.problem(M, N, K, "f32", "uniform", 71, with_c0=True)
    ref, ab = run(False, False, a, b, 0.0, -0.5, c0)
    assert np.array_equal(ref, -0.5 * c0.astype(np.float64))
    assert np.all(ab == 0.0)


def test_k_zero_is_beta_c():
    _, _, c0 = synth.problem(4, 5, 1, "f32", "uniform", 72, with_c0=True)
    A = np.zeros((4, 1), dtype=np.float32)
    B = np.zeros((1, 5), dtype=np.float32)
    ref, _ = oracle.gemm(False, False, 4, 5, 0, 1.0, A, 1, B, 5, 2.0, c0, 5)
    assert np.array_equal(ref, 2.0 * c0.astype(np.float64))


def test_beta_zero_does_not_read_C():
    a, b, _ = synth.problem(6, 7, 8, "f32", "uniform", 73)
    c0 = np.full((6, 7), np.nan, dtype=np.float32)
    ref, _ = run(False, False, a, b, 1.0, 0.0, c0)
    assert np.all(np.isfinite(ref))


def test_beta_one_is_a_two_call_sum():
    a, b, c0 = synth.problem(13, 17, 19, "f32", "int2", 74, with_c0=True)
    r1, _ = run(False, True, a, b, 1.0, 0.0)
    r2, _ = run(False, True, a, b, 1.0, 1.0, c0)
    assert np.array_equal(r2, r1 + c0.astype(np.float64))


# ---------------------------------------------------------------------------
# layout invariance and NaN canaries in padding
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_transpose_variants_agree_and_skip_padding(dtype):
    a, b, c0 = synth.problem(33, 29, 41, dtype, "uniform", 81, with_c0=True)
    outs = [run(ta, tb, a, b, 1.5, -0.5, c0, pad=(8, 8, 8))[0] for ta, tb in TRANS]
    for o in outs:
        assert np.all(np.isfinite(o))
        assert np.array_equal(o, outs[0])


# ---------------------------------------------------------------------------
# the oracle against the exactly rounded sum (its own rounding error bound)
# ---------------------------------------------------------------------------
def test_against_exactly_rounded_sum():
    M, N, K = 8, 8, 512
    a, b, _ = synth.problem(M, N, K, "f32", "uniform", 0)
    ref, ab = run(False, False, a, b, nthreads=2)
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    u = 2.0 ** -53
    for i in range(M):
        for j in range(N):
            exact = math.fsum(a64[i, :] * b64[:, j])  # fp32 x fp32 products are exact in fp64
            assert abs(ref[i, j] - exact) <= (K - 1) * u * ab[i, j] + 1e-300


def test_thread_count_does_not_change_result():
    a, b, c0 = synth.problem(29, 31, 67, "f32", "uniform", 91, with_c0=True)
    r1, a1 = run(True, True, a, b, 1.5, -0.5, c0, nthreads=1)
    r7, a7 = run(True, True, a, b, 1.5, -0.5, c0, nthreads=7)
    assert np.array_equal(r1, r7) and np.array_equal(a1, a7)


def test_points_match_full():
    a, b, c0 = synth.problem(23, 19, 37, "f16", "normal_sqrtk", 92, with_c0=True)
    for ta, tb in TRANS:
        A, lda = synth.store(a, ta, (23 if ta else 37) + 3)
        B, ldb = synth.store(b, tb, (37 if tb else 19) + 5)
        C0, ldc = synth.store(c0, False, 19 + 2)
        full, fab = oracle.gemm(ta, tb, 23, 19, 37, 0.5, A, lda, B, ldb, 0.25, C0, ldc)
        ii, jj = np.meshgrid(np.arange(23), np.arange(19), indexing="ij")
        pts, pab = oracle.gemm_points(ta, tb, 23, 19, 37, 0.5, A, lda, B, ldb, 0.25, C0, ldc,
                                      ii.ravel(), jj.ravel())
        assert np.array_equal(pts.reshape(23, 19), full)
        assert np.array_equal(pab.reshape(23, 19), fab)


# ---------------------------------------------------------------------------
# the pages' worked decomposition of C[35, 93] at 4096^3
# ---------------------------------------------------------------------------
def test_c35_93_index_facts():
    g = read_golden("c35_93.txt")
    r, c = g["row"], g["col"]
    # Kernel 1 / 2-3: 32x32 threadgroups
    T = g["k1_threads_per_group"]
    assert (g["k1_group_x"] * T + g["k1_thread_x"], g["k1_group_y"] * T + g["k1_thread_y"]) == (c, r)
    # Kernel 4: 64x64 tiles, TM = 8 rows per thread, 64 threads per row band
    assert (c // g["k4_bn"], r // g["k4_bm"]) == (g["k4_group_x"], g["k4_group_y"])
    assert (r % g["k4_bm"], c % g["k4_bn"]) == (g["k4_tile_row"], g["k4_tile_col"])
    trow, tcol = g["k4_tile_row"] // g["k4_tm"], g["k4_tile_col"]
    assert (trow, tcol) == (g["k4_trow"], g["k4_tcol"])
    assert trow * g["k4_bn"] + tcol == g["k4_thread"]
    assert g["k4_tile_row"] % g["k4_tm"] == g["k4_sum_index"]
    # Kernel 5: 8x8 tiles
    t = g["k5_tile"]
    assert (r // t * t, c // t * t) == (g["k5_tile_row0"], g["k5_tile_col0"])
    assert (r % t, c % t) == (g["k5_entry_row"], g["k5_entry_col"])
    assert g["size"] // t == g["k5_ksteps"]
    # Kernel 8: 64x64 tiles
    t = g["k8_tile"]
    assert (r // t * t, c // t * t) == (g["k8_tile_row0"], g["k8_tile_col0"])


@pytest.mark.parametrize("dist", ["int2", "uniform"])
def test_c35_93_tile_decomposition(dist):
    """C[35,93] equals the sum over 512 K-steps of the (3,5) entry of the 8x8
    tile products A[32:40, 8t:8t+8] @ B[8t:8t+8, 88:96] (exactly for integers,
    within fp64 rounding for the uniform fp32 data of the 4096^3 problem)."""
    g = read_golden("c35_93.txt")
    S, r, c = g["size"], g["row"], g["col"]
    seed = 1 if dist == "uniform" else 101
    a, b, _ = synth.problem(S, S, S, "f32", dist, seed)
    ref, ab = oracle.gemm_points(False, False, S, S, S, 1.0, a, S, b, S, 0.0, None, S,
                                 np.array([r]), np.array([c]))
    t0r, t0c = g["k5_tile_row0"], g["k5_tile_col0"]
    er, ec = g["k5_entry_row"], g["k5_entry_col"]
    a64 = a[t0r:t0r + 8, :].astype(np.float64)
    b64 = b[:, t0c:t0c + 8].astype(np.float64)
    tiles = [(a64[:, 8 * s:8 * s + 8] @ b64[8 * s:8 * s + 8, :])[er, ec] for s in range(g["k5_ksteps"])]
    total = math.fsum(tiles)
    if dist == "int2":
        assert ref[0] == total
    else:
        assert abs(ref[0] - total) <= 2 * S * 2.0 ** -53 * ab[0]


# ---------------------------------------------------------------------------
# tolerance arithmetic
# ---------------------------------------------------------------------------
def test_bound_reduces_to_stated_form():
    ref = np.array([0.5, -3.0])
    ab = np.array([10.0, 20.0])
    b32 = oracle.bound("f32", ref, ab, 1.0, 0.0)
    assert np.allclose(b32, 2e-5 * ab + 1e-6, rtol=0, atol=0)
    b16 = oracle.bound("f16", ref, ab, 1.0, 0.0)
    half_ulp = np.array([2.0 ** -12, 2.0 ** -10])  # spacing of fp16 at 0.5 and 3.0, halved
    assert np.allclose(b16, 2e-3 * ab + 1e-4 + half_ulp, rtol=0, atol=0)
    bab = oracle.bound("f32", ref, ab, -1.5, -0.5, np.array([4.0, -8.0]))
    assert np.allclose(bab, 2e-5 * (1.5 * ab + np.array([2.0, 4.0])) + 1e-6, rtol=0, atol=0)


def test_compare_flags_nan_and_outliers():
    ref = np.zeros(4)
    ab = np.ones(4)
    ok, bad = oracle.compare("f32", np.array([0.0, 1e-6, -1e-6, 0.0]), ref, ab, 1.0, 0.0)
    assert bad == 0 and ok <= 1.0
    _, bad = oracle.compare("f32", np.array([0.0, np.nan, 0.0, 1e-3]), ref, ab, 1.0, 0.0)
    assert bad == 2


def _adjacent_pairs(dtype):
    """Every pair of adjacent non-negative finite values of a 16-bit format,
    decoded from consecutive bit patterns (fp16 by numpy, bf16 as the upper
    half of an fp32 encoding)."""
    if dtype == "f16":
        v = np.arange(0, 0x7c00, dtype=np.uint16).view(np.float16).astype(np.float64)
    else:
        bits = np.arange(0, 0x7f80, dtype=np.uint32) << np.uint32(16)
        v = bits.view(np.float32).astype(np.float64)
    return v[:-1], v[1:]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_half_ulp_is_half_the_gap_at_every_midpoint(dtype):
    """The output-rounding allowance equals the largest rounding error of its
    binade: at the midpoint of every two adjacent values (a tie, the worst
    case) it is exactly half their gap.  A function that took the spacing of
    the rounded value would be twice too large at the top of each binade."""
    lo, hi = _adjacent_pairs(dtype)
    mid = (lo + hi) / 2
    h = oracle.half_ulp_out(dtype, mid)
    assert np.array_equal(h, (hi - lo) / 2)
    # inside a binade every point's allowance covers its distance to the
    # nearest value
    inner = lo + (hi - lo) * 0.3
    assert np.all(oracle.half_ulp_out(dtype, inner) >= (inner - lo))


def test_half_ulp_f16_binade_tops():
    h = oracle.half_ulp_f16(np.array([2047.5, 2048.0, 1023.75, 1024.0, 65504.0, 65519.99, 65520.0,
                                      2.0 ** -20, 2.0 ** -14, 2.0 ** -13]))
    assert list(h[:6]) == [0.5, 1.0, 0.25, 0.5, 16.0, 16.0]
    assert np.isinf(h[6])
    assert list(h[7:]) == [2.0 ** -25, 2.0 ** -25, 2.0 ** -24]
    # a tie below 2048 moves to 2048 by 0.5; the allowance there is 0.5, not 1
    assert float(np.float16(2047.5)) == 2048.0


def test_overflow_thresholds_match_rounding():
    """Round-to-nearest-even gives an infinity exactly from the thresholds
    on (numpy's conversions as the independent reference)."""
    t16 = oracle.OVERFLOW["f16"]
    with np.errstate(over="ignore"):
        assert np.isinf(np.float16(t16)) and np.float16(np.nextafter(t16, 0)) == 65504.0
    t32 = oracle.OVERFLOW["f32"]
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(t32))
    assert np.float32(np.nextafter(t32, 0)) == np.finfo(np.float32).max
    # bf16: the tie at the threshold rounds to the even neighbour, the infinity
    tb = oracle.OVERFLOW["bf16"]
    top = np.array([0x7f7f0000], dtype=np.uint32).view(np.float32)[0]
    assert float(top) == oracle.BF16_MAX
    assert tb - oracle.BF16_MAX == (2.0 ** 128 - oracle.BF16_MAX) / 2


def test_compare_infinities():
    """An infinite output passes only where the reference can overflow the
    output type, with the reference's sign; a finite output where the
    reference overflows fails; an infinite output of a small reference
    fails."""
    one = np.ones(1)
    cmp = oracle.compare
    # f16: reference beyond the threshold
    assert cmp("f16", [np.inf], [70000.0], one, 1.0, 0.0)[1] == 0
    assert cmp("f16", [-np.inf], [70000.0], one, 1.0, 0.0)[1] == 1
    assert cmp("f16", [65504.0], [70000.0], one, 1.0, 0.0)[1] == 1
    assert cmp("f16", [-np.inf], [-70000.0], one, 1.0, 0.0)[1] == 0
    # f16: just below the threshold, no overflow possible
    assert cmp("f16", [np.inf], [65519.0], one, 1.0, 0.0)[1] == 1
    assert cmp("f16", [65504.0], [65519.0], one, 1.0, 0.0)[1] == 0
    # f16: within bound_pre of the threshold: either neighbour is a correct rounding
    ab = np.array([5000.0])                   # bound_pre = 2e-3 * 5000 + 1e-4 = 10.0001
    assert cmp("f16", [np.inf], [65515.0], ab, 1.0, 0.0)[1] == 0
    assert cmp("f16", [65504.0], [65515.0], ab, 1.0, 0.0)[1] == 0
    # an infinity where the reference is small
    assert cmp("f16", [np.inf], [100.0], one, 1.0, 0.0)[1] == 1
    assert cmp("f32", [np.inf], [1e38], one, 1.0, 0.0)[1] == 1
    assert cmp("f16o32", [np.inf], [70000.0], one, 1.0, 0.0)[1] == 1   # fp32 output holds 70000
    # fp32 and bf16 overflow
    assert cmp("f32", [np.inf], [3.5e38], one, 1.0, 0.0)[1] == 0
    assert cmp("f32", [-np.inf], [3.5e38], one, 1.0, 0.0)[1] == 1
    assert cmp("bf16", [-np.inf], [-4e38], one, 1.0, 0.0)[1] == 0
    assert cmp("bf16", [np.inf], [-4e38], one, 1.0, 0.0)[1] == 1
    # an infinite reference
    assert cmp("f32", [np.inf], [np.inf], one, 1.0, 0.0)[1] == 0
    assert cmp("f32", [1.0], [np.inf], one, 1.0, 0.0)[1] == 1
    assert cmp("f32", [np.nan], [np.inf], one, 1.0, 0.0)[1] == 1


def test_compare_binade_crossing_and_fp32_output():
    """The output rounding is allowed at the far end of bound_pre: an
    unrounded result just past 2048 rounds with spacing 2."""
    ab = np.array([100.0])                    # bound_pre = 0.2001
    assert oracle.compare("f16", [2048.0], [2047.9], ab, 1.0, 0.0)[1] == 0
    assert oracle.compare("f16", [2050.0], [2047.9], ab, 1.0, 0.0)[1] == 1
    # 16-bit operands with an fp32 output: no 16-bit rounding is allowed
    z = np.zeros(1)
    assert oracle.compare("f16", [1000.5], [1000.3], z, 1.0, 0.0)[1] == 0   # half ulp 0.25
    assert oracle.compare("f16o32", [1000.5], [1000.3], z, 1.0, 0.0)[1] == 1
    assert oracle.compare("f16o32", [1000.3 + 5e-5], [1000.3], z, 1.0, 0.0)[1] == 0
    assert oracle.compare("bf16o32", [1000.3 + 2e-4], [1000.3], z, 1.0, 0.0)[1] == 1


# ---------------------------------------------------------------------------
# the LoRA workload recipe against the page's figures
# ---------------------------------------------------------------------------
def test_lora_step_matches_page():
    g = read_golden("lora_step.txt")
    assert (synth.LORA_TOKENS, synth.LORA_DMODEL, synth.LORA_FFN, synth.LORA_RANK) == (
        g["tokens"], g["d_model"], g["ffn"], g["rank"])
    total = sum(2 * M * N * K for _, M, N, K, *_ in synth.LORA_GEMMS)
    assert round(total / 1e9, 1) == g["step_gflop"]
    dga = [e for e in synth.LORA_GEMMS if e[0].startswith("dGa")][0]
    assert dga[1:4] == (g["dga_m"], g["dga_n"], g["dga_k"])
    gf = 2 * dga[1] * dga[2] * dga[3] / 1e9
    assert abs(gf - g["dga_gflop"]) < 1e-3   # the page prints 0.18455 as 0.184
    assert round(gf / (g["dga_ms"] * 1e-3)) == g["dga_gfs"]
    assert len(synth.LORA_GEMMS) == 18
