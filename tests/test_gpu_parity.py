"""Parity of the HIP library with the CPU oracle, on an MI355X.

Every case calls the library through its C ABI (dg_gemm / dg_gemm_with_kernel)
and compares element by element with the oracle within the stated bound:
|C - ref| <= rtol * (|alpha| sum_k |a_ik b_kj| + |beta C0|) + atol
(rtol, atol = 2e-5, 1e-6 for fp32; 2e-3, 1e-4 plus half an fp16 ulp for
fp16), exactly for integer-valued inputs."""
import functools
import itertools

import numpy as np
import pytest

import oracle
import synth
from gpu_util import DTYPES, Problem, check_full

pytestmark = pytest.mark.gpu
TRANS = list(itertools.product([False, True], [False, True]))


@pytest.fixture(scope="module")
def dg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_amd
    return dense_gemm_amd


def kernels_for(dg, dtype):
    return [i for i, n in enumerate(dg.kernel_names()) if n.startswith(dtype + "_")]


def pipe_ok(p):
    """Preconditions of the pipelined 16-byte-load kernels: rows of A and B
    4-byte aligned (the loads sit at 16-byte multiples from a row start), and
    the m/n-contiguous operand's extent a whole number of 16-byte pieces."""
    v = 4 if p.dtype == "f32" else 8
    r = 1 if p.dtype == "f32" else 2
    return (p.lda % r == 0 and p.ldb % r == 0 and (not p.ta or p.M % v == 0)
            and (p.tb or p.N % v == 0))


def run_or_unsupported(dg, p, k, **kw):
    """Runs kernel k; returns None when the library rejects it as unsupported
    for this problem, which is only allowed for the pipelined kernels when
    their preconditions fail."""
    try:
        return p.run_gpu(kernel=k, **kw)
    except dg.GemmError as e:
        assert e.status == dg.DG_ERR_UNSUPPORTED, e
        assert "pipe" in dg.dg_kernel_name(k) and (not pipe_ok(p) or kw.get("offset")), \
            f"{dg.dg_kernel_name(k)} rejected a problem it should take"
        return None


# ---------------------------------------------------------------------------
# every kernel x transpose pair x alignment, ragged shapes over several tiles
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("ta,tb", TRANS)
@pytest.mark.parametrize("aligned", [True, False])
def test_every_kernel_ragged(dg, dtype, ta, tb, aligned):
    if aligned:
        # every row start 16-byte aligned; edges still cut through 16-byte vectors
        M, N, K = 311, 263, 197
        pad = tuple((-x) % 8 + 8 for x in ((M if ta else K), (K if tb else N), N))
    else:
        M, N, K = 300, 270, 200   # row strides not a multiple of 16 bytes
        pad = (3, 5, 1)
    a, b, c0 = synth.problem(M, N, K, dtype, "uniform", 100 + 2 * ta + tb, with_c0=True)
    p = Problem(a, b, c0, ta, tb, 1.5, -0.5, dtype, pad)
    for k in kernels_for(dg, dtype):
        print(f"kernel {dg.dg_kernel_name(k)} {dtype} ta={ta} tb={tb} aligned={aligned}", flush=True)
        out = run_or_unsupported(dg, p, k)
        if out is not None:
            check_full(p, kernel=k, out=out)


@pytest.mark.parametrize("dtype", ["f16", "f32", "bf16"])
@pytest.mark.parametrize("ta,tb", TRANS)
@pytest.mark.parametrize("shape", [(296, 264, 192), (1000, 1032, 512), (136, 8, 64), (8, 136, 128),
                                   (264, 520, 256), (264, 136, 32), (136, 264, 100), (200, 144, 1),
                                   (128, 128, 127), (520, 264, 321), (300, 260, 17)])
def test_pipelined_kernels(dg, dtype, ta, tb, shape):
    """The direct-to-LDS pipelined kernels on shapes meeting their
    preconditions: ragged M and N (clamped loads), one and two K slabs (the
    pipeline tail), a partial last K slab (register-loaded, zero-filled),
    several tiles."""
    M, N, K = shape
    a, b, c0 = synth.problem(M, N, K, dtype, "uniform", 170 + 2 * ta + tb, with_c0=True)
    pad = tuple((-x) % 8 + 8 for x in ((M if ta else K), (K if tb else N), N))
    p = Problem(a, b, c0, ta, tb, 0.75, 0.5, dtype, pad)
    # 16-byte rows; an m/n-contiguous extent that is not a whole number of
    # 16-byte pieces leaves only the 4-byte-load kernels (even extents)
    whole = pipe_ok(p)
    for k in kernels_for(dg, dtype):
        name = dg.dg_kernel_name(k)
        if "pipe" not in name:
            continue
        print(f"kernel {name} {shape} ta={ta} tb={tb}", flush=True)
        out = run_or_unsupported(dg, p, k)
        if out is None:
            assert not whole and "_dw_" not in name and "_kw_" not in name, name
            continue
        assert whole or "_dw_" in name or "_kw_" in name, name
        check_full(p, kernel=k, out=out)


@pytest.mark.parametrize("ta,tb", TRANS)
@pytest.mark.parametrize("tiles_mn", [(24, 32), (25, 31), (32, 32), (33, 32)])
def test_f32_64x64_steady_state_gates(dg, ta, tb, tiles_mn):
    """The two fp32 64x64 kernels on grids at the bounds of their steady-state
    loop, which runs only while every workgroup is resident: at most 768
    workgroups with 32-deep slabs (three per CU), 1024 with 16-deep.  The four
    grids (768, 775, 1024 and 1056 tiles) put each kernel on both sides of its
    bound, so the loop without per-slab tests and the generic loop alone are
    both compared with the oracle; ragged M and N, a partial last K slab."""
    tm, tn = tiles_mn
    M, N, K = 64 * tm - 8, 64 * tn - 4, 269
    a, b, c0 = synth.problem(M, N, K, "f32", "uniform", 190 + 2 * ta + tb, with_c0=True)
    pad = tuple((-x) % 4 + 4 for x in ((M if ta else K), (K if tb else N), N))
    p = Problem(a, b, c0, ta, tb, 1.5, -0.5, "f32", pad)
    assert pipe_ok(p)
    for name in ("f32_64x64_pipe3_k32_mfma32x32x2", "f32_64x64_pipe4_mfma32x32x2"):
        k = dg.kernel_names().index(name)
        print(f"kernel {name} tiles {tm}x{tn} ta={ta} tb={tb}", flush=True)
        check_full(p, kernel=k)


@pytest.mark.parametrize("ta,tb", TRANS)
@pytest.mark.parametrize("shape", [(32, 32, 32), (4, 4, 5), (36, 92, 1), (100, 68, 31), (64, 64, 33),
                                   (300, 260, 257), (512, 252, 4099)])
def test_f32_32x32_k_groups(dg, ta, tb, shape):
    """The fp32 32x32 tile whose four waves each run a quarter of every
    32-deep slab (three and four stages): ragged M and N around the 32-wide
    tile, K of one element, a partial last slab, many slabs; the four
    partial blocks summed in LDS before alpha, beta and C."""
    M, N, K = shape
    a, b, c0 = synth.problem(M, N, K, "f32", "uniform", 200 + 2 * ta + tb, with_c0=True)
    pad = tuple((-x) % 4 + 4 for x in ((M if ta else K), (K if tb else N), N))
    p = Problem(a, b, c0, ta, tb, 1.5, -0.5, "f32", pad)
    for name in ("f32_32x32_pipe3_k32_ksplit4_mfma32x32x2", "f32_32x32_pipe4_k32_ksplit4_mfma32x32x2"):
        k = dg.kernel_names().index(name)
        print(f"kernel {name} {shape} ta={ta} tb={tb}", flush=True)
        assert pipe_ok(p)
        check_full(p, kernel=k)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "f16o32"])
def test_dispatch_random_shapes(dg, dtype):
    """The library's own kernel choice (dg_gemm) on 14 seeded random problems
    per dtype: M, N, K drawn in 1..320 (a third of them multiples of 32, the
    tile edges), a random transpose pair, row strides padded by 0, 8 or 16
    elements in half the cases (16-byte rows when the extents allow: the
    pipelined kernels) and by 0 to 9 in the others (mostly unaligned rows),
    alpha in [-2, 2) and beta 0 or in [-1, 1).  Every output against the
    oracle; the kernel chosen is printed with each case."""
    rng = np.random.default_rng(2024 + ["f32", "f16", "bf16", "f16o32"].index(dtype))
    dist = "uniform" if dtype == "f32" else "normal_sqrtk"
    for case in range(14):
        dims = [int(x) for x in rng.integers(1, 321, 3)]
        if case % 3 == 0:
            dims = [32 * max(1, d // 32) for d in dims]
        ta, tb = bool(rng.integers(2)), bool(rng.integers(2))
        if case % 4 < 2:
            dims = [8 * max(1, d // 8) for d in dims]
            pad = tuple(8 * int(x) for x in rng.integers(0, 3, 3))
        else:
            pad = tuple(int(x) for x in rng.integers(0, 10, 3))
        M, N, K = dims
        alpha = float(rng.uniform(-2, 2))
        beta = 0.0 if case % 2 else float(rng.uniform(-1, 1))
        a, b, c0 = synth.problem(M, N, K, dtype, dist, 300 + case, with_c0=True)
        p = Problem(a, b, c0, ta, tb, alpha, beta, dtype, pad)
        # device buffers start 256-byte aligned, as these stand-in addresses
        name = dg.dg_kernel_name(dg.dg_select_kernel(ta, tb, M, N, K, 256, p.lda, 256, p.ldb, 256, p.ldc,
                                                     DTYPES[dtype]))
        print(f"case {case}: {dtype} {M}x{N}x{K} ta={ta} tb={tb} pad={pad} -> {name}", flush=True)
        check_full(p, out=p.run_gpu())


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False)])
def test_16bit_unaligned_c_rows_route(dg, dtype, ta, tb):
    """The library's own choice for a 16-bit C whose rows are not 4-byte
    aligned (ldc = N + 1, element-wise epilogue), where the dispatcher takes
    the 128x128 tile instead of the model's 256x128: 2048x4096x520, alpha
    1.5, beta -0.5.  Every output against the oracle, C's padding untouched."""
    M, N, K = 2048, 4096, 520
    a, b, c0 = synth.problem(M, N, K, dtype, "normal_sqrtk", 150 + 2 * ta + tb, with_c0=True)
    p = Problem(a, b, c0, ta, tb, 1.5, -0.5, dtype, (0, 0, 1))
    k = dg.dg_select_kernel(ta, tb, M, N, K, 256, p.lda, 256, p.ldb, 256, p.ldc, DTYPES[dtype])
    name = dg.dg_kernel_name(k)
    print(f"kernel {name} {dtype} ta={ta} tb={tb}", flush=True)
    assert "128x128" in name, name
    check_full(p)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("extra", [1, 2, 6])
def test_c_rows_4byte_aligned_take_16byte_accesses(dg, dtype, extra):
    """C rows 4-byte but not 16-byte aligned (ldc = N + 2 or N + 6 for 16-bit
    C; N + 1, 2, 6 for fp32) go through the epilogue's 16-byte loads and
    stores; an odd 16-bit ldc (N + 1) through the element path.  Every kernel
    of the type, beta != 0 (C read), ragged edges; every output against the
    oracle, C's padding untouched."""
    M, N, K = 300, 264, 200
    a, b, c0 = synth.problem(M, N, K, dtype, "uniform", 160 + extra, with_c0=True)
    for ta, tb in TRANS:
        p = Problem(a, b, c0, ta, tb, 1.5, -0.5, dtype, (8, 8, extra))
        for k in kernels_for(dg, dtype):
            out = run_or_unsupported(dg, p, k)
            if out is not None:
                check_full(p, kernel=k, out=out)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_unaligned_pointers(dg, dtype):
    M, N, K = 129, 257, 77
    a, b, c0 = synth.problem(M, N, K, dtype, "uniform", 120, with_c0=True)
    for ta, tb in TRANS:
        p = Problem(a, b, c0, ta, tb, 1.0, 1.0, dtype, (8, 8, 8))
        for k in kernels_for(dg, dtype):
            out = run_or_unsupported(dg, p, k, offset=(1, 3, 1))
            if out is not None:
                check_full(p, kernel=k, out=out)


# ---------------------------------------------------------------------------
# brute force over every tiny shape
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_all_tiny_shapes(dg, dtype):
    for M, N, K in itertools.product(range(1, 9), repeat=3):
        a, b, c0 = synth.problem(M, N, K, dtype, "uniform", M * 100 + N * 10 + K, with_c0=True)
        ta, tb = TRANS[(M * 7 + N * 3 + K) % 4]
        alpha, beta = (1.0, 0.0) if (M + N + K) % 2 else (-2.0, 0.5)
        check_full(Problem(a, b, c0, ta, tb, alpha, beta, dtype, (1, 2, 3)))


# ---------------------------------------------------------------------------
# exact results: integer-valued inputs make every partial sum exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_integer_inputs_exact_and_variants_agree(dg, dtype):
    M, N, K = (259, 131, 515) if dtype == "f32" else (259, 136, 128)  # |sums| exact in fp16
    a, b, c0 = synth.problem(M, N, K, dtype, "int2", 130, with_c0=True)
    exact = a.astype(np.int64) @ b.astype(np.int64) * 2 - c0.astype(np.int64)
    outs = []
    for ta, tb in TRANS:
        for k in kernels_for(dg, dtype):
            p = Problem(a, b, c0, ta, tb, 2.0, -1.0, dtype, (8, 8, 8))
            out = run_or_unsupported(dg, p, k)
            if out is None:
                continue
            out = out[:, :N].astype(np.float64)
            assert np.array_equal(out, exact.astype(np.float64)), (dg.dg_kernel_name(k), ta, tb)
            outs.append(out)


def test_f16_output_rounding_is_rne_and_overflows_to_inf(dg):
    # integer products summed exactly in fp32, then one RNE rounding to fp16:
    # the result must equal numpy's RNE conversion of the exact value
    M, N, K = 64, 96, 256
    st = synth.Stream(140)
    a = st.integers((M, K), 0, 16).astype(np.float16)
    b = st.integers((K, N), 0, 16).astype(np.float16)
    exact = a.astype(np.int64) @ b.astype(np.int64)          # ~16000 (> 2048: rounds)
    for alpha in (1.0, 4.0):                                  # 4x: straddles 65520 -> +inf
        for ta, tb in TRANS:
            p = Problem(a, b, None, ta, tb, alpha, 0.0, "f16", (8, 8, 8))
            out = p.run_gpu()[:, :N]
            with np.errstate(over="ignore"):
                want = (alpha * exact.astype(np.float64)).astype(np.float16)
            got = np.ascontiguousarray(out).astype(np.float16)    # exact: fp16 values
            assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), (alpha, ta, tb)
        if alpha == 4.0:
            assert np.isinf(want).any() and np.isfinite(want).any()


# ---------------------------------------------------------------------------
# alpha / beta / empty cases and what the library does not touch
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_beta_zero_ignores_nan_in_C(dg, dtype):
    a, b, _ = synth.problem(70, 90, 33, dtype, "uniform", 150)
    p = Problem(a, b, None, False, True, 1.0, 0.0, dtype, (4, 4, 4))  # C holds NaN
    check_full(p)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_alpha_zero_and_k_zero_scale_C(dg, dtype):
    a, b, c0 = synth.problem(50, 60, 20, dtype, "uniform", 151, with_c0=True)
    a_nan = np.full_like(a, np.nan)
    p = Problem(a_nan, b, c0, False, False, 0.0, -0.5, dtype, (0, 0, 2))
    out = p.run_gpu()[:, :60].astype(np.float64)
    want = (np.float32(-0.5) * c0.astype(np.float32)).astype(a.dtype).astype(np.float64)
    assert np.array_equal(out, want)
    p0 = Problem(np.zeros((50, 0), a.dtype), np.zeros((0, 60), a.dtype), c0, False, False, 1.0,
                 2.0, dtype, (1, 0, 2))
    out = p0.run_gpu()[:, :60].astype(np.float64)
    assert np.array_equal(out, (2 * c0.astype(np.float64)))
    pz = Problem(np.zeros((50, 0), a.dtype), np.zeros((0, 60), a.dtype), None, False, False, 1.0,
                 0.0, dtype, (1, 0, 2))
    out = pz.run_gpu()[:, :60].astype(np.float64)
    assert np.array_equal(out, np.zeros((50, 60)))


def test_empty_and_invalid_calls_enqueue_nothing(dg):
    import torch
    dev = torch.device("cuda:0")
    C = torch.full((16, 16), 7.0, device=dev)
    A = torch.ones((16, 16), device=dev)
    s = torch.cuda.current_stream().cuda_stream
    ptr = C.data_ptr()
    # M = 0 and N = 0: nothing to do
    assert dg.dg_gemm(0, 0, 0, 16, 16, 1.0, A.data_ptr(), 16, A.data_ptr(), 16, 0.0, ptr, 16, 0, s) == 0
    assert dg.dg_gemm(0, 0, 16, 0, 16, 1.0, A.data_ptr(), 16, A.data_ptr(), 16, 0.0, ptr, 16, 0, s) == 0
    # invalid arguments: -i, the 1-based position of the first bad argument
    bad = [
        ((2, 0, 16, 16, 16, 1.0, A.data_ptr(), 16, A.data_ptr(), 16, 0.0, ptr, 16, 0, s), -1),
        ((0, 5, 16, 16, 16, 1.0, A.data_ptr(), 16, A.data_ptr(), 16, 0.0, ptr, 16, 0, s), -2),
        ((0, 0, -1, 16, 16, 1.0, A.data_ptr(), 16, A.data_ptr(), 16, 0.0, ptr, 16, 0, s), -3),
        ((0, 0, 16, -1, 16, 1.0, A.data_ptr(), 16, A.data_ptr(), 16, 0.0, ptr, 16, 0, s), -4),
        ((0, 0, 16, 16, -2, 1.0, A.data_ptr(), 16, A.data_ptr(), 16, 0.0, ptr, 16, 0, s), -5),
        ((0, 0, 16, 16, 16, 1.0, None, 16, A.data_ptr(), 16, 0.0, ptr, 16, 0, s), -7),
        ((0, 0, 16, 16, 16, 1.0, A.data_ptr(), 15, A.data_ptr(), 16, 0.0, ptr, 16, 0, s), -8),
        ((0, 0, 16, 16, 16, 1.0, A.data_ptr(), 16, None, 16, 0.0, ptr, 16, 0, s), -9),
        ((0, 0, 16, 16, 16, 1.0, A.data_ptr(), 16, A.data_ptr(), 8, 0.0, ptr, 16, 0, s), -10),
        ((0, 0, 16, 16, 16, 1.0, A.data_ptr(), 16, A.data_ptr(), 16, 0.0, None, 16, 0, s), -12),
        ((0, 0, 16, 16, 16, 1.0, A.data_ptr(), 16, A.data_ptr(), 16, 0.0, ptr, 15, 0, s), -13),
        ((0, 0, 16, 16, 16, 1.0, A.data_ptr(), 16, A.data_ptr(), 16, 0.0, ptr, 16, 9, s), -14),
    ]
    for args, want in bad:
        assert dg.dg_gemm(*args) == want, (args, want)
    torch.cuda.synchronize()
    assert (C == 7.0).all()


def test_side_stream_ordering(dg):
    """The call is asynchronous on the given stream: work queued before it on
    that stream is seen, and the result is there after the stream syncs."""
    import torch
    dev = torch.device("cuda:0")
    M = N = K = 512
    a, b, _ = synth.problem(M, N, K, "f32", "int2", 160)
    s = torch.cuda.Stream(device=dev)
    At = torch.from_numpy(a).to(dev)
    Bt = torch.from_numpy(b).to(dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        Bt.mul_(2.0)                     # queued on s before the GEMM
        C = dg.gemm(At, Bt)              # runs on s (the current stream)
    s.synchronize()
    want = (a.astype(np.int64) @ (2 * b.astype(np.int64))).astype(np.float32)
    assert np.array_equal(C.cpu().numpy(), want)


# ---------------------------------------------------------------------------
# the measured workloads at their full sizes (sampled elements)
# ---------------------------------------------------------------------------
def test_sgemm_512_full(dg):
    a, b, _ = synth.problem(512, 512, 512, "f32", "uniform", 0)
    p = Problem(a, b, None, False, False, 1.0, 0.0, "f32")
    check_full(p)


def test_sgemm_4096_nn_full(dg):
    a, b, _ = synth.problem(4096, 4096, 4096, "f32", "uniform", 1)
    p = Problem(a, b, None, False, False, 1.0, 0.0, "f32")
    worst = check_full(p)
    print(f"sgemm 4096^3 nn: max err/bound {worst:.4f}", flush=True)


@pytest.mark.parametrize("ta,tb", [(False, False), (True, False), (False, True)])
def test_hgemm_2048_full(dg, ta, tb):
    a, b, _ = synth.problem(2048, 2048, 2048, "f16", "normal_sqrtk", 2)
    p = Problem(a, b, None, ta, tb, 1.0, 0.0, "f16")
    worst = check_full(p)
    print(f"hgemm 2048^3 ta={ta} tb={tb}: max err/bound {worst:.4f}", flush=True)


@pytest.mark.parametrize("index", range(len(synth.LORA_GEMMS)))
def test_lora_step_gemm(dg, index):
    name, M, N, K, ta, tb, beta, _ = synth.LORA_GEMMS[index]
    a, b, c0 = synth.lora_problem(index, seed=3)
    p = Problem(a, b, c0, ta, tb, 1.0, beta, "f16")
    print(f"LoRA GEMM {name} ({M}x{N}x{K})", flush=True)
    worst = check_full(p)
    print(f"LoRA GEMM {name}: max err/bound {worst:.4f}", flush=True)


@pytest.mark.parametrize("pair", synth.LORA_PAIRS)
def test_lora_pair_strided_batch(dg, pair):
    # two LoRA products of one shape, stored one after the other, in one
    # strided-batch launch: every output of both against the oracle
    import torch
    i0, i1 = pair
    name, M, N, K, ta, tb, beta, _ = synth.LORA_GEMMS[i0]
    assert synth.LORA_GEMMS[i1][1:7] == (M, N, K, ta, tb, beta)
    probs = [synth.lora_problem(i, seed=3) for i in pair]
    dev = torch.device("cuda:0")
    A = torch.from_numpy(np.stack([np.ascontiguousarray(a.T if ta else a) for a, _, _ in probs])).to(dev)
    B = torch.from_numpy(np.stack([np.ascontiguousarray(b.T if tb else b) for _, b, _ in probs])).to(dev)
    if beta != 0.0:
        C = torch.from_numpy(np.stack([c0 for _, _, c0 in probs])).to(dev)
    else:
        C = torch.full((2, M, N), float("nan"), dtype=torch.float16, device=dev)
    lda, ldb = (M if ta else K), (K if tb else N)
    print(f"LoRA pair {name} and {synth.LORA_GEMMS[i1][0]} ({M}x{N}x{K}), batch 2", flush=True)
    rc = dg.dg_gemm_ex(ta, tb, M, N, K, 1.0, A.data_ptr(), lda, M * K, B.data_ptr(), ldb, K * N, beta,
                       C.data_ptr(), N, M * N, 2, None, dg.DG_EPI_NONE, dg.DG_F16_F32ACC,
                       torch.cuda.current_stream().cuda_stream)
    assert rc == 0, dg.dg_status_string(rc)
    torch.cuda.synchronize()
    got = C.float().cpu().numpy().astype(np.float64)
    for h, (a, b, c0) in enumerate(probs):
        ref, ab = oracle.gemm(False, False, M, N, K, 1.0, a, K, b, N, beta, c0, N)
        worst, bad = oracle.compare("f16", got[h], ref, ab, 1.0, beta, c0)
        assert bad == 0, f"{synth.LORA_GEMMS[pair[h]][0]}: {bad} out of bound, max err/bound {worst:.3g}"


# ---------------------------------------------------------------------------
# split-K: fp32 partials in a caller workspace, then one reduction
# ---------------------------------------------------------------------------
def run_splitk(dg, p, splits):
    import torch
    dev = torch.device("cuda:0")
    dtype = torch.float32 if p.dtype == "f32" else torch.float16
    A = torch.from_numpy(np.ascontiguousarray(p.A)).to(dev)
    B = torch.from_numpy(np.ascontiguousarray(p.B)).to(dev)
    C = torch.from_numpy(np.ascontiguousarray(p.C0)).to(dev)
    n = splits if splits > 0 else max(1, dg.dg_gemm_splitk_choose(p.ta, p.tb, p.M, p.N, p.K, DT[p.dtype]))
    wsb = max(16, dg.dg_gemm_splitk_workspace_size(p.M, p.N, n))
    ws = torch.full((wsb // 4,), float("nan"), dtype=torch.float32, device=dev)
    rc = dg.dg_gemm_splitk(p.ta, p.tb, p.M, p.N, p.K, p.alpha, A.data_ptr(), p.lda, B.data_ptr(),
                           p.ldb, p.beta, C.data_ptr(), p.ldc, DT[p.dtype],
                           torch.cuda.current_stream().cuda_stream, splits, ws.data_ptr(), wsb)
    if rc != 0:
        raise dg.GemmError(rc)
    torch.cuda.synchronize()
    assert C.dtype == dtype
    return C.cpu().numpy()


DT = {"f32": 0, "f16": 1}


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("ta,tb", TRANS)
@pytest.mark.parametrize("shape,splits", [((200, 40, 1000), 0), ((72, 264, 777), 3), ((136, 32, 640), 7),
                                          ((96, 96, 64), 2), ((520, 48, 2048), 0),
                                          # N not a multiple of 4 (element loads of the partials);
                                          # N > 4096 (a reduction thread takes several column groups)
                                          ((100, 37, 900), 3), ((40, 5000, 1024), 2)])
def test_splitk(dg, dtype, ta, tb, shape, splits):
    M, N, K = shape
    a, b, c0 = synth.problem(M, N, K, dtype, "uniform", 180 + 2 * ta + tb, with_c0=True)
    pad = tuple((-x) % 8 + 8 for x in ((M if ta else K), (K if tb else N), N))
    p = Problem(a, b, c0, ta, tb, -1.25, 0.5, dtype, pad)
    out = run_splitk(dg, p, splits)
    p.check_padding(out)
    ref, ab, _ = p.oracle_full()
    worst, bad = oracle.compare(dtype, out[:, :N].astype(np.float64), ref, ab, p.alpha, p.beta, c0)
    assert bad == 0, f"{bad} elements out of bound, max err/bound {worst:.3g}"


@pytest.mark.parametrize("index", [i for i, g in enumerate(synth.LORA_GEMMS) if g[2] == 32 or g[1] == 32])
def test_lora_skinny_splitk(dg, index):
    name, M, N, K, ta, tb, beta, _ = synth.LORA_GEMMS[index]
    a, b, c0 = synth.lora_problem(index, seed=3)
    p = Problem(a, b, c0, ta, tb, 1.0, beta, "f16")
    out = run_splitk(dg, p, 0)
    ref, ab, _ = p.oracle_full()
    worst, bad = oracle.compare("f16", out[:, :N].astype(np.float64), ref, ab, 1.0, beta, c0)
    assert bad == 0, f"{name}: {bad} elements out of bound, max err/bound {worst:.3g}"


@functools.lru_cache(maxsize=1)
def ragged_problem(shape):
    M, N, K = shape
    return synth.problem(M, N, K, "f32", "uniform", 4, with_c0=True)


@pytest.mark.parametrize("shape", [(4095, 4097, 1031), (8192, 256, 8192)])
@pytest.mark.parametrize("ta,tb", TRANS)
def test_sgemm_ragged_full_form(dg, shape, ta, tb):
    a, b, c0 = ragged_problem(shape)
    p = Problem(a, b, c0, ta, tb, 1.5, -0.5, "f32", (8, 8, 8))
    print(f"ragged {shape} ta={ta} tb={tb}", flush=True)
    worst = check_full(p)
    print(f"ragged {shape} ta={ta} tb={tb}: max err/bound {worst:.4f}", flush=True)


# ---------------------------------------------------------------------------
# 4-byte direct loads: rows 4-byte but not 16-byte aligned (ld padded so)
# ---------------------------------------------------------------------------
def _pad_4byte_rows(base, dtype):
    """Padding d >= 1 that makes base + d a row stride of 4-byte but not
    16-byte multiples (fp32: not a multiple of 4 elements; 16-bit: even, not
    a multiple of 8)."""
    for d in range(1, 9):
        ld = base + d
        if dtype == "f32" and ld % 4 != 0:
            return d
        if dtype != "f32" and ld % 2 == 0 and ld % 8 != 0:
            return d
    raise AssertionError(base)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("ta,tb", TRANS)
@pytest.mark.parametrize("shape", [(300, 258, 131), (130, 66, 70), (520, 514, 1030)])
def test_four_byte_direct_loads(dg, dtype, ta, tb, shape):
    """The library's own choice on row strides that rule out 16-byte
    alignment: the 16-byte-load kernels where the m/n-contiguous extents are
    whole 16-byte pieces (the loads need 4-byte aligned rows only), else a
    pipelined kernel with 4-byte loads (`_dw`), or for fp32 on the 64x64 tile
    16-byte loads of a k-contiguous operand (`_kw`); every output against the
    oracle, alpha/beta applied, C's padding untouched.  Odd K puts a pair of
    16-bit elements across the end of K in the last slab."""
    M, N, K = shape
    dist = "uniform" if dtype == "f32" else "normal_sqrtk"
    a, b, c0 = synth.problem(M, N, K, dtype, dist, 540 + M + K, with_c0=True)
    pa = _pad_4byte_rows(M if ta else K, dtype)
    pb = _pad_4byte_rows(K if tb else N, dtype)
    p = Problem(a, b, c0, ta, tb, 1.5, -0.5, dtype, pad=(pa, pb, 3))
    k = dg.dg_select_kernel(int(ta), int(tb), M, N, K, 256, p.lda, 256, p.ldb, 256, p.ldc,
                            {"f32": 0, "f16": 1, "bf16": 2}[dtype])
    name = dg.dg_kernel_name(k)
    assert "pipe" in name, name
    assert pipe_ok(p) or "_dw_" in name or (dtype == "f32" and "_kw_" in name), name
    print(f"4-byte loads {dtype} {shape} ta={ta} tb={tb} lda={p.lda} ldb={p.ldb} "
          f"kernel={dg.dg_kernel_name(k)}", flush=True)
    check_full(p, out=p.run_gpu())
