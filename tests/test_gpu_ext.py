"""Parity of the extended entry point (dg_gemm_ex) with the CPU oracle, on an
MI355X: bf16 operands, the fused bias + activation epilogue, and strided
batches (attention's per-head products), through the C ABI, against the
oracle's extended form within the stated bounds (carried through the
activation; bf16 outputs allowed half a bf16 ulp)."""
import itertools

import numpy as np
import pytest

import oracle
import synth
from gpu_util import Batched, Problem, check_full

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


def aligned_pad(M, N, K, ta, tb, extra=8):
    """Row padding that keeps every row start 16-byte aligned."""
    return tuple((-x) % 8 + extra for x in ((M if ta else K), (K if tb else N), N))


def bias_for(N, dtype, seed, scale=1.0):
    return synth.round_to(synth.Stream(seed).uniform((N,)) * scale, dtype)


# ---------------------------------------------------------------------------
# bf16
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("ta,tb", [(False, False), (True, False), (False, True)])
def test_bf16_2048_full(dg, ta, tb):
    """The fp16 headline workload's recipe (N(0,1)/sqrt(K), seed 2) in bf16."""
    S = 2048
    a, b, _ = synth.problem(S, S, S, "bf16", "normal_sqrtk", 2)
    worst = check_full(Problem(a, b, None, ta, tb, 1.0, 0.0, "bf16"))
    print(f"bf16 2048^3 ta={ta} tb={tb}: max err/bound {worst:.4f}", flush=True)


def test_bf16_output_rounding_is_rne(dg):
    """Integer products summed exactly in fp32 and rounded once to bf16: the
    result equals the nearest-even bf16 of the exact integer."""
    M, N, K = 64, 96, 256
    st = synth.Stream(141)
    a = synth.round_to(st.integers((M, K), 0, 12), "bf16")
    b = synth.round_to(st.integers((K, N), 0, 12), "bf16")
    exact = oracle.values(a).astype(np.int64) @ oracle.values(b).astype(np.int64)   # > 256: rounds
    want = oracle.values(synth.round_to(exact.astype(np.float64), "bf16"))
    for ta, tb in TRANS:
        out = Problem(a, b, None, ta, tb, 1.0, 0.0, "bf16", (8, 8, 8)).run_gpu()[:, :N]
        assert np.array_equal(out, want), (ta, tb)
    assert not np.array_equal(want, exact.astype(np.float64))     # rounding did happen


def test_bf16_integer_inputs_exact(dg):
    M, N, K = 264, 136, 24            # |2 ab - c0| <= 194 < 256: exact in bf16
    a, b, c0 = synth.problem(M, N, K, "bf16", "int2", 131, with_c0=True)
    av, bv, cv = (oracle.values(x).astype(np.int64) for x in (a, b, c0))
    exact = (2 * (av @ bv) - cv).astype(np.float64)
    for ta, tb in TRANS:
        p = Problem(a, b, c0, ta, tb, 2.0, -1.0, "bf16", aligned_pad(M, N, K, ta, tb))
        for k in kernels_for(dg, "bf16"):
            out = p.run_gpu(kernel=k)[:, :N]
            assert np.array_equal(out, exact), (dg.dg_kernel_name(k), ta, tb)


# ---------------------------------------------------------------------------
# the fused epilogue, on every kernel of every type
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("act", ["none", "relu", "gelu"])
@pytest.mark.parametrize("ta,tb", TRANS)
def test_epilogue_every_kernel(dg, dtype, act, ta, tb):
    M, N, K = 264, 200, 150     # ragged against every tile; whole 16-byte pieces for any layout
    a, b, c0 = synth.problem(M, N, K, dtype, "uniform", 200 + 2 * ta + tb, with_c0=True)
    bias = bias_for(N, dtype, 201, 4.0)
    p = Problem(a, b, c0, ta, tb, 1.25, -0.5, dtype, aligned_pad(M, N, K, ta, tb), bias=bias,
                act=act)
    for k in kernels_for(dg, dtype):
        print(f"kernel {dg.dg_kernel_name(k)} {dtype} {act} ta={ta} tb={tb}", flush=True)
        check_full(p, kernel=k)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("act", ["relu", "gelu"])
def test_epilogue_without_bias_and_unaligned_rows(dg, dtype, act):
    M, N, K = 130, 98, 70                   # row strides not whole 16-byte pieces
    a, b, c0 = synth.problem(M, N, K, dtype, "uniform", 210, with_c0=True)
    p = Problem(a, b, c0, False, True, 1.0, 1.0, dtype, (1, 3, 5), act=act)
    check_full(p)
    p = Problem(a, b, None, True, False, -1.0, 0.0, dtype, (3, 1, 1), bias=bias_for(N, dtype, 211),
                act=act)
    check_full(p)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("act", ["none", "relu", "gelu"])
def test_epilogue_without_product(dg, dtype, act):
    """alpha = 0 (or K = 0): C = act(beta * C + bias), A and B unread."""
    M, N, K = 50, 60, 20
    a, b, c0 = synth.problem(M, N, K, dtype, "uniform", 212, with_c0=True)
    bias = bias_for(N, dtype, 213, 2.0)
    check_full(Problem(a, b, c0, False, False, 0.0, -0.75, dtype, (0, 0, 2), bias=bias, act=act))
    z = np.zeros((M, 0), a.dtype), np.zeros((0, N), a.dtype)
    check_full(Problem(z[0], z[1], c0, False, False, 1.0, 2.0, dtype, (1, 0, 2), bias=bias, act=act))
    check_full(Problem(z[0], z[1], None, False, False, 1.0, 0.0, dtype, (1, 0, 2), bias=bias,
                       act=act))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("act", ["relu", "gelu"])
@pytest.mark.parametrize("kernel_kind", ["auto", "simple"])
def test_activation_over_a_dense_range(dg, dtype, act, kernel_kind):
    """alpha = beta = 0: every row is act(bias), with the bias swept densely
    over [-12, 12] (the activation alone, both tails of gelu included), in
    the no-product kernel; and a K = 1 product that lands on the same values
    through the matrix-core (or generic) epilogue."""
    N = 4096
    xs = synth.round_to(np.linspace(-12.0, 12.0, N), dtype)
    M = 8
    a, b, _ = synth.problem(M, N, 1, dtype, "uniform", 240)
    check_full(Problem(a, b, None, False, False, 0.0, 0.0, dtype, bias=xs, act=act))
    # K = 1 product a * b with a = 1: act(b + 0) = act(x) for x = b
    one = synth.round_to(np.ones((M, 1)), dtype)
    bvals = xs.reshape(1, N)
    k = -1 if kernel_kind == "auto" else dg.kernel_names().index(f"{dtype}_64x64_simple")
    p = Problem(one, bvals, None, False, False, 1.0, 0.0, dtype, act=act)
    check_full(p, kernel=k)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_epilogue_mlp_projection_full(dg, dtype):
    """The LoRA block's up-projection shape (512 x 5632 x 2048, nt) with a
    bias and gelu fused, every output against the oracle."""
    M, N, K = 512, 5632, 2048
    st = synth.Stream(220)
    a = synth.round_to(st.normal((M, K), 1.0), dtype)
    b = synth.round_to(st.normal((K, N), 0.02), dtype)
    bias = synth.round_to(st.normal((N,), 0.5), dtype)
    p = Problem(a, b, None, False, True, 1.0, 0.0, dtype, bias=bias, act="gelu")
    check_full(p)


def test_epilogue_relu_integer_exact(dg):
    M, N, K = 136, 72, 40
    a, b, c0 = synth.problem(M, N, K, "f16", "int2", 230, with_c0=True)
    bias = synth.round_to(synth.Stream(231).integers((N,), -8, 8), "f16")
    av, bv, cv, bsv = (x.astype(np.int64) for x in (a, b, c0, bias))
    want = np.maximum((av @ bv) - cv + bsv[None, :], 0).astype(np.float64)
    for ta, tb in TRANS:
        p = Problem(a, b, c0, ta, tb, 1.0, -1.0, "f16", aligned_pad(M, N, K, ta, tb), bias=bias,
                    act="relu")
        for k in kernels_for(dg, "f16"):
            out = p.run_gpu(kernel=k)[:, :N]
            assert np.array_equal(out, want), (dg.dg_kernel_name(k), ta, tb)


# ---------------------------------------------------------------------------
# strided batches
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("ta,tb", TRANS)
def test_batched_every_kernel(dg, dtype, ta, tb):
    bp = Batched(136, 104, 72, dtype, 3, ta, tb, 1.5, -0.5, 300 + 2 * ta + tb, gap=(8, 16, 24))
    for k in kernels_for(dg, dtype):
        print(f"kernel {dg.dg_kernel_name(k)} {dtype} batched ta={ta} tb={tb}", flush=True)
        bp.check(bp.run_gpu(kernel=k))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shared", [(True, False), (False, True)])
def test_batched_shared_operand(dg, dtype, shared):
    """Stride 0: one matrix of A (or B) serves every batch."""
    bp = Batched(200, 96, 130, dtype, 4, False, True, 1.0, 0.0, 310, gap=(0, 8, 8), shared=shared)
    bp.check(bp.run_gpu())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("act", ["relu", "gelu"])
def test_batched_with_epilogue(dg, dtype, act):
    bp = Batched(72, 136, 96, dtype, 5, True, False, 0.5, 0.25, 320, gap=(8, 8, 8),
                 bias=bias_for(136, dtype, 321, 2.0), act=act)
    bp.check(bp.run_gpu())


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("product", ["QK^T", "PV", "P^T dO"])
def test_attention_heads(dg, dtype, product):
    """The per-head products of "Metal GEMM Kernels for LoRA Training",
    section 8, for 512 tokens and 32 heads of 64 (Q, K, V head-major): one
    call covers every head; sampled per head."""
    T, D, H = 512, 64, 32
    shape = {"QK^T": (T, T, D, False, True), "PV": (T, D, T, False, False),
             "P^T dO": (T, D, T, True, False)}[product]
    M, N, K, ta, tb = shape
    bp = Batched(M, N, K, dtype, H, ta, tb, 1.0, 0.0, 330, dist="normal_sqrtk")
    bp.check(bp.run_gpu(), full=False, n=200, seed=12)


def test_batch_of_one_equals_plain_call(dg):
    a, b, c0 = synth.problem(160, 136, 96, "f16", "uniform", 340, with_c0=True)
    p = Problem(a, b, c0, False, False, 1.0, 0.5, "f16", (8, 8, 8))
    plain = p.run_gpu()
    ext = Problem(a, b, c0, False, False, 1.0, 0.5, "f16", (8, 8, 8), act="relu")
    ext.act = "none"
    ext.bias = np.zeros(136, np.float16)      # forces the extended entry point
    assert np.array_equal(ext.run_gpu(), plain, equal_nan=True)   # the padding holds NaN canaries


def test_torch_convenience_batched_bias_gelu(dg):
    import torch
    dev = torch.device("cuda:0")
    H, M, N, K = 4, 96, 80, 64
    st = synth.Stream(350)
    a = synth.round_to(st.uniform((H, M, K)), "f32")
    b = synth.round_to(st.uniform((K, N)), "f32")
    bias = synth.round_to(st.uniform((N,)), "f32")
    C = dg.gemm(torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev),
                bias=torch.from_numpy(bias).to(dev), activation="gelu")
    torch.cuda.synchronize()
    assert tuple(C.shape) == (H, M, N)
    got = C.cpu().numpy().astype(np.float64)
    ref, pre, ab = oracle.gemm_ex(False, False, M, N, K, 1.0, a, K, b, N, 0.0, None, N, bias=bias,
                                  act="gelu", batch=H, strideA=M * K, strideB=0)
    worst, bad = oracle.compare("f32", got, ref, ab, 1.0, 0.0, None, bias[None, None, :], "gelu", pre)
    assert bad == 0, worst
