"""Parity of the fp32-output form (fp16 or bf16 operands, fp32 accumulation,
fp32 C: DG_F16_F32OUT / DG_BF16_F32OUT) with the CPU oracle, on an MI355X.

The fp32-output variant is the one "Metal GEMM Kernels for LoRA Training on
Apple Silicon", section 4 measured against its fp16 store.  The bound is the
16-bit path's (rtol 2e-3, atol 1e-4 on the fp32 sums) with no output-rounding
term: the result is the fp32 value itself.  Every kernel of each operand type
is run with the fp32 output, through the C ABI."""
import itertools

import numpy as np
import pytest

import oracle
import synth
from gpu_util import Batched, Problem, check_full

pytestmark = pytest.mark.gpu
TRANS = list(itertools.product([False, True], [False, True]))
O32 = {"f16o32": "f16", "bf16o32": "bf16"}


@pytest.fixture(scope="module")
def dg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_amd
    return dense_gemm_amd


def kernels_for(dg, dtype):
    prefix = O32[dtype] + "_"
    return [i for i, n in enumerate(dg.kernel_names()) if n.startswith(prefix)]


def even_pad(base):
    """The smallest padding that makes base + pad even but not a multiple of 8."""
    return next(d for d in range(1, 9) if (base + d) % 2 == 0 and (base + d) % 8 != 0)


def run_or_unsupported(dg, p, k):
    try:
        return p.run_gpu(kernel=k)
    except dg.GemmError as e:
        assert e.status == dg.DG_ERR_UNSUPPORTED, e
        assert "pipe" in dg.dg_kernel_name(k), dg.dg_kernel_name(k)
        return None


@pytest.mark.parametrize("dtype", ["f16o32", "bf16o32"])
@pytest.mark.parametrize("ta,tb", TRANS)
@pytest.mark.parametrize("layout", ["aligned", "even", "odd"])
def test_every_kernel_fp32_output(dg, dtype, ta, tb, layout):
    """Every 16-bit kernel writing fp32 C: ragged shapes over several tiles, a
    partial K slab, alpha and beta (an fp32 C read), NaN canaries in the
    padding.  16-byte rows reach the 16-byte-load kernels, even strides the
    4-byte-load ones, odd strides the register-staged ones."""
    M, N, K = 311, 264, 197
    if layout == "aligned":
        pad = tuple((-x) % 8 + 8 for x in ((M if ta else K), (K if tb else N), N))
    elif layout == "even":
        # even row strides that are not 16-byte multiples, an even m/n-contiguous extent
        M = 312 if ta else M
        pad = tuple(even_pad(x) for x in ((M if ta else K), (K if tb else N), N))
    else:
        pad = (3, 5, 1)
    a, b, c0 = synth.problem(M, N, K, dtype, "normal_sqrtk", 300 + 2 * ta + tb, with_c0=True)
    assert c0.dtype == np.float32
    p = Problem(a, b, c0, ta, tb, 1.5, -0.5, dtype, pad)
    ran = 0
    for k in kernels_for(dg, dtype):
        print(f"kernel {dg.dg_kernel_name(k)} {dtype} ta={ta} tb={tb} {layout}", flush=True)
        out = run_or_unsupported(dg, p, k)
        if out is not None:
            check_full(p, kernel=k, out=out)
            ran += 1
    assert ran >= 3


@pytest.mark.parametrize("dtype", ["f16o32", "bf16o32"])
def test_fp32_output_is_not_rounded_to_16_bits(dg, dtype):
    """Integer products whose exact sums need more than the 16-bit
    significand: the fp32 output holds them exactly (every partial sum is an
    integer below 2^24), a 16-bit output would have rounded them."""
    M, N, K = 136, 264, 1024
    st = synth.Stream(310)
    opnd = O32[dtype]
    a = synth.round_to(st.integers((M, K), -16, 16), opnd)
    b = synth.round_to(st.integers((K, N), -16, 16), opnd)
    exact = oracle.values(a).astype(np.int64) @ oracle.values(b).astype(np.int64)
    assert np.abs(exact).max() < 2 ** 24
    for ta, tb in TRANS:
        p = Problem(a, b, None, ta, tb, 1.0, 0.0, dtype, (8, 8, 8))
        for k in [-1] + kernels_for(dg, dtype):
            out = run_or_unsupported(dg, p, k)
            if out is None:
                continue
            assert np.array_equal(out[:, :N], exact.astype(np.float64)), (dg.dg_kernel_name(k), ta, tb)
    # the same sums do not fit the 16-bit output type
    assert not np.array_equal(oracle.values(synth.round_to(exact.astype(np.float64), opnd)), exact)


@pytest.mark.parametrize("ta,tb", [(False, False), (True, False), (False, True)])
def test_hgemm_2048_fp32_output_full(dg, ta, tb):
    """The headline fp16 workload (N(0,1)/sqrt(K), seed 2) with an fp32 C."""
    S = 2048
    a, b, _ = synth.problem(S, S, S, "f16o32", "normal_sqrtk", 2)
    worst = check_full(Problem(a, b, None, ta, tb, 1.0, 0.0, "f16o32"))
    print(f"f16->f32 2048^3 ta={ta} tb={tb}: max err/bound {worst:.4f}", flush=True)


@pytest.mark.parametrize("index", range(len(synth.LORA_GEMMS)))
def test_lora_step_gemm_fp32_output(dg, index):
    """Every LoRA-step GEMM with an fp32 C (the "+=" products read an fp32 C),
    every output against the oracle."""
    name, M, N, K, ta, tb, beta, _ = synth.LORA_GEMMS[index]
    a, b, c0 = synth.lora_problem(index, seed=3, out="f32")
    p = Problem(a, b, c0, ta, tb, 1.0, beta, "f16o32")
    worst = check_full(p)
    print(f"LoRA GEMM {name} fp32 out: max err/bound {worst:.4f}", flush=True)


@pytest.mark.parametrize("dtype", ["f16o32", "bf16o32"])
@pytest.mark.parametrize("act", ["relu", "gelu"])
def test_fp32_output_epilogue_and_batch(dg, dtype, act):
    """dg_gemm_ex with an fp32 bias, an activation and a strided batch, fp32 C."""
    M, N, K, nb = 200, 136, 96, 3
    bias = synth.round_to(synth.Stream(320).uniform((N,)), "f32")
    for ta, tb in TRANS:
        bt = Batched(M, N, K, dtype, nb, ta, tb, 0.5, 0.25, 330 + 2 * ta + tb, dist="normal_sqrtk",
                     gap=(8, 8, 8), bias=bias, act=act)
        bt.check(bt.run_gpu())


@pytest.mark.parametrize("dtype", ["f16o32", "bf16o32"])
@pytest.mark.parametrize("shape,splits", [((512, 32, 5632), 0), ((200, 40, 1000), 3),
                                          ((100, 37, 900), 3), ((520, 48, 2048), 0)])
def test_fp32_output_splitk(dg, dtype, shape, splits):
    """Split-K with an fp32 C: fp32 partials, then the reduction writes fp32."""
    import torch
    M, N, K = shape
    a, b, c0 = synth.problem(M, N, K, dtype, "normal_sqrtk", 340 + M, with_c0=True)
    for ta, tb in TRANS:
        p = Problem(a, b, c0, ta, tb, -1.25, 0.5, dtype, (8, 8, 8))
        dev = torch.device("cuda:0")
        from gpu_util import to_device, to_host
        A = to_device(p.A, O32[dtype], dev)
        B = to_device(p.B, O32[dtype], dev)
        C = torch.from_numpy(np.ascontiguousarray(p.C0)).to(dev)
        code = {"f16o32": dg.DG_F16_F32OUT, "bf16o32": dg.DG_BF16_F32OUT}[dtype]
        n = splits if splits > 0 else max(1, dg.dg_gemm_splitk_choose(ta, tb, M, N, K, code))
        wsb = max(16, dg.dg_gemm_splitk_workspace_size(M, N, n))
        ws = torch.full((wsb // 4,), float("nan"), dtype=torch.float32, device=dev)
        rc = dg.dg_gemm_splitk(ta, tb, M, N, K, p.alpha, A.data_ptr(), p.lda, B.data_ptr(), p.ldb,
                               p.beta, C.data_ptr(), p.ldc, code,
                               torch.cuda.current_stream().cuda_stream, splits, ws.data_ptr(), wsb)
        if rc != 0:
            raise dg.GemmError(rc)
        torch.cuda.synchronize()
        out = to_host(C)
        p.check_padding(out)
        check_full(p, out=out)


def test_torch_convenience_fp32_output(dg):
    """dg.gemm with fp16 operands and an fp32 C (given, or allocated through
    out_dtype) selects the fp32-output type."""
    import torch
    M, N, K = 264, 136, 72
    a, b, c0 = synth.problem(M, N, K, "f16o32", "int2", 350, with_c0=True)
    dev = torch.device("cuda:0")
    A, B = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    C = torch.from_numpy(c0).to(dev)
    dg.gemm(A, B, C, alpha=2.0, beta=-1.0)
    want = 2 * (a.astype(np.int64) @ b.astype(np.int64)) - c0.astype(np.int64)
    assert C.dtype == torch.float32 and np.array_equal(C.cpu().numpy(), want.astype(np.float32))
    D = dg.gemm(A, B, out_dtype=torch.float32)
    assert D.dtype == torch.float32
    assert np.array_equal(D.cpu().numpy(), (a.astype(np.int64) @ b.astype(np.int64)).astype(np.float32))
