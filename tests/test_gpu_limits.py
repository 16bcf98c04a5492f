"""Parity at the limits, on an MI355X through the C ABI: an output of more
than 2^31 elements (64-bit offsets in every store path), thousands of
batches in one call (the batch grid dimension), a split-K over a very
long K, and row strides at the pipelined kernels' 32-bit panel-offset limit
(operands of more than 4 GiB on either side of it)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import Batched, sample_points

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_amd
    return dense_gemm_amd


@pytest.mark.parametrize("aligned", [True, False])
def test_output_beyond_2_pow_31_elements(dg, aligned):
    """C with 46400^2 (or 46341 x 46343, odd strides: element stores) fp16
    elements, K small; sampled against the oracle, every element checked
    finite on the device, the last row's tail included."""
    import torch
    dev = torch.device("cuda:0")
    if aligned:
        M, N, K, lda, ldc = 46400, 46400, 32, 32, 46400
    else:
        M, N, K, lda, ldc = 46341, 46343, 33, 35, 46345
    assert M * N > 2 ** 31
    a, b, _ = synth.problem(M, N, K, "f16", "uniform", 500)
    A, _ = synth.store(a, False, lda)
    B, ldb = synth.store(b, False)
    At = torch.from_numpy(A).to(dev)
    Bt = torch.from_numpy(B).to(dev)
    Ct = torch.full((M, ldc), float("nan"), dtype=torch.float16, device=dev)
    print(f"large output {M}x{N} aligned={aligned}", flush=True)
    rc = dg.dg_gemm(0, 0, M, N, K, 1.0, At.data_ptr(), lda, Bt.data_ptr(), ldb, 0.0, Ct.data_ptr(),
                    ldc, dg.DG_F16_F32ACC, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, dg.dg_status_string(rc)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(Ct[:, :N]).all())
    if ldc > N:
        assert bool(torch.isnan(Ct[:, N:]).all())
    rows, cols = sample_points(M, N, 3000, 501)
    rows = np.concatenate([rows, [M - 1] * 4])
    cols = np.concatenate([cols, [N - 1, N - 2, N - 17, 0]])
    got = Ct[torch.from_numpy(rows).to(dev), torch.from_numpy(cols).to(dev)].float().cpu().numpy()
    ref, ab = oracle.gemm_points(False, False, M, N, K, 1.0, A, lda, B, ldb, 0.0, None, ldc, rows,
                                 cols)
    worst, bad = oracle.compare("f16", got, ref, ab, 1.0, 0.0)
    assert bad == 0, worst


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_thousands_of_batches(dg, dtype):
    bp = Batched(24, 40, 16, dtype, 2000, False, True, 1.0, 0.5, 510, gap=(8, 8, 8),
                 bias=synth.round_to(synth.Stream(511).uniform((40,)), dtype), act="relu")
    bp.check(bp.run_gpu())


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_splitk_very_long_k(dg, dtype):
    """K = 40000 over an 96 x 80 output: the library's split choice, fp32
    partials in a caller workspace, one reduction."""
    import torch
    dev = torch.device("cuda:0")
    M, N, K = 96, 80, 40000
    dist = "uniform" if dtype == "f32" else "normal_sqrtk"
    a, b, c0 = synth.problem(M, N, K, dtype, dist, 520, with_c0=True)
    tdt = torch.float32 if dtype == "f32" else torch.float16
    A = torch.from_numpy(a).to(dev)
    B = torch.from_numpy(b).to(dev)
    C = torch.from_numpy(c0.copy()).to(dev)
    code = dg.DG_F32 if dtype == "f32" else dg.DG_F16_F32ACC
    splits = dg.dg_gemm_splitk_choose(0, 0, M, N, K, code)
    assert splits > 1
    wsb = dg.dg_gemm_splitk_workspace_size(M, N, splits)
    ws = torch.empty(wsb // 4, dtype=torch.float32, device=dev)
    rc = dg.dg_gemm_splitk(0, 0, M, N, K, 0.5, A.data_ptr(), K, B.data_ptr(), N, -1.0, C.data_ptr(),
                           N, code, torch.cuda.current_stream().cuda_stream, 0, ws.data_ptr(), wsb)
    assert rc == 0, dg.dg_status_string(rc)
    torch.cuda.synchronize()
    assert C.dtype == tdt
    ref, ab = oracle.gemm(False, False, M, N, K, 0.5, a, K, b, N, -1.0, c0, N)
    worst, bad = oracle.compare(dtype, C.float().cpu().numpy(), ref, ab, 0.5, -1.0, c0)
    assert bad == 0, worst


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_panel_offsets_near_2_pow_31(dg, dtype):
    """A (k-contiguous) with the largest row stride the pipelined kernels
    take: 256 rows of it span just under 2^31 bytes, so the direct loads'
    32-bit byte offsets of the last row come within 1/256 of 2^31.  Only the
    logical K columns of each row are written; every output is compared with
    the oracle."""
    import torch
    dev = torch.device("cuda:0")
    esize = 4 if dtype == "f32" else 2
    lda = (1 << 31) // (256 * esize) - 64
    M, N, K = 256, 128, 64
    assert 255 * lda * esize > (1 << 31) - (1 << 24)
    a, b, _ = synth.problem(M, N, K, dtype, "uniform" if dtype == "f32" else "normal_sqrtk", 530)
    tdt = torch.float32 if dtype == "f32" else torch.float16
    code = dg.DG_F32 if dtype == "f32" else dg.DG_F16_F32ACC
    At = torch.empty((M, lda), dtype=tdt, device=dev)
    At[:, :K] = torch.from_numpy(a).to(dev)
    Bt = torch.from_numpy(b).to(dev)
    Ct = torch.full((M, N), float("nan"), dtype=tdt, device=dev)
    k = dg.dg_select_kernel(0, 0, M, N, K, At.data_ptr(), lda, Bt.data_ptr(), N, Ct.data_ptr(), N, code)
    assert "pipe" in dg.dg_kernel_name(k), dg.dg_kernel_name(k)
    print(f"panel offsets near 2^31: {dtype} lda={lda} kernel={dg.dg_kernel_name(k)}", flush=True)
    rc = dg.dg_gemm(0, 0, M, N, K, 1.0, At.data_ptr(), lda, Bt.data_ptr(), N, 0.0, Ct.data_ptr(), N,
                    code, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, dg.dg_status_string(rc)
    torch.cuda.synchronize()
    got = Ct.float().cpu().numpy()
    del At
    ref, ab = oracle.gemm(False, False, M, N, K, 1.0, a, K, b, N, 0.0, None, N)
    worst, bad = oracle.compare(dtype, got, ref, ab, 1.0, 0.0)
    assert bad == 0, worst


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False), (True, True)])
def test_row_strides_at_the_panel_offset_limit(dg, dtype, ta, tb):
    """A, B and C have 600 rows of the same stride ld, so each spans more
    than 4 GiB.  With 256 rows just under 2^31 bytes (ld = limit - 64) the
    dispatcher's kernel and the 256-row pipelined kernel run, the latter
    addressing a k-contiguous panel with offsets up to about 2^31 from its
    per-panel base.  At the limit the dispatcher takes a register-staged
    kernel (64-bit addressing) and the pipelined one is refused.  Every output
    against the oracle; C's padding keeps its NaN canaries."""
    import torch
    from gpu_util import DTYPES, OPND, OUTT, Problem, check_full, to_device, to_host, torch_dtype
    dev = torch.device("cuda:0")
    s = torch.cuda.current_stream(dev)
    M = N = K = 600
    esize = 4 if dtype == "f32" else 2
    limit = (1 << 31) // (256 * esize)      # first stride whose 256 rows reach 2^31 bytes
    wide = {"f32": "f32_256x128_pipe3_mfma32x32x2", "f16": "f16_256x128_pipe2_w8_mfma32x32x16"}[dtype]
    wide = dg.kernel_names().index(wide)
    a, b, c0 = synth.problem(M, N, K, dtype, "uniform", 131, with_c0=True)
    p = Problem(a, b, c0, ta, tb, 1.5, -0.5, dtype)      # compact operands for the oracle

    def wide_buffer(x, st, ld):
        buf = torch.full((x.shape[0], ld), float("nan"), dtype=torch_dtype(st), device=dev)
        buf[:, :x.shape[1]] = to_device(x, st, dev).view(x.shape)
        return buf

    for ld in (limit - 64, limit):
        A = wide_buffer(p.A, OPND[dtype], ld)
        B = wide_buffer(p.B, OPND[dtype], ld)
        C = wide_buffer(p.C0, OUTT[dtype], ld)
        assert A.numel() * A.element_size() > 1 << 32
        auto = dg.dg_select_kernel(ta, tb, M, N, K, A.data_ptr(), ld, B.data_ptr(), ld,
                                   C.data_ptr(), ld, DTYPES[dtype])
        assert ("pipe" in dg.dg_kernel_name(auto)) == (ld < limit), dg.dg_kernel_name(auto)
        for k in (-1, wide):
            C[:, :N] = to_device(p.C0, OUTT[dtype], dev).view(M, N)
            print(f"\n  {dtype} {'t' if ta else 'n'}{'t' if tb else 'n'} ld={ld} kernel="
                  f"{dg.dg_kernel_name(auto if k < 0 else k)}", flush=True)
            rc = dg.dg_gemm_with_kernel(ta, tb, M, N, K, 1.5, A.data_ptr(), ld, B.data_ptr(), ld,
                                        -0.5, C.data_ptr(), ld, DTYPES[dtype], s.cuda_stream, k)
            if k == wide and ld >= limit:
                assert rc == dg.DG_ERR_UNSUPPORTED, rc
                continue
            assert rc == 0, rc
            s.synchronize()
            assert torch.isnan(C[:, N:N + 64]).all() and torch.isnan(C[:, -64:]).all()
            check_full(p, out=to_host(C[:, :N]))
        del A, B, C
        torch.cuda.empty_cache()
