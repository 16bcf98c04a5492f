"""dg_gemm_splitk_noalloc on an MI355X: the split-K form that keeps its fp32
partials in the library's own device array instead of a caller workspace.

Checked against dg_gemm_splitk with the same K ranges on a caller workspace
(the same kernels in the same order, so bit-identical) and against the CPU
oracle within the stated bound, on two calls in a row, the second with a
smaller problem; a problem whose partials exceed the scratch is refused with
nothing enqueued; a call changes no device memory allocation."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import Problem, to_device, to_host

pytestmark = pytest.mark.gpu
CODE = {"f32": 0, "f16": 1, "bf16": 2, "f16o32": 3, "bf16o32": 4}


@pytest.fixture(scope="module")
def dg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_amd
    return dense_gemm_amd


def _buffers(p):
    import torch
    dev = torch.device("cuda:0")
    A = to_device(p.A, synth.OPERAND_TYPE[p.dtype], dev)
    B = to_device(p.B, synth.OPERAND_TYPE[p.dtype], dev)
    return A, B, dev


def run_noalloc(dg, p, splits):
    import torch
    A, B, dev = _buffers(p)
    C = to_device(p.C0, synth.OUTPUT_TYPE[p.dtype], dev)
    rc = dg.dg_gemm_splitk_noalloc(p.ta, p.tb, p.M, p.N, p.K, p.alpha, A.data_ptr(), p.lda,
                                   B.data_ptr(), p.ldb, p.beta, C.data_ptr(), p.ldc, CODE[p.dtype],
                                   torch.cuda.current_stream().cuda_stream, splits)
    torch.cuda.synchronize()
    return rc, to_host(C).reshape(p.C0.shape)


def run_workspace(dg, p, splits):
    import torch
    A, B, dev = _buffers(p)
    C = to_device(p.C0, synth.OUTPUT_TYPE[p.dtype], dev)
    n = splits if splits > 0 else max(1, dg.dg_gemm_splitk_choose(p.ta, p.tb, p.M, p.N, p.K, CODE[p.dtype]))
    wsb = max(16, dg.dg_gemm_splitk_workspace_size(p.M, p.N, n))
    ws = torch.full((wsb // 4,), float("nan"), dtype=torch.float32, device=dev)
    rc = dg.dg_gemm_splitk(p.ta, p.tb, p.M, p.N, p.K, p.alpha, A.data_ptr(), p.lda, B.data_ptr(),
                           p.ldb, p.beta, C.data_ptr(), p.ldc, CODE[p.dtype],
                           torch.cuda.current_stream().cuda_stream, splits, ws.data_ptr(), wsb)
    assert rc == 0, dg.dg_status_string(rc)
    torch.cuda.synchronize()
    return to_host(C).reshape(p.C0.shape)


def check_oracle(p, out):
    p.check_padding(out)
    ref, ab, _ = p.oracle_full()
    worst, bad = oracle.compare(p.dtype, out[:, :p.N], ref, ab, p.alpha, p.beta, p.logical_c0())
    assert bad == 0, f"{bad} elements out of bound, max err/bound {worst:.3g}"


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "f16o32"])
def test_two_calls_second_smaller(dg, dtype):
    """A large split problem, then a smaller one on the same scratch: each
    equals the workspace form bit for bit and matches the oracle."""
    dist = "uniform" if dtype == "f32" else "normal_sqrtk"
    cases = [((512, 96, 5632), 0, (False, True)), ((136, 40, 1000), 3, (True, False))]
    for (M, N, K), splits, (ta, tb) in cases:
        a, b, c0 = synth.problem(M, N, K, dtype, dist, 400 + M, with_c0=True)
        p = Problem(a, b, c0, ta, tb, 1.25, -0.5, dtype, (8, 8, 8))
        used = splits if splits > 0 else dg.dg_gemm_splitk_choose(ta, tb, M, N, K, CODE[dtype])
        assert used > 1
        rc, out = run_noalloc(dg, p, splits)
        assert rc == 0, dg.dg_status_string(rc)
        want = run_workspace(dg, p, splits)
        assert np.array_equal(np.isnan(out), np.isnan(want))
        assert np.array_equal(out[:, :N], want[:, :N]), (M, N, K)
        check_oracle(p, out)


def test_too_many_partials_are_refused(dg):
    """Partials beyond the scratch: DG_ERR_SCRATCH, C untouched; the same
    problem without a split runs (the scratch is not used)."""
    M, N, K = 1024, 2048, 4096           # 4 ranges of 1024: 32 MiB of partials
    a, b, c0 = synth.problem(M, N, K, "f32", "uniform", 410, with_c0=True)
    p = Problem(a, b, c0, False, False, 1.0, 1.0, "f32", (0, 0, 0))
    assert 4 * M * N * 4 > dg.DG_SCRATCH_BYTES
    rc, out = run_noalloc(dg, p, 4)
    assert rc == dg.DG_ERR_SCRATCH
    assert np.array_equal(out, c0.astype(np.float64))
    rc, out = run_noalloc(dg, p, 1)
    assert rc == 0
    check_oracle(p, out)


def test_no_allocation(dg):
    """A call does not change the device's free memory (no allocation by the
    library or by any routine it calls)."""
    import torch
    M, N, K = 512, 32, 5632
    a, b, c0 = synth.problem(M, N, K, "f16", "normal_sqrtk", 420, with_c0=True)
    p = Problem(a, b, c0, False, False, 1.0, 0.0, "f16")
    A, B, dev = _buffers(p)
    C = to_device(p.C0, "f16", dev)
    s = torch.cuda.current_stream().cuda_stream

    def call():
        rc = dg.dg_gemm_splitk_noalloc(0, 0, M, N, K, 1.0, A.data_ptr(), p.lda, B.data_ptr(), p.ldb,
                                       0.0, C.data_ptr(), p.ldc, 1, s, 0)
        assert rc == 0
        torch.cuda.synchronize()

    call()                                  # the first call on a device looks the scratch up
    free0, _ = torch.cuda.mem_get_info(dev)
    for _ in range(3):
        call()
    free1, _ = torch.cuda.mem_get_info(dev)
    assert free1 == free0
    check_oracle(p, to_host(C).reshape(p.C0.shape))
