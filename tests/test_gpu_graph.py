"""Library calls recorded in a HIP graph.  The library only enqueues kernels
on the caller's stream (no allocation, no memset, no synchronisation), so a
sequence of calls can be captured once and replayed; each replay must read the
buffers' current contents and give exactly what the same calls give eagerly.
Replays are separated by the program's own eager work (new inputs copied in,
C reset, the eager calls) and synchronisations, and every replay is compared
bit for bit with the eager result; the first one is also checked against the
oracle."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_amd
    return dense_gemm_amd


def _bf16_tensor(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16).to(dev)


def test_graph_replay_matches_eager_and_oracle(dg):
    import torch
    dev = torch.device("cuda:0")

    # 1) fp32 nn, several tiles and a ragged tail, beta != 0
    M1, N1, K1 = 520, 390, 264
    # 2) fp16 skinny product through split-K with a caller workspace
    M2, N2, K2 = 64, 96, 6000
    # 3) bf16 batched, shared B, bias + gelu epilogue
    M3, N3, K3, NB = 136, 136, 72, 3

    A1 = torch.empty((M1, K1), dtype=torch.float32, device=dev)
    B1 = torch.empty((K1, N1), dtype=torch.float32, device=dev)
    C1 = torch.empty((M1, N1), dtype=torch.float32, device=dev)
    A2 = torch.empty((M2, K2), dtype=torch.float16, device=dev)
    B2 = torch.empty((K2, N2), dtype=torch.float16, device=dev)
    C2 = torch.empty((M2, N2), dtype=torch.float16, device=dev)
    A3 = torch.empty((NB, M3, K3), dtype=torch.bfloat16, device=dev)
    B3 = torch.empty((K3, N3), dtype=torch.bfloat16, device=dev)
    C3 = torch.empty((NB, M3, N3), dtype=torch.bfloat16, device=dev)
    bias3 = torch.empty((N3,), dtype=torch.bfloat16, device=dev)

    splits = dg.dg_gemm_splitk_choose(0, 0, M2, N2, K2, dg.DG_F16_F32ACC)
    assert splits > 1
    wsb = dg.dg_gemm_splitk_workspace_size(M2, N2, splits)
    ws = torch.empty(max(wsb, 16) // 4, dtype=torch.float32, device=dev)

    def calls(sptr):
        rc = dg.dg_gemm(0, 0, M1, N1, K1, 0.75, A1.data_ptr(), K1, B1.data_ptr(), N1, -0.5,
                        C1.data_ptr(), N1, dg.DG_F32, sptr)
        assert rc == 0, dg.dg_status_string(rc)
        rc = dg.dg_gemm_splitk(0, 0, M2, N2, K2, 1.0, A2.data_ptr(), K2, B2.data_ptr(), N2, 1.0,
                               C2.data_ptr(), N2, dg.DG_F16_F32ACC, sptr, 0, ws.data_ptr(), wsb)
        assert rc == 0, dg.dg_status_string(rc)
        rc = dg.dg_gemm_ex(0, 0, M3, N3, K3, 1.0, A3.data_ptr(), K3, M3 * K3, B3.data_ptr(), N3, 0,
                           0.0, C3.data_ptr(), N3, M3 * N3, NB, bias3.data_ptr(), dg.DG_EPI_GELU,
                           dg.DG_BF16_F32ACC, sptr)
        assert rc == 0, dg.dg_status_string(rc)

    def load(seed):
        """Fresh inputs (host arrays) copied into the captured buffers."""
        a1, b1, c1 = synth.problem(M1, N1, K1, "f32", "uniform", seed, with_c0=True)
        a2, b2, c2 = synth.problem(M2, N2, K2, "f16", "normal_sqrtk", seed + 1, with_c0=True)
        st = synth.Stream(seed + 2)
        a3 = synth.round_to(st.uniform((NB, M3, K3)), "bf16")
        b3 = synth.round_to(st.uniform((K3, N3)), "bf16")
        bb = synth.round_to(st.uniform((N3,)), "bf16")
        A1.copy_(torch.from_numpy(a1))
        B1.copy_(torch.from_numpy(b1))
        A2.copy_(torch.from_numpy(a2))
        B2.copy_(torch.from_numpy(b2))
        A3.copy_(_bf16_tensor(a3, dev))
        B3.copy_(_bf16_tensor(b3, dev))
        bias3.copy_(_bf16_tensor(bb, dev))
        return (a1, b1, c1), (a2, b2, c2), (a3, b3, bb)

    def reset(host):
        (_, _, c1), (_, _, c2), _ = host
        C1.copy_(torch.from_numpy(c1))
        C2.copy_(torch.from_numpy(c2))
        C3.fill_(float("nan"))

    # warm-up outside the capture (first launch of each kernel)
    host = load(600)
    reset(host)
    calls(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()

    for rep in range(4):
        print(f"graph replay {rep}", flush=True)
        host = load(610 + 10 * rep)
        reset(host)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [C1.clone(), C2.clone(), C3.clone()]
        reset(host)
        calls(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for g, e in zip(got, (C1, C2, C3)):
            assert torch.equal(g.view(torch.int16) if g.element_size() == 2 else g.view(torch.int32),
                               e.view(torch.int16) if e.element_size() == 2 else e.view(torch.int32))
        if rep == 0:
            (a1, b1, c1), (a2, b2, c2), (a3, b3, bb) = host
            ref, ab = oracle.gemm(False, False, M1, N1, K1, 0.75, a1, K1, b1, N1, -0.5, c1, N1)
            worst, bad = oracle.compare("f32", got[0].cpu().numpy(), ref, ab, 0.75, -0.5, c1)
            assert bad == 0, worst
            ref, ab = oracle.gemm(False, False, M2, N2, K2, 1.0, a2, K2, b2, N2, 1.0, c2, N2)
            worst, bad = oracle.compare("f16", got[1].float().cpu().numpy(), ref, ab, 1.0, 1.0, c2)
            assert bad == 0, worst
            ref, pre, ab = oracle.gemm_ex(False, False, M3, N3, K3, 1.0, a3.ravel(), K3, b3, N3, 0.0,
                                          None, N3, bias=bb, act="gelu", batch=NB, strideA=M3 * K3,
                                          strideB=0)
            out = got[2].float().cpu().numpy().astype(np.float64)
            worst, bad = oracle.compare("bf16", out, ref, ab, 1.0, 0.0, None,
                                        oracle.values(bb)[None, None, :], "gelu", pre)
            assert bad == 0, worst
