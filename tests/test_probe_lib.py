"""The control-probe library (libdense_gemm_probe.so, include/dense_gemm_probe.h):
on the CPU it loads, exports every declared symbol, counts its flops in closed
form and rejects invalid arguments before any HIP call; on a GPU its copy is
exact and its matrix-core probe reports a plausible rate and shader clock."""
import ctypes
import os
import re
import subprocess

import pytest

import dense_gemm_amd.probe as pr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dense_gemm_probe.h")


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(dgp_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(pr.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", pr.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if " T " in line}
    lib = ctypes.CDLL(pr.LIB_PATH)
    for name in declared_functions():
        assert name in syms, name
        assert hasattr(lib, name), name


def test_header_compiles_as_c99(tmp_path):
    src = tmp_path / "p.c"
    refs = "\n".join(f"    (void)&{f};" for f in declared_functions())
    src.write_text(f'#include "dense_gemm_probe.h"\nint main(void) {{\n{refs}\n    return DGP_MFMA_F32;\n}}\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only",
                    "-I", os.path.dirname(HEADER), str(src)], check=True, capture_output=True, text=True)


def test_flop_count_closed_form():
    # 8 MFMAs per round, 4 waves per workgroup; 2*32*32*2 and 2*32*32*16 flops each
    assert pr.dgp_mfma_flops(pr.DGP_MFMA_F32, 512, 1000) == 512 * 4 * 1000 * 8 * 4096
    assert pr.dgp_mfma_flops(pr.DGP_MFMA_F16, 3, 7) == 3 * 4 * 7 * 8 * 32768
    assert pr.dgp_mfma_flops(pr.DGP_MFMA_F16_RANDOM, 3, 7) == 3 * 4 * 7 * 8 * 32768
    assert pr.dgp_mfma_flops(9, 512, 1000) == 0.0


@pytest.mark.parametrize("args,code", [
    ((7, 512, 10), -1),
    ((pr.DGP_MFMA_F32, 0, 10), -2),
    ((pr.DGP_MFMA_F32, 65537, 10), -2),
    ((pr.DGP_MFMA_F16, 4, 0), -3),
    ((pr.DGP_MFMA_F16, 4, (1 << 24) + 1), -3),
])
def test_mfma_probe_invalid_arguments(args, code):
    assert pr.dgp_mfma_peak(*args, 16, 16, None) == code


def test_mfma_probe_null_buffers():
    assert pr.dgp_mfma_peak(pr.DGP_MFMA_F32, 4, 10, None, 16, None) == -4
    assert pr.dgp_mfma_peak(pr.DGP_MFMA_F32, 4, 10, 16, None, None) == -5


def test_copy_invalid_arguments():
    assert pr.dgp_copy(None, 16, 16, None) == -1
    assert pr.dgp_copy(8, 16, 16, None) == -1            # not 16-byte aligned
    assert pr.dgp_copy(16, None, 16, None) == -2
    assert pr.dgp_copy(16, 24, 16, None) == -2
    assert pr.dgp_copy(16, 32, 15, None) == -3
    assert pr.dgp_copy(16, 32, -16, None) == -3
    assert pr.dgp_copy(16, 32, 0, None) == 0              # empty: nothing enqueued


@pytest.mark.parametrize("args,code", [
    ((0, 4, 10, 1, 128, 16, 32768), -1),
    ((8, 4, 10, 1, 128, 16, 32768), -1),                      # depth alone: no part
    ((64, 4, 10, 1, 128, 16, 32768), -1),
    ((pr.DGP_SLAB_SWIZZLE, 4, 10, 1, 128, 16, 32768), -1),    # no part
    ((pr.DGP_SLAB_MFMA, 0, 10, 1, 128, 16, 32768), -2),
    ((pr.DGP_SLAB_MFMA, 65537, 10, 1, 128, 16, 32768), -2),
    ((pr.DGP_SLAB_LOADS, 4, 0, 1, 128, 16, 32768), -3),
    ((pr.DGP_SLAB_LOADS, 4, (1 << 20) + 1, 1, 128, 16, 32768), -3),
    ((pr.DGP_SLAB_LOADS, 4, 10, 0, 128, 16, 32768), -4),
    ((pr.DGP_SLAB_LOADS, 4, 10, 33, 128, 16, 32768), -4),
    ((pr.DGP_SLAB_LOADS, 4, 10, 1, 64, 16, 32768), -5),
    ((pr.DGP_SLAB_LOADS, 4, 10, 1, 192, 16, 256 * 192), -5),    # not a multiple of 128
    ((pr.DGP_SLAB_LOADS, 4, 10, 1, 65536 + 128, 16, 1 << 25), -5),
    ((pr.DGP_SLAB_READS, 4, 10, 1, 128, None, 32768), -6),
    ((pr.DGP_SLAB_READS, 4, 10, 1, 128, 8, 32768), -6),        # not 16-byte aligned
    ((pr.DGP_SLAB_MFMA, 4, 10, 1, 128, 16, 0), -7),
    ((pr.DGP_SLAB_MFMA, 4, 10, 1, 128, 16, 32768 + 16), -7),  # not whole groups of 256 rows
    ((pr.DGP_SLAB_MFMA, 4, 10, 1, 4096, 16, 1 << 19), -7),    # less than one group at this pitch
    ((pr.DGP_SLAB_MFMA, 4, 10, 1, 128, 16, 1 << 31), -7),
    # a GEMM tile grid: T x T workgroups for src = 2 * T * 128 rows, at most T rows per group
    ((pr.DGP_SLAB_LOADS | pr.DGP_SLAB_PANELS, 15, 10, 1, 128, 16, 4 * 128 * 128), -2),
    ((pr.DGP_SLAB_LOADS | pr.DGP_SLAB_PANELS, 4, 10, 3, 128, 16, 4 * 128 * 128), -4),
])
def test_slab_probe_invalid_arguments(args, code):
    assert pr.dgp_slab_probe(*args, 16, 16, None) == code


def test_slab_probe_null_buffers():
    assert pr.dgp_slab_probe(pr.DGP_SLAB_MFMA, 4, 10, 1, 128, 16, 32768, None, 16, None) == -8
    assert pr.dgp_slab_probe(pr.DGP_SLAB_MFMA, 4, 10, 1, 128, 16, 32768, 16, None, None) == -9


@pytest.mark.gpu
def test_copy_is_exact():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    n = (3 << 20) + 4                                       # not a multiple of the block size
    src = torch.arange(n, dtype=torch.int32, device=dev)
    dst = torch.full((n + 4,), -1, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream()
    assert pr.dgp_copy(src.data_ptr(), dst.data_ptr(), n * 4, s.cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src)
    assert bool((dst[n:] == -1).all())                    # nothing past the end


@pytest.mark.gpu
@pytest.mark.parametrize("kind", [pr.DGP_MFMA_F32, pr.DGP_MFMA_F16, pr.DGP_MFMA_F16_RANDOM])
def test_mfma_probe_runs(kind):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    wgs, iters = 64, 200
    sink = torch.full((wgs * 256,), float("nan"), dtype=torch.float32, device=dev)
    clocks = torch.zeros(wgs * 2, dtype=torch.int64, device=dev)
    s = torch.cuda.current_stream()
    print(f"mfma probe kind={kind} wgs={wgs} iters={iters}", flush=True)
    assert pr.dgp_mfma_peak(kind, wgs, iters, sink.data_ptr(), clocks.data_ptr(), s.cuda_stream) == 0
    torch.cuda.synchronize()
    assert bool(torch.isfinite(sink).all())
    c = clocks.view(wgs, 2).cpu()
    assert bool((c > 0).all())
    khz = pr.dgp_wall_clock_khz()
    assert khz > 0
    mhz = (c[:, 0].double() / c[:, 1].double()).median().item() * khz / 1e3
    assert 500 < mhz < 3000, mhz                           # a shader clock, in MHz


@pytest.mark.gpu
def test_slab_probe_runs():
    """Every combination of the slab probe's parts on one workgroup per CU:
    every workgroup reports its cycles, a slab with MFMAs takes at least
    their 512 cycles per SIMD (less would mean the instructions were not
    run), and a combination takes at least as long as each of its parts."""
    import statistics
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    wgs = torch.cuda.get_device_properties(dev).multi_processor_count
    slabs = 500
    src = torch.ones(1 << 18, dtype=torch.float32, device=dev)             # 1 MiB
    sink = torch.empty(wgs * 512, dtype=torch.float32, device=dev)
    clocks = torch.zeros(wgs * 2, dtype=torch.int64, device=dev)
    s = torch.cuda.current_stream()
    cyc = {}
    for mode in list(range(1, 8)) + [pr.DGP_SLAB_DEPTH1 | m for m in (1, 3, 5, 7)]:
        print(f"slab probe mode={mode} wgs={wgs} slabs={slabs}", flush=True)
        assert pr.dgp_slab_probe(mode, wgs, slabs, 1, 128, src.data_ptr(), src.numel() * 4, sink.data_ptr(),
                                 clocks.data_ptr(), s.cuda_stream) == 0
        torch.cuda.synchronize()
        c = clocks.view(wgs, 2).cpu().tolist()
        assert all(x > 0 and y > 0 for x, y in c)
        cyc[mode] = statistics.median(x for x, _ in c) / slabs
        mhz = statistics.median(x / y for x, y in c) * pr.dgp_wall_clock_khz() / 1e3
        assert 500 < mhz < 3000, (mode, mhz)                 # a shader clock, in MHz
    for mode in cyc:
        if mode & pr.DGP_SLAB_MFMA:
            assert cyc[mode] >= 0.95 * 512, cyc
        for part in (pr.DGP_SLAB_LOADS, pr.DGP_SLAB_MFMA, pr.DGP_SLAB_READS):
            if mode & part and mode & 7 != part:
                assert cyc[mode] >= 0.9 * cyc[part], (mode, part, cyc)


@pytest.mark.gpu
def test_slab_probe_groups_wrap():
    """Group counts that do not divide the source's groups, more groups than
    it holds, and pitches from contiguous to 64 KB rows: every load stays
    inside the source (the group index wraps) and the probe completes."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    wgs = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(wgs * 512, dtype=torch.float32, device=dev)
    clocks = torch.zeros(wgs * 2, dtype=torch.int64, device=dev)
    s = torch.cuda.current_stream()
    for pitch, groups in ((128, 5), (4096, 3), (65536, 1)):
        src = torch.ones(groups * 256 * pitch // 4, dtype=torch.float32, device=dev)
        for windows in (1, 3, 5, 7, 32):
            print(f"slab probe pitch={pitch} groups={groups} windows={windows}", flush=True)
            assert pr.dgp_slab_probe(pr.DGP_SLAB_LOADS | pr.DGP_SLAB_READS | pr.DGP_SLAB_MFMA, wgs, 37, windows,
                                     pitch, src.data_ptr(), src.numel() * 4, sink.data_ptr(), clocks.data_ptr(),
                                     s.cuda_stream) == 0
            torch.cuda.synchronize()
            assert all(x > 0 for x in clocks.cpu().tolist())
        del src


@pytest.mark.gpu
def test_slab_probe_gemm_panels():
    """The probe with a GEMM tile grid's panel loads (T x T workgroups, T =
    16 for 256 CUs), at two row pitches and several tile rows per group:
    completes, every workgroup reports."""
    import math
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    wgs = torch.cuda.get_device_properties(dev).multi_processor_count
    T = math.isqrt(wgs)
    if T * T != wgs:
        pytest.skip("compute-unit count is not a square")
    sink = torch.empty(wgs * 512, dtype=torch.float32, device=dev)
    clocks = torch.zeros(wgs * 2, dtype=torch.int64, device=dev)
    s = torch.cuda.current_stream()
    for pitch in (4096, 128 * 3):
        src = torch.ones(2 * T * 128 * pitch // 4, dtype=torch.float32, device=dev)
        for gm in (1, 4, T):
            print(f"slab probe panels T={T} pitch={pitch} group_m={gm}", flush=True)
            for swz in (0, pr.DGP_SLAB_SWIZZLE):
                mode = pr.DGP_SLAB_LOADS | pr.DGP_SLAB_READS | pr.DGP_SLAB_MFMA | pr.DGP_SLAB_PANELS | swz
                assert pr.dgp_slab_probe(mode, wgs, 50, gm, pitch, src.data_ptr(), src.numel() * 4,
                                         sink.data_ptr(), clocks.data_ptr(), s.cuda_stream) == 0
                torch.cuda.synchronize()
                assert all(x > 0 for x in clocks.cpu().tolist())
        del src
