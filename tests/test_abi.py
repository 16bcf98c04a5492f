"""The C-ABI library on the CPU: it loads, exports every symbol the public
header declares, and its host logic (argument validation, quick returns,
kernel table and selection) behaves as documented.  No call here reaches a
GPU: invalid calls and empty problems return before any HIP call."""
import ctypes
import os
import re

import pytest

import dense_gemm_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dense_gemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    assert "dg_gemm" in names and "dg_status_string" in names and "dg_last_hip_error" in names
    assert sorted(names) == sorted(dg.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(dg.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_nm_lists_symbols_as_global_text():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", dg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in syms, name


NULL = None
GOOD = dict(ta=0, tb=0, M=16, N=16, K=16, alpha=1.0, A=0x1000, lda=16, B=0x2000, ldb=16, beta=0.0,
            C=0x3000, ldc=16, dtype=0, stream=NULL)


def call(**kw):
    a = dict(GOOD)
    a.update(kw)
    return dg.dg_gemm(a["ta"], a["tb"], a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"],
                      a["B"], a["ldb"], a["beta"], a["C"], a["ldc"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(ta=2), -1), (dict(ta=-1), -1), (dict(tb=7), -2),
    (dict(M=-1), -3), (dict(N=-5), -4), (dict(K=-1), -5), (dict(M=2 ** 31), -3),
    (dict(A=NULL), -7), (dict(lda=15), -8), (dict(ta=1, lda=15), -8),
    (dict(B=NULL), -9), (dict(ldb=15), -10), (dict(tb=1, ldb=15), -10),
    (dict(C=NULL), -12), (dict(ldc=15), -13), (dict(dtype=5), -14), (dict(dtype=-1), -14),
    # the first invalid argument is the one reported
    (dict(ta=9, M=-1, dtype=5), -1), (dict(lda=1, ldc=1), -8),
])
def test_invalid_arguments(kw, code):
    assert call(**kw) == code
    assert dg.dg_status_string(code).startswith("invalid")


def test_ld_minimums_follow_the_stored_shape():
    # A transposed is stored K x M: lda >= M, not K
    assert call(ta=1, M=32, K=8, lda=8, C=0x3000, ldc=16) == -8
    assert call(tb=1, N=8, K=32, lda=32, ldb=16, ldc=16) == -10   # B stored N x K: ldb >= K
    # minimum of 1 on empty extents
    assert call(M=0, lda=0) == -8


def test_empty_problems_return_ok_without_gpu():
    assert call(M=0) == 0
    assert call(N=0) == 0
    assert call(M=0, N=0, A=NULL, B=NULL, C=NULL) == 0


def test_null_A_B_allowed_when_not_read():
    # alpha == 0 or K == 0: A and B are never read, so NULL is accepted by the
    # checks (the call then only scales C, which needs a GPU: not made here)
    assert dg.dg_select_kernel(0, 0, 16, 16, 0, NULL, 1, NULL, 16, NULL, 16, 0) >= 0


def test_kernel_table():
    n = dg.dg_kernel_count()
    names = dg.kernel_names()
    assert n == len(names) >= 4
    assert len(set(names)) == n
    for i, name in enumerate(names):
        assert name.split("_")[0] in ("f32", "f16", "bf16")
        bm, bn = dg.dg_kernel_tile_m(i), dg.dg_kernel_tile_n(i)
        assert f"{bm}x{bn}" in name
    assert dg.dg_kernel_name(n) is None and dg.dg_kernel_name(-1) is None
    assert dg.dg_kernel_tile_m(n) == -1


def test_forced_kernel_out_of_range_is_unsupported():
    a = dict(GOOD)
    rc = dg.dg_gemm_with_kernel(0, 0, 16, 16, 16, 1.0, 0x1000, 16, 0x2000, 16, 0.0, 0x3000, 16, 0,
                                NULL, dg.dg_kernel_count())
    assert rc == dg.DG_ERR_UNSUPPORTED
    del a


def test_fp32_output_types_choose_the_operand_types_kernels():
    """A 16-bit-operand problem with an fp32 output runs the kernel the same
    problem with a 16-bit output would run (the kernels take the output type
    as a parameter); forcing a kernel of the other operand type is refused."""
    for dt16, dt32 in ((dg.DG_F16_F32ACC, dg.DG_F16_F32OUT), (dg.DG_BF16_F32ACC, dg.DG_BF16_F32OUT)):
        for ta, tb in ((0, 0), (1, 0), (0, 1), (1, 1)):
            for M, N, K in ((2048, 2048, 2048), (512, 32, 5632), (4096, 4096, 4096), (130, 66, 70)):
                lda, ldb = (M if ta else K), (K if tb else N)
                k16 = dg.dg_select_kernel(ta, tb, M, N, K, 256, lda, 256, ldb, 256, N, dt16)
                k32 = dg.dg_select_kernel(ta, tb, M, N, K, 256, lda, 256, ldb, 256, N, dt32)
                assert k16 == k32 >= 0
                assert dg.dg_gemm_splitk_choose(ta, tb, M, N, K, dt16) == \
                    dg.dg_gemm_splitk_choose(ta, tb, M, N, K, dt32)
    f32k = dg.dg_select_kernel(0, 0, 64, 64, 64, 256, 64, 256, 64, 256, 64, dg.DG_F32)
    rc = dg.dg_gemm_with_kernel(0, 0, 64, 64, 64, 1.0, 0x1000, 64, 0x2000, 64, 0.0, 0x3000, 64,
                                dg.DG_F16_F32OUT, NULL, f32k)
    assert rc == dg.DG_ERR_UNSUPPORTED


def test_fp32_output_bias_alignment_is_c_elements():
    """dg_gemm_ex's bias has C's type: 4-byte alignment for an fp32 output,
    2-byte for a 16-bit one (checked before any GPU call)."""
    def ex(dtype, bias):
        return dg.dg_gemm_ex(0, 0, 16, 16, 16, 1.0, 0x1000, 16, 0, 0x2000, 16, 0, 0.0, 0x3000, 16, 0,
                             1, bias, dg.DG_EPI_NONE, dtype, NULL)
    assert ex(dg.DG_F16_F32OUT, 0x4002) == -18
    assert ex(dg.DG_BF16_F32OUT, 0x4001) == -18
    assert ex(dg.DG_F16_F32ACC, 0x4001) == -18
    # a valid call with an empty batch returns before any GPU work
    assert dg.dg_gemm_ex(0, 0, 16, 16, 16, 1.0, 0x1000, 16, 0, 0x2000, 16, 0, 0.0, 0x3000, 16, 0,
                         0, 0x4004, dg.DG_EPI_NONE, dg.DG_F16_F32OUT, NULL) == 0


def test_selection_picks_matrix_core_kernels_of_the_right_type():
    for dtype, prefix in ((0, "f32_"), (1, "f16_"), (2, "bf16_"), (3, "f16_"), (4, "bf16_")):
        for M, N, K in ((4096, 4096, 4096), (2048, 2048, 2048), (512, 32, 5632), (1, 1, 1),
                        (8192, 256, 8192), (4095, 4097, 1031)):
            k = dg.dg_select_kernel(0, 0, M, N, K, NULL, K, NULL, N, NULL, N, dtype)
            name = dg.dg_kernel_name(k)
            assert name.startswith(prefix), (M, N, K, name)
            # every type has matrix-core kernels for any alignment
            assert "mfma" in name, (M, N, K, name)
    # the headline shapes get the large tiles
    k = dg.dg_select_kernel(0, 0, 4096, 4096, 4096, NULL, 4096, NULL, 4096, NULL, 4096, 0)
    assert (dg.dg_kernel_tile_m(k), dg.dg_kernel_tile_n(k)) == (256, 128)
    k = dg.dg_select_kernel(0, 0, 4096, 4096, 4096, NULL, 4096, NULL, 4096, NULL, 4096, 1)
    assert (dg.dg_kernel_tile_m(k), dg.dg_kernel_tile_n(k)) == (256, 256)
    k = dg.dg_select_kernel(0, 0, 2048, 2048, 2048, NULL, 2048, NULL, 2048, NULL, 2048, 1)
    assert (dg.dg_kernel_tile_m(k), dg.dg_kernel_tile_n(k)) == (128, 128)


def tile_of(M, N, K, dtype=1):
    k = dg.dg_select_kernel(0, 0, M, N, K, 256, K, 256, N, 256, N, dtype)
    return dg.dg_kernel_tile_m(k), dg.dg_kernel_tile_n(k)


def test_underfilled_16bit_grids_take_64x64_tiles_unsplit():
    # at most 128 tiles of 128x128 but >= 256 of 64x64, K <= 8192: 64x64, no split
    for dtype in (1, 2):
        for M, N, K in ((512, 2048, 5632), (512, 2048, 1024), (1024, 1024, 4096), (512, 4096, 4096)):
            assert tile_of(M, N, K, dtype) == (64, 64), (M, N, K, dtype)
            assert dg.dg_gemm_splitk_choose(0, 0, M, N, K, dtype) == 1
    # longer K: the 128x128 tile split over K
    assert tile_of(512, 2048, 16384) == (128, 128)
    assert dg.dg_gemm_splitk_choose(0, 0, 512, 2048, 16384, 1) > 1
    # enough 128x128 tiles (176 for the LoRA gate projection): unchanged
    assert tile_of(512, 5632, 2048) == (128, 128)
    # fp32 has its own rule (at most 256 tiles of 128x128: 64x64, whatever K)
    assert tile_of(512, 2048, 5632, 0) == (64, 64)
    assert tile_of(4096, 4096, 512, 0) != (64, 64)


def test_16bit_large_grids_take_the_tile_that_fills_the_cus_in_one_wave():
    for dtype in (1, 2):
        # the tile with the least time in rounds of 256 workgroups (a round: a
        # fixed part and a part per unit of K; a partly filled round counting
        # 0.82); each of these was the fastest tile when measured, every
        # transpose pair
        for M, N, K, tile in ((4096, 4096, 4096, (256, 256)), (3072, 3072, 3072, (256, 256)),
                              (8192, 8192, 2048, (256, 256)), (6144, 6144, 6144, (256, 256)),
                              (1536, 8192, 2048, (256, 256)), (5120, 5120, 1024, (256, 256)),
                              (3000, 3000, 3000, (256, 256)), (3584, 3584, 3584, (256, 256)),
                              (2048, 4096, 4096, (256, 128)), (2560, 2560, 2560, (256, 128)),
                              (2304, 2048, 2048, (256, 128)), (8192, 1024, 1024, (256, 128)),
                              (4096, 2048, 4096, (256, 128)), (8448, 4096, 2048, (256, 256)),
                              (6400, 6400, 2048, (256, 256)), (5120, 4096, 2048, (128, 128)),
                              (4608, 4608, 2048, (256, 128)), (4608, 4096, 4096, (128, 128)),
                              (4096, 4224, 4096, (128, 128)), (4224, 4224, 4224, (128, 128)),
                              (4096, 4608, 1024, (128, 128)),
                              (4352, 4096, 4096, (128, 128))):
            for ta, tb in ((0, 0), (1, 0), (0, 1)):
                k = dg.dg_select_kernel(ta, tb, M, N, K, 256, M if ta else K, 256, K if tb else N, 256, N,
                                        dtype)
                assert (dg.dg_kernel_tile_m(k), dg.dg_kernel_tile_n(k)) == tile, (M, N, K, ta, tb)
        # at most 128 such tiles: 128x128
        assert tile_of(2048, 2048, 2048, dtype) == (128, 128)
        assert tile_of(2048, 2048, 8192, dtype) == (128, 128)
        # the two-workgroup 128x128 kernel is never chosen
        for M, N, K in ((2048, 4096, 1024), (3072, 3072, 3072), (4096, 4096, 512)):
            k = dg.dg_select_kernel(0, 0, M, N, K, 256, K, 256, N, 256, N, dtype)
            assert "pipe2_ksplit2" not in dg.dg_kernel_name(k)


def test_fp32_tile_by_rounds():
    # the tile with the fewest tile-times per CU (ceil(tiles / 256) times a
    # tile's time relative to 128x128: 1.933, 1, 0.51, 0.2636), 256x128 only
    # where its tiles fill whole rounds of two per CU; each of these was the
    # fastest of the four tiles when measured
    for M, N, K, tile in ((4096, 4096, 4096, (256, 128)), (8192, 8192, 2048, (256, 128)),
                          (2048, 8192, 4096, (256, 128)), (4096, 4096, 1024, (256, 128)),
                          (1024, 16384, 4096, (256, 128)), (6144, 6144, 6144, (128, 128)),
                          (3072, 4096, 4096, (128, 128)), (5120, 4096, 2048, (128, 128)),
                          (6144, 6144, 2048, (128, 128)), (2048, 3072, 2048, (128, 64)),
                          (4096, 4224, 4096, (64, 64)), (2560, 2560, 2560, (64, 64)),
                          (3584, 3584, 3584, (64, 64)), (2304, 2048, 2048, (64, 64))):
        assert tile_of(M, N, K, 0) == tile, (M, N, K)
    # at most one 128x128 tile per CU and at least one 64x64 tile per CU: the
    # 64x64 tile, every transpose pair (the tall-skinny 8192x256x8192 of the
    # full-form workload, 1024^3, 2048^3);
    # 32-deep slabs in three stages (three workgroups per CU) unless the grid
    # has 769 to 1024 tiles, which four 16-deep workgroups per CU hold in one
    # round
    for M, N, K, name in ((8192, 256, 8192, "f32_64x64_pipe3_k32_mfma32x32x2"),
                          (1024, 1024, 1024, "f32_64x64_pipe3_k32_mfma32x32x2"),
                          (2048, 2048, 2048, "f32_64x64_pipe4_mfma32x32x2"),
                          (1792, 1792, 2048, "f32_64x64_pipe4_mfma32x32x2"),
                          (256, 8192, 8192, "f32_64x64_pipe3_k32_mfma32x32x2"),
                          (3072, 1024, 2048, "f32_64x64_pipe3_k32_mfma32x32x2"),
                          (2304, 2048, 2048, "f32_64x64_pipe3_k32_mfma32x32x2")):
        for ta, tb in ((0, 0), (1, 0), (0, 1), (1, 1)):
            lda, ldb = (M if ta else K) + 8, (K if tb else N) + 8
            k = dg.dg_select_kernel(ta, tb, M, N, K, 256, lda, 256, ldb, 256, N + 8, 0)
            assert dg.dg_kernel_name(k) == name, (M, N, K, ta, tb)
    # fewer 64x64 tiles than CUs: the 32x32 tile with four K groups, four
    # stages from K = 512
    for M, N, K in ((512, 512, 512), (256, 256, 256), (768, 768, 768), (512, 512, 8192), (900, 900, 64),
                    (64, 4096, 1024), (128, 128, 508), (128, 128, 4096)):
        name = f"f32_32x32_pipe{4 if K >= 512 else 3}_k32_ksplit4_mfma32x32x2"
        for ta, tb in ((0, 0), (1, 0), (0, 1), (1, 1)):
            lda, ldb = (M if ta else K) + 8, (K if tb else N) + 8
            k = dg.dg_select_kernel(ta, tb, M, N, K, 256, lda, 256, ldb, 256, N + 8, 0)
            assert dg.dg_kernel_name(k) == name, (M, N, K, ta, tb)
    # the 4-byte-load kernels follow the same rule (K and N not multiples of 4):
    # 4097 columns end in a partly filled round of the larger tiles.  On the
    # 64x64 tile a k-contiguous operand takes 16-byte loads (nn, tt: 16-deep
    # slabs); tn, with none, keeps the 4-byte kernel; nt (both operands
    # k-contiguous, rows 4-byte aligned) runs the 16-byte kernel itself
    M, N, K = 4095, 4097, 1031
    for (ta, tb), name in (((0, 0), "f32_64x64_pipe4_kw_mfma32x32x2"), ((1, 1), "f32_64x64_pipe4_kw_mfma32x32x2"),
                           ((0, 1), "f32_64x64_pipe3_k32_mfma32x32x2"), ((1, 0), "f32_64x64_pipe4_dw_mfma32x32x2")):
        lda, ldb = (M if ta else K) + 8, (K if tb else N) + 8
        k = dg.dg_select_kernel(ta, tb, M, N, K, 256, lda, 256, ldb, 256, N + 8, 0)
        assert dg.dg_kernel_name(k) == name, (ta, tb)
    k = dg.dg_select_kernel(0, 0, 4096, 4096, 4095, 256, 4095, 256, 4096, 256, 4096, 0)
    assert dg.dg_kernel_name(k) == "f32_256x128_pipe3_mfma32x32x2"      # 4-byte rows suffice
    k = dg.dg_select_kernel(0, 0, 4096, 4095, 4095, 256, 4095, 256, 4095, 256, 4096, 0)
    assert dg.dg_kernel_name(k) == "f32_256x128_pipe3_dw_mfma32x32x2"   # N not a multiple of 4


def test_pipelined_kernels_need_32bit_panel_offsets():
    # a tile panel is addressed with 32-bit byte offsets: 256 rows of the
    # stored matrix must span less than 2^31 bytes, else the register-staged
    # kernels take the problem
    for dtype, esize in ((0, 4), (1, 2), (2, 2)):
        big = (1 << 31) // (256 * esize)          # the first row stride that does not fit
        for ld, pipe in ((big - 64, True), (big, False)):
            k = dg.dg_select_kernel(0, 0, 512, 512, 512, 256, ld, 256, 512, 256, 512, dtype)
            assert ("pipe" in dg.dg_kernel_name(k)) == pipe, (dtype, ld, dg.dg_kernel_name(k))
            k = dg.dg_select_kernel(0, 0, 512, 512, 512, 256, 512, 256, ld, 256, 512, dtype)
            assert ("pipe" in dg.dg_kernel_name(k)) == pipe, (dtype, ld, dg.dg_kernel_name(k))


def test_16bit_unaligned_c_rows_take_the_128x128_tile():
    # 16-bit C rows not 4-byte aligned (odd ldc): the 128x128 tile replaces
    # the one-round 256x256 / 256x128 tiles of the model; an even ldc keeps
    # the 16-byte epilogue and the model's tile
    for dtype, tile in ((dg.DG_F16_F32ACC, "f16_128x128_pipe4_ksplit2_mfma32x32x16"),
                        (dg.DG_BF16_F32ACC, "bf16_128x128_pipe4_ksplit2_mfma32x32x16")):
        for M, N, K in ((4096, 4096, 1032), (2048, 4096, 520), (4096, 4096, 4096), (8192, 8192, 1032)):
            for ta, tb in ((0, 0), (0, 1), (1, 0), (1, 1)):
                lda, ldb = (M if ta else K), (K if tb else N)
                sel = lambda ldc: dg.dg_kernel_name(
                    dg.dg_select_kernel(ta, tb, M, N, K, 256, lda, 256, ldb, 256, ldc, dtype))
                assert sel(N + 1) == tile, (dtype, M, N, K, ta, tb)
                assert sel(N + 8) == sel(N + 2) == sel(N)
                assert "256x" in sel(N), sel(N)


def test_forced_pipelined_kernel_refused_past_the_panel_limit():
    # forcing a pipelined kernel on such a stride is refused before anything
    # is enqueued (no device is touched, so this runs without a GPU)
    names = dg.kernel_names()
    for dtype, esize in ((dg.DG_F32, 4), (dg.DG_F16_F32ACC, 2), (dg.DG_BF16_F32ACC, 2)):
        big = (1 << 31) // (256 * esize)
        prefix = ("f32", "f16", "bf16")[dtype] + "_"
        pipes = [i for i, n in enumerate(names) if n.startswith(prefix) and "pipe" in n]
        assert pipes
        for k in pipes:
            for lda, ldb in ((big, 600), (600, big)):
                rc = dg.dg_gemm_with_kernel(0, 0, 600, 600, 600, 1.0, 0x1000, lda, 0x2000, ldb,
                                            0.0, 0x3000, 600, dtype, NULL, k)
                assert rc == dg.DG_ERR_UNSUPPORTED, (names[k], lda, ldb, rc)


def test_tile_grid_matches_the_pages_decompositions():
    """Output tiles of side T cover C[35,93] at ((35//T)*T, (93//T)*T): the
    8x8 tile at (32,88) entry (3,5) and the 64x64 tile at (0,64) of the pages
    (golden file), and for this library's tiles the same arithmetic."""
    from test_oracle import read_golden
    g = read_golden("c35_93.txt")
    r, c = g["row"], g["col"]
    for t, r0, c0 in ((g["k5_tile"], g["k5_tile_row0"], g["k5_tile_col0"]),
                      (g["k8_tile"], g["k8_tile_row0"], g["k8_tile_col0"])):
        assert (r // t * t, c // t * t) == (r0, c0)
    for i in range(dg.dg_kernel_count()):
        bm, bn = dg.dg_kernel_tile_m(i), dg.dg_kernel_tile_n(i)
        assert 0 <= r - (r // bm) * bm < bm and 0 <= c - (c // bn) * bn < bn


def test_status_strings():
    assert dg.dg_status_string(0) == "ok"
    assert "HIP" in dg.dg_status_string(dg.DG_ERR_HIP)
    assert dg.dg_status_string(12345) == "unknown status"
    assert dg.dg_last_hip_error() == 0
    assert dg.dg_version() >= 100


def test_splitk_host_logic():
    # the library's choice: split only grids that leave compute units idle
    assert dg.dg_gemm_splitk_choose(0, 0, 512, 32, 5632, 1) > 1          # LoRA dGa
    assert dg.dg_gemm_splitk_choose(0, 0, 4096, 4096, 4096, 0) == 1
    assert dg.dg_gemm_splitk_choose(0, 0, 512, 32, 64, 1) == 1            # too little K
    assert dg.dg_gemm_splitk_choose(2, 0, 512, 32, 64, 1) == -1
    assert dg.dg_gemm_splitk_workspace_size(512, 32, 22) == 22 * 512 * 32 * 4
    assert dg.dg_gemm_splitk_workspace_size(512, 32, 1) == 0
    assert dg.dg_gemm_splitk_workspace_size(0, 32, 4) == 0


def test_splitk_invalid_arguments():
    def sk(**kw):
        a = dict(GOOD, splits=2, ws=0x10000, wsb=1 << 20)
        a.update(kw)
        return dg.dg_gemm_splitk(a["ta"], a["tb"], a["M"], a["N"], a["K"], a["alpha"], a["A"],
                                 a["lda"], a["B"], a["ldb"], a["beta"], a["C"], a["ldc"],
                                 a["dtype"], a["stream"], a["splits"], a["ws"], a["wsb"])
    assert sk(ta=3) == -1                       # dg_gemm's checks come first
    assert sk(splits=-1) == -16
    assert sk(splits=5000) == -16
    assert sk(ws=None) == -17
    assert sk(ws=0x10004) == -17                # not 16-byte aligned
    # a workspace too small for the ranges used: rejected before any launch
    assert sk(M=512, N=32, K=5632, lda=5632, ldb=32, ldc=32, splits=8, wsb=1024) == -18
    assert sk(M=0, ws=None) == 0                # empty output: nothing to do
    assert "workspace too small" in dg.dg_status_string(-18)


# ---- the extended entry point (bias + activation epilogue, strided batches) ----
GOOD_EX = dict(ta=0, tb=0, M=16, N=16, K=16, alpha=1.0, A=0x1000, lda=16, sA=256, B=0x2000, ldb=16,
               sB=256, beta=0.0, C=0x3000, ldc=16, sC=256, batch=2, bias=0x4000, epi=1, dtype=1,
               stream=NULL)


def call_ex(**kw):
    a = dict(GOOD_EX)
    a.update(kw)
    return dg.dg_gemm_ex(a["ta"], a["tb"], a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"],
                         a["sA"], a["B"], a["ldb"], a["sB"], a["beta"], a["C"], a["ldc"], a["sC"],
                         a["batch"], a["bias"], a["epi"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(ta=2), -1), (dict(tb=-1), -2), (dict(M=-1), -3), (dict(N=-1), -4), (dict(K=-1), -5),
    (dict(A=NULL), -7), (dict(lda=15), -8), (dict(sA=-1), -9),
    (dict(B=NULL), -10), (dict(ldb=15), -11), (dict(sB=-16), -12),
    (dict(C=NULL), -14), (dict(ldc=15), -15),
    # batches of C overlap: batch 1 would start inside batch 0 (needs >= 15*16+16)
    (dict(sC=-1), -16), (dict(sC=255), -16), (dict(ldc=32, sC=256 + 16), -16),
    (dict(batch=-1), -17), (dict(batch=65536), -17),
    (dict(bias=0x4001), -18),            # fp16 bias not aligned to its element
    (dict(epi=3), -19), (dict(epi=-1), -19),
    (dict(dtype=5), -20),
    (dict(ta=9, sA=-1, epi=7), -1),      # the first invalid argument is the one reported
])
def test_ex_invalid_arguments(kw, code):
    assert call_ex(**kw) == code
    assert dg.dg_status_string(code).startswith("invalid")


def test_ex_quick_returns_and_valid_strides():
    assert call_ex(M=0) == 0
    assert call_ex(batch=0, A=NULL, B=NULL, C=NULL) == 0      # nothing to do, nothing read
    assert call_ex(M=0, C=NULL, batch=3) == 0
    # the tightest non-overlapping C stride, and stride 0 for a shared A or B, pass the checks:
    # M = 0 keeps the call on the CPU
    assert call_ex(M=0, sC=0, batch=1) == 0
    assert call_ex(M=0, sA=0, sB=0) == 0
    # fp32 bias needs 4-byte alignment
    assert call_ex(dtype=0, bias=0x4002) == -18
    assert call_ex(dtype=0, bias=0x4004, M=0) == 0


def test_ex_forced_kernel_checks():
    n = dg.dg_kernel_count()
    a = dict(GOOD_EX)
    rc = dg.dg_gemm_ex_with_kernel(0, 0, 16, 16, 16, 1.0, 0x1000, 16, 256, 0x2000, 16, 256, 0.0,
                                   0x3000, 16, 256, 2, NULL, 0, 1, NULL, n)
    assert rc == dg.DG_ERR_UNSUPPORTED
    # a kernel of another dtype is refused before any launch
    f32_kernel = dg.kernel_names().index("f32_64x64_simple")
    rc = dg.dg_gemm_ex_with_kernel(0, 0, 16, 16, 16, 1.0, 0x1000, 16, 256, 0x2000, 16, 256, 0.0,
                                   0x3000, 16, 256, 2, NULL, 0, 1, NULL, f32_kernel)
    assert rc == dg.DG_ERR_UNSUPPORTED
    del a


def test_bf16_kernels_listed():
    names = dg.kernel_names()
    for n in ("bf16_64x64_simple", "bf16_128x128_pipe4_ksplit2_mfma32x32x16",
              "bf16_256x128_pipe2_w8_mfma32x32x16", "bf16_256x256_pipe2_w8_mfma32x32x16"):
        assert n in names
