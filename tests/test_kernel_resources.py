"""Every kernel of the library compiles without scratch memory or spilled
vector registers, by the compiler's resource-usage report (a device-only
compile of each kernel source with the library's own flags; no GPU needed).
Scalar registers may spill: they go to lanes of vector registers, not to
memory, and the kernels that do it keep the spills out of their main loop."""
import importlib.util
import os
import shutil

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("dg_build", os.path.join(ROOT, "dense_gemm_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is not installed")
def test_no_kernel_uses_scratch_or_spills_vector_registers():
    rows = _build_module().resources()
    names = [r["kernel"] for r in rows]
    # the pipelined, register-staged, simple and reduction kernels of all dtypes
    assert len(rows) >= 250, len(rows)
    assert any("gemm_pipe_kernel" in n for n in names) and any("splitk_reduce" in n for n in names)
    bad = [(r["kernel"], r.get("scratch"), r.get("vgpr_spill")) for r in rows
           if r.get("scratch") != 0 or r.get("vgpr_spill") != 0]
    assert not bad, bad
    # the one-workgroup-per-CU 16-bit tiles keep two waves per SIMD
    for r in rows:
        if "gemm_pipe_kernelIDF16_Li128ELi128ELi64ELi64E" in r["kernel"] and "Li4ELi2ELi16E" in r["kernel"]:
            assert r["occupancy"] >= 2, r
