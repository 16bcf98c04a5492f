"""Build libdense_gemm_amd.so for gfx950 with hipcc, in place.

    python dense_gemm_amd/build.py                # build
    python dense_gemm_amd/build.py --resources    # registers, scratch, LDS per kernel

(run by path: importing the package would load the library being rebuilt)

Each source compiles to an object in _build/ (in parallel), then one link.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdense_gemm_amd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.cpp", "gemm_simple.hip", "gemm_f32.hip", "gemm_f16.hip", "gemm_bf16.hip",
           "gemm_f16_o32.hip", "gemm_bf16_o32.hip"]
# the control probes of the measurements, a library of their own
PROBE_LIB = os.path.join(PKG, "libdense_gemm_probe.so")
PROBE_SOURCES = ["probe.hip"]
HEADERS = ["gemm_common.hpp", "gemm_mfma.hpp", "gemm_pipe.hpp", "gemm_tables16.hpp"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops off (v_pk_fma_f32 and friends are not emitted)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = SOURCES + PROBE_SOURCES
    jobs = min(len(sources), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, sources))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


# ---- register, scratch and LDS use of every kernel ------------------------
# The compiler's resource-usage remarks (-Rpass-analysis=kernel-resource-usage)
# for a device-only compile of each kernel source: the VGPR, AGPR and SGPR
# counts, scratch bytes per lane, spills, occupancy and LDS of every kernel.
_RES_KEYS = {"TotalSGPRs": "sgpr", "VGPRs": "vgpr", "AGPRs": "agpr",
             "ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "occupancy",
             "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill", "LDS Size [bytes/block]": "lds"}


def _resources_of(src: str) -> list:
    cmd = [HIPCC] + FLAGS + ["--cuda-device-only", "-c", "-Rpass-analysis=kernel-resource-usage",
                             os.path.join(CSRC, src), "-o", os.devnull]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    rows, cur = [], None
    for line in r.stderr.splitlines():
        if "remark:" not in line:
            continue
        text = line.split("remark:", 1)[1].split("[-Rpass", 1)[0].strip()
        if text.startswith("Function Name:"):
            cur = {"source": src, "kernel": text.split(":", 1)[1].strip()}
            rows.append(cur)
        elif cur is not None and ":" in text:
            key, val = text.rsplit(":", 1)
            if key.strip() in _RES_KEYS:
                v = val.strip()
                cur[_RES_KEYS[key.strip()]] = int(v) if v.lstrip("-").isdigit() else v
    return rows


def resources() -> list:
    """Resource use of every kernel of the library, one dict per kernel."""
    srcs = [s for s in SOURCES if s.endswith(".hip")]
    with ThreadPoolExecutor(len(srcs)) as ex:
        return [row for rows in ex.map(_resources_of, srcs) for row in rows]


def resources_table(rows: list) -> str:
    cols = ["vgpr", "agpr", "sgpr", "scratch", "vgpr_spill", "sgpr_spill", "occupancy", "lds"]
    out = ["| source | kernel | " + " | ".join(cols) + " |", "|---|---|" + "---|" * len(cols)]
    for r in rows:
        out.append(f"| {r['source']} | `{r['kernel']}` | " + " | ".join(str(r.get(c, "")) for c in cols) + " |")
    return "\n".join(out)


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--resources":
        print(resources_table(resources()))
    else:
        build()
    sys.exit(0)
