"""The C ABI from plain C: the public header compiles as strict C99 and as
C++, a C program (tests/c_abi/gemm_from_c.c) builds against it with gcc, and
on a GPU that program -- HIP runtime only, no Python or torch in its process --
computes results that match the oracle."""
import os
import re
import struct
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")
C_ABI = os.path.join(ROOT, "tests", "c_abi")


def _c_build():
    """tests/c_abi/build.py, loaded by path."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("c_abi_build", os.path.join(C_ABI, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def declared_functions():
    text = open(os.path.join(HEADER_DIR, "dense_gemm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z_0-9]+)\s*\(", text)))


@pytest.mark.parametrize("lang,std", [("c", "c99"), ("c", "c11"), ("c++", "c++11")])
def test_header_compiles_strictly(tmp_path, lang, std):
    """Every declaration is valid strict C99 / C11 / C++11 without any HIP
    header (plain pointers and sizes only), and each entry point can be taken
    as a function pointer."""
    src = tmp_path / ("probe.c" if lang == "c" else "probe.cpp")
    refs = "\n".join(f"    (void)&{f};" for f in declared_functions())
    src.write_text(f'#include "dense_gemm.h"\nint main(void) {{\n{refs}\n    return DG_OK;\n}}\n')
    cc = "gcc" if lang == "c" else "g++"
    subprocess.run([cc, f"-std={std}", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only",
                    "-I", HEADER_DIR, str(src)], check=True, capture_output=True, text=True)


def test_c_caller_builds():
    exe = _c_build().build()
    assert os.access(exe, os.X_OK)


def write_problem(path, ta, tb, dtype, entry, M, N, K, lda, ldb, ldc, batch, sA, sB, sC, alpha,
                  beta, epilogue, A, B, C0, bias=None):
    code = {"f32": 0, "f16": 1, "bf16": 2}[dtype]
    with open(path, "wb") as f:
        f.write(struct.pack("<4i", int(ta), int(tb), code, entry))
        f.write(struct.pack("<10q", M, N, K, lda, ldb, ldc, batch, sA, sB, sC))
        f.write(struct.pack("<2f", alpha, beta))
        f.write(struct.pack("<2i", epilogue, 1 if bias is not None else 0))
        for x in (A, B, C0) + ((bias,) if bias is not None else ()):
            x = np.ascontiguousarray(x).ravel()
            f.write(struct.pack("<q", x.size))
            f.write(x.tobytes())


def run_c(tmp_path, *args, **kw):
    cbuild = _c_build()
    exe = cbuild.EXE if os.path.exists(cbuild.EXE) else cbuild.build()
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    write_problem(inp, *args, **kw)
    r = subprocess.run([exe, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    return out.read_bytes()


@pytest.mark.gpu
def test_c_caller_dg_gemm_matches_oracle(tmp_path):
    M, N, K = 257, 131, 97
    a, b, c0 = synth.problem(M, N, K, "f32", "uniform", 400, with_c0=True)
    A, lda = synth.store(a, True, M + 3)
    B, ldb = synth.store(b, False, N + 5)
    C0, ldc = synth.store(c0, False, N + 2)
    raw = run_c(tmp_path, True, False, "f32", 0, M, N, K, lda, ldb, ldc, 1, 0, 0, 0, 1.5, -0.5, 0,
                A, B, C0)
    out = np.frombuffer(raw, dtype=np.float32).reshape(M, ldc)
    ref, ab = oracle.gemm(True, False, M, N, K, 1.5, A, lda, B, ldb, -0.5, C0, ldc)
    worst, bad = oracle.compare("f32", out[:, :N], ref, ab, 1.5, -0.5, c0)
    assert bad == 0, worst
    assert np.isnan(out[:, N:]).all()          # the row padding of C is untouched


@pytest.mark.gpu
def test_c_caller_dg_gemm_ex_batched_bias_gelu(tmp_path):
    M, N, K, nb = 136, 72, 64, 3
    st = synth.Stream(401)
    a = synth.round_to(st.uniform((nb * M * K,)), "f16")
    b = synth.round_to(st.uniform((K * N,)), "f16")           # shared by the batches
    c0 = np.zeros(nb * M * N, np.float16)
    bias = synth.round_to(st.uniform((N,)), "f16")
    raw = run_c(tmp_path, False, False, "f16", 1, M, N, K, K, N, N, nb, M * K, 0, M * N, 1.0, 0.0,
                2, a, b, c0, bias)
    out = np.frombuffer(raw, dtype=np.float16).astype(np.float64).reshape(nb, M, N)
    ref, pre, ab = oracle.gemm_ex(False, False, M, N, K, 1.0, a, K, b, N, 0.0, None, N, bias=bias,
                                  act="gelu", batch=nb, strideA=M * K, strideB=0)
    worst, bad = oracle.compare("f16", out, ref, ab, 1.0, 0.0, None, bias[None, None, :].astype(np.float64),
                                "gelu", pre)
    assert bad == 0, worst
