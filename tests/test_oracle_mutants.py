"""Plant plausible mistakes in a copy of the oracle's C source, build each
mutant on the CPU and check that the pins in test_oracle.py reject it.  This
shows the pins are strong enough that a dropped term, a wrong sign or index or
a transposed operand in the oracle would not go unnoticed."""
import multiprocessing
import os
import shutil
import subprocess

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle_gemm.c")

# (name, text in the source, replacement)
MUTANTS = [
    ("A transpose ignored", "return j->ta ? elem(j->A, j->tyA, k * j->lda + i)",
     "return j->ta ? elem(j->A, j->tyA, i * j->lda + k)"),
    ("B transpose ignored", "return j->tb ? elem(j->B, j->tyB, c * j->ldb + k)",
     "return j->tb ? elem(j->B, j->tyB, k * j->ldb + c)"),
    ("lda used as ldb", "elem(j->B, j->tyB, k * j->ldb + c)", "elem(j->B, j->tyB, k * j->lda + c)"),
    ("last k dropped", "for (int64_t k = 0; k < j->K; ++k) {      /* ikj",
     "for (int64_t k = 0; k < j->K - 1; ++k) {      /* ikj"),
    ("first k dropped", "for (int64_t k = 0; k < j->K; ++k) {      /* ikj",
     "for (int64_t k = 1; k < j->K; ++k) {      /* ikj"),
    ("beta sign flipped", "r += j->beta * elem(j->C0, j->tyC, i * j->ldc + c);\n            j->ref",
     "r -= j->beta * elem(j->C0, j->tyC, i * j->ldc + c);\n            j->ref"),
    ("beta term dropped", "r += j->beta * elem(j->C0, j->tyC, i * j->ldc + c);\n            j->ref",
     "(void)0;\n            j->ref"),
    ("alpha ignored", "double r = use_ab ? j->alpha * acc[c] : 0.0;",
     "double r = use_ab ? acc[c] : 0.0;"),
    ("C0 read with ld = N", "elem(j->C0, j->tyC, i * j->ldc + c);\n            j->ref",
     "elem(j->C0, j->tyC, i * j->N + c);\n            j->ref"),
    ("absum without abs", "abs_[c] += fabs(p);", "abs_[c] += p;"),
    ("fp16 exponent bias off by one", "ldexp((double)(f + 1024), e - 25)",
     "ldexp((double)(f + 1024), e - 24)"),
    ("fp16 subnormals scaled wrong", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    ("C0 read when beta is 0", "if (j->beta != 0.0)\n                r += j->beta",
     "if (1)\n                r += j->beta"),
    ("A read when alpha is 0", "int use_ab = (j->alpha != 0.0) && (j->K > 0);\n    double *acc",
     "int use_ab = (j->K > 0);\n    double *acc"),
    ("row index of A transposed into column", "a = opA(j, i, k);", "a = opA(j, k % j->M, i % j->K);"),
    ("product sign flipped", "double p = a * opB(j, k, c);", "double p = -a * opB(j, k, c);"),
    ("accumulation in fp32", "double p = a * opB(j, k, c);\n                    acc[c] += p;",
     "double p = a * opB(j, k, c);\n                    acc[c] = (float)(acc[c] + p);"),
]

# pins run against each mutant (the full-result entry point is the one mutated)
PIN_CALLS = [
    ("brute force f32", lambda: pins.test_bruteforce_all_tiny_shapes("f32")),
    ("brute force f16", lambda: pins.test_bruteforce_all_tiny_shapes("f16")),
    ("f16 decode", pins.test_f16_decode_every_bit_pattern),
] + [(f"integer {ta}{tb}", (lambda ta=ta, tb=tb: pins.test_integer_inputs_exact(ta, tb, "f32")))
     for ta, tb in pins.TRANS] + [
    ("alpha zero", pins.test_alpha_zero_reads_neither_A_nor_B),
    ("beta zero", pins.test_beta_zero_does_not_read_C),
    ("exact sum", pins.test_against_exactly_rounded_sum),
]


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(name, old, new, workdir):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for '{name}' not found"
    mutated = src.replace(old, new, 1)
    tag = "".join(ch if ch.isalnum() else "_" for ch in name)
    cpath = os.path.join(workdir, f"{tag}.c")
    lpath = os.path.join(workdir, f"lib{tag}.so")
    with open(cpath, "w") as f:
        f.write(mutated)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                    cpath, "-o", lpath, "-lm"], check=True)
    # run the pins in a forked child: a mutant may also crash (that rejects it too)
    ctx = multiprocessing.get_context("fork")
    q = ctx.Queue()
    proc = ctx.Process(target=_run_pins, args=(lpath, q))
    proc.start()
    proc.join(300)
    if proc.is_alive():
        proc.kill()
        proc.join()
        pytest.fail(f"mutant '{name}' hung the pins")
    if proc.exitcode != 0:
        return  # crashed: rejected
    caught = q.get()
    assert caught, f"no pin rejects the mutant '{name}'"


def _run_pins(lpath, q):
    oracle._lib = oracle.bind(lpath)
    caught = []
    for pin_name, fn in PIN_CALLS:
        try:
            fn()
        except AssertionError:
            caught.append(pin_name)
    q.put(caught)
