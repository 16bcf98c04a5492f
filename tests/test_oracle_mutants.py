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
import test_oracle_ext as ext

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle_gemm.c")

# (name, text in the source, replacement)
MUTANTS = [
    ("A transpose ignored", "return j->ta ? elem(j->A, j->tyA, o + k * j->lda + i)",
     "return j->ta ? elem(j->A, j->tyA, o + i * j->lda + k)"),
    ("B transpose ignored", "return j->tb ? elem(j->B, j->tyB, o + c * j->ldb + k)",
     "return j->tb ? elem(j->B, j->tyB, o + k * j->ldb + c)"),
    ("lda used as ldb", "elem(j->B, j->tyB, o + k * j->ldb + c)", "elem(j->B, j->tyB, o + k * j->lda + c)"),
    ("last k dropped", "for (int64_t k = 0; k < j->K; ++k) {      /* ikj",
     "for (int64_t k = 0; k < j->K - 1; ++k) {      /* ikj"),
    ("first k dropped", "for (int64_t k = 0; k < j->K; ++k) {      /* ikj",
     "for (int64_t k = 1; k < j->K; ++k) {      /* ikj"),
    ("beta sign flipped", "r += j->beta * elem(j->C0, j->tyC, b * j->sC + i * j->ldc + c);",
     "r -= j->beta * elem(j->C0, j->tyC, b * j->sC + i * j->ldc + c);"),
    ("beta term dropped", "r += j->beta * elem(j->C0, j->tyC, b * j->sC + i * j->ldc + c);",
     "(void)0;"),
    ("alpha ignored", "double r = use_ab ? j->alpha * acc : 0.0;", "double r = use_ab ? acc : 0.0;"),
    ("C0 read with ld = N", "b * j->sC + i * j->ldc + c", "b * j->sC + i * j->N + c"),
    ("absum without abs", "abs_[c] += fabs(p);", "abs_[c] += p;"),
    ("fp16 exponent bias off by one", "ldexp((double)(f + 1024), e - 25)",
     "ldexp((double)(f + 1024), e - 24)"),
    ("fp16 subnormals scaled wrong", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    ("C0 read when beta is 0", "if (j->beta != 0.0)\n        r += j->beta",
     "if (1)\n        r += j->beta"),
    ("A read when alpha is 0", "int use_ab = (j->alpha != 0.0) && (j->K > 0);\n    double *acc",
     "int use_ab = (j->K > 0);\n    double *acc"),
    ("row index of A transposed into column", "a = opA(j, b, i, k);",
     "a = opA(j, b, k % j->M, i % j->K);"),
    ("product sign flipped", "double p = a * opB(j, b, k, c);", "double p = -a * opB(j, b, k, c);"),
    ("accumulation in fp32", "double p = a * opB(j, b, k, c);\n                    acc[c] += p;",
     "double p = a * opB(j, b, k, c);\n                    acc[c] = (float)(acc[c] + p);"),
    # bf16 decoding
    ("bf16 exponent bias off by one", "ldexp((double)(f + 128), e - 134)",
     "ldexp((double)(f + 128), e - 133)"),
    ("bf16 subnormals scaled wrong", "v = ldexp((double)f, -133);", "v = ldexp((double)f, -134);"),
    ("bf16 read as fp16", "case ORC_BF16: return oracle_bf16_to_f64(",
     "case ORC_BF16: return oracle_f16_to_f64("),
    # epilogue
    ("bias indexed by row", "r += elem(j->bias, j->tyBias, c);", "r += elem(j->bias, j->tyBias, i);"),
    ("bias dropped", "r += elem(j->bias, j->tyBias, c);", "(void)0;"),
    ("relu as absolute value", "return x > 0.0 ? x : (x != x ? x : 0.0);", "return fabs(x);"),
    ("gelu by the tanh approximation", "return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));",
     "return 0.5 * x * (1.0 + tanh(0.7978845608028654 * (x + 0.044715 * x * x * x)));"),
    ("gelu with erf argument unscaled", "erf(x / sqrt(2.0))", "erf(x)"),
    ("activation before the bias", "j->ref[o] = activation(j->act, r);",
     "j->ref[o] = j->bias ? activation(j->act, r - elem(j->bias, j->tyBias, c)) + "
     "elem(j->bias, j->tyBias, c) : activation(j->act, r);"),
    # batches
    ("batch stride of B ignored", "int64_t o = b * j->sB;", "int64_t o = 0;"),
    ("A batch stride used for B", "int64_t o = b * j->sB;", "int64_t o = b * j->sA;"),
    ("C0 batch stride ignored", "elem(j->C0, j->tyC, b * j->sC + i * j->ldc + c)",
     "elem(j->C0, j->tyC, i * j->ldc + c)"),
    ("batch row split wrong", "const int64_t b = g / j->M, i = g % j->M;",
     "const int64_t b = g % (j->batch), i = g / (j->batch);"),
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
    ("bf16 decode", ext.test_bf16_decode_every_bit_pattern),
    ("brute force bf16", ext.test_bruteforce_bf16_tiny_shapes),
    ("relu bias integer", lambda: ext.test_relu_bias_integer_exact(False, True, "bf16")),
    ("relu of bias", lambda: ext.test_activation_of_bias_alone("relu")),
    ("gelu of bias", lambda: ext.test_activation_of_bias_alone("gelu")),
    ("gelu closed forms", ext.test_gelu_closed_forms),
    ("batched integer", lambda: ext.test_batched_integer_exact(True, True)),
    ("batched shared operand", ext.test_batched_shared_operand_stride_zero),
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
    import faulthandler
    faulthandler.disable()        # a crashing mutant is an expected outcome, not a report
    oracle._lib = oracle.bind(lpath)
    caught = []
    for pin_name, fn in PIN_CALLS:
        try:
            fn()
        except AssertionError:
            caught.append(pin_name)
    q.put(caught)
