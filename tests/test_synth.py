"""The seeded input generator: published SplitMix64 outputs, ranges,
determinism, and the layout helper."""
import numpy as np

import synth


def test_splitmix64_reference_outputs():
    # first five outputs of the reference SplitMix64 for seed 1234567
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    got = synth.splitmix64(1234567, 0, 5)
    assert [int(x) for x in got] == want
    # counter based: any window of the stream is the same words
    assert [int(x) for x in synth.splitmix64(1234567, 2, 3)] == want[2:]


def test_uniform_ranges_and_determinism():
    st = synth.Stream(5)
    u = st.uniform((1000,))
    assert u.min() >= -1.0 and u.max() < 1.0
    assert abs(u.mean()) < 0.1
    st2 = synth.Stream(5)
    assert np.array_equal(st2.uniform((1000,)), u)
    n = synth.Stream(6).normal((20000,))
    assert abs(n.mean()) < 0.05 and abs(n.std() - 1.0) < 0.05


def test_problem_rounding_and_shared_operands():
    a, b, c0 = synth.problem(16, 24, 32, "f16", "normal_sqrtk", 2, with_c0=True)
    assert a.dtype == np.float16 and b.shape == (32, 24) and c0.shape == (16, 24)
    a32, b32, _ = synth.problem(16, 24, 32, "f32", "uniform", 4)
    assert a32.dtype == np.float32
    # the logical operands do not depend on the transpose variant: only store() does
    A, lda = synth.store(a32, True, 16 + 8)
    assert A.shape == (32, 24) and lda == 24
    assert np.array_equal(A[:, :16], a32.T)
    assert np.all(np.isnan(A[:, 16:]))


def test_integers_in_range():
    x = synth.Stream(9).integers((5000,), -2, 2)
    assert set(np.unique(x).tolist()) == {-2.0, -1.0, 0.0, 1.0, 2.0}
