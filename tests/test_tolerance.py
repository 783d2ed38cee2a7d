"""Pins of the parity bar (``oracle.tolerance``) to bf16 itself.

The half-ulp term of the bf16 bound must be the real spacing of bf16 values
at the output's binade, and must cover the one rounding of an fp32 result
into bf16.  Both are checked against bf16 bit patterns, not against the
helper's own formula.
"""
import numpy as np

from oracle import tolerance
from workloads import round_to_dtype


def _bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def test_ulp_is_the_spacing_of_bf16_values():
    rng = np.random.default_rng(0)
    # Positive finite bf16 patterns from 2^-20 to 2^20, and the next pattern up.
    bits = rng.integers(0x3580, 0x4980, size=4000).astype(np.uint32)
    x = _bf16_to_f64(bits)
    nxt = _bf16_to_f64(bits + 1)
    assert np.array_equal(tolerance.bf16_ulp(x), nxt - x)
    assert np.array_equal(tolerance.bf16_ulp(-x), nxt - x)


def test_ulp_at_named_points():
    assert tolerance.bf16_ulp(1.0) == 2.0 ** -7
    assert tolerance.bf16_ulp(1.99) == 2.0 ** -7
    assert tolerance.bf16_ulp(2.0) == 2.0 ** -6
    assert tolerance.bf16_ulp(3.9) == 2.0 ** -6
    assert tolerance.bf16_ulp(-4.0) == 2.0 ** -5
    assert tolerance.bf16_ulp(0.75) == 2.0 ** -8


def test_one_rounding_stays_within_half_an_ulp_of_the_result():
    rng = np.random.default_rng(1)
    x = rng.uniform(-9, 9, size=200_000).astype(np.float32)
    # values just below powers of two, where rounding can cross into the next binade
    edges = np.float32(2.0) ** np.arange(-3, 4, dtype=np.float32)
    near = (edges[:, None] * (1 - rng.uniform(0, 2 ** -8, size=(1, 500)))).astype(np.float32).ravel()
    x = np.concatenate([x, near, -near])
    r = _bf16_to_f64(round_to_dtype(x, "bf16"))
    err = np.abs(r - x.astype(np.float64))
    assert (err <= 0.5 * tolerance.bf16_ulp(r)).all()


def test_bars():
    want = np.zeros(1000)
    want[:3] = [0.5, 3.0, -5.0]

    def bump(i, d):
        g = want.copy()
        g[i] += d
        return g
    assert tolerance.check(bump(0, 0.0099), want, "f16")[0]
    ok, st = tolerance.check(bump(0, 0.0101), want, "f16")
    assert not ok and "bound" in st["msg"]
    # bf16 at |o| = 3: 1e-2 plus half of 2^-6
    assert tolerance.check(bump(1, 0.0177), want, "bf16")[0]
    assert not tolerance.check(bump(1, 0.0179), want, "bf16")[0]
    # at |o| = 0.5 the bf16 term is 2^-9
    assert tolerance.check(bump(0, 0.0119), want, "bf16")[0]
    assert not tolerance.check(bump(0, 0.0121), want, "bf16")[0]
    # mean bar
    ok, st = tolerance.check(np.full(10, 1.002), np.ones(10), "f16")
    assert not ok and "mean" in st["msg"]
    assert tolerance.check(np.full(10, 1.0 + 2e-6), np.ones(10), "f32")[0]
    assert not tolerance.check(np.full(10, 1.0 + 2e-5), np.ones(10), "f32")[0]
    ok, st = tolerance.check(np.array([np.nan]), np.array([0.0]), "f32")
    assert not ok and "non-finite" in st["msg"]
