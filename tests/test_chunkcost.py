"""The chunk recomputation-cost table: piecewise-linear interpolation of
measured attention times (Pensieve page, 重算成本估算: measured offline at some
context sizes, interpolated for the others)."""
import math

import pytest

from paged_kv_cache_block_amd.chunkcost import ChunkCostProfile


def test_exact_at_measured_contexts_and_linear_between():
    p = ChunkCostProfile(32, [0, 1024, 4096], [10.0, 30.0, 90.0])
    assert p.attention_us(0) == 10.0 and p.attention_us(1024) == 30.0 and p.attention_us(4096) == 90.0
    assert p.attention_us(512) == pytest.approx(20.0)
    assert p.attention_us(2560) == pytest.approx(60.0)


def test_reproduces_a_linear_cost_everywhere():
    a, b = 7.5, 0.013          # any linear attention cost is interpolated exactly
    xs = [0, 100, 1000, 5000]
    p = ChunkCostProfile(32, xs, [a + b * x for x in xs])
    for x in (0, 1, 57, 999, 1000, 3000, 5000, 20000):
        assert p.attention_us(x) == pytest.approx(a + b * x, rel=1e-12)


def test_extrapolation_and_clamping():
    p = ChunkCostProfile(32, [256, 1024], [20.0, 50.0])
    assert p.attention_us(0) == 20.0                   # before the first measurement
    assert p.attention_us(2048) == pytest.approx(90.0)   # last slope continues
    assert p.cost_us(1024, other_us=12.0) == pytest.approx(62.0)


def test_monotone_input_gives_monotone_cost():
    p = ChunkCostProfile(32, [0, 256, 1024, 4096, 16384], [5.0, 6.0, 9.0, 21.0, 70.0])
    vals = [p.attention_us(x) for x in range(0, 20000, 97)]
    assert all(b >= a for a, b in zip(vals, vals[1:]))
    assert all(math.isfinite(v) for v in vals)


def test_round_trip_and_validation():
    p = ChunkCostProfile(32, [0, 64], [1.0, 2.0], {"batch": 1})
    q = ChunkCostProfile.from_dict(p.to_dict())
    assert q == p
    with pytest.raises(ValueError):
        ChunkCostProfile(32, [0, 0], [1.0, 2.0])
    with pytest.raises(ValueError):
        ChunkCostProfile(32, [0, 1], [1.0])
