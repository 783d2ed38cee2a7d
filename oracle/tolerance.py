"""The parity bar between the GPU output and the float64 oracle.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: ``tests/`` and
``__graft_entry__.smoke()`` use it to judge a GPU result.

Bars, per element of the attention output:

* fp32 inputs: ``|got - want| <= 1e-5``;
* fp16 inputs: ``|got - want| <= 1e-2``;
* bf16 inputs: ``|got - want| <= 1e-2 + ulp_bf16(got) / 2``;

and for fp16 / bf16 the mean of ``|got - want|`` over the compared elements
is at most ``1e-3``.

The bf16 term: the kernels round their fp32 result once, to nearest even,
into the output type.  That rounding alone moves a value by up to half a
unit in the last place of the binade the result lands in (round to nearest
never lands below the binade of the unrounded value), which for bf16 is
``2^-7`` for ``|o|`` in ``[2, 4)`` and ``2^-6`` from 4 on, whatever the
precision of the attention itself.  The 1e-2 budget is kept for the
computation on top of it.  An fp16 output needs no such term: its half ulp
stays below ``2^-7`` up to ``|o| = 16``, and these outputs (convex
combinations of N(0, 1) values) stay far below that.
"""
from __future__ import annotations

import numpy as np

MAX_ABS = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}
MEAN_ABS = {"f32": 1e-5, "f16": 1e-3, "bf16": 1e-3}


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Unit in the last place of bf16 (8 significant bits) at the binade of
    ``|x|``: ``2^(e - 7)`` for ``2^e <= |x| < 2^(e + 1)``; zero maps to the
    ulp at 1 (only ever used as a bound)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    a = np.where(a > 0, a, 1.0)
    _, e = np.frexp(a)              # a = m * 2^e with 0.5 <= m < 1: binade 2^(e-1)
    return np.ldexp(1.0, e - 8)


def element_bound(got: np.ndarray, dtype: str) -> np.ndarray:
    """Allowed ``|got - want|`` per element."""
    if dtype == "bf16":
        return MAX_ABS["bf16"] + 0.5 * bf16_ulp(got)
    return np.full(np.shape(got), MAX_ABS[dtype])


def check(got: np.ndarray, want: np.ndarray, dtype: str):
    """``(ok, stats)`` for a GPU output ``got`` (float64, widened exactly from
    its storage type) against the oracle's ``want``.  ``stats`` holds the
    max and mean of ``|got - want|``, the worst ratio to the element bound,
    and a message naming the first failing bar."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if got.shape != want.shape:
        return False, {"msg": f"shape {got.shape} != {want.shape}"}
    if not np.isfinite(got).all():
        return False, {"msg": "non-finite GPU output"}
    if got.size == 0:
        return True, {"max": 0.0, "mean": 0.0, "worst": 0.0, "msg": ""}
    diff = np.abs(got - want)
    ratio = diff / element_bound(got, dtype)
    stats = {"max": float(diff.max()), "mean": float(diff.mean()), "worst": float(ratio.max())}
    if stats["worst"] > 1.0:
        i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        stats["msg"] = (f"|d| = {diff[i]:.3e} at {tuple(int(j) for j in i)} (got {got[i]:.6g}, "
                        f"want {want[i]:.6g}) exceeds its bound {element_bound(got[i], dtype):.3e}")
        return False, stats
    if stats["mean"] > MEAN_ABS[dtype]:
        stats["msg"] = f"mean |d| = {stats['mean']:.3e} > {MEAN_ABS[dtype]}"
        return False, stats
    stats["msg"] = ""
    return True, stats
