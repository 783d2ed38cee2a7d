"""Attention cost of recomputing one fixed-size chunk, as a function of its context.

Pensieve page (细粒度的缓存驱逐策略; 重算成本估算; figure 4): the eviction policy
ranks a chunk of 32 tokens by a retention value, its recomputation cost over
the time since the conversation was last active.  The cost is an attention
part that grows with the context the chunk attends over, plus a constant for
the rest of the layer; the attention part is measured offline at a few
context sizes and interpolated between them.  This module holds that
measured table and its interpolation; ``bench.py --chunk-cost`` measures the
table with the library's multi-token kernel.  The eviction policy itself is
not part of this library.
"""
from __future__ import annotations

import bisect
from dataclasses import dataclass, field
from typing import Sequence


@dataclass
class ChunkCostProfile:
    """Measured attention time (microseconds) of one chunk at given contexts.

    ``contexts`` are the numbers of cached tokens before the chunk, strictly
    increasing; ``micros`` the measured times.  Between two measured contexts
    the cost is linear; past the last one it continues the last segment's
    slope (attention work grows linearly with the context); before the first
    one it is the first measurement.
    """
    chunk: int
    contexts: Sequence[int]
    micros: Sequence[float]
    meta: dict = field(default_factory=dict)

    def __post_init__(self):
        if len(self.contexts) != len(self.micros) or not self.contexts:
            raise ValueError("contexts and micros must be non-empty and of equal length")
        if any(b <= a for a, b in zip(self.contexts, self.contexts[1:])):
            raise ValueError("contexts must be strictly increasing")

    def attention_us(self, context: float) -> float:
        """Interpolated attention time of the chunk after ``context`` tokens."""
        xs, ys = self.contexts, self.micros
        if context <= xs[0] or len(xs) == 1:
            return float(ys[0])
        i = bisect.bisect_right(xs, context) - 1
        i = min(i, len(xs) - 2)
        x0, x1, y0, y1 = xs[i], xs[i + 1], ys[i], ys[i + 1]
        return float(y0 + (y1 - y0) * (context - x0) / (x1 - x0))

    def cost_us(self, context: float, other_us: float) -> float:
        """Recomputation cost of the chunk: attention plus the context-free rest."""
        return self.attention_us(context) + other_us

    def to_dict(self) -> dict:
        return {"chunk": self.chunk, "contexts": list(self.contexts),
                "micros": [float(y) for y in self.micros], "meta": dict(self.meta)}

    @classmethod
    def from_dict(cls, d: dict) -> "ChunkCostProfile":
        return cls(int(d["chunk"]), [int(x) for x in d["contexts"]], [float(y) for y in d["micros"]],
                   dict(d.get("meta", {})))
