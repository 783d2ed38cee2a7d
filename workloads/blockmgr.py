"""Host-side KV block manager used to build test and benchmark batches.

This is a fixture, not part of the GPU path: it hands out physical block ids,
keeps per-block reference counts and decides copy-on-write, and from that
produces the block tables, slot mappings and copy pairs the library consumes.

Behaviour follows the pages:

* vLLM blog page (devpress.csdn.net), section 1 "vLLM整体架构": a sequence's
  logical blocks fill left to right; a new physical block is taken only when
  the last one is full; the block table records the mapping and how many
  slots of each block are filled.  Worked example: a 7-token prompt with
  block size 4 maps logical blocks 0 and 1 to physical blocks 7 and 1; the
  first decode fills the last free slot of block 1; the second decode takes
  physical block 3.
* vLLM blog page, section 2.1 (parallel sampling): samples share prompt
  blocks with a reference count; a writer that finds its block shared takes
  a new block, has the old one copied into it and drops the old block's
  count by one; the last holder then writes in place.
* vLLM wiki page ("vLLM-SOSP23"), section "核心方法": on-demand allocation
  and copy-on-write sharing through reference counts.
"""
from __future__ import annotations

from collections import deque

import numpy as np


class OutOfBlocks(RuntimeError):
    pass


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        if free_order is None:
            free_order = range(self.num_blocks)
        self.free = deque(int(b) for b in free_order)
        self.ref = np.zeros(self.num_blocks, dtype=np.int64)
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self._preset: dict[int, deque] = {}

    # -- allocation -------------------------------------------------------
    def _take(self) -> int:
        if not self.free:
            raise OutOfBlocks("physical block pool exhausted")
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def reserve(self, blocks) -> None:
        """Remove specific blocks from the free list (they get count 0 until
        a sequence adopts them)."""
        drop = set(int(b) for b in blocks)
        self.free = deque(b for b in self.free if b not in drop)

    # -- sequences --------------------------------------------------------
    def add_sequence(self, seq: int, blocks=None) -> None:
        """Start a sequence, optionally on pre-chosen physical blocks (which
        must have been reserved) that it will fill in order."""
        if seq in self.tables:
            raise ValueError(f"sequence {seq} exists")
        self.tables[seq] = []
        self.lens[seq] = 0
        self._preset[seq] = deque(int(b) for b in (blocks or ()))

    def fork(self, parent: int, child: int) -> None:
        """The child shares every block of the parent (count + 1 each)."""
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        self._preset[child] = deque()
        for b in self.tables[child]:
            self.ref[b] += 1

    def append(self, seq: int, n: int):
        """Append ``n`` tokens; return ``(slots, copy_pairs)``.

        A token at position ``p`` goes to logical block ``p // bs``, offset
        ``p % bs``.  A new physical block is taken when ``offset == 0``.  If the
        target block is shared, it is first replaced by a private copy.
        """
        bs = self.block_size
        table = self.tables[seq]
        slots, pairs = [], []
        for _ in range(int(n)):
            pos = self.lens[seq]
            li, off = divmod(pos, bs)
            if off == 0:
                pre = self._preset[seq]
                if pre:
                    b = pre.popleft()
                    self.ref[b] = 1
                else:
                    b = self._take()
                table.append(b)
            else:
                b = table[li]
                if self.ref[b] > 1:
                    nb = self._take()
                    pairs.append((b, nb))
                    self.ref[b] -= 1
                    table[li] = nb
                    b = nb
            slots.append(b * bs + off)
            self.lens[seq] = pos + 1
        return slots, pairs

    def filled(self, seq: int) -> list[int]:
        """Number of filled slots of each logical block of ``seq``."""
        bs = self.block_size
        n = self.lens[seq]
        return [min(bs, n - i * bs) for i in range(len(self.tables[seq]))]

    def free_sequence(self, seq: int) -> None:
        for b in self.tables.pop(seq):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        self.lens.pop(seq)
