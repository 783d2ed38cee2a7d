"""Seeded synthetic batches for paged KV-cache attention.

Every value is drawn from N(0, 1) with ``numpy.random.default_rng(seed)`` in
float32 and rounded once (round-to-nearest-even) to the storage dtype; both
the GPU path and the oracle consume exactly these rounded values.  Physical
block placement comes from a seeded permutation of the pool, which stands in
for the random physical placement the Pensieve page describes for paged
memory ("多Token注意力内核运算原理", figure 9 caption).

The five named workloads:

1. tiny fp32 mix on a 16-block pool: the worked 7-token prompt on blocks
   [7, 1] plus one decode token (vLLM blog page, section 1), a 5-token
   prefill, and a 9-token history on permuted blocks plus 3 new tokens;
2. 64 decodes at 40 heads x 128, fp16, block size 16, context U{128..2048};
3. a Pensieve-style unified batch: 8 requests with a 256..3072-token history
   held in two separate runs of consecutive physical blocks plus 16..512 new
   tokens, mixed with 56 decodes over 64..2048 tokens; fp16, block size 32;
4. 256 GQA decodes (16 query heads over 2 KV heads), bf16, block size 16,
   lognormal contexts (median 800, sigma 1, capped at 4096); groups of four
   share a prompt and copy-on-write runs before the write;
5. 16 requests with 3000..4096 cached tokens plus 512 new tokens, alongside
   128 decodes over 1024..4096 tokens; 64 query heads over 8 KV heads, bf16,
   block size 32.

Pools start filled with a NaN pattern, so any read outside the written
context shows up in the output.  Unused block-table entries point at a block
that is never written.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .blockmgr import BlockManager

NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
ELT_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def nan_bits(dtype: str):
    """The quiet-NaN bit pattern pools are poisoned with, as a storage scalar."""
    if dtype == "f32":
        return np.array([0x7FC00000], dtype=np.uint32).view(np.float32)[0]
    if dtype == "f16":
        return np.array([0x7E00], dtype=np.uint16).view(np.float16)[0]
    return np.uint16(0x7FC0)


def round_to_dtype(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values once, to nearest even, into the storage dtype."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f32":
        return x32
    if dtype == "f16":
        return x32.astype(np.float16)
    u = x32.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


@dataclass
class Workload:
    name: str
    dtype: str
    num_blocks: int
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    hist_k: np.ndarray          # [T_hist, H_kv, D] history written before the step
    hist_v: np.ndarray
    hist_slots: np.ndarray      # [T_hist] int64
    cow_pairs: np.ndarray       # [n, 2] int32 (src, dst), run before the write
    k_new: np.ndarray           # [T_new, H_kv, D]
    v_new: np.ndarray
    slot_mapping: np.ndarray    # [T_new] int64
    q: np.ndarray               # [T_q, H_q, D]
    block_tables: np.ndarray    # [S, max_blocks] int32
    context_lens: np.ndarray    # [S] int32
    query_start_loc: np.ndarray  # [S + 1] int32
    scale: float
    poison_block: int
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def n_new(self) -> np.ndarray:
        return np.diff(self.query_start_loc).astype(np.int64)

    def pool_shapes(self):
        nb, h, bs, d = self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim
        return (nb, h, bs, d), (nb, h, d, bs)

    def empty_pools(self):
        """Host pools filled with the NaN pattern (K and V layouts differ)."""
        ks, vs = self.pool_shapes()
        fill = nan_bits(self.dtype)
        k = np.full(ks, fill, dtype=NP_STORAGE[self.dtype])
        v = np.full(vs, fill, dtype=NP_STORAGE[self.dtype])
        return k, v

    def kv_bytes_per_token(self) -> int:
        return 2 * self.num_kv_heads * self.head_dim * ELT_BYTES[self.dtype]


def _draw(rng, shape, dtype):
    return round_to_dtype(rng.standard_normal(shape, dtype=np.float32), dtype)


def build_batch(name, dtype, num_q_heads, num_kv_heads, head_dim, block_size,
                num_blocks, seqs, seed, free_order=None, rng=None,
                two_run_gap_max=8) -> Workload:
    """Build a batch from per-sequence ``(history, new, runs)`` triples.

    ``history`` tokens are cached before the step; ``new`` tokens are the
    sequence's query tokens, written by the step and attending causally;
    ``runs == 2`` places the history on two runs of consecutive physical
    blocks that are disjoint and not adjacent (the Pensieve page,
    "丢弃前端Token与非连续缓存的挑战", figure 5: a context split into a
    swapped-in segment and a GPU-resident segment).
    """
    rng = np.random.default_rng(seed) if rng is None else rng
    bs = block_size
    specs = [(int(h), int(n), int(r)) for h, n, r in seqs]

    runs = {}                         # seq -> list of runs (block id lists)
    run_list = []
    for s, (h, n, r) in enumerate(specs):
        if r == 2:
            nbh = -(-h // bs)
            if nbh < 2:
                raise ValueError("a two-run history needs at least two blocks")
            a = int(rng.integers(1, nbh))
            run_list.append((s, 0, a))
            run_list.append((s, 1, nbh - a))
    used = np.zeros(num_blocks, dtype=bool)
    if run_list:
        order = rng.permutation(len(run_list))
        cursor = int(rng.integers(0, two_run_gap_max))
        placed = {}
        for idx in order:
            s, part, length = run_list[idx]
            ids = list(range(cursor, cursor + length))
            placed[(s, part)] = ids
            cursor += length + int(rng.integers(1, two_run_gap_max + 1))
        if cursor > num_blocks:
            raise ValueError("pool too small for the two-run layout")
        for (s, part), ids in placed.items():
            runs.setdefault(s, [None, None])[part] = ids
            used[ids] = True
    if free_order is None:
        rest = np.flatnonzero(~used)
        free_order = rest[rng.permutation(rest.size)]
    mgr = BlockManager(num_blocks, bs, free_order)
    preset = {s: r[0] + r[1] for s, r in runs.items()}
    mgr.reserve([b for ids in preset.values() for b in ids])
    for s in range(len(specs)):
        mgr.add_sequence(s, preset.get(s))
    hist_slots, new_slots = [], []
    for s, (h, n, r) in enumerate(specs):
        sl, pairs = mgr.append(s, h)
        assert not pairs
        hist_slots.extend(sl)
    for s, (h, n, r) in enumerate(specs):
        sl, pairs = mgr.append(s, n)
        assert not pairs
        new_slots.extend(sl)
    return _finish(name, dtype, num_q_heads, num_kv_heads, head_dim, bs,
                   num_blocks, mgr, specs, hist_slots, new_slots, [], rng)


def _finish(name, dtype, hq, hkv, d, bs, nb, mgr, specs, hist_slots, new_slots,
            cow_pairs, rng, extra_meta=None) -> Workload:
    S = len(specs)
    lens = np.array([h + n for h, n, _ in specs], dtype=np.int32)
    qsl = np.zeros(S + 1, dtype=np.int32)
    qsl[1:] = np.cumsum([n for _, n, _ in specs])
    poison = int(mgr.free[0]) if mgr.free else -1
    width = max(1, max(len(mgr.tables[s]) for s in range(S)))
    bt = np.full((S, width), poison if poison >= 0 else 0, dtype=np.int32)
    for s in range(S):
        t = mgr.tables[s]
        bt[s, :len(t)] = t
    t_q = int(qsl[-1])
    q = _draw(rng, (t_q, hq, d), dtype)
    hist_k = _draw(rng, (len(hist_slots), hkv, d), dtype)
    hist_v = _draw(rng, (len(hist_slots), hkv, d), dtype)
    k_new = _draw(rng, (len(new_slots), hkv, d), dtype)
    v_new = _draw(rng, (len(new_slots), hkv, d), dtype)
    meta = {"specs": specs, "manager": mgr}
    if extra_meta:
        meta.update(extra_meta)
    return Workload(
        name=name, dtype=dtype, num_blocks=nb, block_size=bs, num_q_heads=hq,
        num_kv_heads=hkv, head_dim=d, hist_k=hist_k, hist_v=hist_v,
        hist_slots=np.asarray(hist_slots, dtype=np.int64),
        cow_pairs=np.asarray(cow_pairs, dtype=np.int32).reshape(-1, 2),
        k_new=k_new, v_new=v_new,
        slot_mapping=np.asarray(new_slots, dtype=np.int64), q=q,
        block_tables=bt, context_lens=lens, query_start_loc=qsl,
        scale=float(1.0 / np.sqrt(d)), poison_block=poison, meta=meta)


# --------------------------------------------------------------------------
# The five named workloads
# --------------------------------------------------------------------------
def config1(seed=1) -> Workload:
    rng = np.random.default_rng(seed)
    others = np.array([b for b in range(16) if b not in (7, 1, 3)])
    free_order = [7, 1] + list(others[rng.permutation(others.size)]) + [3]
    seqs = [(7, 1, 1), (0, 5, 1), (9, 3, 1)]
    return build_batch("tiny fp32 mix (4 heads x 64, block 4, 16 blocks)", "f32",
                       4, 4, 64, 4, 16, seqs, seed, free_order=free_order, rng=rng)


def config2(seed=2) -> Workload:
    rng = np.random.default_rng(seed)
    lens = rng.integers(128, 2049, size=64)
    seqs = [(int(L) - 1, 1, 1) for L in lens]
    return build_batch("decode 64 seqs, 40 heads x 128, fp16, block 16", "f16",
                       40, 40, 128, 16, 10_000, seqs, seed, rng=rng)


def config3(seed=3) -> Workload:
    rng = np.random.default_rng(seed)
    mt = [(int(rng.integers(256, 3073)), int(rng.integers(16, 513)), 2) for _ in range(8)]
    dec = [(int(L) - 1, 1, 1) for L in rng.integers(64, 2049, size=56)]
    seqs = mt + dec
    seqs = [seqs[i] for i in rng.permutation(len(seqs))]
    return build_batch("unified batch: 8 prefill + 56 decode, 40 heads x 128, fp16, block 32",
                       "f16", 40, 40, 128, 32, 8192, seqs, seed, rng=rng)


def config4(seed=4, groups=64, pool=20_000, lens=None, name=None) -> Workload:
    """256 GQA decodes in groups of 4 sharing a prompt by reference count.

    Per group: ``L = clip(round(exp(N(ln 800, 1))), 2, 4096)``; the shared
    prompt is ``L - 1`` tokens; every member decodes one token at position
    ``L - 1``.  Copy-on-write (vLLM blog page, section 2.1): while the last
    prompt block is shared, a writing member takes a copy; the last holder
    writes in place.
    """
    rng = np.random.default_rng(seed)
    bs = 16
    if lens is None:
        lens = np.clip(np.rint(np.exp(rng.normal(np.log(800.0), 1.0, size=groups))),
                       2, 4096).astype(np.int64)
    free_order = rng.permutation(pool)
    mgr = BlockManager(pool, bs, free_order)
    specs, hist_slots, new_slots, pairs = [], [], [], []
    for gi, L in enumerate(lens):
        base = 4 * gi
        mgr.add_sequence(base)
        sl, pr = mgr.append(base, int(L) - 1)
        assert not pr
        hist_slots.extend(sl)
        for m in range(1, 4):
            mgr.fork(base, base + m)
    for gi, L in enumerate(lens):
        for m in range(4):
            sl, pr = mgr.append(4 * gi + m, 1)
            new_slots.extend(sl)
            pairs.extend(pr)
            specs.append((int(L) - 1, 1, 1))
    name = name or "GQA decode 256 seqs, 16/2 heads x 128, bf16, block 16"
    return _finish(name, "bf16",
                   16, 2, 128, bs, pool, mgr, specs, hist_slots, new_slots, pairs,
                   rng, {"group_lens": lens})


def config5(seed=5) -> Workload:
    rng = np.random.default_rng(seed)
    mt = [(int(rng.integers(3000, 4097)), 512, 1) for _ in range(16)]
    dec = [(int(L) - 1, 1, 1) for L in rng.integers(1024, 4097, size=128)]
    seqs = mt + dec
    seqs = [seqs[i] for i in rng.permutation(len(seqs))]
    return build_batch("long mix: 16 prefill x 512 + 128 decode, 64/8 heads x 128, bf16, block 32",
                       "bf16", 64, 8, 128, 32, 20_480, seqs, seed, rng=rng)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def config_workload(cfg: int, seed: int | None = None) -> Workload:
    return CONFIGS[cfg](cfg if seed is None else seed)


def small_workload(cfg: int, seed: int | None = None) -> Workload:
    """A reduced batch with a named workload's dtype, heads, head dim and
    block size, small enough for the oracle to finish in seconds, yet with
    several KV tiles, ragged tails, length-1 contexts and block-aligned
    contexts."""
    seed = cfg + 1000 if seed is None else seed
    rng = np.random.default_rng(seed)
    if cfg == 1:
        return config1(seed)
    if cfg == 2:
        lens = [1, 2, 16, 17, 255, 300] + list(rng.integers(1, 700, size=4))
        seqs = [(int(L) - 1, 1, 1) for L in lens]
        return build_batch("small decode (fp16, 40 x 128, block 16)", "f16",
                           40, 40, 128, 16, 1024, seqs, seed, rng=rng)
    if cfg == 3:
        seqs = [(70, 33, 2), (200, 140, 2), (64, 1, 1), (0, 1, 1), (31, 1, 1),
                (0, 47, 1), (95, 1, 1)]
        seqs = [seqs[i] for i in rng.permutation(len(seqs))]
        return build_batch("small unified (fp16, 40 x 128, block 32)", "f16",
                           40, 40, 128, 32, 1024, seqs, seed, rng=rng)
    if cfg == 4:
        return config4(seed, groups=6, pool=2048,
                       lens=np.array([2, 17, 33, 150, 400, 1000]),
                       name="small GQA decode (bf16, 16/2 x 128, block 16)")
    if cfg == 5:
        seqs = [(100, 64, 1), (250, 130, 1), (0, 1, 1), (31, 1, 1), (32, 1, 1),
                (700, 1, 1), (1, 1, 1), (0, 37, 1)]
        seqs = [seqs[i] for i in rng.permutation(len(seqs))]
        return build_batch("small long mix (bf16, 64/8 x 128, block 32)", "bf16",
                           64, 8, 128, 32, 1024, seqs, seed, rng=rng)
    raise KeyError(cfg)
