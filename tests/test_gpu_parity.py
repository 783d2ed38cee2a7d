"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: scatter, block copy and indexing bit-exact; attention (fp32
accumulation on the GPU, float64 in the oracle) within max |d| <= 1e-5 for
fp32 inputs, max |d| <= 1e-2 for fp16 inputs, and max |d| <= 1e-2 plus half
a bf16 ulp of the output (the one rounding of the result into bf16) for bf16
inputs; for fp16 / bf16 also mean |d| <= 1e-3 (``oracle.tolerance``).
"""
import functools
import os
import sys

import numpy as np
import pytest

import oracle
from oracle import tolerance
from workloads import build_batch, config_workload, small_workload

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]



def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


def _step_mod():
    from paged_kv_cache_block_amd import step
    return step


def oracle_step(w):
    k, v = w.empty_pools()
    oracle.write_kv(k, v, w.hist_k, w.hist_v, w.hist_slots)
    oracle.copy_blocks(k, v, w.cow_pairs)
    oracle.write_kv(k, v, w.k_new, w.v_new, w.slot_mapping)
    return k, v


def compare(got_storage, want64, dtype, rows=None, what=""):
    got = oracle.to_f64(got_storage, dtype)
    if rows is not None:
        got, want64 = got[rows], want64[rows]
    ok, st = tolerance.check(got, want64, dtype)
    say(f"{what}: max|d|={st.get('max', float('nan')):.3e} mean|d|={st.get('mean', float('nan')):.3e} "
        f"worst |d|/bound={st.get('worst', float('nan')):.3f}")
    assert ok, f"{what}: {st['msg']}"


def run_gpu(w, opt=None, write_history=True, fused=False):
    torch = pytest.importorskip("torch")
    db = _step_mod().DeviceBatch(w, opt=opt)
    if write_history:
        db.write_history()
    db.step(fused=fused)
    torch.cuda.synchronize()
    return db


def bits(a):
    return a.view(np.uint32 if a.dtype == np.float32 else np.uint16)


# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_write_and_copy_bit_exact(torch_cuda, cfg):
    w = small_workload(cfg)
    say("write/copy", w.name)
    db = run_gpu(w)
    gk, gv = db.pools_numpy()
    k, v = oracle_step(w)
    assert np.array_equal(bits(gk), bits(k)), "K pool differs"
    assert np.array_equal(bits(gv), bits(v)), "V pool differs"


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_copy_blocks_layers_bit_exact(torch_cuda, dtype):
    """One launch applies the same copy-on-write pairs to every layer's pools."""
    torch = torch_cuda
    from paged_kv_cache_block_amd import binding
    from paged_kv_cache_block_amd.step import TORCH_DTYPE, to_numpy, to_torch
    from workloads import round_to_dtype
    nb, h, bs, d, layers = 40, 2, 16, 64, 5
    rng = np.random.default_rng(9)
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:12], perm[12:24]], 1).astype(np.int32)    # distinct, disjoint
    ks, vs, want = [], [], []
    for l in range(layers):
        k = round_to_dtype(rng.standard_normal((nb, h, bs, d), dtype=np.float32), dtype)
        v = round_to_dtype(rng.standard_normal((nb, h, d, bs), dtype=np.float32), dtype)
        ks.append(to_torch(k, dtype, "cuda"))
        vs.append(to_torch(v, dtype, "cuda"))
        k2, v2 = k.copy(), v.copy()
        oracle.copy_blocks(k2, v2, pairs)
        want.append((k2, v2))
    say("copy layers", dtype)
    binding.pa_copy_blocks_layers(ks, vs, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    for l in range(layers):
        assert np.array_equal(bits(to_numpy(ks[l], dtype)), bits(want[l][0])), l
        assert np.array_equal(bits(to_numpy(vs[l], dtype)), bits(want[l][1])), l


@pytest.mark.parametrize("dtype,scattered", [("bf16", False), ("f32", False), ("bf16", True), ("f16", True)])
def test_swap_out_and_in_bit_exact(torch_cuda, dtype, scattered):
    """Blocks go to a pinned host pool and come back into other device
    blocks: a few runs (DMA engines) or many scattered pairs (the copy kernel
    over the host link), bit-exact."""
    torch = torch_cuda
    from paged_kv_cache_block_amd import binding
    from paged_kv_cache_block_amd.step import TORCH_DTYPE, to_numpy, to_torch
    from workloads import round_to_dtype
    nb, hnb, h, bs, d = 48, 40, 2, 16, 64
    rng = np.random.default_rng(17)
    k = round_to_dtype(rng.standard_normal((nb, h, bs, d), dtype=np.float32), dtype)
    v = round_to_dtype(rng.standard_normal((nb, h, d, bs), dtype=np.float32), dtype)
    dk, dv = to_torch(k, dtype, "cuda"), to_torch(v, dtype, "cuda")
    dt = TORCH_DTYPE[dtype]
    hk = torch.zeros((hnb, h, bs, d), dtype=dt).pin_memory()
    hv = torch.zeros((hnb, h, d, bs), dtype=dt).pin_memory()
    if scattered:      # 20 pairs, no two consecutive: 20 runs
        src = rng.permutation(nb)[:20]
        hdst = rng.permutation(hnb)[:20]
        out_pairs = np.stack([src, hdst], 1).astype(np.int32)
        in_pairs = np.stack([hdst, rng.permutation(nb)[:20]], 1).astype(np.int32)
    else:
        out_pairs = np.array([[5, 10], [6, 11], [7, 12], [30, 0], [2, 39], [3, 20]], dtype=np.int32)
        in_pairs = np.array([[10, 40], [11, 41], [12, 42], [0, 44], [39, 47], [20, 45]], dtype=np.int32)
    say("swap", dtype)
    binding.pa_swap_blocks(dk, dv, hk, hv, torch.from_numpy(out_pairs), binding.PA_SWAP_OUT)
    binding.pa_swap_blocks(dk, dv, hk, hv, torch.from_numpy(in_pairs), binding.PA_SWAP_IN)
    torch.cuda.synchronize()
    wk, wv = k.copy(), v.copy()
    whk = np.zeros_like(to_numpy(hk, dtype))
    whv = np.zeros_like(to_numpy(hv, dtype))
    oracle.swap_blocks(wk, wv, whk, whv, out_pairs)
    oracle.swap_blocks(whk, whv, wk, wv, in_pairs)
    assert np.array_equal(bits(to_numpy(hk, dtype)), bits(whk))
    assert np.array_equal(bits(to_numpy(hv, dtype)), bits(whv))
    assert np.array_equal(bits(to_numpy(dk, dtype)), bits(wk))
    assert np.array_equal(bits(to_numpy(dv, dtype)), bits(wv))


def test_layerwise_swap_in_gates_attention(torch_cuda):
    """Three layers whose history blocks were swapped out (device copies then
    poisoned) are swapped back in on a copy stream; each layer's attention
    waits only for its own layer's event and still matches the oracle."""
    torch = torch_cuda
    from paged_kv_cache_block_amd import binding
    from paged_kv_cache_block_amd.swap import LayerSwap, LayerSwapPipeline
    layers, swaps, wants, dbs = 3, [], [], []
    for l in range(layers):
        w = small_workload(5, 500 + l)
        db = run_gpu(w)                            # history + step written, pools complete
        k, v = oracle_step(w)
        wants.append(oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                                      w.num_kv_heads, w.dtype, w.scale))
        used = np.unique(np.concatenate([w.block_tables[s, :-(-int(L) // w.block_size)]
                                         for s, L in enumerate(w.context_lens)]))
        moved = used[::2].astype(np.int32)          # every other live block goes to the host
        hk = torch.empty((moved.size,) + tuple(db.k_cache.shape[1:]), dtype=db.k_cache.dtype).pin_memory()
        hv = torch.empty((moved.size,) + tuple(db.v_cache.shape[1:]), dtype=db.v_cache.dtype).pin_memory()
        out_pairs = torch.from_numpy(np.stack([moved, np.arange(moved.size, dtype=np.int32)], 1))
        binding.pa_swap_blocks(db.k_cache, db.v_cache, hk, hv, out_pairs, binding.PA_SWAP_OUT)
        torch.cuda.synchronize()
        idx = torch.from_numpy(moved.astype(np.int64)).cuda()
        db.k_cache.index_fill_(0, idx, float("nan"))
        db.v_cache.index_fill_(0, idx, float("nan"))
        in_pairs = torch.from_numpy(np.stack([np.arange(moved.size, dtype=np.int32), moved], 1))
        swaps.append(LayerSwap(db.k_cache, db.v_cache, hk, hv, in_pairs))
        dbs.append(db)
    torch.cuda.synchronize()
    say("layerwise swap-in")
    pipe = LayerSwapPipeline()
    pipe.start_swap_in(swaps)
    outs = []
    for l in range(layers):
        pipe.wait_layer(l)
        outs.append(dbs[l].attention(out=torch.empty_like(dbs[l].q)))
    torch.cuda.synchronize()
    from paged_kv_cache_block_amd.step import to_numpy
    for l in range(layers):
        compare(to_numpy(outs[l], dbs[l].w.dtype), wants[l], dbs[l].w.dtype, what=f"layer {l} after swap-in")


@pytest.mark.parametrize("dtype,bs", [("f16", 16), ("bf16", 32), ("f32", 8), ("f16", 128)])
def test_write_kv_runs_and_gaps(torch_cuda, dtype, bs):
    """The scatter with slot runs that are aligned, misaligned, cross a block
    boundary, skip (negative slots) and end in a ragged tail: bit-exact."""
    torch = torch_cuda
    from paged_kv_cache_block_amd import binding
    from paged_kv_cache_block_amd.step import NAN_FILL, TORCH_DTYPE, to_numpy, to_torch
    from workloads import round_to_dtype
    nb, h, d = 64, 3, 64
    rng = np.random.default_rng(bs)
    runs = [list(range(8 * bs, 8 * bs + 16)),              # two aligned 8-runs
            list(range(5 * bs + 4, 5 * bs + 12)),          # misaligned
            list(range(2 * bs - 4, 2 * bs + 4)),           # crosses a block boundary
            [-1, 3 * bs + 1, -1, 3 * bs + 2, 40 * bs, 41 * bs + 3, -5, 12 * bs + 7],
            list(range(20 * bs, 20 * bs + 5))]             # ragged tail
    slots = np.array([x for r in runs for x in r], dtype=np.int64)
    t = slots.size
    kn = round_to_dtype(rng.standard_normal((t, h, d), dtype=np.float32), dtype)
    vn = round_to_dtype(rng.standard_normal((t, h, d), dtype=np.float32), dtype)
    dt = TORCH_DTYPE[dtype]
    kc = torch.empty((nb, h, bs, d), dtype=dt, device="cuda")
    vc = torch.empty((nb, h, d, bs), dtype=dt, device="cuda")
    it, fill = NAN_FILL[dtype]
    kc.view(it).fill_(fill)
    vc.view(it).fill_(fill)
    say("write runs", dtype, bs)
    binding.pa_write_kv(to_torch(kn, dtype, "cuda"), to_torch(vn, dtype, "cuda"),
                        torch.from_numpy(slots).cuda(), kc, vc)
    torch.cuda.synchronize()
    k0 = to_numpy(kc, dtype).copy()
    v0 = to_numpy(vc, dtype).copy()
    # expected: the poisoned pools with the oracle's scatter applied
    ke, ve = np.empty_like(k0), np.empty_like(v0)
    ke.view(np.uint32 if dtype == "f32" else np.uint16)[...] = fill & (0xFFFFFFFF if dtype == "f32" else 0xFFFF)
    ve.view(np.uint32 if dtype == "f32" else np.uint16)[...] = fill & (0xFFFFFFFF if dtype == "f32" else 0xFFFF)
    oracle.write_kv(ke, ve, kn, vn, slots)
    assert np.array_equal(bits(k0), bits(ke))
    assert np.array_equal(bits(v0), bits(ve))


@pytest.mark.parametrize("seed", range(24))
def test_random_copy_and_write(torch_cuda, seed):
    """Seeded random pools, copy-on-write pairs and slot mappings (distinct
    slots in any order, some negative) over dtypes, head counts, head dims
    and block sizes: copy then write, bit-exact against the oracle."""
    torch = torch_cuda
    from paged_kv_cache_block_amd import binding
    from paged_kv_cache_block_amd.step import TORCH_DTYPE, to_numpy, to_torch
    from workloads import round_to_dtype
    rng = np.random.default_rng(5000 + seed)
    dtype = str(rng.choice(["f16", "bf16", "f32"]))
    bs = int(rng.choice([4, 8, 16, 32, 64] + ([128] if dtype != "f32" else [])))
    h = int(rng.choice([1, 2, 3, 8]))
    d = int(rng.choice([64, 128]))
    nb = int(rng.integers(8, 96))
    k = round_to_dtype(rng.standard_normal((nb, h, bs, d), dtype=np.float32), dtype)
    v = round_to_dtype(rng.standard_normal((nb, h, d, bs), dtype=np.float32), dtype)
    perm = rng.permutation(nb)
    m = int(rng.integers(0, nb // 2 + 1))
    pairs = np.stack([perm[:m], perm[m:2 * m]], 1).astype(np.int32)
    t = int(rng.integers(1, min(nb * bs, 700) + 1))
    slots = rng.choice(nb * bs, size=t, replace=False).astype(np.int64)
    slots[rng.random(t) < 0.1] = -1
    kn = round_to_dtype(rng.standard_normal((t, h, d), dtype=np.float32), dtype)
    vn = round_to_dtype(rng.standard_normal((t, h, d), dtype=np.float32), dtype)
    say("random copy+write", seed, dtype, "bs", bs, "H", h, "D", d, "blocks", nb, "pairs", m, "tokens", t)
    kc, vc = to_torch(k, dtype, "cuda"), to_torch(v, dtype, "cuda")
    binding.pa_copy_blocks(kc, vc, torch.from_numpy(pairs).cuda())
    binding.pa_write_kv(to_torch(kn, dtype, "cuda"), to_torch(vn, dtype, "cuda"),
                        torch.from_numpy(slots).cuda(), kc, vc)
    torch.cuda.synchronize()
    oracle.copy_blocks(k, v, pairs)
    oracle.write_kv(k, v, kn, vn, slots)
    assert np.array_equal(bits(to_numpy(kc, dtype)), bits(k))
    assert np.array_equal(bits(to_numpy(vc, dtype)), bits(v))


@pytest.mark.parametrize("mode", ["default", "split64", "rows", "stream", "tile128", "tile256",
                                  "psplit128", "psplit128w", "nopsplit"])
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_attention_small(torch_cuda, cfg, mode):
    from paged_kv_cache_block_amd import binding
    opt = {"default": None, "split64": binding.options(64),
           "rows": binding.options(0, 0, binding.PA_FLAG_VECTOR_ALU),
           "stream": binding.options(0, 0, binding.PA_FLAG_KV_UNSHARED),
           "tile128": binding.options(prefill_tile_rows=128),
           "tile256": binding.options(prefill_tile_rows=256),
           "psplit128": binding.options(prefill_split_tokens=128),
           "psplit128w": binding.options(prefill_split_tokens=128, prefill_tile_rows=256),
           "nopsplit": binding.options(0, 0, binding.PA_FLAG_NO_PREFILL_SPLIT)}[mode]
    w = small_workload(cfg)
    say("attention", w.name, mode)
    db = run_gpu(w, opt)
    k, v = oracle_step(w)
    want = oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                            w.num_kv_heads, w.dtype, w.scale)
    compare(db.out_numpy(), want, w.dtype, what=f"{w.name} [{mode}]")


@pytest.mark.parametrize("seed", [100, 200, 300])
@pytest.mark.parametrize("cfg", [1, 3, 5])
def test_attention_small_seeds(torch_cuda, cfg, seed):
    w = small_workload(cfg, seed + cfg) if cfg != 1 else config_workload(1, seed + 1)
    say("attention seed", seed, w.name)
    db = run_gpu(w)
    k, v = oracle_step(w)
    want = oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                            w.num_kv_heads, w.dtype, w.scale)
    compare(db.out_numpy(), want, w.dtype, what=f"{w.name} seed {seed}")


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_relabelled_pool_is_bit_identical(torch_cuda, cfg):
    """Physical block ids do not change the result, bit for bit."""
    w = small_workload(cfg)
    say("relabel", w.name)
    a = run_gpu(w).out_numpy()
    perm = np.random.default_rng(cfg + 7).permutation(w.num_blocks)
    bs = w.block_size

    def remap_slots(sl):
        sl = np.asarray(sl, dtype=np.int64)
        return np.where(sl >= 0, perm[sl // bs] * bs + sl % bs, sl)
    import copy
    w2 = copy.copy(w)
    w2.hist_slots = remap_slots(w.hist_slots)
    w2.slot_mapping = remap_slots(w.slot_mapping)
    w2.block_tables = perm[w.block_tables].astype(np.int32)
    w2.cow_pairs = perm[w.cow_pairs].astype(np.int32).reshape(-1, 2)
    b = run_gpu(w2).out_numpy()
    assert np.array_equal(bits(a), bits(b))


SHAPES = [  # (dtype, H_q, H_kv, D, block_size)
    ("f16", 8, 8, 64, 16), ("f16", 8, 4, 128, 32), ("f16", 16, 4, 64, 32), ("f16", 32, 2, 128, 16),
    ("bf16", 8, 8, 128, 16), ("bf16", 16, 8, 64, 16), ("bf16", 32, 4, 128, 32),
    ("f32", 4, 4, 128, 16), ("f32", 8, 2, 64, 32), ("f32", 16, 1, 64, 8),
    ("f16", 4, 2, 128, 8), ("bf16", 8, 1, 64, 4),
    ("f16", 8, 4, 128, 64), ("bf16", 16, 2, 128, 128), ("bf16", 8, 8, 64, 128), ("f32", 8, 8, 64, 64),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_shape_sweep(torch_cuda, shape):
    from paged_kv_cache_block_amd import binding
    dtype, hq, hkv, d, bs = shape
    seqs = [(0, 1, 1), (47, 1, 1), (130, 1, 1), (0, 19, 1), (70, 45, 1), (5, 2, 1), (200, 1, 1)]
    w = build_batch(f"sweep {shape}", dtype, hq, hkv, d, bs, 512, seqs, 21)
    k, v = oracle_step(w)
    want = oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                            w.num_kv_heads, w.dtype, w.scale)
    for rows in (128, 256):
        say("shape", shape, "tile rows", rows)
        db = run_gpu(w, binding.options(prefill_tile_rows=rows))
        compare(db.out_numpy(), want, w.dtype, what=f"shape {shape} tile rows {rows}")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("split", [0, 64])
def test_fused_write_is_bit_identical(torch_cuda, cfg, split):
    """pa_write_kv_attention gives the outputs and pools of pa_write_kv
    followed by pa_attention, bit for bit, on every config (fp32, decode-only,
    mixed).  Unwritten slots hold NaN, so a new token read before it is
    stored would show."""
    from paged_kv_cache_block_amd import binding
    w = small_workload(cfg)
    opt = binding.options(split) if split else None
    say("fused write", w.name, "split", split)
    a = run_gpu(w, opt)
    b = run_gpu(w, opt, fused=True)
    assert np.array_equal(bits(a.out_numpy()), bits(b.out_numpy()))
    ka, va = a.pools_numpy()
    kb, vb = b.pools_numpy()
    assert np.array_equal(bits(ka), bits(kb))
    assert np.array_equal(bits(va), bits(vb))
    k, v = oracle_step(w)
    want = oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                            w.num_kv_heads, w.dtype, w.scale)
    compare(b.out_numpy(), want, w.dtype, what=f"{w.name} fused write")


@pytest.mark.parametrize("dtype,bs", [("f16", 16), ("bf16", 32), ("bf16", 64)])
@pytest.mark.parametrize("split", [0, 64])
def test_fused_write_step_aligned_contexts(torch_cuda, dtype, bs, split):
    """Decode rows whose own token ends a 32-key step (contexts 32, 64, 96,
    160), or starts one, or is alone, over three block sizes: the fused call
    stores every new token before any attention kernel reads it."""
    from paged_kv_cache_block_amd import binding
    seqs = [(31, 1, 1), (63, 1, 1), (95, 1, 1), (159, 1, 1), (32, 1, 1), (0, 1, 1),
            (64, 1, 1), (30, 1, 1)]
    w = build_batch(f"aligned decodes {dtype} bs {bs}", dtype, 16, 4, 128, bs, 256, seqs, 5)
    opt = binding.options(split) if split else None
    say("fused aligned", dtype, bs, "split", split)
    a = run_gpu(w, opt)
    b = run_gpu(w, opt, fused=True)
    assert np.array_equal(bits(a.out_numpy()), bits(b.out_numpy()))
    ka, va = a.pools_numpy()
    kb, vb = b.pools_numpy()
    assert np.array_equal(bits(ka), bits(kb))
    assert np.array_equal(bits(va), bits(vb))
    k, v = oracle_step(w)
    want = oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                            w.num_kv_heads, w.dtype, w.scale)
    compare(b.out_numpy(), want, w.dtype, what=f"aligned decodes {dtype} bs {bs} fused")


@pytest.mark.parametrize("cfg", [2, 4])
def test_fused_write_full_size(torch_cuda, cfg):
    """Full-size decode batches: fused and separate calls agree bit for bit."""
    w = config_workload(cfg)
    say("fused write full", w.name)
    a = run_gpu(w)
    b = run_gpu(w, fused=True)
    assert np.array_equal(bits(a.out_numpy()), bits(b.out_numpy()))
    ka, va = a.pools_numpy()
    kb, vb = b.pools_numpy()
    assert np.array_equal(bits(ka), bits(kb))
    assert np.array_equal(bits(va), bits(vb))


@pytest.mark.parametrize("cfg", [2, 3])
def test_graph_capture_replays(torch_cuda, cfg):
    """The fused write + attention call (plan + write, multi-token and decode
    kernels, split combine) captured in a HIP graph replays to the eager
    result, three times, with eager calls and synchronizations between the
    replays."""
    torch = torch_cuda
    w = small_workload(cfg)
    say("graph capture", w.name)
    db = _step_mod().DeviceBatch(w)
    db.write_history()
    db.copy_blocks()
    db.write_attention()
    torch.cuda.synchronize()
    want = bits(db.out_numpy()).copy()
    out_g = torch.empty_like(db.out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        db.write_attention(out=out_g)
    torch.cuda.synchronize()
    for r in range(3):
        out_g.zero_()
        db.write_attention()          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = bits(db.out_numpy(out_g))
        assert np.array_equal(got, want), f"replay {r}"


@pytest.mark.parametrize("cfg,split", [(2, 0), (3, 0), (5, 0), (2, 64), (3, 64)])
def test_streaming_hint_is_bit_identical(torch_cuda, cfg, split):
    """The no-sharing hint changes the cache policy of the decode loads and
    the order of the decode work (listed longest first, dealt over the XCDs);
    neither changes a bit of the output."""
    from paged_kv_cache_block_amd import binding
    w = small_workload(cfg)
    say("stream hint", w.name, "split", split)
    a = run_gpu(w, binding.options(split)).out_numpy()
    b = run_gpu(w, binding.options(split, 0, binding.PA_FLAG_KV_UNSHARED)).out_numpy()
    assert np.array_equal(bits(a), bits(b))


@pytest.mark.parametrize("cfg,split", [(2, 0), (2, 64), (3, 0), (5, 0)])
def test_dealt_row_list_is_longest_first(torch_cuda, cfg, split):
    """With the no-sharing hint the planner lists the decode work longest
    first: every full split, then the last splits in buckets of descending
    length.  White-box: reads the row list the plan leaves in the workspace
    (16-byte records (seq, row, split, first partial slot) right after the
    256-byte status block) and checks it is exactly the expected set of
    splits, in that order."""
    torch = torch_cuda
    from paged_kv_cache_block_amd import binding
    w = config_workload(cfg)
    opt = binding.options(split, 0, binding.PA_FLAG_KV_UNSHARED)
    db = run_gpu(w, opt, fused=True)
    desc = binding.cache_desc(db.k_cache, db.v_cache)
    st, info = binding.pa_attention_plan(desc, w.num_q_heads, w.block_tables.shape[1],
                                         w.context_lens, w.query_start_loc,
                                         db.workspace.numel(), opt)
    assert st == 0
    S = info.decode_split_tokens
    n_items = int(info.row_items)
    torch.cuda.synchronize()
    raw = db.workspace[256:256 + 16 * n_items].cpu().numpy().view(np.int32).reshape(-1, 4)
    n_new = np.diff(w.query_start_loc)
    want = set()
    for s_ in np.flatnonzero(n_new == 1):
        L = int(w.context_lens[s_])
        for k in range(-(-L // S)):
            want.add((int(s_), 0, k))
    got = [(int(a), int(b), int(c)) for a, b, c, _ in raw]
    assert len(got) == len(want) and set(got) == want
    shift = 0
    while (S - 1) >> shift >= 64:
        shift += 1
    keys = [min(int(w.context_lens[a]), (c + 1) * S) - c * S for a, _, c in got]
    buckets = [(S - k) >> shift for k in keys]
    assert buckets == sorted(buckets), "row items not listed longest first"


def test_split_lengths_agree(torch_cuda):
    from paged_kv_cache_block_amd import binding
    w = small_workload(5)
    k, v = oracle_step(w)
    want = oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                            w.num_kv_heads, w.dtype, w.scale)
    for split in (64, 128, 192, 512, 4096):
        say("split", split)
        db = run_gpu(w, binding.options(split))
        compare(db.out_numpy(), want, w.dtype, what=f"split {split}")


@pytest.mark.parametrize("cfg", [3, 5])
def test_prefill_split_lengths_agree(torch_cuda, cfg):
    """Multi-token contexts split into 128..4096-key ranges, merged by the
    combine kernel (tokens with one, two and three splits), on both tile
    sizes and together with split decode rows."""
    from paged_kv_cache_block_amd import binding
    w = small_workload(cfg)
    k, v = oracle_step(w)
    want = oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                            w.num_kv_heads, w.dtype, w.scale)
    for psplit in (100, 128, 256, 384, 4096):
        for rows in (128, 256):
            for dsplit in (0, 64):
                say("prefill split", psplit, "tile rows", rows, "decode split", dsplit)
                db = run_gpu(w, binding.options(dsplit, psplit, prefill_tile_rows=rows))
                compare(db.out_numpy(), want, w.dtype,
                        what=f"{w.name} prefill split {psplit} rows {rows} decode split {dsplit}")


@pytest.mark.parametrize("psplit", [-1, 0, 128, 1024])
def test_chunk_recompute_shape(torch_cuda, psplit):
    """32-token chunks after 0..3000 cached tokens (the chunk recomputation
    the cost profile measures), whole (-1), with the automatic split (0) and
    with given split lengths."""
    from paged_kv_cache_block_amd import binding
    seqs = [(0, 32, 1), (31, 32, 1), (700, 32, 2), (3000, 32, 1)]
    w = build_batch("32-token chunks bf16", "bf16", 64, 8, 128, 32, 256, seqs, 77)
    k, v = oracle_step(w)
    want = oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                            w.num_kv_heads, w.dtype, w.scale)
    for rows in (128, 256):
        say("chunk shape split", psplit, "rows", rows)
        opt = (binding.options(0, 0, binding.PA_FLAG_NO_PREFILL_SPLIT, prefill_tile_rows=rows)
               if psplit < 0 else binding.options(0, psplit, prefill_tile_rows=rows))
        db = run_gpu(w, opt)
        compare(db.out_numpy(), want, w.dtype, what=f"chunks split {psplit} rows {rows}")


def test_long_contexts(torch_cuda):
    """A decode row after 100K cached tokens and a 16-token chunk after 60K
    (hundreds of block-table windows, up to 1563 key splits of one row merged
    by the combine), beside a short decode, against the oracle: automatic
    splits, 64-key splits, and the vector-ALU row path."""
    from paged_kv_cache_block_amd import binding
    seqs = [(100_000, 1, 1), (60_000, 16, 2), (5, 1, 1)]
    nblocks = sum(-(-(h + n) // 16) for h, n, _ in seqs) + 64
    w = build_batch("long contexts bf16", "bf16", 16, 2, 128, 16, nblocks, seqs, 31)
    k, v = oracle_step(w)
    want = oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                            w.num_kv_heads, w.dtype, w.scale)
    for mode, opt in [("default", None), ("split64", binding.options(64, 64)),
                      ("rows", binding.options(0, 0, binding.PA_FLAG_VECTOR_ALU))]:
        say("long contexts", mode)
        db = run_gpu(w, opt)
        compare(db.out_numpy(), want, w.dtype, what=f"long contexts [{mode}]")
        del db


@pytest.mark.parametrize("nseq", [37, 300])
@pytest.mark.parametrize("psplit", [0, 128])
def test_many_multi_token_sequences(torch_cuda, nseq, psplit):
    """Many short multi-token sequences (more than the planner's 256
    threads), many with equal context lengths, whole and with split
    contexts, on both tile sizes, against the oracle."""
    from paged_kv_cache_block_amd import binding
    rng = np.random.default_rng(nseq)
    seqs = [(int(rng.choice([0, 9, 130, 131])), int(rng.integers(2, 6)), 1) for _ in range(nseq)]
    w = build_batch(f"{nseq} multi-token f16", "f16", 8, 2, 64, 16, 10 * nseq + 8, seqs, 5)
    k, v = oracle_step(w)
    want = oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                            w.num_kv_heads, w.dtype, w.scale)
    for rows in (128, 256):
        say("multi-token sequences", nseq, "prefill split", psplit, "rows", rows)
        db = run_gpu(w, binding.options(0, psplit, prefill_tile_rows=rows))
        compare(db.out_numpy(), want, w.dtype, what=f"{nseq} seqs split {psplit} rows {rows}")


def _random_batch_spec(seed):
    """A seeded random batch: dtype, head dim, block size, GQA group, and a
    mix of decode rows, prompts, prompts after history (some on two block
    runs), sequences without new tokens and a few long histories, with one
    option set."""
    rng = np.random.default_rng(1000 + seed)
    dtype = str(rng.choice(["f16", "bf16", "f32"]))
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([4, 8, 16, 32, 64] + ([128] if dtype != "f32" else [])))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8, 16]))
    seqs = []
    for _ in range(int(rng.integers(1, 10))):
        kind = rng.choice(["decode", "prefill", "mixed", "empty", "long"], p=[0.38, 0.2, 0.3, 0.07, 0.05])
        if kind == "long":     # a long history: automatic key splits of decode rows and tiles
            h, n = int(rng.integers(1000, 6000)), int(rng.choice([1, int(rng.integers(2, 33))]))
        elif kind == "decode":
            h, n = int(rng.integers(0, 700)), 1
        elif kind == "prefill":
            h, n = 0, int(rng.integers(2, 81))
        elif kind == "mixed":
            h, n = int(rng.integers(1, 500)), int(rng.integers(2, 49))
        else:
            h, n = int(rng.integers(1, 300)), 0
        seqs.append((h, n, 2 if h >= 2 * bs and rng.random() < 0.3 else 1))
    mode = str(rng.choice(["default", "split64", "psplit128", "nopsplit", "tile128", "tile256",
                           "rows", "stream", "stream64"]))
    if bs == 128 and mode == "rows":     # 128-token blocks have no vector-ALU path
        mode = "default"
    nblocks = 2 * sum(-(-(h + n) // bs) for h, n, _ in seqs) + 64
    return dtype, d, bs, hkv, g, seqs, mode, nblocks


@pytest.mark.parametrize("seed", range(int(os.environ.get("PA_RANDOM_SEEDS", "48"))))
def test_random_batches(torch_cuda, seed):
    """Seeded random batches over the supported shapes and options, against
    the oracle (48 seeds; PA_RANDOM_SEEDS=N runs seeds 0..N-1)."""
    from paged_kv_cache_block_amd import binding
    dtype, d, bs, hkv, g, seqs, mode, nblocks = _random_batch_spec(seed)
    opt = {"default": None, "split64": binding.options(64),
           "psplit128": binding.options(prefill_split_tokens=128),
           "nopsplit": binding.options(0, 0, binding.PA_FLAG_NO_PREFILL_SPLIT),
           "tile128": binding.options(prefill_tile_rows=128),
           "tile256": binding.options(prefill_tile_rows=256),
           "rows": binding.options(0, 0, binding.PA_FLAG_VECTOR_ALU),
           "stream": binding.options(0, 0, binding.PA_FLAG_KV_UNSHARED),
           "stream64": binding.options(64, 0, binding.PA_FLAG_KV_UNSHARED)}[mode]
    w = build_batch(f"random {seed}", dtype, hkv * g, hkv, d, bs, nblocks, seqs, seed)
    say("random", seed, dtype, "D", d, "bs", bs, "H", hkv * g, "/", hkv, "seqs", seqs, mode)
    db = run_gpu(w, opt)
    if int(w.query_start_loc[-1]) == 0:   # no new tokens anywhere: nothing to attend
        assert db.out_numpy().size == 0
        return
    k, v = oracle_step(w)
    want = oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                            w.num_kv_heads, w.dtype, w.scale)
    compare(db.out_numpy(), want, w.dtype, what=f"random {seed} [{mode}]")


def test_edge_cases(torch_cuda):
    """Sequences with no new tokens, one-token contexts, prefills without
    history, sub-requests sharing one block-table row, and a ragged tail."""
    seqs = [(5, 0, 1), (0, 1, 1), (0, 2, 1), (40, 0, 1), (31, 33, 1), (0, 0, 1), (63, 1, 1)]
    w = build_batch("edges bf16", "bf16", 16, 2, 64, 16, 256, seqs, 11)
    # Sequence 5 becomes a sub-request of sequence 4: its first 9 positions
    # recomputed as queries over themselves.
    w.block_tables[5] = w.block_tables[4]
    w.context_lens[5] = 9
    lens = w.context_lens
    n = np.diff(w.query_start_loc)
    n[5] = 9
    qsl = np.zeros_like(w.query_start_loc)
    qsl[1:] = np.cumsum(n)
    rng = np.random.default_rng(3)
    from workloads import round_to_dtype
    q = round_to_dtype(rng.standard_normal((int(qsl[-1]), 16, 64), dtype=np.float32), "bf16")
    w.q, w.query_start_loc, w.context_lens = q, qsl.astype(np.int32), lens
    say("edge cases", w.name)
    db = run_gpu(w)
    k, v = oracle_step(w)
    want = oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                            w.num_kv_heads, w.dtype, w.scale)
    compare(db.out_numpy(), want, w.dtype, what="edge cases")


def test_empty_and_error_paths(torch_cuda, monkeypatch):
    torch = torch_cuda
    from paged_kv_cache_block_amd import binding
    w = small_workload(2)
    db = _step_mod().DeviceBatch(w)
    db.write_history()
    say("validate: block id out of range")
    monkeypatch.setenv("PA_VALIDATE", "1")
    bad = db.block_tables.clone()
    bad[0, 0] = w.num_blocks + 5
    with pytest.raises(binding.PagedAttnError) as ei:
        binding.pa_attention(db.out, db.q, db.k_cache, db.v_cache, bad, db.context_lens,
                             db.query_start_loc, db.context_lens_host, db.qsl_host, w.scale,
                             db.workspace)
    assert ei.value.status == -5
    say("validate: duplicate slot")
    dup = db.slot_mapping.clone()
    dup[1] = dup[0]
    with pytest.raises(binding.PagedAttnError) as ei:
        binding.pa_write_kv(db.k_new, db.v_new, dup, db.k_cache, db.v_cache)
    assert ei.value.status == -5
    say("validate: fused write with a duplicate slot")
    with pytest.raises(binding.PagedAttnError) as ei:
        binding.pa_write_kv_attention(db.out, db.q, db.k_new, db.v_new, dup, db.k_cache,
                                      db.v_cache, db.block_tables, db.context_lens,
                                      db.query_start_loc, db.context_lens_host, db.qsl_host,
                                      w.scale, db.workspace)
    assert ei.value.status == -5
    monkeypatch.delenv("PA_VALIDATE")
    say("workspace too small")
    with pytest.raises(binding.PagedAttnError) as ei:
        binding.pa_attention(db.out, db.q, db.k_cache, db.v_cache, db.block_tables,
                             db.context_lens, db.query_start_loc, db.context_lens_host,
                             db.qsl_host, w.scale, db.workspace[:64])
    assert ei.value.status == -3
    torch.cuda.synchronize()


def test_attention_check_reports_disagreeing_mirrors(torch_cuda):
    """pa_attention_check: OK after a consistent call; PA_ERR_BOUNDS when the
    device context_lens say 64 keys fewer than the host mirror for one row
    (the device plan then lists one split item less than the host sized the
    grid and partial states for).  The shorter context reads a subset of what
    the consistent call reads, so nothing is read out of bounds."""
    torch = torch_cuda
    from paged_kv_cache_block_amd import binding
    w = small_workload(2)
    opt = binding.options(64)
    db = _step_mod().DeviceBatch(w, opt=opt)
    db.write_history()
    db.step()
    say("attention check: consistent call")
    binding.pa_attention_check(db.workspace)
    s = int(np.argmax(w.context_lens))                 # room in its table row
    lens = db.context_lens.clone()
    lens[s] -= 64                                      # device: fewer keys, host unchanged
    assert int(lens[s]) >= 1
    say("attention check: device context_lens differ from the host mirror")
    binding.pa_attention(db.out, db.q, db.k_cache, db.v_cache, db.block_tables, lens,
                         db.query_start_loc, db.context_lens_host, db.qsl_host, w.scale,
                         db.workspace, opt)
    with pytest.raises(binding.PagedAttnError) as ei:
        binding.pa_attention_check(db.workspace)
    assert ei.value.status == -5
    # the next consistent call clears the status
    db.attention()
    binding.pa_attention_check(db.workspace)
    torch.cuda.synchronize()


# --------------------------------------------------------------------------
# Full-size workloads: whole pools bit-exact, every output row vs the oracle
# --------------------------------------------------------------------------
@functools.lru_cache(maxsize=1)
def _full_reference(cfg):
    """The full workload, the oracle's pools after the step, and the oracle's
    output for every query row (kept for the split variants of one config)."""
    w = config_workload(cfg)
    k, v = oracle_step(w)
    want = oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                            w.num_kv_heads, w.dtype, w.scale)
    return w, k, v, want


@pytest.mark.parametrize("cfg,psplit", [(1, 0), (2, 0), (3, 0), (3, 512), (4, 0), (5, 0), (5, 1024)])
def test_full_config(torch_cuda, cfg, psplit):
    """Each named workload at full size through the bench's step (copy-on-write,
    then the fused write + attention call): both pools bit-exact against the
    oracle's, and every output row (decode and multi-token) within the bar."""
    from paged_kv_cache_block_amd import binding
    say("full: oracle for config", cfg)
    w, k, v, want = _full_reference(cfg)
    say("full", w.name, "prefill split", psplit)
    db = run_gpu(w, binding.options(prefill_split_tokens=psplit) if psplit else None, fused=True)
    gk, gv = db.pools_numpy()
    assert np.array_equal(bits(gk), bits(k)), "K pool differs"
    assert np.array_equal(bits(gv), bits(v)), "V pool differs"
    del gk, gv
    n = w.n_new
    for kind, sel in (("decode", n == 1), ("multi-token", n > 1)):
        seqs = np.flatnonzero(sel)
        if seqs.size == 0:
            continue
        rows = np.concatenate([np.arange(w.query_start_loc[s], w.query_start_loc[s + 1]) for s in seqs])
        compare(db.out_numpy(), want, w.dtype, rows=rows,
                what=f"{w.name} split {psplit}: all {seqs.size} {kind} sequences")
