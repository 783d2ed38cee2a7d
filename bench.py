#!/usr/bin/env python3
"""Benchmark one step of the paged-attention hot path on one MI355X.

A step is the whole path over one synthetic batch with its inputs resident in
HBM: copy-on-write block copies, the slot-mapping write of the new tokens,
and causal paged attention of every query row (plan, multi-token MFMA
kernel, decode kernel, split combine).  The write and attention go through
one pa_write_kv_attention call (the write shares the planner's launch);
``--separate-write`` times pa_write_kv + pa_attention.  The default workload is
the long mixed bf16 batch (16 requests of 512 new tokens over 3000..4096
cached tokens, beside 128 decodes over 1024..4096 tokens; 64 query / 8 KV
heads of 128, block size 32), the largest named workload and the one with
both a multi-token and a decode part; ``--config`` picks another.

Prints one JSON line.  ``value`` is whole-step throughput in GB/s of
algorithmic bytes; ``roofline`` rates the dominant kernel from its own
per-launch HIP events (the multi-token kernel against the bf16 MFMA peak, or
the decode kernel against HBM), and ``roofline_decode`` /
``roofline_multi_token`` rate the other attention kernel of a mixed batch the
same way; ``cpu_baseline`` times the CPU oracle on a bounded sample of the
same batch.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "paged-attn KV GB/s (decode) & TFLOP/s (multi-token) vs MI355X peak"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}
ELT = {"f32": 4, "f16": 2, "bf16": 2}


def work_model(w):
    """Algorithmic bytes and flops of one step, per part of the path."""
    elt = ELT[w.dtype]
    kvb = w.kv_bytes_per_token()
    n = w.n_new
    L = w.context_lens.astype(np.int64)
    dec = n == 1
    mt = n > 1
    row_q = int(n[dec].sum()) * w.num_q_heads * w.head_dim * elt
    m = {}
    m["rows_bytes"] = int((L[dec] * kvb).sum()) + 2 * row_q       # KV once per KV head + q + out
    # The same with each cached slot counted once however many decode rows
    # read it (sequences sharing prompt blocks by reference count).
    used = {}
    for s in np.flatnonzero(dec):
        nb = (int(L[s]) + w.block_size - 1) // w.block_size
        for j in range(nb):
            b = int(w.block_tables[s, j])
            used[b] = max(used.get(b, 0), min(w.block_size, int(L[s]) - j * w.block_size))
    m["rows_unique_bytes"] = sum(used.values()) * kvb + 2 * row_q
    m["tile_bytes"] = int((L[mt] * kvb).sum()) + 2 * int(n[mt].sum()) * w.num_q_heads * w.head_dim * elt
    m["tile_flops"] = int(4 * w.head_dim * w.num_q_heads *
                          (n[mt] * (L[mt] - n[mt]) + n[mt] * (n[mt] + 1) // 2).sum())
    m["write_bytes"] = 2 * int(w.k_new.shape[0]) * kvb
    blk_bytes = w.num_kv_heads * w.block_size * w.head_dim * elt * 2
    m["copy_bytes"] = 2 * int(w.cow_pairs.shape[0]) * blk_bytes
    m["table_bytes"] = int(((L + w.block_size - 1) // w.block_size).sum()) * 4
    m["step_bytes"] = (m["rows_bytes"] + m["tile_bytes"] + m["write_bytes"] + m["copy_bytes"]
                       + m["table_bytes"])
    return m


def blocks_unshared(w) -> bool:
    """True when no physical block is read by two sequences of the batch --
    what a caller's block manager knows from its reference counts."""
    bs = w.block_size
    used = [w.block_tables[s, :(int(L) + bs - 1) // bs] for s, L in enumerate(w.context_lens)]
    ids = np.concatenate(used) if used else np.zeros(0, np.int32)
    return np.unique(ids).size == ids.size


def cpu_baseline(w, target_s: float):
    """The oracle, as it stands, on a bounded sample of sequences."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    k, v = w.empty_pools()
    oracle.write_kv(k, v, w.hist_k, w.hist_v, w.hist_slots)
    oracle.copy_blocks(k, v, w.cow_pairs)
    oracle.write_kv(k, v, w.k_new, w.v_new, w.slot_mapping)
    order = np.random.default_rng(0).permutation(w.num_seqs)
    kvb = w.kv_bytes_per_token()
    elt = ELT[w.dtype]
    # Sequences in a seeded order, passing over the batch again while the
    # time used is short of the target (a small batch is timed several times).
    done, nbytes, nflops, t_used, passes = [], 0, 0, 0.0, 0
    while t_used < target_s and passes < 50:
        passes += 1
        for s in order:
            n = int(w.n_new[s])
            if n == 0:
                continue
            t0 = time.perf_counter()
            oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                             w.num_kv_heads, w.dtype, w.scale, seqs=[int(s)])
            t_used += time.perf_counter() - t0
            L = int(w.context_lens[s])
            done.append(int(s))
            nbytes += L * kvb + 2 * n * w.num_q_heads * w.head_dim * elt
            nflops += 4 * w.head_dim * w.num_q_heads * (n * (L - n) + n * (n + 1) // 2)
            if t_used >= target_s:
                break
    if not done:
        return None
    return {"value": nbytes / t_used / 1e9, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"oracle attention, {len(done)} sequence evaluations over {len(set(done))} of "
                      f"{w.num_seqs} sequences in {passes} pass(es) ({nbytes / 1e6:.1f} MB KV+q+out, "
                      f"{nflops / 1e9:.2f} GFLOP) in {t_used:.2f} s",
            "gflops": nflops / t_used / 1e9}


def copy_calibration(steps: int) -> int:
    """pa_copy_blocks over 4096 distinct block pairs of a 40 x 16 x 128 fp16
    pool: each launch reads and writes exactly 2 x 4096 x 163840 bytes."""
    import torch
    from paged_kv_cache_block_amd import binding
    nb, h, bs, d = 8192, 40, 16, 128
    k = torch.zeros((nb, h, bs, d), dtype=torch.float16, device="cuda")
    v = torch.zeros((nb, h, d, bs), dtype=torch.float16, device="cuda")
    pairs = torch.stack([torch.arange(4096), torch.arange(4096, 8192)], 1).to(torch.int32).cuda()
    for _ in range(steps):
        binding.pa_copy_blocks(k, v, pairs)
    torch.cuda.synchronize()
    per_launch = 2 * 4096 * h * bs * d * 2
    print(json.dumps({"copy_calibration": {"launches": steps, "read_bytes_per_launch": per_launch,
                                           "write_bytes_per_launch": per_launch}}), flush=True)
    return 0


def hbm_reference() -> int:
    """Reference HBM rates on this GPU, for context beside the kernel figures."""
    import torch
    from paged_kv_cache_block_amd import binding

    def timed(fn, n=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    x = torch.randn(1 << 30, dtype=torch.float16, device="cuda")      # 2 GiB
    out = {"torch_sum_read_GBs": 2 * 2**30 / timed(lambda: x.sum(dtype=torch.float32)) / 1e6}
    y = torch.empty_like(x)
    out["torch_copy_read_write_GBs"] = 4 * 2**30 / timed(lambda: y.copy_(x)) / 1e6
    del x, y
    nb, h, bs, d = 8192, 40, 16, 128
    k = torch.zeros((nb, h, bs, d), dtype=torch.float16, device="cuda")
    v = torch.zeros((nb, h, d, bs), dtype=torch.float16, device="cuda")
    pairs = torch.stack([torch.arange(4096), torch.arange(4096, 8192)], 1).to(torch.int32).cuda()
    ms = timed(lambda: binding.pa_copy_blocks(k, v, pairs))
    out["pa_copy_blocks_read_write_GBs"] = 2 * 2 * 4096 * h * bs * d * 2 / ms / 1e6
    print(json.dumps({"hbm_reference": {k2: round(v2, 1) for k2, v2 in out.items()}}), flush=True)
    return 0


def mfma_reference() -> int:
    """Reference bf16 matrix-core rate on this GPU: a large dense torch GEMM
    (hipBLASLt), for context beside the multi-token kernel's TFLOP/s."""
    import torch

    n = 8192
    a = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"mfma_reference": {"torch_bf16_gemm_8192_TFLOPs": round(2 * n**3 / ms / 1e9, 1)}}),
          flush=True)
    return 0


def chunk_cost(args) -> int:
    """Attention time of one 32-token chunk after 0..32K cached tokens (and of
    16 such chunks after up to 8K), on the long-mix head shape (64 query / 8 KV
    heads of 128, bf16, block size 32): the table a recomputation cost model
    interpolates.  Each context is timed without and with a key split sized to
    give the GPU at least 256 workgroups."""
    import torch
    from paged_kv_cache_block_amd import binding
    from paged_kv_cache_block_amd.chunkcost import ChunkCostProfile
    from paged_kv_cache_block_amd.step import DeviceBatch
    from workloads import build_batch

    chunk, hq, hkv, d, bs = 32, 64, 8, 128, 32
    contexts = [0, 256, 1024, 2048, 4096, 8192, 16384, 32768]
    reps = max(args.steps, 5)
    rows = []
    for batch, ctxs in ((1, contexts), (16, contexts[:6])):
        for split_mode in ("none", "auto", "split"):
            times = []
            for ctx in ctxs:
                L = ctx + chunk
                nb = batch * ((L + bs - 1) // bs) + 8
                w = build_batch(f"chunk {chunk} after {ctx}", "bf16", hq, hkv, d, bs, nb,
                                [(ctx, chunk, 1)] * batch, 4242 + ctx)
                psplit, flags = 0, binding.PA_FLAG_KV_UNSHARED | binding.PA_FLAG_NO_PREFILL_SPLIT
                if split_mode == "auto":      # the library's own choice
                    flags = binding.PA_FLAG_KV_UNSHARED
                if split_mode == "split":
                    items = batch * hkv           # one 256-row tile per chunk and KV head
                    want = max(1, -(-256 // items))
                    psplit = max(128, -(-L // want))
                    flags = binding.PA_FLAG_KV_UNSHARED
                opt = binding.options(0, psplit, flags, prefill_tile_rows=256)
                db = DeviceBatch(w, opt=opt)
                db.write_history()
                db.write_new()
                torch.cuda.synchronize()
                for _ in range(3):
                    db.attention()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    db.attention()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) / reps * 1e3
                flops = 4 * d * hq * batch * (chunk * ctx + chunk * (chunk + 1) // 2)
                times.append(us)
                line = {"chunk_cost": {"chunk": chunk, "context": ctx, "batch": batch,
                                       "split_mode": split_mode,
                                       "prefill_split": psplit, "us": round(us, 2),
                                       "us_per_chunk": round(us / batch, 2),
                                       "tflops": round(flops / us / 1e6, 1)}}
                rows.append(line)
                print(json.dumps(line), flush=True)
                del db
            prof = ChunkCostProfile(chunk, ctxs, [t / batch for t in times],
                                    {"batch": batch, "split": split_mode, "heads": [hq, hkv, d],
                                     "dtype": "bf16", "block_size": bs})
            print(json.dumps({"chunk_cost_profile": prof.to_dict()}), flush=True)
    return 0


def _time_ms(fn, reps: int) -> float:
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _contiguous(w):
    """The same batch with every sequence's blocks renumbered to consecutive
    physical ids in table order (identity-like placement)."""
    import copy
    bs = w.block_size
    perm = np.full(w.num_blocks, -1, np.int64)
    nxt = 0
    for si, L in enumerate(w.context_lens):
        for b in w.block_tables[si, :-(-int(L) // bs)]:
            if perm[b] < 0:
                perm[b] = nxt
                nxt += 1
    rest = np.flatnonzero(perm < 0)
    perm[rest] = np.arange(nxt, nxt + rest.size)

    def slots(sl):
        sl = np.asarray(sl, dtype=np.int64)
        return np.where(sl >= 0, perm[sl // bs] * bs + sl % bs, sl)
    w2 = copy.copy(w)
    w2.hist_slots = slots(w.hist_slots)
    w2.slot_mapping = slots(w.slot_mapping)
    w2.block_tables = perm[w.block_tables].astype(np.int32)
    w2.cow_pairs = perm[np.asarray(w.cow_pairs, dtype=np.int64)].astype(np.int32).reshape(-1, 2)
    return w2


def paging(args) -> int:
    """Paging-overhead and batching diagnostics on the two headline shapes.

    The vLLM wiki page (实验与结果: the paged kernel is 20-26% slower than a
    contiguous one; block sizes 16-128 work well) and the Pensieve page
    (figures 12-13: copying K/V out before attending costs a lot; one
    unified call for prefill and decode) measure these effects.  For the
    decode shape (64 fp16 decodes, 40 heads x 128) and the multi-token shape
    (16 x 512-token prefills over 3000-4096 cached tokens, 64/8 heads x 128,
    bf16) this prints, one JSON line each:
    - block size 16, 32, 64, 128: attention time, and the slots allocated
      but unused in each sequence's last block;
    - contiguous (identity) block placement vs a shuffled pool;
    - copy-out: gathering every context into contiguous blocks with
      pa_copy_blocks and then attending, vs attending in place;
    - for the two mixed batches, one unified call vs separate prefill and
      decode calls.
    """
    import torch
    from paged_kv_cache_block_amd import binding
    from paged_kv_cache_block_amd.step import DeviceBatch
    from workloads import build_batch, config_workload

    reps = max(args.steps, 5)
    rng = np.random.default_rng(11)
    dec_lens = rng.integers(128, 2049, size=64)
    shapes = {
        "decode": ("f16", 40, 40, 128, [(int(L) - 1, 1, 1) for L in dec_lens]),
        "multi_token": ("bf16", 64, 8, 128,
                        [(int(h), 512, 1) for h in rng.integers(3000, 4097, size=16)]),
    }

    def emit(d):
        print(json.dumps({"paging": d}), flush=True)

    def attend_ms(db, tables=None):
        bt = db.block_tables if tables is None else tables
        return _time_ms(lambda: binding.pa_attention(
            db.out, db.q, db.k_cache, db.v_cache, bt, db.context_lens, db.query_start_loc,
            db.context_lens_host, db.qsl_host, db.w.scale, db.workspace, db.opt), reps)

    for name, (dt, hq, hkv, d, seqs) in shapes.items():
        tokens = sum(h + n for h, n, _ in seqs)
        for bs in (16, 32, 64, 128):
            need = sum(-(-(h + n) // bs) for h, n, _ in seqs)
            nb = 2 * need + 16                        # room for a contiguous copy
            shuffled = build_batch(f"{name} bs {bs}", dt, hq, hkv, d, bs, nb, seqs, 5)
            for placement in ("shuffled", "contiguous"):
                w = shuffled if placement == "shuffled" else _contiguous(shuffled)
                db = DeviceBatch(w, opt=binding.options(0, 0, binding.PA_FLAG_KV_UNSHARED))
                db.write_history()
                db.write_new()
                torch.cuda.synchronize()
                ms = attend_ms(db)
                rec = {"shape": name, "block_size": bs, "placement": placement,
                       "attention_ms": round(ms, 4),
                       "unused_slots_frac": round(1 - tokens / (need * bs), 4)}
                if placement == "shuffled":
                    # Copy-out: gather every context into blocks no sequence
                    # uses (in table order), then attend there.
                    tbl = w.block_tables
                    live = np.zeros(nb, bool)
                    for si, L in enumerate(w.context_lens):
                        live[tbl[si, :-(-int(L) // bs)]] = True
                    free = iter(np.flatnonzero(~live).tolist())
                    pairs, ctab = [], np.zeros_like(tbl)
                    for si, L in enumerate(w.context_lens):
                        for j in range(-(-int(L) // bs)):
                            dst = next(free)
                            pairs.append((int(tbl[si, j]), dst))
                            ctab[si, j] = dst
                    pairs_t = torch.tensor(pairs, dtype=torch.int32, device="cuda")
                    ctab_t = torch.from_numpy(ctab).to("cuda")

                    def copy_then_attend():
                        binding.pa_copy_blocks(db.k_cache, db.v_cache, pairs_t)
                        binding.pa_attention(db.out, db.q, db.k_cache, db.v_cache, ctab_t,
                                             db.context_lens, db.query_start_loc,
                                             db.context_lens_host, db.qsl_host, w.scale,
                                             db.workspace, db.opt)
                    rec["copy_out_then_attend_ms"] = round(_time_ms(copy_then_attend, reps), 4)
                emit(rec)
                del db
                torch.cuda.empty_cache()

    for cfg in (3, 5):
        w = config_workload(cfg)
        db = DeviceBatch(w)
        db.write_history()
        db.write_new()
        torch.cuda.synchronize()
        unified = attend_ms(db)
        n = np.diff(w.query_start_loc)
        parts = []
        for sel in (n > 1, n == 1):
            idx = np.flatnonzero(sel)
            qsl = np.zeros(idx.size + 1, np.int32)
            qsl[1:] = np.cumsum(n[idx])
            rows = np.concatenate([np.arange(w.query_start_loc[i], w.query_start_loc[i + 1]) for i in idx])
            sub = dict(bt=torch.from_numpy(np.ascontiguousarray(w.block_tables[idx])).to("cuda"),
                       lens=torch.from_numpy(np.ascontiguousarray(w.context_lens[idx])).to("cuda"),
                       qsl=torch.from_numpy(qsl).to("cuda"),
                       lens_h=torch.from_numpy(np.ascontiguousarray(w.context_lens[idx])),
                       qsl_h=torch.from_numpy(qsl.copy()),
                       q=db.q[torch.from_numpy(rows).to("cuda")].contiguous())
            sub["out"] = torch.empty_like(sub["q"])
            sub["ws"] = torch.empty(binding.pa_attention_workspace_size(
                db.desc, w.num_q_heads, idx.size, int(qsl[-1]), int(w.context_lens[idx].max())),
                dtype=torch.uint8, device="cuda")
            parts.append(sub)

        def separate():
            for sb in parts:
                binding.pa_attention(sb["out"], sb["q"], db.k_cache, db.v_cache, sb["bt"], sb["lens"],
                                     sb["qsl"], sb["lens_h"], sb["qsl_h"], w.scale, sb["ws"])
        # Alternate the two forms and keep each one's best: the first timing in
        # a process runs a few percent slow (clocks still settling), which
        # would otherwise always land on whichever form goes first.
        sep = _time_ms(separate, reps)
        unified = min(unified, attend_ms(db))
        sep = min(sep, _time_ms(separate, reps))

        # Each kernel on its own (events the library records around it): the
        # same kernels in the same times whichever form the call takes.
        def kernel_ms(form, kid):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(reps)]
            for a, b in evs:
                o = binding.options(0, 0, 0, kid, a, b)
                if form == "unified":
                    binding.pa_attention(db.out, db.q, db.k_cache, db.v_cache, db.block_tables,
                                         db.context_lens, db.query_start_loc, db.context_lens_host,
                                         db.qsl_host, w.scale, db.workspace, o)
                else:   # the events are recorded by whichever call runs that kernel
                    for sb in parts:
                        binding.pa_attention(sb["out"], sb["q"], db.k_cache, db.v_cache, sb["bt"],
                                             sb["lens"], sb["qsl"], sb["lens_h"], sb["qsl_h"], w.scale,
                                             sb["ws"], o)
            torch.cuda.synchronize()
            return round(float(np.mean([a.elapsed_time(b) for a, b in evs])), 4)
        kinds = (("tile", binding.PA_TIME_TILE), ("decode", binding.PA_TIME_ROWS),
                 ("combine", binding.PA_TIME_COMBINE))
        per = {form: {k: kernel_ms(form, kid) for k, kid in kinds} for form in ("unified", "separate")}
        emit({"batch": w.name, "unified_call_ms": round(unified, 4),
              "separate_calls_ms": round(sep, 4), "kernels_ms": per})
        del db, parts
        torch.cuda.empty_cache()

    # Copy-on-write copies of one step on a 32-layer model: one launch for all
    # layers vs one launch per layer (the config-4 shape: 180 pairs of bf16
    # blocks, 2 KV heads x 16 tokens x 128).
    layers, nb, h, bs, d = 32, 4096, 2, 16, 128
    ks = [torch.zeros((nb, h, bs, d), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    vs = [torch.zeros((nb, h, d, bs), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    perm = np.random.default_rng(4).permutation(nb)
    pairs = torch.from_numpy(np.stack([perm[:180], perm[180:360]], 1).astype(np.int32)).cuda()
    moved = 2 * 2 * 180 * h * bs * d * 2 * layers            # read + write, K + V
    one = _time_ms(lambda: binding.pa_copy_blocks_layers(ks, vs, pairs), reps)
    per = _time_ms(lambda: [binding.pa_copy_blocks(k, v, pairs) for k, v in zip(ks, vs)], reps)
    emit({"copy_on_write_layers": layers, "pairs": 180, "bytes_moved": moved,
          "one_launch_ms": round(one, 4), "one_launch_GBs": round(moved / one / 1e6, 1),
          "launch_per_layer_ms": round(per, 4), "launch_per_layer_GBs": round(moved / per / 1e6, 1),
          "note": "call times from Python, host time included (one call checks and passes 64 pool "
                  "pointers); the kernel's own time is in a kernel trace of this command"})
    return 0


def swap(args) -> int:
    """Host <-> device block swaps on the DMA engines (pa_swap_blocks).

    - rates for one run of consecutive blocks and for scattered blocks, both
      directions (bf16, 8 KV heads x 128, block 32: 128 KB of K+V a block);
    - swap-in and swap-out at the same time on two streams vs one after the
      other (the Pensieve page, 实现细节与优化, saw both directions slow down
      by 18-20% when concurrent);
    - a 16-layer step: every layer swaps 64 blocks in and runs the 64-decode
      attention batch; all swaps first, then all attention, vs the layer-wise
      pipeline that gates each layer's attention on its own event.
    """
    import torch
    from paged_kv_cache_block_amd import binding
    from paged_kv_cache_block_amd.step import DeviceBatch
    from paged_kv_cache_block_amd.swap import LayerSwap, LayerSwapPipeline
    from workloads import config_workload

    reps = max(args.steps, 5)

    def emit(d):
        print(json.dumps({"swap": d}), flush=True)

    nb, h, bs, d = 4096, 8, 32, 128
    blk = 2 * h * bs * d * 2
    dk = torch.zeros((nb, h, bs, d), dtype=torch.bfloat16, device="cuda")
    dv = torch.zeros((nb, h, d, bs), dtype=torch.bfloat16, device="cuda")
    hk = torch.zeros((nb, h, bs, d), dtype=torch.bfloat16).pin_memory()
    hv = torch.zeros((nb, h, d, bs), dtype=torch.bfloat16).pin_memory()
    n = 1024
    rng = np.random.default_rng(1)
    run = np.stack([np.arange(n), np.arange(n) + 2048], 1).astype(np.int32)
    scat = np.stack([rng.permutation(nb)[:n], rng.permutation(nb)[:n]], 1).astype(np.int32)
    for name, pairs in (("run", run), ("scattered", scat)):
        pt = torch.from_numpy(pairs)
        for dname, dirn in (("in", binding.PA_SWAP_IN), ("out", binding.PA_SWAP_OUT)):
            ms = _time_ms(lambda: binding.pa_swap_blocks(dk, dv, hk, hv, pt, dirn), reps)
            emit({"pairs": name, "direction": dname, "blocks": n, "bytes": n * blk,
                  "ms": round(ms, 4), "GBs": round(n * blk / ms / 1e6, 1)})
    pin, pout = torch.from_numpy(run), torch.from_numpy(run[:, ::-1].copy())
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()

    def concurrent():
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        binding.pa_swap_blocks(dk, dv, hk, hv, pin, binding.PA_SWAP_IN, stream=s1)
        binding.pa_swap_blocks(dk, dv, hk, hv, pout, binding.PA_SWAP_OUT, stream=s2)
        torch.cuda.current_stream().wait_stream(s1)
        torch.cuda.current_stream().wait_stream(s2)

    def ordered():
        binding.pa_swap_blocks(dk, dv, hk, hv, pin, binding.PA_SWAP_IN)
        binding.pa_swap_blocks(dk, dv, hk, hv, pout, binding.PA_SWAP_OUT)
    emit({"both_directions": 2 * n * blk, "concurrent_ms": round(_time_ms(concurrent, reps), 4),
          "ordered_ms": round(_time_ms(ordered, reps), 4)})
    del dk, dv, hk, hv

    w = config_workload(2)
    db = DeviceBatch(w)
    db.write_history()
    db.write_new()
    layers, per = 16, 64
    free = np.setdiff1d(np.arange(w.num_blocks), np.unique(w.block_tables))
    hkl = torch.zeros((per,) + tuple(db.k_cache.shape[1:]), dtype=db.k_cache.dtype).pin_memory()
    hvl = torch.zeros((per,) + tuple(db.v_cache.shape[1:]), dtype=db.v_cache.dtype).pin_memory()
    plan = [LayerSwap(db.k_cache, db.v_cache, hkl, hvl,
                      torch.from_numpy(np.stack([np.arange(per), free[l * per:(l + 1) * per]], 1)
                                       .astype(np.int32))) for l in range(layers)]
    pipe = LayerSwapPipeline()

    def serial():
        pipe.start_swap_in(plan)
        torch.cuda.current_stream().wait_stream(pipe.copy_stream)
        for _ in range(layers):
            db.attention()

    def pipelined():
        pipe.start_swap_in(plan)
        for l in range(layers):
            pipe.wait_layer(l)
            db.attention()
    one_layer_bytes = per * w.num_kv_heads * w.block_size * w.head_dim * 2 * 2
    emit({"layers": layers, "swap_in_per_layer_bytes": one_layer_bytes,
          "attention_per_layer_ms": round(_time_ms(db.attention, reps), 4),
          "swaps_then_attention_ms": round(_time_ms(serial, reps), 4),
          "layerwise_pipeline_ms": round(_time_ms(pipelined, reps), 4)})
    # Release what the swaps used while the runtime is fully up: wait for the
    # copy streams, drop the pipeline (streams, events) and the pinned host
    # pools, and return torch's cached pinned blocks, so that none of it is
    # left for the interpreter's exit.
    torch.cuda.synchronize()
    for st in (pipe.copy_stream, pipe.out_stream, s1, s2):
        st.synchronize()
    del plan, pipe, hkl, hvl, pin, pout, s1, s2, db
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch._C._host_emptyCache()
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed steps for this much wall time before the warmup steps (clock ramp)")
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split", type=int, default=0, help="decode split length (0 = auto)")
    ap.add_argument("--prefill-split", type=int, default=0,
                    help="keys per split of a multi-token context (0 = auto, -1 = none)")
    ap.add_argument("--cold-cache", action="store_true",
                    help="also time the dominant kernel with L2 and MALL flushed before each step")
    ap.add_argument("--separate-write", action="store_true",
                    help="time pa_write_kv then pa_attention instead of pa_write_kv_attention")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once in a HIP graph and replayed (launch gaps out)")
    ap.add_argument("--tile-rows", type=int, default=0, choices=[0, 128, 256],
                    help="rows per multi-token MFMA work item (0 = auto)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run pa_copy_blocks over a known byte count (scales HBM counters)")
    ap.add_argument("--hbm-reference", action="store_true",
                    help="only measure reference HBM rates (torch sum and copy, pa_copy_blocks)")
    ap.add_argument("--paging", action="store_true",
                    help="paging diagnostics: block sizes, contiguous vs shuffled, copy-out, unified vs split calls")
    ap.add_argument("--swap", action="store_true",
                    help="host<->device block swap rates and the layer-wise swap-in pipeline, then exit")
    ap.add_argument("--chunk-cost", action="store_true",
                    help="time one 32-token chunk (and 16 of them) after 0..32K cached tokens, then exit")
    ap.add_argument("--mfma-reference", action="store_true",
                    help="time a large bf16 torch GEMM as a matrix-core reference rate, then exit")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the attention would shard by KV head or by sequence, with no exchange).",
              file=sys.stderr)
        return 2

    import torch
    from paged_kv_cache_block_amd import binding
    from paged_kv_cache_block_amd.step import DeviceBatch
    from workloads import config_workload

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 3
    if args.copy_calibration:
        return copy_calibration(args.steps)
    if args.hbm_reference:
        return hbm_reference()
    if args.mfma_reference:
        return mfma_reference()
    if args.chunk_cost:
        return chunk_cost(args)
    if args.paging:
        return paging(args)
    if args.swap:
        return swap(args)
    t0 = time.time()
    w = config_workload(args.config, args.seed)
    print(f"[bench] built {w.name} in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    unshared = blocks_unshared(w)
    flags = binding.PA_FLAG_KV_UNSHARED if unshared else 0
    if args.prefill_split < 0:
        flags |= binding.PA_FLAG_NO_PREFILL_SPLIT
        args.prefill_split = 0
    db = DeviceBatch(w, opt=binding.options(args.split, args.prefill_split, flags, prefill_tile_rows=args.tile_rows))
    db.write_history()
    torch.cuda.synchronize()
    model = work_model(w)
    has_tiles = bool((w.n_new > 1).any()) and w.dtype != "f32" and w.block_size in (16, 32)
    has_rows = bool((w.n_new == 1).any()) or (bool((w.n_new > 1).any()) and not has_tiles)
    kernels = []
    if has_tiles:
        kernels.append(("tile", binding.PA_TIME_TILE))
    if has_rows:
        kernels.append(("rows", binding.PA_TIME_ROWS))
    if has_tiles and w.dtype != "f32":
        dominant = "tile" if model["tile_flops"] / (MFMA_PEAK_TFLOPS[w.dtype] * 1e12) > \
            model["rows_bytes"] / (HBM_PEAK_GBS * 1e9) else ("rows" if has_rows else "tile")
    else:
        dominant = "rows"

    def run_step(opt):
        db.copy_blocks()
        if args.separate_write:
            db.write_new()
            db.attention(opt=opt)
        else:
            db.write_attention(opt=opt)

    base_opt = binding.options(args.split, args.prefill_split, flags, prefill_tile_rows=args.tile_rows)
    # Settle: untimed steps for about --settle-ms of wall time before the
    # warmup steps.  A process's first tens of milliseconds of load run a few
    # percent slow while the chip's clocks come up (config 5's multi-token
    # kernel: about 1.05 ms over the first 20 calls, 0.975 ms after), so a
    # short warmup alone would time the ramp, not the steady state.
    settle_steps = 0
    torch.cuda.synchronize()
    t_settle = time.time()
    while (time.time() - t_settle) * 1e3 < args.settle_ms and settle_steps < 20_000:
        run_step(base_opt)
        settle_steps += 1
        if settle_steps % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    settle_ms = (time.time() - t_settle) * 1e3
    for _ in range(args.warmup):
        run_step(base_opt)
    torch.cuda.synchronize()
    print(f"[bench] settled ({settle_steps} steps, {settle_ms:.0f} ms), warmup done ({args.warmup} steps)",
          file=sys.stderr, flush=True)

    K = args.steps
    dom_id = dict(kernels)[dominant]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    opts = [binding.options(args.split, args.prefill_split, flags, dom_id, a, b, args.tile_rows) for a, b in evs]
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(K):
        run_step(opts[i])
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / K
    dom_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    print(f"[bench] timed {K} steps: {ms_step:.4f} ms/step", file=sys.stderr, flush=True)

    # The other kernels, timed the same way in a second pass (reported only).
    per_kernel = {dominant: dom_ms}
    for name, kid in kernels:
        if name == dominant:
            continue
        evs2 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(K)]
        opts2 = [binding.options(args.split, args.prefill_split, flags, kid, a, b, args.tile_rows) for a, b in evs2]
        for i in range(K):
            run_step(opts2[i])
        torch.cuda.synchronize()
        per_kernel[name] = float(np.mean([a.elapsed_time(b) for a, b in evs2]))

    # --cold-cache: the dominant kernel once more with L2 and the MALL flushed
    # before every step (a 512 MiB write between steps).  The timed steps
    # above run back to back, as a serving loop does.
    dom_cold_ms = None
    if args.cold_cache:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=db.device)
        evs3 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(K)]
        opts3 = [binding.options(args.split, args.prefill_split, flags, dom_id, a, b, args.tile_rows)
                 for a, b in evs3]
        for i in range(K):
            scratch.fill_(i & 255)
            run_step(opts3[i])
        torch.cuda.synchronize()
        dom_cold_ms = float(np.mean([a.elapsed_time(b) for a, b in evs3]))
        del scratch

    # --graph: the same step captured once in a HIP graph and replayed K
    # times, back to back.  The replay has the same kernels and work; what it
    # removes is the host's per-launch cost and the gaps between launches,
    # which is what a launch-bound step (few, short kernels) spends beyond its
    # kernels.  Reported beside the eager step, never as `value`.
    graph_ms = None
    if args.graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_step(base_opt)
        torch.cuda.synchronize()
        for _ in range(max(args.warmup, 1)):
            g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(K):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / K
        del g

    value = model["step_bytes"] / (ms_step * 1e-3) / 1e9
    rows_kernel = ("decode_mfma_kernel" if w.dtype != "f32" and w.block_size in (16, 32)
                   else "row_attn_kernel")
    from paged_kv_cache_block_amd.profiling import counter_record_for, traffic_record_for
    stored_ok = (args.split == 0 and args.tile_rows == 0 and args.prefill_split == 0
                 and not flags & binding.PA_FLAG_NO_PREFILL_SPLIT)

    def roof_block(which, ms):
        """Roofline of one attention kernel from its mean launch time."""
        if which == "rows":
            achieved = model["rows_bytes"] / (ms * 1e-3) / 1e9
            r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                 "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                 "kernel": rows_kernel, "algorithmic_bytes": model["rows_bytes"],
                 "avg_ms": round(ms, 5)}
            if model["rows_unique_bytes"] < model["rows_bytes"]:
                # Blocks shared by several rows (reference counts): the bytes
                # that must cross from HBM count each cached slot once.  The
                # fraction of peak is stated on those, so it cannot pass 1.
                au = model["rows_unique_bytes"] / (ms * 1e-3) / 1e9
                r.update({"unique_bytes": model["rows_unique_bytes"], "achieved_unique": round(au, 1),
                          "frac": round(au / HBM_PEAK_GBS, 4),
                          "frac_logical": round(achieved / HBM_PEAK_GBS, 4),
                          "frac_note": "frac on unique bytes (each cached slot once); "
                                       "frac_logical counts each row's context once per KV head"})
        else:
            achieved = model["tile_flops"] / (ms * 1e-3) / 1e12
            peak = MFMA_PEAK_TFLOPS[w.dtype]
            r = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                 "frac": round(achieved / peak, 4), "traffic": None, "kernel": "tile_attn_kernel",
                 "algorithmic_flops": model["tile_flops"], "avg_ms": round(ms, 5)}
        rec = traffic_record_for(r["kernel"], args.config) if stored_ok else None
        if rec is not None:
            r["traffic"] = rec["fetch_bytes"] + rec["write_bytes"]
            r["traffic_note"] = ("HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                 "scaled by pa_copy_blocks over a known byte count")
        if which == "tile":
            mrec = counter_record_for("mfma-record", "tile_attn_kernel", args.config) if stored_ok else None
            if mrec is not None:
                r["mfma_busy"] = mrec["mfma_busy_frac"]
                r["mfma_busy_note"] = ("SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE per XCD), "
                                       "rocprofv3 --pmc of the same command")
        return r

    roof = roof_block(dominant, dom_ms)
    others = {}
    for name, _ in kernels:
        if name != dominant:
            others["roofline_decode" if name == "rows" else "roofline_multi_token"] = \
                roof_block(name, per_kernel[name])
    if dom_cold_ms is not None:
        unit_work = model["rows_bytes"] if dominant == "rows" else model["tile_flops"]
        roof["cold_cache"] = {
            "avg_ms": round(dom_cold_ms, 5),
            "achieved": round(unit_work / (dom_cold_ms * 1e-3) / (1e9 if dominant == "rows" else 1e12), 1),
            "note": "the same kernel with a 512 MiB write before every step (L2 and MALL flushed)"}
        if dominant == "rows" and "unique_bytes" in roof:
            roof["cold_cache"]["achieved_unique"] = round(
                model["rows_unique_bytes"] / (dom_cold_ms * 1e-3) / 1e9, 1)
    extra = {}
    if "tile" in per_kernel:
        extra["multi_token_tflops"] = round(model["tile_flops"] / (per_kernel["tile"] * 1e-3) / 1e12, 1)
    if "rows" in per_kernel:
        extra["decode_kv_gbs"] = round(model["rows_bytes"] / (per_kernel["rows"] * 1e-3) / 1e9, 1)

    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        cpu = cpu_baseline(w, args.cpu_seconds)
        print(f"[bench] cpu baseline in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
        if cpu is not None:
            cpu = {k2: (round(v, 3) if isinstance(v, float) else v) for k2, v in cpu.items()}

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "settle_steps": settle_steps, "settle_ms": round(settle_ms, 1),
        "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "config": args.config, "seqs": w.num_seqs,
                   "query_rows": int(w.q.shape[0]), "new_tokens": int(w.k_new.shape[0]),
                   "cow_pairs": int(w.cow_pairs.shape[0]), "kv_unshared_hint": unshared,
                   "step": ("pa_copy_blocks, pa_write_kv, pa_attention" if args.separate_write
                            else "pa_copy_blocks, pa_write_kv_attention"),
                   "step_bytes": model["step_bytes"], "multi_token_flops": model["tile_flops"]},
        "roofline": roof,
        **others,
        "kernels_ms": {k2: round(v, 5) for k2, v in per_kernel.items()},
        **({"graph_replay": {"ms_per_step": round(graph_ms, 5),
                             "note": "the same step captured once in a HIP graph and replayed"}}
           if graph_ms is not None else {}),
        "derived": extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
