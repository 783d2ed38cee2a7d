"""Pins for the CPU oracle: each check ties it to something other than itself.

* golden integers from the pages (block mapping, copy-on-write);
* exact conversions of known bit patterns;
* brute force on tiny inputs: the token-level causal formula of the
  PagedAttention wiki page ("数学表述") in plain Python loops, and
  ``torch.nn.functional.scaled_dot_product_attention`` in float64 on the CPU
  with an explicit mask;
* closed forms (one key, constant values, shifted keys, identical keys);
* invariants: relabelling physical blocks, decode = last prefill row,
  sub-requests and chunked prefill (Pensieve page, "非连续Query张量的子请求
  处理"), and the split-context combination.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from workloads import BlockManager, build_batch, config_workload, round_to_dtype, small_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def run_oracle(w, k=None, v=None):
    """Apply the workload's step to host pools with the oracle: history,
    copy-on-write, new tokens, attention."""
    if k is None:
        k, v = w.empty_pools()
    oracle.write_kv(k, v, w.hist_k, w.hist_v, w.hist_slots)
    oracle.copy_blocks(k, v, w.cow_pairs)
    oracle.write_kv(k, v, w.k_new, w.v_new, w.slot_mapping)
    out = oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                           w.num_kv_heads, w.dtype, w.scale)
    return out, k, v


# --------------------------------------------------------------------------
# Golden integers from the pages
# --------------------------------------------------------------------------
def test_worked_block_mapping():
    g = _golden("worked_block_mapping.json")
    bs = g["block_size"]
    mgr = BlockManager(16, bs, [7, 1, 3] + [b for b in range(16) if b not in (7, 1, 3)])
    mgr.add_sequence(0)
    slots, pairs = mgr.append(0, g["prompt_tokens"])
    assert mgr.tables[0] == g["prompt_physical_blocks"]
    assert mgr.filled(0) == g["filled_after_prompt"]
    exp = [b * bs + o for b, n in zip(g["prompt_physical_blocks"], g["filled_after_prompt"])
           for o in range(n)]
    assert slots == exp == [28, 29, 30, 31, 4, 5, 6]
    s1, _ = mgr.append(0, 1)
    assert s1 == [g["decode1_block"] * bs + 3] == [7]
    assert mgr.filled(0) == g["filled_after_decode1"]
    s2, _ = mgr.append(0, 1)
    assert mgr.tables[0] == g["physical_blocks_after_decode2"]
    assert s2 == [g["decode2_new_physical_block"] * bs] == [12]
    assert mgr.filled(0) == g["filled_after_decode2"]
    assert not pairs


def test_config1_uses_worked_example():
    w = config_workload(1)
    assert list(w.block_tables[0, :2]) == [7, 1]
    assert list(w.hist_slots[:7]) == [28, 29, 30, 31, 4, 5, 6]
    assert w.slot_mapping[0] == 7
    assert list(w.context_lens) == [8, 5, 12]
    assert list(w.query_start_loc) == [0, 1, 6, 9]


def test_cow_parallel_sampling():
    g = _golden("cow_parallel_sampling.json")
    bs = g["block_size"]
    mgr = BlockManager(16, bs, [7, 1, 3] + [b for b in range(16) if b not in (7, 1, 3)])
    mgr.add_sequence(0)
    mgr.append(0, g["prompt_tokens"])
    mgr.fork(0, 1)
    assert {str(b): int(mgr.ref[b]) for b in g["shared_physical_blocks"]} == g["refcounts_before"]
    a1_slots, a1_pairs = mgr.append(0, 1)
    assert a1_pairs == [tuple(g["a1_copy_pair"])]
    assert mgr.tables[0][1] == g["a1_writer_new_block"]
    assert int(mgr.ref[1]) == g["refcount_block1_after_a1"]
    assert a1_slots == [g["a1_writer_new_block"] * bs + 3] == [15]
    a2_slots, a2_pairs = mgr.append(1, 1)
    assert a2_pairs == []
    assert a2_slots == [g["a2_writes_in_place_to_block"] * bs + 3] == [7]

    # The oracle's copy + write then give each sample its own last token and
    # leave the shared prompt intact for both.
    rng = np.random.default_rng(0)
    k = np.full((16, 2, bs, 8), np.nan, np.float32)
    v = np.full((16, 2, 8, bs), np.nan, np.float32)
    prompt_k = rng.standard_normal((7, 2, 8)).astype(np.float32)
    prompt_v = rng.standard_normal((7, 2, 8)).astype(np.float32)
    oracle.write_kv(k, v, prompt_k, prompt_v, [28, 29, 30, 31, 4, 5, 6])
    oracle.copy_blocks(k, v, a1_pairs)
    new_k = rng.standard_normal((2, 2, 8)).astype(np.float32)
    new_v = rng.standard_normal((2, 2, 8)).astype(np.float32)
    oracle.write_kv(k, v, new_k, new_v, a1_slots + a2_slots)
    for seq, t in ((0, 0), (1, 1)):
        kc, vc = oracle.gather_context(k, v, mgr.tables[seq], 8, "f32")
        np.testing.assert_array_equal(kc[:7], prompt_k)
        np.testing.assert_array_equal(vc[:7], prompt_v)
        np.testing.assert_array_equal(kc[7], new_k[t])
        np.testing.assert_array_equal(vc[7], new_v[t])


# --------------------------------------------------------------------------
# Exact conversions
# --------------------------------------------------------------------------
def test_to_f64_bit_patterns():
    bf = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F80, 0x8000], dtype=np.uint16)
    got = oracle.to_f64(bf, "bf16")
    assert list(got[:4]) == [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133]
    assert got[4] == math.inf and got[5] == 0.0 and math.copysign(1, got[5]) < 0
    hf = np.array([0x3C00, 0xC000, 0x3C01, 0x0001], dtype=np.uint16).view(np.float16)
    assert list(oracle.to_f64(hf, "f16")) == [1.0, -2.0, 1.0 + 2.0 ** -10, 2.0 ** -24]


def test_generator_rounding_is_nearest_even():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -9), 3.0],
                 dtype=np.float32)
    got = oracle.to_f64(round_to_dtype(x, "bf16"), "bf16")
    assert list(got) == [1.0, 1.0 + 2.0 ** -6, -1.0, 3.0]


# --------------------------------------------------------------------------
# Scatter / gather round trip and layout
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_write_gather_roundtrip(dtype):
    w = small_workload(3)
    k, v = w.empty_pools()
    oracle.write_kv(k, v, w.hist_k, w.hist_v, w.hist_slots)
    oracle.write_kv(k, v, w.k_new, w.v_new, w.slot_mapping)
    # token t of sequence s: history tokens first, then the new ones
    hist_at = 0
    new_at = 0
    for s, (h, n, _) in enumerate(w.meta["specs"]):
        kc, vc = oracle.gather_context(k, v, w.block_tables[s], h + n, w.dtype)
        want_k = np.concatenate([w.hist_k[hist_at:hist_at + h], w.k_new[new_at:new_at + n]])
        want_v = np.concatenate([w.hist_v[hist_at:hist_at + h], w.v_new[new_at:new_at + n]])
        np.testing.assert_array_equal(kc, oracle.to_f64(want_k, w.dtype))
        np.testing.assert_array_equal(vc, oracle.to_f64(want_v, w.dtype))
        hist_at += h
        new_at += n
    # explicit layout: V is head-dim major inside a block
    t = 5
    blk, off = divmod(int(w.slot_mapping[t]), w.block_size)
    np.testing.assert_array_equal(v[blk, 3, :, off], w.v_new[t, 3])
    np.testing.assert_array_equal(k[blk, 3, off, :], w.k_new[t, 3])


def test_negative_slot_is_skipped():
    k = np.zeros((2, 1, 4, 2), np.float32)
    v = np.zeros((2, 1, 2, 4), np.float32)
    oracle.write_kv(k, v, np.ones((2, 1, 2), np.float32), np.ones((2, 1, 2), np.float32), [-1, 5])
    assert k.sum() == 2 and k[1, 0, 1].tolist() == [1, 1] and v[1, 0, :, 1].tolist() == [1, 1]


# --------------------------------------------------------------------------
# Brute force on tiny inputs
# --------------------------------------------------------------------------
def _brute_python(q, kc, vc, n, hkv):
    """Token-level causal formula, plain loops and math.exp."""
    r, hq, d = q.shape
    L = kc.shape[0]
    g = hq // hkv
    out = np.zeros_like(q)
    for i in range(r):
        p = L - n + i
        for h in range(hq):
            kh = h // g
            e = [math.exp(sum(q[i, h, x] * kc[j, kh, x] for x in range(d)) / math.sqrt(d))
                 for j in range(p + 1)]
            z = sum(e)
            for x in range(d):
                out[i, h, x] = sum(e[j] * vc[j, kh, x] for j in range(p + 1)) / z
    return out


def _brute_torch(q, kc, vc, n, hkv):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    r, hq, d = q.shape
    L = kc.shape[0]
    g = hq // hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]                     # [1, Hq, r, D]
    kt = torch.from_numpy(kc).permute(1, 0, 2).repeat_interleave(g, 0)[None]
    vt = torch.from_numpy(vc).permute(1, 0, 2).repeat_interleave(g, 0)[None]
    pos = L - n + torch.arange(r)
    mask = torch.arange(L)[None, :] <= pos[:, None]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return o[0].permute(1, 0, 2).numpy()


TINY = [  # (hq, hkv, d, bs, [(hist, new)])
    (2, 2, 4, 4, [(0, 1), (3, 1), (0, 5), (6, 3)]),
    (4, 2, 8, 2, [(5, 1), (0, 7), (9, 2)]),
    (6, 3, 4, 4, [(11, 1), (2, 4)]),
    (4, 1, 16, 4, [(4, 4), (0, 12)]),
]


@pytest.mark.parametrize("case", range(len(TINY)))
def test_brute_force_tiny(case):
    hq, hkv, d, bs, seqs = TINY[case]
    w = build_batch("tiny", "f32", hq, hkv, d, bs, 64, [(h, n, 1) for h, n in seqs], 77 + case)
    out, k, v = run_oracle(w)
    for s, (h, n) in enumerate(seqs):
        q0, q1 = w.query_start_loc[s], w.query_start_loc[s + 1]
        # contiguous K/V straight from the generator, no paging involved
        kc = np.concatenate([w.hist_k[sum(x for x, _ in seqs[:s]):][:h],
                             w.k_new[q0:q1]]).astype(np.float64)
        vc = np.concatenate([w.hist_v[sum(x for x, _ in seqs[:s]):][:h],
                             w.v_new[q0:q1]]).astype(np.float64)
        qs = w.q[q0:q1].astype(np.float64)
        np.testing.assert_allclose(out[q0:q1], _brute_python(qs, kc, vc, n, hkv), rtol=0, atol=1e-12)
        np.testing.assert_allclose(out[q0:q1], _brute_torch(qs, kc, vc, n, hkv), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------
def _one_seq(L, n, hq=4, hkv=2, d=8, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, hq, d))
    kc = rng.standard_normal((L, hkv, d))
    vc = rng.standard_normal((L, hkv, d))
    return q, kc, vc


def test_single_key_returns_its_value_exactly():
    q, kc, vc = _one_seq(1, 1)
    out = oracle.attention_seq(q, kc, vc, 1, [0], 2, 0.3)
    for h in range(4):
        assert np.array_equal(out[0, h], vc[0, h // 2])


def test_constant_values_give_that_constant():
    q, kc, vc = _one_seq(13, 4)
    vc[:] = np.array([0.5, -1.25, 2.0, 0.0, 3.0, -0.75, 1.0, 0.25])
    out = oracle.attention_seq(q, kc, vc, 4, np.arange(4), 2, 1 / math.sqrt(8))
    np.testing.assert_allclose(out, np.broadcast_to(vc[0, 0], out.shape), atol=1e-12, rtol=0)


def test_shifting_all_keys_changes_nothing():
    q, kc, vc = _one_seq(17, 5)
    a = oracle.attention_seq(q, kc, vc, 5, np.arange(5), 2, 0.35)
    b = oracle.attention_seq(q, kc + np.array([0.3, -2, 1, 0.5, 0, 1.5, -1, 2]), vc, 5,
                             np.arange(5), 2, 0.35)
    np.testing.assert_allclose(a, b, atol=1e-12, rtol=0)


def test_identical_keys_average_visible_values():
    q, kc, vc = _one_seq(9, 3)
    kc[:] = kc[0]
    out = oracle.attention_seq(q, kc, vc, 3, np.arange(3), 2, 0.5)
    for i in range(3):
        p = 9 - 3 + i
        for h in range(4):
            np.testing.assert_allclose(out[i, h], vc[:p + 1, h // 2].mean(axis=0), atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [1, 3, 4, 5])
def test_physical_relabelling_is_bit_identical(cfg):
    w = small_workload(cfg)
    out, k, v = run_oracle(w)
    perm = np.random.default_rng(cfg).permutation(w.num_blocks)   # new id of block b
    k2 = np.empty_like(k)
    v2 = np.empty_like(v)
    k2[perm] = k
    v2[perm] = v
    bt2 = perm[w.block_tables]
    out2 = oracle.attention(w.q, k2, v2, bt2, w.context_lens, w.query_start_loc,
                            w.num_kv_heads, w.dtype, w.scale)
    assert np.array_equal(out, out2, equal_nan=True)


def test_decode_equals_last_prefill_row():
    q, kc, vc = _one_seq(23, 23, seed=3)
    full = oracle.attention_seq(q, kc, vc, 23, np.arange(23), 2, 0.35)
    for L in (1, 7, 23):
        dec = oracle.attention_seq(q[L - 1:L], kc[:L], vc[:L], 1, [0], 2, 0.35)
        np.testing.assert_allclose(dec[0], full[L - 1], atol=1e-12, rtol=0)


def test_sub_requests_and_chunked_prefill_match_one_prefill():
    # Pensieve page, "处理丢弃的Token" / figure 8: a dropped prefix recomputed
    # as one sub-request (attending to itself) and the new prompt as another
    # (attending to the whole context) give the rows of one full prefill.
    q, kc, vc = _one_seq(40, 40, seed=4)
    full = oracle.attention_seq(q, kc, vc, 40, np.arange(40), 2, 0.35)
    r = 9                                  # dropped prefix length
    sub1 = oracle.attention_seq(q[:r], kc[:r], vc[:r], r, np.arange(r), 2, 0.35)
    sub2 = oracle.attention_seq(q[30:], kc, vc, 10, np.arange(10), 2, 0.35)
    np.testing.assert_allclose(sub1, full[:r], atol=1e-12, rtol=0)
    np.testing.assert_allclose(sub2, full[30:], atol=1e-12, rtol=0)
    c1 = oracle.attention_seq(q[:25], kc[:25], vc[:25], 25, np.arange(25), 2, 0.35)
    c2 = oracle.attention_seq(q[25:], kc, vc, 15, np.arange(15), 2, 0.35)
    np.testing.assert_allclose(np.concatenate([c1, c2]), full, atol=1e-12, rtol=0)


def test_split_context_combination():
    q, kc, vc = _one_seq(50, 6, seed=5)
    full = oracle.attention_seq(q, kc, vc, 6, np.arange(6), 2, 0.35)
    for i in range(6):
        limit = 50 - 6 + i
        bounds = [0, 7, 20, 21, 48, 50]            # the last split is fully masked for i = 0
        parts = [oracle.partial_state(q[i], kc, vc, a, b, limit, 2, 0.35)
                 for a, b in zip(bounds[:-1], bounds[1:])]
        comb = oracle.combine_partials(*zip(*parts))
        np.testing.assert_allclose(comb, full[i], atol=1e-12, rtol=0)


def test_unused_slots_never_reach_the_output():
    for cfg in (1, 2, 3, 4, 5):
        out, _, _ = run_oracle(small_workload(cfg))
        rows = out[~np.isnan(out).all(axis=(1, 2))]
        assert rows.shape[0] == out.shape[0]
        assert np.isfinite(out).all()


def test_swap_out_then_in_restores_the_pool_and_matches_copy_blocks():
    """Swapping blocks to a second pool and back is the identity on those
    blocks; within one pool it is exactly the copy-on-write copy."""
    rng = np.random.default_rng(5)
    k = rng.standard_normal((12, 2, 4, 8))
    v = rng.standard_normal((12, 2, 8, 4))
    hk, hv = np.zeros((5, 2, 4, 8)), np.zeros((5, 2, 8, 4))
    out_pairs = [(3, 0), (7, 4), (8, 1)]
    oracle.swap_blocks(k, v, hk, hv, out_pairs)
    assert np.array_equal(hk[[0, 4, 1]], k[[3, 7, 8]]) and np.array_equal(hv[4], v[7])
    assert not hk[[2, 3]].any()                 # untouched host blocks stay as they were
    k2, v2 = k.copy(), v.copy()
    k2[[3, 7, 8]] = 0
    v2[[3, 7, 8]] = 0
    oracle.swap_blocks(hk, hv, k2, v2, [(s, d) for d, s in out_pairs])
    assert np.array_equal(k2, k) and np.array_equal(v2, v)
    k3, v3, k4, v4 = k.copy(), v.copy(), k.copy(), v.copy()
    oracle.swap_blocks(k3, v3, k3, v3, [(1, 9), (2, 10)])
    oracle.copy_blocks(k4, v4, [(1, 9), (2, 10)])
    assert np.array_equal(k3, k4) and np.array_equal(v3, v4)
