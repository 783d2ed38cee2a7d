"""CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The HIP
library never imports it, and it imports nothing from the HIP library.

Plain NumPy, float64 throughout.  Every function states the passage of the
source pages it follows.  The pages are cited by title and section:

* Pensieve page  -- "Stateful Large Language Model Serving with Pensieve"
  (papercache.org summary).
* vLLM wiki page -- "vLLM-SOSP23" (Awesome System Papers Wiki, papers.lqhl.me).
* vLLM blog page -- the devpress.csdn.net article on vLLM.
* PagedAttention wiki page -- "PagedAttention" (lib.yinfer.top).

Storage conventions (the same contract the C header documents; restated here,
not shared):

* fp32 arrays are ``np.float32``; fp16 arrays are ``np.float16``; bf16 arrays
  are ``np.uint16`` holding the raw bf16 bit pattern.
* K pool: ``[num_blocks][num_kv_heads][block_size][head_dim]``.
* V pool: ``[num_blocks][num_kv_heads][head_dim][block_size]`` (head-dim
  major inside a block).
* A slot is ``block * block_size + offset``; token ``j`` of a sequence lives
  in block ``block_table[j // block_size]`` at offset ``j % block_size``.
* The new query tokens of a sequence are its last ``n`` context positions.

What pins each function is listed in ``tests/test_oracle_pins.py``.  Every
function here has at least one pin other than itself.
"""
from __future__ import annotations

import numpy as np

DTYPES = ("f32", "f16", "bf16")


# --------------------------------------------------------------------------
# Element conversion (exact widening to float64)
# --------------------------------------------------------------------------
def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values to float64 exactly.

    bf16 is the upper half of an IEEE binary32 word, so the widening places
    the 16 stored bits in the high half of a 32-bit word.
    """
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# a1: block copy (copy-on-write)
# --------------------------------------------------------------------------
def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs) -> None:
    """Copy whole physical blocks, K and V, for each ``(src, dst)`` pair.

    vLLM blog page, section 2.1 (parallel sampling): a writer that finds its
    block shared (reference count above one) gets a fresh block and the block
    engine copies the old block's contents into it.  vLLM wiki page, section
    "Kernel 层实现", names the batched block copy.  The copy is bitwise.
    """
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        k_cache[dst] = k_cache[src]
        v_cache[dst] = v_cache[src]


def swap_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray, dst_v: np.ndarray,
                pairs) -> None:
    """Copy whole blocks from one pool pair into another, for each ``(src, dst)``.

    Pensieve page, "流水线KV缓存恢复" and "提前交换": K/V tokens are copied
    from the GPU cache to a CPU cache (swap-out) and back (swap-in) a block of
    tokens at a time; vLLM wiki page, "调度与抢占": preempted sequences' blocks
    are swapped between GPU and CPU memory.  The copy is bitwise; the two pools
    have the same per-block layout and may differ in block count.
    """
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        dst_k[dst] = src_k[src]
        dst_v[dst] = src_v[src]


# --------------------------------------------------------------------------
# a2: slot-mapping scatter of new K/V
# --------------------------------------------------------------------------
def write_kv(k_cache, v_cache, k_new, v_new, slot_mapping) -> None:
    """Store each new token's K and V into its slot, bitwise.

    Pensieve page, "统一Prefill和Generation阶段的执行过程": the newly made KV
    tokens are stored into the slots allocated in the GPU cache before the
    attention kernel runs.  vLLM wiki page, "Kernel 层实现": the reshape and
    block write are one operation.  A negative slot means "no slot" and the
    token is skipped.
    """
    bs = k_cache.shape[2]
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), bs)
        k_cache[blk, :, off, :] = k_new[t]
        v_cache[blk, :, :, off] = v_new[t]


# --------------------------------------------------------------------------
# a3: block-table gather
# --------------------------------------------------------------------------
def gather_context(k_cache, v_cache, block_table, context_len: int, dtype: str):
    """Gather one sequence's K and V into contiguous float64 arrays.

    vLLM wiki page, "核心方法 / PagedAttention": logical block ``j`` of a
    sequence maps through its block table to an arbitrary physical block; the
    kernel reads K/V by that indirection.  Only positions below the context
    length are read (vLLM blog page, section 1: only the last block of a
    sequence is partly filled).

    Returns ``Kc, Vc`` of shape ``[context_len, num_kv_heads, head_dim]``.
    """
    bs = k_cache.shape[2]
    j = np.arange(context_len, dtype=np.int64)
    blocks = np.asarray(block_table, dtype=np.int64)[j // bs]
    offs = j % bs
    kc = k_cache[blocks, :, offs, :]            # [L, H_kv, D]
    vc = v_cache[blocks, :, :, offs]            # [L, H_kv, D]
    return to_f64(kc, dtype), to_f64(vc, dtype)


# --------------------------------------------------------------------------
# a4 + a5: causal attention over the gathered context
# --------------------------------------------------------------------------
def attention_seq(q_rows, kc, vc, n_new: int, query_index, num_kv_heads: int,
                  scale: float) -> np.ndarray:
    """Causal softmax attention for some query rows of one sequence.

    Pensieve page, "LLM与注意力机制": ``A = Q K^T / scale`` then
    ``O = softmax(A) V`` per head.  PagedAttention wiki page, "数学表述":
    query ``i`` attends to key positions ``1..i`` only, normalised over the
    same range.  Pensieve page, "融合因果掩码与内核实现": earlier query tokens
    do not see later ones.  Pensieve page, "统一Prefill和Generation阶段的执行
    过程": single-token decode is the one-query case.

    ``q_rows``      float64 ``[r, H_q, D]``: the selected query rows.
    ``query_index`` int ``[r]``: each row's index ``i`` among the sequence's
                    ``n_new`` new tokens; its absolute position is
                    ``L - n_new + i`` and it sees keys ``0..L - n_new + i``.
    ``scale``       multiplies the dot product (``1/sqrt(D)`` by default at
                    the call sites).
    Returns float64 ``[r, H_q, D]``.
    """
    L = kc.shape[0]
    r, hq, d = q_rows.shape
    group = hq // num_kv_heads
    pos = L - n_new + np.asarray(query_index, dtype=np.int64)      # [r]
    visible = np.arange(L)[None, :] <= pos[:, None]                 # [r, L]
    out = np.empty((r, hq, d), dtype=np.float64)
    for h in range(hq):
        g = h // group
        a = scale * (q_rows[:, h, :] @ kc[:, g, :].T)               # [r, L]
        a = np.where(visible, a, -np.inf)
        a = a - a.max(axis=1, keepdims=True)
        w = np.exp(a)
        out[:, h, :] = (w @ vc[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out


def attention(q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
              num_kv_heads: int, dtype: str, scale: float | None = None,
              seqs=None) -> np.ndarray:
    """Paged attention for a ragged batch, as one float64 array.

    Pensieve page, "多Token注意力内核运算原理" and "统一Prefill和Generation
    阶段的执行过程": the batch concatenates every request's new tokens; each
    request's region is given by auxiliary per-request data
    (``query_start_loc``), and each request attends to its own paged context.

    ``seqs`` restricts the work to some sequences (rows of other sequences
    are left as NaN); used for sampled checks at large sizes.
    """
    qf = to_f64(q, dtype)
    t, hq, d = qf.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.full((t, hq, d), np.nan, dtype=np.float64)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    lens = np.asarray(context_lens, dtype=np.int64)
    todo = range(len(lens)) if seqs is None else seqs
    for s in todo:
        q0, q1 = int(qsl[s]), int(qsl[s + 1])
        n = q1 - q0
        if n == 0:
            continue
        kc, vc = gather_context(k_cache, v_cache, block_tables[s], int(lens[s]), dtype)
        out[q0:q1] = attention_seq(qf[q0:q1], kc, vc, n, np.arange(n),
                                   num_kv_heads, scale)
    return out


# --------------------------------------------------------------------------
# a6: split-context partial states and their combination
# --------------------------------------------------------------------------
def partial_state(q_row, kc, vc, key_lo: int, key_hi: int, limit: int,
                  num_kv_heads: int, scale: float):
    """Softmax state of one query row over the keys ``[key_lo, key_hi)``.

    Not on the pages (they never split one context); it restates the
    exponent-shift identity of softmax.  Keys above ``limit`` are masked.
    Returns ``m[H_q]`` (max score, ``-inf`` if every key is masked),
    ``l[H_q]`` (sum of ``exp(score - m)``) and ``acc[H_q, D]``
    (``sum exp(score - m) v``, unnormalised).
    """
    hq, d = q_row.shape
    group = hq // num_kv_heads
    keys = np.arange(key_lo, key_hi)
    keys = keys[keys <= limit]
    m = np.full(hq, -np.inf)
    lsum = np.zeros(hq)
    acc = np.zeros((hq, d))
    if keys.size == 0:
        return m, lsum, acc
    for h in range(hq):
        g = h // group
        a = scale * (kc[keys, g, :] @ q_row[h])
        m[h] = a.max()
        w = np.exp(a - m[h])
        lsum[h] = w.sum()
        acc[h] = w @ vc[keys, g, :]
    return m, lsum, acc


def combine_partials(ms, ls, accs) -> np.ndarray:
    """Merge split states: ``m = max m_k``; ``l = sum l_k e^(m_k - m)``;
    ``o = sum e^(m_k - m) acc_k / l``.  Splits whose every key was masked
    (``l_k = 0``) contribute nothing."""
    ms = np.asarray(ms)          # [K, H]
    ls = np.asarray(ls)          # [K, H]
    accs = np.asarray(accs)      # [K, H, D]
    m = ms.max(axis=0)
    w = np.where(ls > 0, np.exp(ms - m[None, :]), 0.0)
    lsum = (w * ls).sum(axis=0)
    return (w[:, :, None] * accs).sum(axis=0) / lsum[:, None]
