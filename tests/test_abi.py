"""CPU checks of the C ABI: the library loads, exports every declared entry
point, and rejects bad arguments on the host before touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def binding():
    from paged_kv_cache_block_amd import binding as b
    return b


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for s in ("pa_write_kv", "pa_copy_blocks", "pa_attention", "pa_attention_workspace_size",
              "pa_last_error"):
        assert s in syms


def test_library_exports_every_declared_symbol(binding):
    lib = ctypes.CDLL(binding.LIB_PATH)
    missing = [s for s in declared_symbols() if not hasattr(lib, s)]
    assert not missing, missing
    assert binding.version() >= 100


def _desc(b, nb=16, bs=4, h=4, d=64, dt=0):
    return b.PaCacheDesc(nb, bs, h, d, dt)


def test_workspace_size_is_host_only(binding):
    d = _desc(binding, 10_000, 16, 40, 128, 1)
    n = binding.pa_attention_workspace_size(d, 40, 64, 64, 2048)
    assert n > 0 and n % 256 == 0
    # forcing short splits needs more room for partial states
    small = binding.pa_attention_workspace_size(d, 40, 64, 64, 2048, binding.options(64))
    assert small > n
    # so does splitting multi-token contexts
    psplit = binding.pa_attention_workspace_size(d, 40, 64, 64, 2048, binding.options(0, 512))
    assert psplit > n
    # the default (automatic) multi-token split is never shorter than 1024
    # keys, so its bound covers an explicit 1024-key split; without splits
    # less room is needed
    p1024 = binding.pa_attention_workspace_size(d, 40, 64, 64, 2048, binding.options(0, 1024))
    nosplit = binding.pa_attention_workspace_size(
        d, 40, 64, 64, 2048, binding.options(0, 0, binding.PA_FLAG_NO_PREFILL_SPLIT))
    assert n >= p1024 > nosplit
    assert binding.pa_attention_workspace_size(d, 41, 64, 64, 2048) == 0   # 41 % 40 != 0


def _call_attention(b, desc, hq, lens, qsl, ws_bytes=1 << 20, opt=None):
    S = len(lens)
    lh = (ctypes.c_int32 * S)(*lens)
    qh = (ctypes.c_int32 * (S + 1))(*qsl)
    fake = 1 << 20   # never dereferenced: every case fails on the host
    return b.LIB.pa_attention(fake, fake, fake, fake, ctypes.byref(desc), hq, fake, 8, fake, fake,
                              S, qsl[-1], lh, qh, 0.125, fake, ws_bytes,
                              ctypes.byref(opt) if opt else None, None)


@pytest.mark.parametrize("case,expect", [
    ("bad_dtype", -2), ("bad_head_dim", -2), ("bad_block", -2), ("heads", -1),
    ("group", -2), ("n_gt_L", -1), ("qsl_order", -1), ("qsl_total", -1), ("too_long", -1),
    ("workspace", -3), ("flags", -1), ("neg_split", -1), ("block128_vector", -2)])
def test_attention_argument_errors(binding, case, expect):
    b = binding
    desc = _desc(b)
    hq, lens, qsl, ws, opt = 4, [8, 5], [0, 1, 6], 1 << 20, None
    if case == "bad_dtype":
        desc.dtype = 7
    elif case == "bad_head_dim":
        desc.head_dim = 96
    elif case == "bad_block":
        desc.block_size = 12
    elif case == "heads":
        hq = 6
    elif case == "group":
        hq = 12
    elif case == "n_gt_L":
        lens = [8, 4]
    elif case == "qsl_order":
        qsl = [0, 2, 1]
    elif case == "qsl_total":
        qsl = [1, 2, 6]
    elif case == "too_long":
        lens = [8, 33]          # 8 blocks x 4 slots = 32 < 33
        qsl = [0, 1, 6]
    elif case == "workspace":
        ws = 10
    elif case == "flags":
        opt = b.options(0, 0, 8)
    elif case == "neg_split":
        opt = b.options(0, -128)
    elif case == "block128_vector":   # fp32 rows take the vector-ALU kernel: no 128-token blocks
        desc.block_size = 128
        ws = 1 << 30
    st = _call_attention(b, desc, hq, lens, qsl, ws, opt)
    assert st == expect, (case, st, b.LIB.pa_last_error())
    assert b.LIB.pa_last_error()


@pytest.mark.parametrize("case,expect", [("null_k_new", -1), ("null_slots", -1),
                                         ("misaligned_v_new", -1), ("n_gt_L", -1),
                                         ("workspace", -3)])
def test_write_attention_argument_errors(binding, case, expect):
    """The fused entry point checks its write arguments with the attention
    ones, on the host, before anything is enqueued."""
    b = binding
    desc = _desc(b)
    lens, qsl, ws = [8, 5], [0, 1, 6], 1 << 20
    fake = 1 << 20
    k_new, v_new, slots = fake, fake, fake
    if case == "null_k_new":
        k_new = None
    elif case == "null_slots":
        slots = None
    elif case == "misaligned_v_new":
        v_new = fake + 4
    elif case == "n_gt_L":
        lens = [8, 4]
    elif case == "workspace":
        ws = 10
    S = len(lens)
    lh = (ctypes.c_int32 * S)(*lens)
    qh = (ctypes.c_int32 * (S + 1))(*qsl)
    st = b.LIB.pa_write_kv_attention(fake, fake, k_new, v_new, slots, fake, fake,
                                     ctypes.byref(desc), 4, fake, 8, fake, fake, S, qsl[-1], lh,
                                     qh, 0.125, fake, ws, None, None)
    assert st == expect, (case, st, b.LIB.pa_last_error())
    assert b.LIB.pa_last_error()


def test_write_and_copy_argument_errors(binding):
    b = binding
    desc = _desc(b)
    assert b.LIB.pa_write_kv(None, None, None, 0, None, None, ctypes.byref(desc), None) == 0
    assert b.LIB.pa_write_kv(None, None, None, 3, None, None, ctypes.byref(desc), None) == -1
    assert b.LIB.pa_write_kv(16, 16, 16, -1, 16, 16, ctypes.byref(desc), None) == -1
    assert b.LIB.pa_write_kv(8, 16, 16, 2, 16, 16, ctypes.byref(desc), None) == -1   # misaligned
    # more than 2^31 - 1 16-byte chunks in one call: refused on the host
    cpr = desc.head_dim * (4 if desc.dtype == 0 else 2) // 16
    big = (1 << 31) // (desc.num_kv_heads * cpr) + 32
    assert b.LIB.pa_write_kv(16, 16, 16, big, 16, 16, ctypes.byref(desc), None) == -2
    assert b"too many new tokens" in b.LIB.pa_last_error()
    assert b.LIB.pa_copy_blocks(None, None, ctypes.byref(desc), None, 0, None) == 0
    assert b.LIB.pa_copy_blocks(None, None, ctypes.byref(desc), None, 2, None) == -1
    desc.block_size = 3
    assert b.LIB.pa_copy_blocks(16, 16, ctypes.byref(desc), 16, 1, None) == -2


def test_copy_blocks_layers_argument_errors(binding):
    b = binding
    desc = _desc(b)
    lib = b.LIB
    ptrs = (ctypes.c_void_p * 200)(*([1 << 20] * 200))
    arr = ctypes.cast(ptrs, ctypes.c_void_p)
    assert lib.pa_copy_blocks_layers(arr, arr, 0, ctypes.byref(desc), 16, 3, None) == 0     # no layers
    assert lib.pa_copy_blocks_layers(arr, arr, 4, ctypes.byref(desc), 16, 0, None) == 0     # no pairs
    assert lib.pa_copy_blocks_layers(arr, arr, 129, ctypes.byref(desc), 16, 3, None) == -1  # > 128 layers
    assert lib.pa_copy_blocks_layers(None, arr, 2, ctypes.byref(desc), 16, 3, None) == -1
    assert lib.pa_copy_blocks_layers(arr, arr, 2, ctypes.byref(desc), None, 3, None) == -1
    assert lib.pa_copy_blocks_layers(arr, arr, 2, ctypes.byref(desc), 16, -1, None) == -1
    bad = (ctypes.c_void_p * 2)(1 << 20, 8)                                       # misaligned layer 1
    assert lib.pa_copy_blocks_layers(ctypes.cast(bad, ctypes.c_void_p), arr, 2, ctypes.byref(desc),
                                     16, 3, None) == -1
    desc.block_size = 3
    assert lib.pa_copy_blocks_layers(arr, arr, 2, ctypes.byref(desc), 16, 3, None) == -2
    assert b.MAX_LAYERS == 128


def test_swap_blocks_argument_errors(binding):
    b = binding
    desc = _desc(b)                       # 16 device blocks
    lib = b.LIB

    def call(pairs, direction=0, host_blocks=8, n=None):
        arr = (ctypes.c_int32 * max(1, 2 * len(pairs)))(*[x for p in pairs for x in p])
        n = len(pairs) if n is None else n
        return lib.pa_swap_blocks(1 << 20, 1 << 20, ctypes.byref(desc), 1 << 21, 1 << 21, host_blocks,
                                  ctypes.cast(arr, ctypes.c_void_p), n, direction, None)
    assert call([]) == 0                                   # nothing to do
    assert call([(1, 2)], direction=2) == -1               # unknown direction
    assert call([(16, 2)], direction=0) == -5              # device block out of range (swap-out source)
    assert call([(1, 8)], direction=0) == -5               # host block out of range
    assert call([(8, 1)], direction=1) == -5               # host source out of range (swap-in)
    assert call([(1, 3), (2, 3)], direction=0) == -5       # duplicate destination
    assert call([(1, 2)], n=-1) == -1
    assert lib.pa_swap_blocks(None, 1 << 20, ctypes.byref(desc), 1 << 21, 1 << 21, 8,
                              ctypes.cast((ctypes.c_int32 * 2)(1, 2), ctypes.c_void_p), 1, 0, None) == -1


def test_empty_batch_is_ok_without_a_gpu(binding):
    b = binding
    desc = _desc(b)
    S = 2
    lh = (ctypes.c_int32 * S)(3, 0)
    qh = (ctypes.c_int32 * (S + 1))(0, 0, 0)
    st = b.LIB.pa_attention(None, None, None, None, ctypes.byref(desc), 4, None, 1, None, None,
                            S, 0, lh, qh, 0.125, None, 0, None, None)
    assert st == 0
