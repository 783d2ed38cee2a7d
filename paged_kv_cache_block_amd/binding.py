"""ctypes binding of libpagedattn.so: argument marshalling only.

Every function here takes torch tensors (for device memory and the current
HIP stream), checks shapes and dtypes, and calls the C entry point of the
same name.  No part of the computation happens in Python.  If the library
has not been built the import raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

PA_F32, PA_F16, PA_BF16 = 0, 1, 2
STATUS = {0: "PA_OK", -1: "PA_ERR_INVALID_ARG", -2: "PA_ERR_UNSUPPORTED", -3: "PA_ERR_WORKSPACE",
          -4: "PA_ERR_HIP", -5: "PA_ERR_BOUNDS"}
TORCH_TO_PA = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
SYMBOLS = ("pa_write_kv", "pa_copy_blocks", "pa_copy_blocks_layers", "pa_swap_blocks",
           "pa_attention_workspace_size", "pa_attention_plan", "pa_attention",
           "pa_write_kv_attention", "pa_write_kv_attention_static", "pa_attention_check",
           "pa_last_error", "pa_version")
PA_SWAP_OUT, PA_SWAP_IN = 0, 1
MAX_LAYERS = 128


class PaCacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class PaOptions(ctypes.Structure):
    _fields_ = [("decode_split_tokens", ctypes.c_int32), ("prefill_split_tokens", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("timed_kernel", ctypes.c_int32),
                ("timing_start", ctypes.c_void_p), ("timing_end", ctypes.c_void_p),
                ("prefill_tile_rows", ctypes.c_int32)]


class PaPlanInfo(ctypes.Structure):
    _fields_ = [("row_items", ctypes.c_int64), ("tile_items", ctypes.c_int64),
                ("combine_items", ctypes.c_int64), ("partial_slots", ctypes.c_int64),
                ("decode_split_tokens", ctypes.c_int32), ("prefill_split_tokens", ctypes.c_int32),
                ("prefill_tile_rows", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t)]


PA_TIME_NONE, PA_TIME_TILE, PA_TIME_ROWS, PA_TIME_COMBINE = 0, 1, 2, 3
PA_FLAG_VECTOR_ALU, PA_FLAG_KV_UNSHARED, PA_FLAG_NO_PREFILL_SPLIT = 1, 2, 4


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with "
                          "`python -m paged_kv_cache_block_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64p, i32p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p
    desc_p = ctypes.POINTER(PaCacheDesc)
    opt_p = ctypes.POINTER(PaOptions)
    lib.pa_write_kv.argtypes = [vp, vp, i64p, i32, vp, vp, desc_p, vp]
    lib.pa_write_kv.restype = ctypes.c_int
    lib.pa_copy_blocks.argtypes = [vp, vp, desc_p, i32p, i32, vp]
    lib.pa_copy_blocks.restype = ctypes.c_int
    lib.pa_copy_blocks_layers.argtypes = [vp, vp, i32, desc_p, i32p, i32, vp]
    lib.pa_copy_blocks_layers.restype = ctypes.c_int
    lib.pa_swap_blocks.argtypes = [vp, vp, desc_p, vp, vp, i32, i32p, i32, i32, vp]
    lib.pa_swap_blocks.restype = ctypes.c_int
    lib.pa_attention_workspace_size.argtypes = [desc_p, i32, i32, i32, i32, opt_p]
    lib.pa_attention_workspace_size.restype = ctypes.c_size_t
    lib.pa_attention.argtypes = [vp, vp, vp, vp, desc_p, i32, i32p, i32, i32p, i32p, i32, i32,
                                 i32p, i32p, ctypes.c_float, vp, ctypes.c_size_t, opt_p, vp]
    lib.pa_attention.restype = ctypes.c_int
    lib.pa_write_kv_attention.argtypes = [vp, vp, vp, vp, i64p, vp, vp, desc_p, i32, i32p, i32,
                                          i32p, i32p, i32, i32, i32p, i32p, ctypes.c_float, vp,
                                          ctypes.c_size_t, opt_p, vp]
    lib.pa_write_kv_attention.restype = ctypes.c_int
    lib.pa_write_kv_attention_static.argtypes = [vp, vp, vp, vp, i64p, vp, vp, desc_p, i32, i32p,
                                                 i32, i32p, i32p, i32, i32, i32p, i32p,
                                                 ctypes.c_float, opt_p, vp]
    lib.pa_write_kv_attention_static.restype = ctypes.c_int
    lib.pa_attention_plan.argtypes = [desc_p, i32, i32, i32, i32, i32p, i32p, ctypes.c_size_t, opt_p,
                                      ctypes.POINTER(PaPlanInfo)]
    lib.pa_attention_plan.restype = ctypes.c_int
    lib.pa_attention_check.argtypes = [vp, vp]
    lib.pa_attention_check.restype = ctypes.c_int
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_version.argtypes = []
    lib.pa_version.restype = ctypes.c_int32
    return lib


LIB = _load()


def _check(status: int) -> None:
    if status != 0:
        raise PagedAttnError(status, LIB.pa_last_error().decode(errors="replace"))


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _on_device(dev: torch.device, **tensors) -> None:
    """Every named tensor must live on ``dev`` (the pools' GPU): a host
    pointer handed to a kernel would fault the GPU."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.device != dev:
            where = t.device if isinstance(t, torch.Tensor) else type(t).__name__
            raise ValueError(f"{name} must be a tensor on {dev}, got {where}")


def _on_host(**tensors) -> None:
    for name, t in tensors.items():
        if not isinstance(t, torch.Tensor) or t.device.type != "cpu":
            where = t.device if isinstance(t, torch.Tensor) else type(t).__name__
            raise ValueError(f"{name} must be a CPU tensor, got {where}")


def _pairs(block_pairs) -> int:
    if block_pairs.dtype != torch.int32 or block_pairs.dim() != 2 or block_pairs.shape[1] != 2 \
            or not block_pairs.is_contiguous():
        raise ValueError("block_pairs must be a contiguous int32 [n][2] tensor")
    return int(block_pairs.shape[0])


def cache_desc(k_cache: torch.Tensor, v_cache: torch.Tensor) -> PaCacheDesc:
    """Descriptor of a pool pair: K [NB][H][bs][D], V [NB][H][D][bs]."""
    if k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("pools must be 4-D")
    nb, h, bs, d = k_cache.shape
    if tuple(v_cache.shape) != (nb, h, d, bs):
        raise ValueError(f"v_cache shape {tuple(v_cache.shape)} != {(nb, h, d, bs)}")
    if k_cache.dtype != v_cache.dtype or k_cache.dtype not in TORCH_TO_PA:
        raise ValueError("pools must share a dtype among float32, float16, bfloat16")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("pools must be contiguous")
    if k_cache.device.type == "cuda" and v_cache.device != k_cache.device:
        raise ValueError("k_cache and v_cache must be on the same GPU")
    return PaCacheDesc(nb, bs, h, d, TORCH_TO_PA[k_cache.dtype])


def options(decode_split_tokens: int = 0, prefill_split_tokens: int = 0, flags: int = 0,
            timed_kernel: int = 0, timing_start=None, timing_end=None, prefill_tile_rows: int = 0):
    """``timing_start`` / ``timing_end`` are ``torch.cuda.Event(enable_timing=True)``
    objects (or raw hipEvent_t handles) recorded around ``timed_kernel``."""
    def handle(ev):
        if ev is None:
            return None
        if not isinstance(ev, int):
            ev.record()          # materialise the underlying hipEvent_t
            ev = ev.cuda_event
        return ev
    return PaOptions(decode_split_tokens, prefill_split_tokens, flags, timed_kernel,
                     handle(timing_start), handle(timing_end), prefill_tile_rows)


def pa_write_kv(k_new, v_new, slot_mapping, k_cache, v_cache, stream=None) -> None:
    desc = cache_desc(k_cache, v_cache)
    t = int(k_new.shape[0])
    for x in (k_new, v_new):
        if tuple(x.shape) != (t, desc.num_kv_heads, desc.head_dim) or x.dtype != k_cache.dtype \
                or not x.is_contiguous():
            raise ValueError("k_new/v_new must be contiguous [T][H_kv][D] in the pool dtype")
    if slot_mapping.dtype != torch.int64 or tuple(slot_mapping.shape) != (t,) \
            or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 [T] tensor")
    _on_device(k_cache.device, k_cache=k_cache, v_cache=v_cache, k_new=k_new, v_new=v_new,
               slot_mapping=slot_mapping)
    _check(LIB.pa_write_kv(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), t, _ptr(k_cache),
                           _ptr(v_cache), ctypes.byref(desc), _stream(stream)))


def pa_copy_blocks_layers(k_caches, v_caches, block_pairs, stream=None) -> None:
    """The block copies of ``pa_copy_blocks`` on every layer's pools, one launch."""
    if len(k_caches) != len(v_caches) or not k_caches:
        raise ValueError("one K and one V pool per layer")
    desc = cache_desc(k_caches[0], v_caches[0])
    for k, v in zip(k_caches, v_caches):
        if tuple(k.shape) != tuple(k_caches[0].shape) or k.dtype != k_caches[0].dtype or \
                tuple(v.shape) != tuple(v_caches[0].shape):
            raise ValueError("every layer's pools must have the same shape and dtype")
    npairs = _pairs(block_pairs)
    dev = k_caches[0].device
    for l, (k, v) in enumerate(zip(k_caches, v_caches)):
        _on_device(dev, **{f"k_caches[{l}]": k, f"v_caches[{l}]": v})
        if not (k.is_contiguous() and v.is_contiguous()):
            raise ValueError("every layer's pools must be contiguous")
    _on_device(dev, block_pairs=block_pairs)
    n = len(k_caches)
    kp = (ctypes.c_void_p * n)(*[_ptr(k) for k in k_caches])
    vp_ = (ctypes.c_void_p * n)(*[_ptr(v) for v in v_caches])
    _check(LIB.pa_copy_blocks_layers(ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(vp_, ctypes.c_void_p),
                                     n, ctypes.byref(desc), _ptr(block_pairs), npairs,
                                     _stream(stream)))


def pa_swap_blocks(dev_k, dev_v, host_k, host_v, block_pairs, direction: int, stream=None) -> None:
    """Copy whole blocks device -> host (PA_SWAP_OUT) or host -> device
    (PA_SWAP_IN) on the DMA engines.  ``host_k`` / ``host_v`` are pinned CPU
    tensors shaped like the device pools (any block count); ``block_pairs``
    is an int32 CPU tensor [n][2] of (src, dst)."""
    desc = cache_desc(dev_k, dev_v)
    if host_k.device.type != "cpu" or host_v.device.type != "cpu":
        raise ValueError("host pools must be CPU tensors")
    if tuple(host_k.shape[1:]) != tuple(dev_k.shape[1:]) or tuple(host_v.shape[1:]) != tuple(dev_v.shape[1:]) \
            or host_k.dtype != dev_k.dtype or host_v.dtype != dev_v.dtype or host_k.shape[0] != host_v.shape[0]:
        raise ValueError("host pools must match the device pools' block shape and dtype")
    if not (host_k.is_contiguous() and host_v.is_contiguous()):
        raise ValueError("host pools must be contiguous")
    _on_device(dev_k.device, dev_k=dev_k, dev_v=dev_v)
    _on_host(block_pairs=block_pairs)
    npairs = _pairs(block_pairs)
    _check(LIB.pa_swap_blocks(_ptr(dev_k), _ptr(dev_v), ctypes.byref(desc), _ptr(host_k), _ptr(host_v),
                              int(host_k.shape[0]), _ptr(block_pairs), npairs, int(direction),
                              _stream(stream)))


def pa_copy_blocks(k_cache, v_cache, block_pairs, stream=None) -> None:
    desc = cache_desc(k_cache, v_cache)
    npairs = _pairs(block_pairs)
    _on_device(k_cache.device, k_cache=k_cache, v_cache=v_cache, block_pairs=block_pairs)
    _check(LIB.pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), ctypes.byref(desc),
                              _ptr(block_pairs), npairs, _stream(stream)))


def pa_attention_workspace_size(desc: PaCacheDesc, num_q_heads: int, num_seqs: int, total_q: int,
                                max_context_len: int, opt: PaOptions | None = None) -> int:
    return int(LIB.pa_attention_workspace_size(ctypes.byref(desc), num_q_heads, num_seqs,
                                               total_q, max_context_len,
                                               ctypes.byref(opt) if opt is not None else None))


def pa_attention_plan(desc: PaCacheDesc, num_q_heads: int, max_blocks_per_seq: int,
                      context_lens_host, query_start_loc_host, workspace_bytes: int,
                      opt: PaOptions | None = None) -> tuple[int, PaPlanInfo]:
    """Host-only: the plan ``pa_attention`` would make for this batch given a
    workspace of ``workspace_bytes``.  Returns ``(status, info)``; status 0
    when the plan fits, -3 when it does not (``info`` is filled either way)."""
    lens = np.ascontiguousarray(context_lens_host, dtype=np.int32)
    qsl = np.ascontiguousarray(query_start_loc_host, dtype=np.int32)
    if qsl.shape[0] != lens.shape[0] + 1:
        raise ValueError("query_start_loc must have one more entry than context_lens")
    info = PaPlanInfo()
    st = LIB.pa_attention_plan(ctypes.byref(desc), num_q_heads, max_blocks_per_seq, lens.shape[0],
                               int(qsl[-1]) if qsl.size else 0, lens.ctypes.data, qsl.ctypes.data,
                               int(workspace_bytes), ctypes.byref(opt) if opt is not None else None,
                               ctypes.byref(info))
    return int(st), info


def pa_attention_check(workspace, stream=None) -> None:
    """Wait for the stream; raise PagedAttnError if the last attention call
    that used ``workspace`` skipped work (device batch != host mirrors)."""
    _on_device(workspace.device, workspace=workspace)
    _check(LIB.pa_attention_check(_ptr(workspace), _stream(stream)))


def _attention_args(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                    context_lens_host, query_start_loc_host, workspace):
    tq, hq, d = q.shape
    if tuple(out.shape) != (tq, hq, d) or out.dtype != q.dtype or q.dtype != k_cache.dtype:
        raise ValueError("q/out must be [T_q][H_q][D] in the pool dtype")
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q/out must be contiguous")
    s = int(context_lens.shape[0])
    for x in (block_tables, context_lens, query_start_loc):
        if x.dtype != torch.int32 or not x.is_contiguous():
            raise ValueError("block_tables, context_lens, query_start_loc must be contiguous int32")
    for x in (context_lens_host, query_start_loc_host):
        if x.dtype != torch.int32 or x.device.type != "cpu" or not x.is_contiguous():
            raise ValueError("host mirrors must be contiguous int32 CPU tensors")
    if block_tables.dim() != 2 or block_tables.shape[0] != s or query_start_loc.shape[0] != s + 1:
        raise ValueError("block_tables [S][max_blocks] and query_start_loc [S+1] expected")
    if context_lens_host.shape[0] != s or query_start_loc_host.shape[0] != s + 1:
        raise ValueError("host mirrors must match context_lens [S] and query_start_loc [S+1]")
    _on_device(k_cache.device, k_cache=k_cache, v_cache=v_cache, out=out, q=q,
               block_tables=block_tables, context_lens=context_lens,
               query_start_loc=query_start_loc, workspace=workspace)
    return tq, hq, s


def pa_attention(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                 context_lens_host, query_start_loc_host, scale: float, workspace,
                 opt: PaOptions | None = None, stream=None) -> None:
    """Causal paged attention of a ragged batch; writes ``out`` in place.

    ``context_lens_host`` / ``query_start_loc_host`` are contiguous int32 CPU
    tensors with the same contents as their device counterparts.
    """
    desc = cache_desc(k_cache, v_cache)
    tq, hq, s = _attention_args(out, q, k_cache, v_cache, block_tables, context_lens,
                                query_start_loc, context_lens_host, query_start_loc_host,
                                workspace)
    _check(LIB.pa_attention(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc),
                            hq, _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens),
                            _ptr(query_start_loc), s, tq, _ptr(context_lens_host),
                            _ptr(query_start_loc_host), float(scale), _ptr(workspace),
                            0 if workspace is None else int(workspace.numel() * workspace.element_size()),
                            ctypes.byref(opt) if opt is not None else None, _stream(stream)))


def pa_write_kv_attention(out, q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                          context_lens, query_start_loc, context_lens_host, query_start_loc_host,
                          scale: float, workspace, opt: PaOptions | None = None,
                          stream=None) -> None:
    """``pa_write_kv`` of the batch's new tokens (row t of ``k_new`` /
    ``v_new`` is query row t's token, stored at ``slot_mapping[t]``) followed
    by ``pa_attention``, in one call (the write shares the planner's
    launch)."""
    desc = cache_desc(k_cache, v_cache)
    tq, hq, s = _attention_args(out, q, k_cache, v_cache, block_tables, context_lens,
                                query_start_loc, context_lens_host, query_start_loc_host,
                                workspace)
    if tuple(k_new.shape) != (tq, desc.num_kv_heads, desc.head_dim) or k_new.shape != v_new.shape:
        raise ValueError("k_new/v_new must be [T_q][H_kv][D]")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise ValueError("k_new/v_new must have the pool dtype")
    if not (k_new.is_contiguous() and v_new.is_contiguous()):
        raise ValueError("k_new/v_new must be contiguous")
    if (slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous()
            or slot_mapping.numel() != tq):
        raise ValueError("slot_mapping must be a contiguous int64 [T_q] tensor")
    _on_device(k_cache.device, k_new=k_new, v_new=v_new, slot_mapping=slot_mapping)
    _check(LIB.pa_write_kv_attention(
        _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_cache),
        _ptr(v_cache), ctypes.byref(desc), hq, _ptr(block_tables), int(block_tables.shape[1]),
        _ptr(context_lens), _ptr(query_start_loc), s, tq, _ptr(context_lens_host),
        _ptr(query_start_loc_host), float(scale), _ptr(workspace),
        0 if workspace is None else int(workspace.numel() * workspace.element_size()),
        ctypes.byref(opt) if opt is not None else None, _stream(stream)))


def pa_write_kv_attention_static(out, q, k_new, v_new, slot_mapping, k_cache, v_cache,
                                 block_tables, context_lens, query_start_loc, context_lens_host,
                                 query_start_loc_host, scale: float, opt: PaOptions | None = None,
                                 stream=None) -> None:
    """``pa_write_kv_attention`` with the library's static device scratch in
    place of a workspace: the call allocates no device memory.  Calls that
    overlap on one GPU share the scratch and must be serialized."""
    desc = cache_desc(k_cache, v_cache)
    tq, hq, s = _attention_args(out, q, k_cache, v_cache, block_tables, context_lens,
                                query_start_loc, context_lens_host, query_start_loc_host, None)
    if tuple(k_new.shape) != (tq, desc.num_kv_heads, desc.head_dim) or k_new.shape != v_new.shape:
        raise ValueError("k_new/v_new must be [T_q][H_kv][D]")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise ValueError("k_new/v_new must have the pool dtype")
    if not (k_new.is_contiguous() and v_new.is_contiguous()):
        raise ValueError("k_new/v_new must be contiguous")
    if (slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous()
            or slot_mapping.numel() != tq):
        raise ValueError("slot_mapping must be a contiguous int64 [T_q] tensor")
    _on_device(k_cache.device, k_new=k_new, v_new=v_new, slot_mapping=slot_mapping)
    _check(LIB.pa_write_kv_attention_static(
        _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_cache),
        _ptr(v_cache), ctypes.byref(desc), hq, _ptr(block_tables), int(block_tables.shape[1]),
        _ptr(context_lens), _ptr(query_start_loc), s, tq, _ptr(context_lens_host),
        _ptr(query_start_loc_host), float(scale),
        ctypes.byref(opt) if opt is not None else None, _stream(stream)))


STATIC_SCRATCH_BYTES = 64 << 20


def version() -> int:
    return int(LIB.pa_version())
