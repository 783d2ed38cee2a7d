"""Device-resident batch and one step of the hot path.

A step is: copy-on-write block copies, the slot-mapping write of the new
tokens' K/V, then causal paged attention of every query row (the last two as
one call when ``fused``) -- the order the pages give (vLLM blog page, section 2.1: the copy happens before the write;
Pensieve page, 统一Prefill和Generation阶段的执行过程: K/V are stored before
attention).

The batch object only needs these attributes (numpy arrays in storage form:
float32, float16, or uint16 bit patterns for bf16): ``dtype`` ('f32', 'f16',
'bf16'), ``num_blocks``, ``block_size``, ``num_kv_heads``, ``head_dim``,
``num_q_heads``, ``hist_k``, ``hist_v``, ``hist_slots``, ``cow_pairs``,
``k_new``, ``v_new``, ``slot_mapping``, ``q``, ``block_tables``,
``context_lens``, ``query_start_loc``, ``scale``.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
NAN_FILL = {"f32": (torch.int32, 0x7FC00000), "f16": (torch.int16, 0x7E00),
            "bf16": (torch.int16, 0x7FC0)}


def to_torch(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Storage-form numpy array -> torch tensor of the element type."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def to_numpy(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Torch tensor -> storage-form numpy array (bit patterns for bf16)."""
    t = t.detach().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class DeviceBatch:
    def __init__(self, w, device="cuda", opt=None, pools=None):
        self.w = w
        self.device = torch.device(device)
        self.opt = opt
        dt = TORCH_DTYPE[w.dtype]
        nb, h, bs, d = w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim
        if pools is None:
            self.k_cache = torch.empty((nb, h, bs, d), dtype=dt, device=self.device)
            self.v_cache = torch.empty((nb, h, d, bs), dtype=dt, device=self.device)
            self.poison_pools()
        else:
            self.k_cache, self.v_cache = pools
        up = lambda a: to_torch(a, w.dtype, self.device)
        self.hist_k, self.hist_v = up(w.hist_k), up(w.hist_v)
        self.k_new, self.v_new = up(w.k_new), up(w.v_new)
        self.q = up(w.q)
        i64 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(self.device)
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(self.device)
        self.hist_slots = i64(w.hist_slots)
        self.slot_mapping = i64(w.slot_mapping)
        self.cow_pairs = i32(np.asarray(w.cow_pairs).reshape(-1, 2))
        self.block_tables = i32(w.block_tables)
        self.context_lens = i32(w.context_lens)
        self.query_start_loc = i32(w.query_start_loc)
        self.context_lens_host = torch.from_numpy(np.ascontiguousarray(w.context_lens, dtype=np.int32))
        self.qsl_host = torch.from_numpy(np.ascontiguousarray(w.query_start_loc, dtype=np.int32))
        self.out = torch.empty_like(self.q)
        self.desc = binding.cache_desc(self.k_cache, self.v_cache)
        max_len = int(np.max(w.context_lens)) if len(w.context_lens) else 0
        self.ws_bytes = binding.pa_attention_workspace_size(
            self.desc, w.num_q_heads, len(w.context_lens), int(w.q.shape[0]), max_len, opt)
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)

    def poison_pools(self) -> None:
        it, bits = NAN_FILL[self.w.dtype]
        self.k_cache.view(it).fill_(bits)
        self.v_cache.view(it).fill_(bits)

    def write_history(self) -> None:
        binding.pa_write_kv(self.hist_k, self.hist_v, self.hist_slots, self.k_cache, self.v_cache)

    def copy_blocks(self) -> None:
        if self.cow_pairs.shape[0]:
            binding.pa_copy_blocks(self.k_cache, self.v_cache, self.cow_pairs)

    def write_new(self) -> None:
        binding.pa_write_kv(self.k_new, self.v_new, self.slot_mapping, self.k_cache, self.v_cache)

    def attention(self, out=None, opt="default") -> torch.Tensor:
        out = self.out if out is None else out
        opt = self.opt if opt == "default" else opt
        binding.pa_attention(out, self.q, self.k_cache, self.v_cache, self.block_tables,
                             self.context_lens, self.query_start_loc, self.context_lens_host,
                             self.qsl_host, self.w.scale, self.workspace, opt)
        return out

    def write_attention(self, out=None, opt="default") -> torch.Tensor:
        """The new-token write and attention in one call (pa_write_kv_attention)."""
        out = self.out if out is None else out
        opt = self.opt if opt == "default" else opt
        binding.pa_write_kv_attention(out, self.q, self.k_new, self.v_new, self.slot_mapping,
                                      self.k_cache, self.v_cache, self.block_tables,
                                      self.context_lens, self.query_start_loc,
                                      self.context_lens_host, self.qsl_host, self.w.scale,
                                      self.workspace, opt)
        return out

    def step(self, fused: bool = False) -> torch.Tensor:
        self.copy_blocks()
        if fused:
            return self.write_attention()
        self.write_new()
        return self.attention()

    def out_numpy(self, out=None) -> np.ndarray:
        return to_numpy(self.out if out is None else out, self.w.dtype)

    def pools_numpy(self):
        return to_numpy(self.k_cache, self.w.dtype), to_numpy(self.v_cache, self.w.dtype)
