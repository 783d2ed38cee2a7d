"""Paged KV-cache attention for AMD Instinct MI355X (gfx950).

The compute path lives in ``libpagedattn.so`` (hand-written HIP kernels
behind the C ABI declared in ``include/pagedattn.h``).  ``binding`` is the
ctypes layer over it; importing any entry point below loads the library and
raises ``ImportError`` when it has not been built.  Build with
``python -m paged_kv_cache_block_amd.build``.
"""

_API = ("pa_write_kv", "pa_copy_blocks", "pa_copy_blocks_layers", "pa_swap_blocks",
        "pa_attention", "pa_write_kv_attention", "pa_attention_workspace_size",
        "pa_attention_plan", "pa_attention_check",
        "cache_desc", "options", "version", "PagedAttnError", "LIB_PATH")


def __getattr__(name):
    if name in _API:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
