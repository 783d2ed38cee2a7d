"""pa_write_kv_attention_static (no workspace argument, static device
scratch) against pa_write_kv_attention, through the C ABI.

Two calls in a row on one GPU, the second with a smaller batch: both equal
the workspace entry point's output and pools bit for bit (the plans are the
same, so the arithmetic is), and both are within the parity bar of the
oracle.  A batch whose plan exceeds the scratch is refused on the host.
"""
import numpy as np
import pytest

import oracle
from oracle import tolerance
from workloads import build_batch, small_workload

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


def _bits(a):
    return a.view(np.uint32 if a.dtype == np.float32 else np.uint16)


def _oracle(w):
    k, v = w.empty_pools()
    oracle.write_kv(k, v, w.hist_k, w.hist_v, w.hist_slots)
    oracle.copy_blocks(k, v, w.cow_pairs)
    oracle.write_kv(k, v, w.k_new, w.v_new, w.slot_mapping)
    return oracle.attention(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc,
                            w.num_kv_heads, w.dtype, w.scale)


def _static_call(binding, db, out):
    binding.pa_write_kv_attention_static(out, db.q, db.k_new, db.v_new, db.slot_mapping,
                                         db.k_cache, db.v_cache, db.block_tables,
                                         db.context_lens, db.query_start_loc,
                                         db.context_lens_host, db.qsl_host, db.w.scale, db.opt)


@pytest.mark.parametrize("hint", [False, True], ids=["default", "kv_unshared"])
def test_static_scratch_matches_the_workspace_entry_point(hint):
    """With the no-sharing hint the plan also lists the decode work longest
    first (for dealing over the XCDs), in the same static scratch."""
    import torch
    assert torch.cuda.is_available()
    from paged_kv_cache_block_amd import binding
    from paged_kv_cache_block_amd.step import DeviceBatch
    opt = binding.options(0, 0, binding.PA_FLAG_KV_UNSHARED) if hint else None
    big = small_workload(5)           # multi-token and decode rows, split decode contexts
    small = small_workload(3)         # a smaller batch on the second call
    for i, w in enumerate((big, small)):
        print(f"[case] static scratch call {i} (hint {hint}): {w.name}", flush=True)
        ref = DeviceBatch(w, opt=opt)
        ref.write_history()
        ref.copy_blocks()
        ref.write_attention()
        st = DeviceBatch(w, opt=opt)
        st.write_history()
        st.copy_blocks()
        out = torch.empty_like(st.q)
        _static_call(binding, st, out)
        torch.cuda.synchronize()
        got = st.out_numpy(out)
        assert np.array_equal(_bits(got), _bits(ref.out_numpy())), f"call {i}: outputs differ"
        for a, b in zip(st.pools_numpy(), ref.pools_numpy()):
            assert np.array_equal(_bits(a), _bits(b)), f"call {i}: pools differ"
        ok, stats = tolerance.check(oracle.to_f64(got, w.dtype), _oracle(w), w.dtype)
        assert ok, f"call {i}: {stats['msg']}"
        del ref, st


def test_static_scratch_refuses_a_plan_that_does_not_fit():
    import torch
    from paged_kv_cache_block_amd import binding
    from paged_kv_cache_block_amd.step import DeviceBatch
    # 40 decode rows over 4096-token contexts split every 64 keys: 2560
    # partial states of 64 heads x 128 floats (84 MB), beyond the scratch.
    seqs = [(4095, 1, 1)] * 40
    w = build_batch("scratch overflow", "bf16", 64, 8, 128, 32, 40 * 128 + 8, seqs, 3)
    opt = binding.options(64)
    st, info = binding.pa_attention_plan(binding.PaCacheDesc(w.num_blocks, w.block_size, w.num_kv_heads,
                                                             w.head_dim, 2),
                                         w.num_q_heads, w.block_tables.shape[1], w.context_lens,
                                         w.query_start_loc, binding.STATIC_SCRATCH_BYTES, opt)
    if st == 0:
        pytest.skip("this batch fits the scratch")
    db = DeviceBatch(w, opt=opt)
    out = torch.empty_like(db.q)
    with pytest.raises(binding.PagedAttnError) as ei:
        _static_call(binding, db, out)
    assert ei.value.status == -3 and "static scratch" in str(ei.value)
