"""Planted mistakes: each plausible error in the oracle must fail a pin.

Every mutant below is a copy of the oracle's attention with one mistake
planted (CPU only).  The test runs the pins against the mutant and requires
at least one of them to fail, showing that the pin set would catch it.
"""
import numpy as np
import pytest

import oracle
import oracle.pa_oracle as po
import tests.test_oracle_pins as pins

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _make(mistake):
    def attention_seq(q_rows, kc, vc, n_new, query_index, num_kv_heads, scale):
        L = kc.shape[0]
        r, hq, d = q_rows.shape
        group = hq // num_kv_heads
        idx = np.asarray(query_index, dtype=np.int64)
        pos = (idx if mistake == "position_from_start" else L - n_new + idx)
        if mistake == "mask_off_by_one":
            visible = np.arange(L)[None, :] < pos[:, None]
            visible[:, 0] = True
        else:
            visible = np.arange(L)[None, :] <= pos[:, None]
        out = np.empty((r, hq, d))
        for h in range(hq):
            g = (h % num_kv_heads) if mistake == "gqa_modulo" else h // group
            sc = scale * scale if mistake == "scale_no_sqrt" else scale
            a = sc * (q_rows[:, h, :] @ kc[:, g, :].T)
            a = np.where(visible, a, -np.inf)
            a = a - a.max(axis=1, keepdims=True)
            w = np.exp(a)
            vals = kc[:, g, :] if mistake == "values_from_keys" else vc[:, g, :]
            den = 1.0 if mistake == "no_normalise" else w.sum(axis=1, keepdims=True)
            out[:, h, :] = (w @ vals) / den
        return out
    return attention_seq


PIN_TESTS = [
    lambda: [pins.test_brute_force_tiny(c) for c in range(len(pins.TINY))],
    pins.test_single_key_returns_its_value_exactly,
    pins.test_constant_values_give_that_constant,
    pins.test_identical_keys_average_visible_values,
    pins.test_decode_equals_last_prefill_row,
    pins.test_sub_requests_and_chunked_prefill_match_one_prefill,
]


@pytest.mark.parametrize("mistake", ["position_from_start", "mask_off_by_one", "gqa_modulo",
                                     "scale_no_sqrt", "values_from_keys", "no_normalise"])
def test_pins_catch_planted_mistake(monkeypatch, mistake):
    mutant = _make(mistake)
    monkeypatch.setattr(po, "attention_seq", mutant)
    monkeypatch.setattr(oracle, "attention_seq", mutant)
    failures = 0
    for t in PIN_TESTS:
        try:
            t()
        except AssertionError:
            failures += 1
    assert failures >= 1, f"no pin caught the planted mistake {mistake!r}"


def test_pins_catch_transposed_value_layout(monkeypatch):
    """A gather that reads V with the K layout (token-major) must fail."""
    def bad_gather(k_cache, v_cache, block_table, context_len, dtype):
        bs = k_cache.shape[2]
        j = np.arange(context_len)
        blocks = np.asarray(block_table)[j // bs]
        flat = v_cache.reshape(v_cache.shape[0], v_cache.shape[1], -1)
        d = k_cache.shape[3]
        vt = flat.reshape(v_cache.shape[0], v_cache.shape[1], bs, d)[blocks, :, j % bs, :]
        return po.to_f64(k_cache[blocks, :, j % bs, :], dtype), po.to_f64(vt, dtype)
    monkeypatch.setattr(po, "gather_context", bad_gather)
    monkeypatch.setattr(oracle, "gather_context", bad_gather)
    with pytest.raises(AssertionError):
        for c in range(len(pins.TINY)):
            pins.test_brute_force_tiny(c)
