"""Pins for the INT8 KV-cache oracle ([KV2P] §5.2: INT8 halves the cache;
group-wise scales, one per 128-element group).  Each test checks the oracle
against something other than itself: integers that must round-trip, ties that
must go to even, the closed form of the scale, the half-step error bound,
the page's paging example and SDPA on dequantised contiguous data.  CPU only."""

import numpy as np
import pytest

import oracle
from tests import pins


def test_integers_round_trip_at_scale_one():
    assert pins.quant_integers_exact(oracle.quantize_rows_ref)


def test_ties_round_to_even():
    assert pins.quant_rounds_half_to_even(oracle.quantize_rows_ref)


def test_scale_is_amax_over_127_and_zero_rows():
    assert pins.quant_scale_is_amax_over_127(oracle.quantize_rows_ref)


def test_error_within_half_a_step_per_row():
    assert pins.quant_error_within_half_step(oracle.quantize_rows_ref, oracle.dequantize_ref)


@pytest.mark.parametrize("d", [64, 128])
def test_group_is_one_head_row(d):
    """One scale per (token, head) row of head_dim values: codes and scales of
    a row do not depend on the other rows or heads."""
    rng = np.random.default_rng(d)
    x = rng.standard_normal((5, 4, d)).astype(np.float16)
    codes, scales = oracle.quantize_rows_ref(x)
    assert codes.shape == x.shape and scales.shape == (5, 4) and scales.dtype == np.float32
    for t in range(5):
        for h in range(4):
            row = x[t, h].astype(np.float32)
            s = np.float32(np.abs(row).max()) / np.float32(127)
            assert scales[t, h] == s
            want = np.clip(np.rint(row / s), -127, 127)
            assert np.array_equal(codes[t, h], want.astype(np.int8))


def test_dequantize_is_exact_product():
    codes = np.array([[-127, 0, 5, 127]], dtype=np.int8)
    scales = np.array([0.1], dtype=np.float32)
    s = float(np.float32(0.1))
    assert np.array_equal(oracle.dequantize_ref(codes, scales)[0], [-127 * s, 0.0, 5 * s, 127 * s])


def test_i8_cache_write_round_trip_page_example():
    assert pins.i8_cache_round_trip(oracle.cache_write_i8_ref, oracle.quantize_rows_ref,
                                    oracle.dequantize_ref)


def test_i8_cow_copies_codes_and_scales_first():
    assert pins.i8_cow_before_scatter(oracle.cache_write_i8_ref)


def test_i8_negative_slot_writes_nothing():
    rng = np.random.default_rng(4)
    codes = rng.integers(-127, 128, (3, 2, 1, 4, 8)).astype(np.int8)
    scales = rng.uniform(0.1, 1, (3, 1, 2, 4)).astype(np.float32)
    key = np.ones((2, 1, 8), dtype=np.float16)
    c2, s2 = oracle.cache_write_i8_ref(codes, scales, key, key, np.array([-1, -5]))
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_i8_decode_is_sdpa_on_dequantised_contiguous():
    assert pins.i8_decode_is_sdpa_on_dequantised(oracle.decode_i8_ref, oracle.dequantize_ref)


def test_i8_decode_close_to_fp16_decode():
    """Quantisation error bound carried through attention: outputs move by at
    most a few quantisation steps of V (plus the change in weights from K)."""
    import synth
    x = synth.make_decode_inputs([50, 200], 8, 2, 64, 16, dtype="f16", seed=9)
    kv = x.kv_cache.numpy()
    codes, scales = oracle.quantize_rows_ref(kv)
    args = (x.q.numpy(), x.block_tables.numpy(), x.context_lens.numpy(), x.scale)
    a = oracle.decode_ref(args[0], kv, *args[1:])
    b = oracle.decode_i8_ref(args[0], codes, np.swapaxes(scales, 1, 2), *args[1:])
    assert np.abs(a - b).max() < 0.05 and not np.array_equal(a, b)


@pytest.mark.parametrize("window", [0, 1, 6, 30])
def test_i8_prefill_is_masked_sdpa_on_dequantised_contiguous(window):
    assert pins.i8_prefill_is_masked_sdpa_on_dequantised(oracle.prefill_i8_ref, window)


def test_i8_prefill_single_token_is_i8_decode():
    """T = 1 per sequence is the INT8 decode, exactly (with and without a
    window)."""
    rng = np.random.default_rng(19)
    codes = rng.integers(-127, 128, (12, 2, 2, 8, 16)).astype(np.int8)
    scales = rng.uniform(0.01, 0.1, (12, 2, 2, 8)).astype(np.float32)
    bt = np.array([[3, 1, 7], [4, 0, 11]])
    lens = np.array([20, 9])
    q = rng.standard_normal((2, 4, 16))
    for w in (0, 4, 15):
        assert np.array_equal(
            oracle.prefill_i8_ref(q, codes, scales, bt, lens, np.array([0, 1, 2]), 0.5, window=w),
            oracle.decode_i8_ref(q, codes, scales, bt, lens, 0.5, window=w))
