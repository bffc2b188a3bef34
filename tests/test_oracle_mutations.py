"""Planted mistakes in the oracle must be caught by its pins.

Each case swaps one oracle function for a plausibly wrong version (on the CPU,
inside this process only) and checks that at least one pin test then fails.
"""
import numpy as np
import pytest

import tests.test_oracle_pins as pins
from oracle import fp, layout, ref


def _fails(fn):
    try:
        fn()
    except (AssertionError, layout.FormatError, ValueError):
        return True
    return False


def test_wrong_group_axis_is_caught(monkeypatch):
    def bad(codes, scales_bits):
        s = fp.decode_f16(scales_bits)
        return codes.astype(np.float64) * np.tile(s, (1, layout.GROUP))  # k % G instead of k // 128
    monkeypatch.setattr(ref, "weights_f64", bad)
    assert _fails(pins.test_group_axis_is_128_consecutive_weights_of_a_row)


def test_flipped_sign_map_is_caught(monkeypatch):
    orig = layout.unpack

    def bad(fmt, blob, N, K, rows=None):
        c, s = orig(fmt, blob, N, K, rows)
        return (-c if fmt == "q1" else c), s
    monkeypatch.setattr(layout, "unpack", bad)
    assert _fails(pins.test_golden_byte_value_maps)


def test_tq2_code_offset_is_caught(monkeypatch):
    orig = layout.unpack

    def bad(fmt, blob, N, K, rows=None):
        c, s = orig(fmt, blob, N, K, rows)
        return (np.clip(c + 1, -1, 1).astype(np.int8) if fmt == "tq2" else c), s
    monkeypatch.setattr(layout, "unpack", bad)
    assert _fails(pins.test_golden_byte_value_maps)


def test_abs_outside_sum_is_caught(monkeypatch):
    orig = ref.product

    def bad(codes, scales_bits, x_bits, x_dtype):
        y, _ = orig(codes, scales_bits, x_bits, x_dtype)
        return y, np.abs(y)  # |sum| instead of sum of |.|
    monkeypatch.setattr(ref, "product", bad)
    assert _fails(lambda: pins.test_product_matches_rational_brute_force("f16"))


def test_transposed_scales_are_caught(monkeypatch):
    def bad(codes, scales_bits):
        s = fp.decode_f16(scales_bits)
        N, G = s.shape
        s = s.T.reshape(N, G) if N * G > 1 else s  # scales read in the wrong order
        return codes.astype(np.float64) * np.repeat(s, layout.GROUP, axis=1)
    monkeypatch.setattr(ref, "weights_f64", bad)
    assert _fails(lambda: pins.test_product_matches_rational_brute_force("bf16"))


def test_wrong_bf16_bias_is_caught(monkeypatch):
    orig = fp.decode_bf16

    def bad(bits):
        return 2.0 * orig(bits)  # exponent bias 126 instead of 127
    monkeypatch.setattr(fp, "decode_bf16", bad)
    assert _fails(pins.test_decode_bf16_all_patterns_match_float32_view)


@pytest.mark.parametrize("swap", ["uq", "qe"])
def test_layout_index_swaps_are_caught(monkeypatch, swap):
    orig = layout._in_group

    def bad(k):
        u, q, e = orig(k)
        return (q, u, e) if swap == "uq" else (u, e % 4, q + 4 * (e // 4))
    monkeypatch.setattr(layout, "_in_group", bad)
    assert _fails(pins.test_golden_layout_positions)


def test_mlx_reversed_bit_order_is_caught(monkeypatch):
    from oracle import mlx

    def bad(wq):
        wq = np.asarray(wq, dtype=np.uint32)
        N, W = wq.shape
        shifts = np.arange(31, -1, -1, dtype=np.uint32)  # highest bit first
        return ((wq[:, :, None] >> shifts[None, None, :]) & np.uint32(1)).reshape(N, 32 * W).astype(np.uint8)
    monkeypatch.setattr(mlx, "bits_q", bad)
    assert _fails(pins.test_mlx_golden_example)
    assert _fails(pins.test_mlx_bit_order_single_bits)


def test_mlx_scale_from_scale_not_bias_is_caught(monkeypatch):
    from oracle import mlx
    orig = mlx.to_binary

    def bad(wq, scales_bits, biases_bits, dtype):
        r = orig(wq, scales_bits, biases_bits, dtype)
        if r is None:
            return None
        codes, _ = r
        a = fp.decode(scales_bits, dtype)  # s = a instead of a / 2 = -b
        return codes, a.astype(np.float16).view(np.uint16)
    monkeypatch.setattr(mlx, "to_binary", bad)
    assert _fails(pins.test_mlx_golden_example)


def test_mlx_missing_bias_is_caught(monkeypatch):
    from oracle import mlx

    def bad(wq, scales_bits, biases_bits, dtype):
        q = mlx.bits_q(wq).astype(np.float64)
        return np.repeat(fp.decode(scales_bits, dtype), mlx.GROUP, axis=1) * q  # bias dropped
    monkeypatch.setattr(mlx, "dequant", bad)
    assert _fails(pins.test_mlx_golden_example)
