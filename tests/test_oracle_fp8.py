"""Pins of the oracle's FP8 (E4M3FN) control cache (CPU only)."""
import numpy as np
import pytest

from oracle import attention, cache, codec, fp8cache
import pins


def test_fp8_encode_exhaustive_vs_exact_rationals():
    pins.check_fp8_encode_exhaustive(codec)


def test_fp8_round_trip_of_representable_values():
    v = codec.e4m3_value(np.arange(256))
    ok = np.isfinite(v)
    codes = codec.e4m3_encode_signed(v[ok])
    assert np.array_equal(codes, np.arange(256)[ok].astype(np.uint8))


def test_fp8_saturation_and_global_scale():
    x = np.array([448.0, 464.0, 1e6, -1e6, 0.0, -0.0], np.float32)
    assert list(codec.quantize_fp8(x)) == [0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x80]
    y = np.array([3.0, -0.5], np.float32)
    assert np.array_equal(codec.dequantize_fp8(codec.quantize_fp8(y * 4, 4.0), 4.0), [12.0, -2.0])


def test_fp8_dequant_exhaustive_vs_exact_rationals():
    pins.check_fp8_dequant(codec, fp8cache)


def test_pins_catch_fp8_dequant_without_global_scale():
    class C(fp8cache.Fp8PagedCache):
        def dequant_slots(self, slot_mapping, out_dtype="bf16"):
            g = self.v_global
            self.v_global = 1.0  # drops the per-tensor scale
            try:
                return super().dequant_slots(slot_mapping, out_dtype)
            finally:
                self.v_global = g
    import types
    with pytest.raises(AssertionError):
        pins.check_fp8_dequant(codec, types.SimpleNamespace(Fp8PagedCache=C))


def test_fp8_attention_bruteforce():
    pins.check_attention_bruteforce(
        codec, cache, attention, make_cache=fp8cache.Fp8PagedCache,
        round_trip=lambda x: codec.dequantize_fp8(codec.quantize_fp8(x)))


def test_fp8_cache_layout_and_footprint():
    c = fp8cache.Fp8PagedCache(3, 8)
    assert c.k_data.shape == (3, 8, 16, 128) and c.nbytes() == 3 * 8 * 16 * 128 * 2
    # 2048 B per token and layer at 8 KV heads against 1,152 B for NVFP4 (ratio 0.5625)
    n = cache.PagedCache(3, 8)
    assert n.nbytes() / c.nbytes() == 0.5625


def test_pins_catch_fp8_ties_away_from_zero():
    def enc(y):
        y = np.asarray(y, np.float64)
        grid = codec.e4m3_value(np.arange(0x7F))
        a = np.minimum(np.abs(y), 448.0)
        idx = np.searchsorted(grid, a)
        idx = np.clip(idx, 1, len(grid) - 1)
        lo, hi = grid[idx - 1], grid[idx]
        mag = np.where(a - lo >= hi - a, idx, idx - 1)  # ties upward
        return ((np.signbit(y).astype(np.uint8) << 7) | mag.astype(np.uint8)).astype(np.uint8)
    class M:
        pass
    m = M(); m.e4m3_encode_signed = enc
    with pytest.raises(AssertionError):
        pins.check_fp8_encode_exhaustive(m)
