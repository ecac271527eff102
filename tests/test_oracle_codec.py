"""Pins of the oracle's NVFP4 codec (CPU only)."""
import numpy as np
import pytest

from oracle import codec, cache
import pins


def test_e2m1_grid():
    pins.check_e2m1_grid(codec)


def test_e4m3_definition_points():
    pins.check_e4m3_values(codec)


def test_scale_rounding_exhaustive_vs_exact_rationals():
    pins.check_scale_rounding_exhaustive(codec)


def test_element_rounding_exhaustive_vs_threshold_form():
    pins.check_element_rounding_exhaustive(codec)


def test_fp16_input_decode():
    pins.check_fp16_decode(codec)


def test_scale_rounding_exhaustive_fp16_inputs():
    pins.check_scale_rounding_exhaustive_fp16(codec)


def test_element_rounding_exhaustive_fp16_inputs():
    pins.check_element_rounding_exhaustive_fp16(codec)


def test_output_rounding_vs_exact_rationals():
    pins.check_round_to_dtype(codec)


def test_dequant_routes_agree():
    pins.check_dequant_routes_agree(codec, cache)


def test_repack_is_exact_fp16_of_the_block_values():
    pins.check_repack(codec, cache)


def test_worked_block():
    pins.check_worked_block(codec)


def test_saturating_tie():
    # amax 6.375: 6.375/6 = 1.0625 is an exact tie between 1.0 (0x38) and 1.125 (0x39):
    # the even code 0x38 wins, and 6.375 / 1.0 > 6 saturates to code 7 (6.0).
    x = np.zeros(16, np.float32); x[3] = 6.375; x[4] = -6.375
    codes, sc = codec.quantize(x)
    assert sc[0] == 0x38 and codes[3] == 0x7 and codes[4] == 0xF


def test_zero_and_underflow_blocks_keep_signs():
    x = np.array([0.0, -0.0] * 8, np.float32)
    codes, sc = codec.quantize(x)
    assert sc[0] == 0 and list(codes) == [0, 8] * 8
    tiny = np.full(16, 2.0 ** -20, np.float32); tiny[1::2] *= -1
    codes, sc = codec.quantize(tiny)
    assert sc[0] == 0 and list(codes) == [0, 8] * 8
    deq = codec.dequantize(codec.pack(codes), sc)
    assert np.all(deq == 0)


def test_error_bound_over_random_blocks():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20000, 16)).astype(np.float32)
    x[::7, 2] *= 8
    x[::11] *= 1e-3
    codes, sc = codec.quantize(x)
    s = codec.e4m3_value(sc)[:, :1]
    xh = codec.dequantize(codec.pack(codes), sc)
    err = np.abs(x.astype(np.float64) - xh)
    amax = np.abs(x).max(axis=1, keepdims=True).astype(np.float64)
    in_range = np.abs(x) <= 6 * s
    assert np.all(err[in_range] <= np.broadcast_to(s, x.shape)[in_range])
    sat = ~in_range
    assert np.all(err[sat] <= np.broadcast_to(amax - 6 * s, x.shape)[sat])
    # dequantized values are exact bf16 numbers (at most 6 significant bits)
    m, _ = np.frexp(xh)
    assert np.all((m * 64) == np.round(m * 64))


def test_grid_values_round_trip_exactly():
    rng = np.random.default_rng(4)
    sc = rng.integers(1, 127, size=500)
    s = codec.e4m3_value(sc)
    q = rng.integers(0, 16, size=(500, 16))
    q[:, 0] = 7  # put 6*s in every block, so the chosen scale is s itself
    x = (codec.e2m1_value(q) * s[:, None]).astype(np.float32)
    codes, sc2 = codec.quantize(x)
    assert np.array_equal(sc2[:, 0], sc.astype(np.uint8))
    q_exp = np.where(codec.e2m1_value(q) == 0, q & 8, q)  # +-0 keep their sign bit
    assert np.array_equal(codes, q_exp.astype(np.uint8))


def test_nibble_order():
    assert codec.pack(np.array([1, 2, 3, 4], np.uint8)).tobytes() == bytes([0x21, 0x43])
    assert np.array_equal(codec.unpack(np.array([0x21, 0x43], np.uint8)), [1, 2, 3, 4])


def test_global_scale_divides_before_quantizing():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 16)).astype(np.float32)
    c1, s1 = codec.quantize(x, 1.0)
    c2, s2 = codec.quantize(x * np.float32(4.0), 4.0)  # exact power-of-two rescale
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    d = codec.dequantize(codec.pack(c2), s2, 4.0)
    assert np.array_equal(d, 4.0 * codec.dequantize(codec.pack(c1), s1))


def test_footprint_figures_from_the_pages():
    pins.check_footprint(cache)


# --- planted mistakes: each pin must fail on a copy of the oracle with one error ---------

class _Mutant:
    def __init__(self, **over):
        self.__dict__.update({k: getattr(codec, k) for k in dir(codec) if not k.startswith("__")})
        self.__dict__.update(over)


def test_pins_catch_swapped_nibbles():
    m = _Mutant(pack=lambda c: (np.asarray(c)[..., 1::2] | (np.asarray(c)[..., 0::2] << 4)).astype(np.uint8))
    with pytest.raises(AssertionError):
        pins.check_worked_block(m)


def test_pins_catch_ties_away_from_zero():
    def enc(y, s):
        y = np.asarray(y, np.float64); s = np.broadcast_to(np.asarray(s, np.float64), y.shape)
        r = np.where(s > 0, np.abs(y) / np.where(s > 0, s, 1), 0)
        grid = np.array(pins.E2M1_GRID)
        mag = np.abs(r[..., None] - grid[::-1]).argmin(axis=-1)  # ties resolve upward
        mag = 7 - mag
        return ((np.signbit(y).astype(np.int64) << 3) | mag).astype(np.uint8)
    m = _Mutant(e2m1_encode=enc)
    with pytest.raises(AssertionError):
        pins.check_element_rounding_exhaustive(m, scale_codes=[0x38])


def test_pins_catch_reciprocal_multiply_scaling():
    def enc(y, s):
        y = np.asarray(y, np.float64); s = np.broadcast_to(np.asarray(s, np.float64), y.shape)
        inv = (np.float32(1.0) / s.astype(np.float32)).astype(np.float32)
        r = (np.abs(y).astype(np.float32) * inv).astype(np.float64)
        return codec.e2m1_encode(np.copysign(r, y), np.ones_like(r))
    m = _Mutant(e2m1_encode=enc)
    with pytest.raises(AssertionError):
        pins.check_element_rounding_exhaustive(m, scale_codes=range(1, 127))


def test_pins_catch_scale_from_amax_over_4():
    def bsc(y):
        yb = np.asarray(y, np.float32).reshape(*y.shape[:-1], y.shape[-1] // 16, 16)
        return codec.e4m3_encode((np.abs(yb).max(axis=-1) / np.float32(4)).astype(np.float64))
    m = _Mutant(block_scale_codes=bsc)
    with pytest.raises(AssertionError):
        pins.check_scale_rounding_exhaustive(m)


def test_pins_catch_e4m3_bias_8():
    def val(code):
        code = np.asarray(code).astype(np.int64)
        e, mm = (code >> 3) & 15, (code & 7).astype(np.float64)
        return np.where(e == 0, np.ldexp(mm / 8, -7), np.ldexp(1 + mm / 8, (e - 8)))
    m = _Mutant(e4m3_value=val)
    with pytest.raises(AssertionError):
        pins.check_e4m3_values(m)


def test_pins_catch_fp16_exponent_bias_off_by_one():
    m = _Mutant(fp16_to_f32=lambda b: codec.fp16_to_f32(b) * np.float32(2.0))
    with pytest.raises(AssertionError):
        pins.check_fp16_decode(m)


def test_pins_catch_truncating_output_rounding():
    def rnd(x, out):
        x = np.asarray(x, np.float32)
        if out == "bf16":
            return (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation, not nearest-even
        return codec.round_to_dtype(x, out)
    m = _Mutant(round_to_dtype=rnd)
    with pytest.raises(AssertionError):
        pins.check_round_to_dtype(m)


def test_pins_catch_dequant_without_scale():
    class C(cache.PagedCache):
        def dequant_slots(self, slot_mapping, out_dtype="bf16"):
            k, v = super().dequant_slots(slot_mapping, "f32")
            g = np.where(k != 0, np.sign(k), 0).astype(np.float32)  # drops the block scale
            return codec.round_to_dtype(g, out_dtype), codec.round_to_dtype(v, out_dtype)
    import types
    mod = types.SimpleNamespace(PagedCache=C)
    with pytest.raises(AssertionError):
        pins.check_dequant_routes_agree(codec, mod)


def test_pins_catch_repack_applying_the_global_scale():
    class C(cache.PagedCache):
        def repack(self, block_table, kv_lens):
            k, v = super().repack(block_table, kv_lens)
            val = pins.fp16_value_by_fields(k) * self.k_global  # applies g, which the reader does
            return codec.round_to_dtype(val.astype(np.float32), "fp16"), v
    import types
    with pytest.raises(AssertionError):
        pins.check_repack(codec, types.SimpleNamespace(PagedCache=C))


def test_quantize_at_non_power_of_two_g_vs_exact_rationals():
    pins.check_quantize_general_g(codec)


def test_nvfp4_dequant_at_g_not_one_vs_exact_rationals():
    pins.check_nvfp4_dequant_general_g(codec, cache)


def test_pins_catch_quantize_without_float32_quotient():
    def q64(x, g=1.0):  # y = x / g kept in float64: no float32 rounding of the quotient
        y = np.asarray(x, np.float32).astype(np.float64) / g
        yb = y.reshape(*y.shape[:-1], y.shape[-1] // 16, 16)
        sc = codec.e4m3_encode(np.abs(yb).max(axis=-1) / 6.0)
        return codec.e2m1_encode(y, np.repeat(codec.e4m3_value(sc), 16, axis=-1)), sc
    with pytest.raises(AssertionError):
        pins.check_quantize_general_g(_Mutant(quantize=q64))


def test_pins_catch_dequant_without_float32_product():
    class C(cache.PagedCache):
        def dequant_slots(self, slot_mapping, out_dtype="bf16"):
            k, v = super().dequant_slots(slot_mapping, "f32")
            out = []
            for x, data, scale, g in ((k, self.k_data, self.k_scale, self.k_global),
                                      (v, self.v_data, self.v_scale, self.v_global)):
                slots = np.asarray(slot_mapping, np.int64)
                keep = slots >= 0
                pg, off = np.where(keep, slots // 16, 0), np.where(keep, slots % 16, 0)
                s = np.repeat(codec.e4m3_value(scale[pg, :, off, :]), 16, axis=-1)
                ex = np.where(keep[:, None, None], s * codec.e2m1_value(codec.unpack(data[pg, :, off, :])) * g, 0)
                if out_dtype == "bf16":  # exact product rounded once, straight to bf16
                    m, e = np.frexp(ex)
                    out.append(codec.round_to_dtype(np.ldexp(np.round(np.ldexp(m, 8)), e - 8).astype(np.float32), "bf16"))
                else:
                    out.append(codec.round_to_dtype(ex.astype(np.float32), out_dtype))
            return out[0], out[1]
    import types
    with pytest.raises(AssertionError):
        pins.check_nvfp4_dequant_general_g(codec, types.SimpleNamespace(PagedCache=C))
