"""Checks that tie the oracle to facts outside itself.

Each check raises AssertionError when the oracle disagrees with what the
pages print, with a format definition, with exact rational arithmetic, or
with brute force.  The CPU tests run them on the oracle as it is, and run
some of them again on copies of the oracle with a planted mistake, to show
that each pin would catch that mistake.
"""
from __future__ import annotations

import bisect
import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def finite_bf16_patterns() -> np.ndarray:
    """Every finite bfloat16 bit pattern (both signs, both zeros): 65,280 values."""
    p = np.arange(65536, dtype=np.uint32)
    finite = ((p >> 7) & 0xFF) != 0xFF
    return p[finite].astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def finite_fp16_patterns() -> np.ndarray:
    """Every finite IEEE binary16 bit pattern (both signs, both zeros): 63,488 values."""
    p = np.arange(65536, dtype=np.uint32)
    return p[((p >> 10) & 0x1F) != 0x1F].astype(np.uint16)


def fp16_value_by_fields(bits: np.ndarray) -> np.ndarray:
    """binary16 value from its fields (sign, 5-bit exponent of bias 15, 10-bit fraction),
    exact in float64."""
    b = bits.astype(np.int64)
    e, m = (b >> 10) & 0x1F, (b & 0x3FF).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m, -24), np.ldexp(1024.0 + m, (e - 25).astype(np.int64)))
    return np.where((b >> 15) & 1, -mag, mag)


def nearest_even_fraction(x: Fraction, grid_exp_min: int, mant_bits: int) -> Fraction:
    """x rounded to nearest (ties to even significand) in a binary format with `mant_bits`
    stored fraction bits and least exponent grid_exp_min (no overflow handling)."""
    if x == 0:
        return Fraction(0)
    sgn = -1 if x < 0 else 1
    a = abs(x)
    e = max(math.floor(math.log2(a)) if a.numerator else 0, grid_exp_min)
    while Fraction(2) ** e > a and e > grid_exp_min:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, grid_exp_min)
    ulp = Fraction(2) ** (e - mant_bits)
    q, r = divmod(a, ulp)
    if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
        q += 1
    return sgn * q * ulp


# ---------------------------------------------------------------------------------------
# Formats
# ---------------------------------------------------------------------------------------

E2M1_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def check_e2m1_grid(codec):
    vals = codec.e2m1_value(np.arange(16))
    assert list(vals[:8]) == E2M1_GRID, vals[:8]
    assert list(-vals[8:]) == E2M1_GRID, vals[8:]
    assert np.signbit(vals[8]) and not np.signbit(vals[0])


def check_e4m3_values(codec):
    """Fixed points of the E4M3FN definition: bias 7, 2^-9 smallest subnormal,
    2^-6 smallest normal, 448 largest, 0x7F NaN, strictly increasing codes."""
    v = codec.e4m3_value(np.arange(256))
    assert v[0x00] == 0.0 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6 and v[0x38] == 1.0 and v[0x39] == 1.125
    assert v[0x7E] == 448.0 and math.isnan(v[0x7F]) and math.isnan(v[0xFF])
    assert v[0x80 | 0x38] == -1.0
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0) and len(pos) == 127


def _fraction_e4m3_table():
    out = []
    for c in range(127):
        e, m = c >> 3, c & 7
        out.append(Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return out


def expected_scale_code(amax: Fraction, table=None) -> int:
    """Exact E4M3 rounding (nearest, ties to even code, saturating) of amax/6."""
    return expected_e4m3_code(amax / 6, table)


def expected_e4m3_code(q: Fraction, table=None) -> int:
    """Exact E4M3 rounding (nearest, ties to even code, saturating) of q >= 0."""
    table = table or _fraction_e4m3_table()
    if q >= table[-1]:
        return 126
    i = bisect.bisect_left(table, q)
    if table[i] == q:
        return i
    lo, hi = i - 1, i
    dl, dh = q - table[lo], table[hi] - q
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    return lo if lo % 2 == 0 else hi


def check_scale_rounding_exhaustive(codec):
    """Every positive finite bf16 amax, against exact rational rounding of amax/6."""
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    amax = bf16_value(bits)
    blocks = np.zeros((len(bits), 16), np.float32)
    blocks[:, 5] = amax
    got = codec.block_scale_codes(blocks)[:, 0]
    table = _fraction_e4m3_table()
    exp = np.array([expected_scale_code(Fraction(float(a)), table) for a in amax], np.uint8)
    bad = np.nonzero(got != exp)[0]
    assert len(bad) == 0, f"{len(bad)} mismatches, first amax={amax[bad[0]]!r} got {got[bad[0]]} want {exp[bad[0]]}"


def threshold_code(y: np.ndarray, s: float) -> np.ndarray:
    """E2M1 code from comparisons against exact midpoints t*s (ties to the even code)."""
    a = np.abs(y.astype(np.float64))
    mag = ((a > 0.25 * s).astype(np.int64) + (a >= 0.75 * s) + (a > 1.25 * s) + (a >= 1.75 * s)
           + (a > 2.5 * s) + (a >= 3.5 * s) + (a > 5.0 * s))
    if s == 0:
        mag = np.zeros_like(mag)
    return ((np.signbit(y).astype(np.int64) << 3) | mag).astype(np.uint8)


def check_element_rounding_exhaustive(codec, scale_codes=range(0, 127)):
    """All finite bf16 values (both signs) under every E4M3 scale, against the threshold form."""
    y = bf16_value(finite_bf16_patterns())
    for c in scale_codes:
        s = float(codec.e4m3_value(c))
        got = codec.e2m1_encode(y.astype(np.float64), s)
        exp = threshold_code(y, s)
        bad = np.nonzero(got != exp)[0]
        assert len(bad) == 0, f"scale code {c:#x}: {len(bad)} mismatches, first y={y[bad[0]]!r}"


def check_fp16_decode(codec):
    """The writer's fp16 input decoding against the field definition, every finite pattern."""
    bits = finite_fp16_patterns()
    got = codec.fp16_to_f32(bits).astype(np.float64)
    exp = fp16_value_by_fields(bits)
    assert np.array_equal(got, exp) and np.array_equal(np.signbit(got), np.signbit(exp))


def check_scale_rounding_exhaustive_fp16(codec):
    """Every positive finite fp16 amax, against exact rational rounding of amax/6."""
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    amax = fp16_value_by_fields(bits).astype(np.float32)
    blocks = np.zeros((len(bits), 16), np.float32)
    blocks[:, 9] = -amax
    got = codec.block_scale_codes(blocks)[:, 0]
    table = _fraction_e4m3_table()
    exp = np.array([expected_scale_code(Fraction(float(a)), table) for a in amax], np.uint8)
    bad = np.nonzero(got != exp)[0]
    assert len(bad) == 0, f"{len(bad)} mismatches, first amax={amax[bad[0]]!r}"


def check_element_rounding_exhaustive_fp16(codec, scale_codes=range(0, 127)):
    """All finite fp16 values (both signs) under every E4M3 scale, against the threshold form."""
    y = fp16_value_by_fields(finite_fp16_patterns())
    for c in scale_codes:
        s = float(codec.e4m3_value(c))
        got = codec.e2m1_encode(y, s)
        exp = threshold_code(y.astype(np.float32), s)
        bad = np.nonzero(got != exp)[0]
        assert len(bad) == 0, f"scale code {c:#x}: {len(bad)} mismatches, first y={y[bad[0]]!r}"


def check_round_to_dtype(codec, seed=11):
    """bf16 / fp16 output rounding against exact rational nearest-even, on random float32 values,
    exact ties of both formats, subnormal and near-limit values."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(3000) * np.exp(rng.uniform(-20, 12, 3000))).astype(np.float32)
    ties_bf16 = (((rng.integers(0, 1 << 15, 500) << 16) | 0x8000)).astype(np.uint32).view(np.float32)
    ties_fp16 = (rng.integers(1, 1 << 10, 500) * 2.0 ** -11 + 1.0) * 2.0 ** rng.integers(-14, 15, 500)
    extra = np.array([0.0, -0.0, 2.0 ** -25, 3 * 2.0 ** -26, 65504.0, 6e-8, -1e-40], np.float32)
    x = np.concatenate([x, ties_bf16[np.isfinite(ties_bf16)], ties_fp16.astype(np.float32), extra])
    got_b = codec.round_to_dtype(x, "bf16")
    got_h = codec.round_to_dtype(x, "fp16")
    for xi, gb, gh in zip(x, got_b, got_h):
        f = Fraction(float(xi))
        eb = nearest_even_fraction(f, -126, 7)                     # bf16: 7 fraction bits
        assert Fraction(float(bf16_value(np.array([gb], np.uint16))[0])) == eb, (xi, gb)
        if abs(f) < 65520:                                          # below fp16 overflow
            eh = nearest_even_fraction(f, -14, 10)                   # fp16: 10 fraction bits
            assert Fraction(float(fp16_value_by_fields(np.array([gh], np.uint16))[0])) == eh, (xi, gh)


def check_dequant_routes_agree(codec, cache_mod, seed=5):
    """The standalone dequantization (float32 product, rounded to the output type) equals the
    float64 read path used by attention, for g = 1 where every value is exact in bf16 and fp16,
    and slot < 0 gives zero rows."""
    rng = np.random.default_rng(seed)
    c = cache_mod.PagedCache(6, 2)
    x = (rng.standard_normal((40, 2, 128)) * np.exp(rng.uniform(-6, 6, (40, 2, 1)))).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)          # truncation: any bf16 pattern
    slots = rng.permutation(96)[:40].astype(np.int64)
    c.append(bits, bits[::-1].copy(), slots)
    q = np.concatenate([slots, [-1]])
    for out in ("bf16", "fp16", "f32"):
        k, v = c.dequant_slots(q, out)
        for got, data, scale in ((k, c.k_data, c.k_scale), (v, c.v_data, c.v_scale)):
            ref = codec.dequantize(data[slots // 16, :, slots % 16, :], scale[slots // 16, :, slots % 16, :])
            if out == "bf16":
                val = bf16_value(got[:-1])
            elif out == "fp16":
                val = fp16_value_by_fields(got[:-1])
            else:
                val = got[:-1]
            assert np.array_equal(np.asarray(val, np.float64), ref), out
            assert not np.any(np.asarray(got[-1], np.float64)), out


def check_fp8_encode_exhaustive(codec):
    """FP8 cache encoding of every finite bf16 and fp16 value (both signs) against exact
    rational nearest-even rounding onto the E4M3FN values, saturating at 448."""
    table = _fraction_e4m3_table()
    for vals in (bf16_value(finite_bf16_patterns()), fp16_value_by_fields(finite_fp16_patterns())):
        got = codec.e4m3_encode_signed(np.asarray(vals, np.float64))
        mags = np.abs(np.asarray(vals, np.float64))
        uniq, inv = np.unique(mags, return_inverse=True)
        exp_mag = np.array([expected_e4m3_code(Fraction(float(a)), table) for a in uniq], np.uint8)[inv]
        exp = (np.signbit(vals).astype(np.uint8) << 7) | exp_mag
        bad = np.nonzero(got != exp)[0]
        assert len(bad) == 0, f"{len(bad)} mismatches, first y={vals[bad[0]]!r}"


def check_fp8_dequant(codec, fp8_mod):
    """FP8 standalone dequantization of every finite E4M3FN code (both signs) against exact
    rationals: g * e4m3(code) rounded to float32, then nearest-even to the output type; g = 1 for
    K (every product exact) and fl32(1/3) for V (the product rounds); slot < 0 gives zeros."""
    table = _fraction_e4m3_table()
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    c = fp8_mod.Fp8PagedCache(1, 1, k_global=1.0, v_global=float(np.float32(1 / 3)))
    c.k_data[0, 0, :2, :] = np.resize(codes, (2, 128))
    c.v_data[0, 0, :2, :] = np.resize(codes, (2, 128))
    value = {int(x): (-1 if x & 0x80 else 1) * table[x & 0x7F] for x in codes}
    flat = np.resize(codes, 256)
    for out, (emin, mant, decode) in {"bf16": (-126, 7, bf16_value), "fp16": (-14, 10, fp16_value_by_fields),
                                      "f32": (-126, 23, None)}.items():
        k, v = c.dequant_slots(np.array([0, 1, -1]), out)
        for got, g in ((k, Fraction(1)), (v, Fraction(float(np.float32(1 / 3))))):
            vals = np.asarray(got[:2, 0].reshape(-1) if decode is None else decode(got[:2, 0].reshape(-1)), np.float64)
            for i, x in enumerate(flat):
                f32 = nearest_even_fraction(value[int(x)] * g, -126, 23)
                exp = nearest_even_fraction(f32, emin, mant)
                assert Fraction(float(vals[i])) == exp, (out, int(x), float(vals[i]), float(exp))
                if exp == 0:
                    assert np.signbit(vals[i]) == bool(x & 0x80), (out, int(x))
            assert not np.any(np.asarray(got[2], np.float64)), out


def check_repack(codec, cache_mod, seed=9):
    """The repacked fp16 copy decodes (by its fields) to the exact s * e2m1 of every element of
    the reached pages, with g != 1 left out; pages beyond a sequence's length and pages no
    sequence reaches stay zero."""
    rng = np.random.default_rng(seed)
    c = cache_mod.PagedCache(12, 2, k_global=1.5, v_global=0.75)
    x = (rng.standard_normal((96, 2, 128)) * np.exp(rng.uniform(-8, 8, (96, 2, 1)))).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    c.append(bits, bits[::-1].copy(), np.arange(96, dtype=np.int64) + 16)  # pages 1..6
    bt = np.array([[3, 1, 5, 0], [6, 4, 2, 9]], np.int32)
    lens = [40, 33]  # sequence 0 reaches pages 3, 1, 5; sequence 1 reaches 6, 4, 2
    k, v = c.repack(bt, lens)
    reached = [3, 1, 5, 6, 4, 2]
    for got, data, scale in ((k, c.k_data, c.k_scale), (v, c.v_data, c.v_scale)):
        exact = codec.dequantize(data[reached], scale[reached])  # g = 1: the repack leaves g out
        assert np.array_equal(fp16_value_by_fields(got[reached]), exact)
        others = [p for p in range(12) if p not in reached]
        assert not np.any(got[others])
        assert np.any(exact)


def check_worked_block(codec):
    g = golden("worked_block.json")
    x = np.array(g["values"], np.float32)
    codes, sc = codec.quantize(x)
    assert int(sc[0]) == int(g["scale_code"], 16)
    assert [int(c) for c in codes] == [int(c, 16) for c in g["element_codes"]]
    assert codec.pack(codes).tobytes().hex() == g["packed_hex"]
    assert list(codec.dequantize(codec.pack(codes), sc)) == g["dequantized"]


# ---------------------------------------------------------------------------------------
# Footprint figures printed on the pages
# ---------------------------------------------------------------------------------------

def check_footprint(cache_mod):
    g = golden("footprint.json")
    one = cache_mod.PagedCache(num_pages=1, num_kv_heads=1, head_dim=128, page_size=16)
    per_token_head_x = one.nbytes() // 16 // 2  # bytes per (token, head) for one of K or V
    bits_per_block = per_token_head_x * 8 // (128 // 16)
    assert bits_per_block == g["bits_per_block_of_16"]["value"]
    assert bits_per_block / 16 == g["bits_per_value"]["value"]
    ratio = (bits_per_block / 16) / 8
    assert ratio == g["ratio_to_fp8"]["value"]
    assert round(1 / ratio, 2) == g["capacity_multiplier_rounded"]["value"]

    h8 = cache_mod.PagedCache(num_pages=1, num_kv_heads=8, head_dim=128, page_size=16)
    per_token_layer = h8.nbytes() // 16
    fp8_64 = 2 * 64 * 8 * 128
    assert fp8_64 == g["fp8_bytes_per_token_L64_H8_D128"]["value"]
    assert per_token_layer * 64 == g["nvfp4_bytes_per_token_L64_H8_D128"]["value"]
    assert 131072 * fp8_64 == g["fp8_gib_at_131072_tokens"]["value"] * 2 ** 30
    assert 131072 * per_token_layer * 64 == g["nvfp4_gib_at_131072_tokens"]["value"] * 2 ** 30
    vals80 = 2 * 80 * 8 * 128
    assert vals80 == g["values_per_token_L80_H8_D128"]["value"]
    assert vals80 * 2 == g["bf16_bytes_per_token_L80"]["value"]
    assert vals80 == g["fp8_kib_per_token_L80"]["value"] * 1024
    nv80 = per_token_layer * 80
    assert nv80 == g["nvfp4_bytes_per_token_L80"]["value"]
    assert round(32768 * nv80 / 2 ** 30, 2) == g["nvfp4_gib_32768_tokens_L80_about"]["value"]
    assert 32768 * vals80 * 2 == g["bf16_gib_32768_tokens_L80"]["value"] * 2 ** 30
    assert 32768 * vals80 == g["fp8_gib_32768_tokens_L80"]["value"] * 2 ** 30
    assert round(8 * 32768 * nv80 / 2 ** 30, 1) == g["nvfp4_gib_8_seqs_about"]["value"]
    assert 8 * 32768 * vals80 * 2 == g["bf16_gib_8_seqs"]["value"] * 2 ** 30


# ---------------------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------------------

def brute_force_attention(q, k, v, last_visible, sm_scale):
    """Python-float loops: z, max, exp, sum and the weighted sum of V, row by row."""
    n, d = len(q), len(q[0])
    out, lses = [], []
    for i in range(n):
        z = []
        for j in range(last_visible[i] + 1):
            z.append(sm_scale * math.fsum(float(q[i][t]) * float(k[j][t]) for t in range(d)))
        m = max(z)
        e = [math.exp(x - m) for x in z]
        den = math.fsum(e)
        out.append([math.fsum(e[j] * float(v[j][t]) for j in range(len(e))) / den for t in range(d)])
        lses.append(m + math.log(den))
    return np.array(out), np.array(lses)


def _nvfp4_round_trip(codec, x):
    c, sc = codec.quantize(x)
    return codec.dequantize(codec.pack(c), sc)


def check_attention_bruteforce(codec, cache_mod, attention, seed=7, head_dim=32,
                               make_cache=None, round_trip=None):
    """Tiny ragged shapes, all rows, GQA 2, vs Python loops over independently dequantized K/V
    (NVFP4 by default; `make_cache` / `round_trip` select another cache format)."""
    make_cache = make_cache or cache_mod.PagedCache
    round_trip = round_trip or (lambda x: _nvfp4_round_trip(codec, x))
    rng = np.random.default_rng(seed)
    q_lens, kv_lens = [1, 3, 5], [1, 7, 9]
    hq, hkv, ps = 4, 2, 16
    pages = [(n + ps - 1) // ps for n in kv_lens]
    perm = rng.permutation(sum(pages) + 2)
    bt = np.zeros((len(kv_lens), max(pages)), np.int32)
    off = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[off:off + n]; off += n
    cache = make_cache(sum(pages) + 2, hkv, head_dim=head_dim, page_size=ps)
    sm = 1 / math.sqrt(head_dim)
    qs, ks, vs = [], [], []
    for b, (ql, kl) in enumerate(zip(q_lens, kv_lens)):
        k = (rng.standard_normal((kl, hkv, head_dim)) * 2).astype(np.float32)
        v = rng.standard_normal((kl, hkv, head_dim)).astype(np.float32)
        kb = (k.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 input will do
        vb = (v.view(np.uint32) >> 16).astype(np.uint16)
        pos = np.arange(kl)
        slots = bt[b][pos // ps].astype(np.int64) * ps + pos % ps
        cache.append(kb, vb, slots)
        qs.append((rng.standard_normal((ql, hq, head_dim)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
        ks.append(kb); vs.append(vb)
    qb = np.concatenate(qs)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    o, lse = attention.prefill(cache, qb, cu, kv_lens, bt, sm)
    for b, (ql, kl) in enumerate(zip(q_lens, kv_lens)):
        for kvh in range(hkv):
            kd = round_trip(bf16_value(ks[b][:, kvh]))
            vd = round_trip(bf16_value(vs[b][:, kvh]))
            for h in range(kvh * (hq // hkv), (kvh + 1) * (hq // hkv)):
                qv = bf16_value(qs[b][:, h]).astype(np.float64)
                ref_o, ref_l = brute_force_attention(qv, kd, vd, [kl - ql + i for i in range(ql)], sm)
                np.testing.assert_allclose(o[cu[b]:cu[b + 1], h], ref_o, rtol=0, atol=1e-12)
                np.testing.assert_allclose(lse[cu[b]:cu[b + 1], h], ref_l, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------
# Per-tensor scale g != 1 ("NVFP4 KV cache vs NVFP4 weights": a second, per-tensor scale maps
# the tensor into the range the block format covers; the writer divides by it, the reader
# multiplies by it)
# ---------------------------------------------------------------------------------------

def rne32(x: Fraction) -> Fraction:
    """x rounded to the nearest float32 (ties to even), normal and subnormal range."""
    return nearest_even_fraction(x, -126, 23)


_E2M1_MIDPOINTS = [Fraction(1, 4), Fraction(3, 4), Fraction(5, 4), Fraction(7, 4), Fraction(5, 2),
                   Fraction(7, 2), Fraction(5)]


def expected_block(xs, g: Fraction, table=None):
    """Scale code and element codes of one 16-value block of float32 inputs under per-tensor
    scale g, by exact rationals: y = RNE32(x / g); s = E4M3(RNE32(amax_y / 6)); magnitude code =
    number of midpoints below |y| / s (a midpoint itself counts when the lower grid code is odd,
    which sends ties to the even code); sign bit copied from y (from x, as g > 0)."""
    table = table or _fraction_e4m3_table()
    ys = [rne32(Fraction(float(x)) / g) for x in xs]
    amax = max(abs(y) for y in ys)
    sc = expected_e4m3_code(rne32(amax / 6), table)
    s = table[sc]
    codes = []
    for x, y in zip(xs, ys):
        mag = 0
        if s > 0:
            r = abs(y) / s
            for i, t in enumerate(_E2M1_MIDPOINTS):
                if r > t or (r == t and i % 2 == 1):
                    mag += 1
        codes.append((8 if math.copysign(1.0, float(x)) < 0 else 0) | mag)
    return sc, codes


def near_threshold_inputs(g: float, seed=31, n=192) -> np.ndarray:
    """Float32 blocks whose quotients x / g sit within a few float32 ulps of an E2M1 rounding
    midpoint t * s (x = fl32(t s g) and its float32 neighbours), each block holding 6 s g so that
    its scale is s (or one code away): inputs on which y = fl32(x / g) and the exact x / g round
    differently."""
    rng = np.random.default_rng(seed)
    out = np.zeros((n, 16), np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for i in range(n):
        s = float(2.0 ** rng.integers(-8, 6) * (1 + rng.integers(0, 8) / 8))
        out[i, 0] = np.float32(6 * s * g)
        t = mids[rng.integers(0, 7, 15)]
        base = (t * s * g).astype(np.float32)
        step = rng.integers(-3, 4, 15)
        vals = np.array([np.nextafter(b, np.float32(np.inf) if k > 0 else np.float32(-np.inf))
                         if k else b for b, k in zip(base, step)], np.float32)
        for j, k in enumerate(step):  # |k| float32 steps
            for _ in range(abs(int(k)) - 1):
                vals[j] = np.nextafter(vals[j], np.float32(np.inf) if k > 0 else np.float32(-np.inf))
        out[i, 1:] = vals * np.where(rng.random(15) < 0.5, -1, 1).astype(np.float32)
    return out


def check_quantize_general_g(codec, gs=(float(np.float32(1 / 3)), 1.5, 0.75), seed=32):
    """codec.quantize at non-power-of-two g against exact rationals (y = RNE32(x / g), then the
    block rule), on random blocks over a wide range and on blocks built next to rounding
    midpoints."""
    rng = np.random.default_rng(seed)
    table = _fraction_e4m3_table()
    for g in gs:
        gf = Fraction(g)
        rand = (rng.standard_normal((160, 16)) * np.exp(rng.uniform(-12, 9, (160, 1)))).astype(np.float32)
        rand[0] = 0.0
        rand[1, ::2] = -0.0
        x = np.concatenate([rand, near_threshold_inputs(g, seed=seed + int(g * 1000))])
        codes, sc = codec.quantize(x, g)
        for i in range(x.shape[0]):
            esc, ecodes = expected_block(x[i], gf, table)
            assert int(sc[i, 0]) == esc, (g, i, int(sc[i, 0]), esc)
            assert [int(c) for c in codes[i]] == ecodes, (g, i, list(codes[i]), ecodes)


# g pairs (K, V) for the NVFP4 dequantization pin: fl32(1/3) and 1.5 are plain non-powers of two;
# 2.8187499 (bf16 output) and 1.1714844 (fp16 output) are float32 values for which a product
# s * e2m1 * g rounded first to float32 and then to the output type differs from rounding the
# exact product once (19 of the 127 x 7 magnitudes each), so the pin sees the float32 step.
DEQUANT_G_PAIRS = ((float(np.float32(1 / 3)), 1.5), (2.8187499046325684, 1.171484351158142))


def check_nvfp4_dequant_general_g(codec, cache_mod, g_pairs=DEQUANT_G_PAIRS):
    """NVFP4 standalone dequantization at g != 1 of every element code under every scale code,
    against exact rationals: RNE32(s * e2m1(code) * g) (s * e2m1 is exact), then nearest-even to
    the output type; slot < 0 gives zero rows."""
    table = _fraction_e4m3_table()
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
            Fraction(4), Fraction(6)]
    fmts = {"bf16": (-126, 7, bf16_value), "fp16": (-14, 10, fp16_value_by_fields),
            "f32": (-126, 23, None)}
    memo = {}

    def expected(sc, e, g, out):
        key = (sc, e, g, out)
        if key not in memo:
            exact = (-1 if e & 8 else 1) * table[sc] * grid[e & 7] * Fraction(g)
            memo[key] = nearest_even_fraction(rne32(exact), fmts[out][0], fmts[out][1])
        return memo[key]

    for gk, gv in g_pairs:
        c = cache_mod.PagedCache(8, 2, k_global=gk, v_global=gv)
        # 127 scale codes x 16 element codes: token t of page p, head h holds scale code
        # (8 (16 p + t) + 4 h + block) % 127 in block `block`, and every block holds all 16
        # element codes (a rotated 0..15 ramp)
        nslots = 8 * 16
        codes = np.tile(np.arange(16, dtype=np.uint8), 8)
        packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
        for slot in range(nslots):
            p, t = divmod(slot, 16)
            for h in range(2):
                for plane_d, plane_s in ((c.k_data, c.k_scale), (c.v_data, c.v_scale)):
                    plane_d[p, h, t] = np.roll(packed, slot % 7)
                    plane_s[p, h, t] = [(8 * slot + 4 * h + bb) % 127 for bb in range(8)]
        slots = np.concatenate([np.arange(nslots), [-1]]).astype(np.int64)
        for out, (_, _, decode) in fmts.items():
            k, v = c.dequant_slots(slots, out)
            for got, data, scale, g in ((k, c.k_data, c.k_scale, gk), (v, c.v_data, c.v_scale, gv)):
                vals = np.asarray(got if decode is None else decode(got), np.float64)
                for slot in range(nslots):
                    p, t = divmod(slot, 16)
                    for h in range(2):
                        row = data[p, h, t]
                        el = np.empty(128, np.int64)
                        el[0::2], el[1::2] = row & 0xF, row >> 4
                        for j in range(128):
                            exp = expected(int(scale[p, h, t, j // 16]), int(el[j]), g, out)
                            assert Fraction(float(vals[slot, h, j])) == exp, (out, g, slot, h, j)
                assert not np.any(vals[-1]), out


def expected_nvfp4_dual_row(q_row):
    """Two-level NVFP4 quantization of one float32 query row by exact rationals: g =
    RNE32(amax / RNE32(6 * 448)) (1 for a zero row); y = RNE32(q / g); each 16-block of y gets
    s = E4M3(RNE32(amax_b / 6)) and E2M1 nearest-even codes; value g * s * e2m1 (no further
    rounding)."""
    table = _fraction_e4m3_table()
    fr = [Fraction(float(x)) for x in q_row]
    amax = max(abs(x) for x in fr)
    g = rne32(amax / rne32(Fraction(6 * 448))) if amax > 0 else Fraction(1)
    out = []
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
            Fraction(4), Fraction(6)]
    for b0 in range(0, len(fr), 16):
        ys = [rne32(x / g) for x in fr[b0:b0 + 16]]
        s = table[expected_e4m3_code(rne32(max(abs(y) for y in ys) / 6), table)]
        for y in ys:
            mag = 0
            if s > 0:
                r = abs(y) / s
                for i, t in enumerate(_E2M1_MIDPOINTS):
                    if r > t or (r == t and i % 2 == 1):
                        mag += 1
            out.append(float((-1 if y < 0 else 1) * grid[mag] * s * g))
    return out


def dual_level_rows(seed=33) -> np.ndarray:
    """Query rows for the two-level pin: N(0,1) rows over a wide range of magnitudes, zero rows,
    and rows whose blocks span many binades (some blocks 2^-10 .. 2^-20 of the row maximum, where
    the level-one scale decides whether their block scales are normal or subnormal)."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((40, 128)) * np.exp(rng.uniform(-30, 30, (40, 1)))).astype(np.float32)
    x[0] = 0.0
    for i in range(1, 12):
        x[i] *= np.repeat(np.float32(2.0) ** -rng.integers(0, 21, 8), 16).astype(np.float32)
    return x


def check_nvfp4_dual(a4q_mod):
    x = dual_level_rows()
    got = a4q_mod.quantize_q(x, "nvfp4_dual")
    for i in range(x.shape[0]):
        assert list(got[i]) == expected_nvfp4_dual_row(x[i]), i
