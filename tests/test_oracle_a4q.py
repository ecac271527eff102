"""Pins of the oracle's A4Q-style QK numerics (CPU only)."""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import a4q, cache, codec
import pins

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def _mx_block_brute(vals):
    """MXFP4 of one 32-value block by exhaustive search: X = 2^(e - 2) with e the integer
    2^e <= amax < 2^(e+1); each |v| / X goes to the nearest grid magnitude (ties: the even code),
    beyond 6 to 6; the sign is kept."""
    fr = [Fraction(float(v)) for v in vals]
    amax = max(abs(v) for v in fr)
    if amax == 0:
        return [0.0] * len(vals)
    e = 0
    while Fraction(2) ** e > amax:
        e -= 1
    while Fraction(2) ** (e + 1) <= amax:
        e += 1
    X = Fraction(2) ** (e - 2)
    out = []
    for v in fr:
        r = abs(v) / X
        best = None
        for code, gv in enumerate(GRID):
            d = abs(r - gv)
            if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
                best = (d, code, gv)
        mag = GRID[7] if r > GRID[7] else best[2]
        out.append(float((-1 if v < 0 else 1) * mag * X))
    return out


def test_mxfp4_worked_block():
    b = np.zeros(32)
    b[:5] = [7.0, 1.0, 2.5, -0.3, -2.5]
    got = a4q.mxfp4_values(b)
    # amax 7: e = 2, X = 1; 7 saturates to 6, 2.5 ties to the even code (2.0), 0.3 -> 0.5
    assert list(got[:5]) == [6.0, 1.0, 2.0, -0.5, -2.0]
    assert not np.any(got[5:])


def test_mxfp4_against_exhaustive_search():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((200, 64)) * np.exp(rng.uniform(-10, 10, (200, 1)))
    x[5, :32] = 0.0
    x[6, :32] = 2.0 ** -30
    x[7, 3] = 4.0  # amax exactly a power of two
    x = x.astype(np.float32).astype(np.float64)
    got = a4q.mxfp4_values(x)
    for i in range(x.shape[0]):
        for j in (0, 32):
            assert list(got[i, j:j + 32]) == _mx_block_brute(x[i, j:j + 32]), (i, j)


def test_nvfp4_scheme_is_the_cache_writers_rule():
    rng = np.random.default_rng(22)
    q = (rng.standard_normal((50, 4, 128)) * 3).astype(np.float32)
    got = a4q.quantize_q(q, "nvfp4")
    codes, sc = codec.quantize(q)
    assert np.array_equal(got, codec.dequantize(codec.pack(codes), sc))
    s = np.repeat(codec.e4m3_value(sc), 16, axis=-1)
    assert np.all(np.abs(got - q) <= s + np.maximum(0, np.abs(q) - 6 * s))


def test_dual_level_keeps_small_rows_that_one_level_flushes():
    rng = np.random.default_rng(23)
    q = (rng.standard_normal((8, 128)) * 1e-5).astype(np.float32)
    one = a4q.quantize_q(q, "nvfp4")
    two = a4q.quantize_q(q, "nvfp4_dual")
    assert not np.any(one)  # amax / 6 is below half the smallest E4M3 scale: every block is 0
    rel = np.linalg.norm(two - q, axis=1) / np.linalg.norm(q, axis=1)
    assert np.all(rel < 0.25)
    # exact power-of-two rescaling commutes with the dual-level scheme
    assert np.array_equal(a4q.quantize_q(q * np.float32(2.0 ** 20), "nvfp4_dual"), two * 2.0 ** 20)


def _bf16(x):
    b = struct.unpack("<I", struct.pack("<f", x))[0]
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return struct.unpack("<f", struct.pack("<I", b << 16))[0]


def test_attention_against_python_brute_force():
    rng = np.random.default_rng(24)
    d, m, n = 64, 21, 5
    k = rng.standard_normal((m, d))
    v = rng.standard_normal((m, d))
    q = rng.standard_normal((n, d)).astype(np.float32)
    last = np.array([20, 3, 0, 11, 20])
    sm = 1 / math.sqrt(d)
    for scheme in a4q.SCHEMES:
        qh = a4q.quantize_q(q, scheme)
        got = a4q.attend_a4q(qh, k, v, last, sm)
        for i in range(n):
            z = [sm * sum(float(qh[i, t]) * float(k[j, t]) for t in range(d)) for j in range(last[i] + 1)]
            zm = max(z)
            p = [math.exp(x - zm) for x in z]
            den = sum(p)
            for t in range(0, d, 7):
                ref = sum(_bf16(p[j]) * float(v[j, t]) for j in range(len(p))) / den
                assert abs(got[i, t] - ref) < 1e-12, (scheme, i, t)


def test_prefill_a4q_reduces_to_the_rows_it_was_given():
    """Same rows, heads and masks as the stock oracle: the output is finite where the stock one
    is, and the A4Q error stays within a few percent on N(0,1) inputs."""
    from oracle import attention
    import workload as W
    pc = W.prefill_case(W.get("tiny"))
    oc = cache.PagedCache(pc.layout.num_pages, pc.w.num_kv_heads)
    oc.append(pc.k_bits, pc.v_bits, pc.slot_mapping)
    ref, _ = attention.prefill(oc, pc.q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table,
                               pc.w.sm_scale)
    for scheme in a4q.SCHEMES:
        o = a4q.prefill_a4q(oc, pc.q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table,
                            pc.w.sm_scale, scheme)
        assert np.array_equal(np.isnan(o), np.isnan(ref))
        err = np.abs(o - ref)[~np.isnan(ref)]
        assert 0 < err.mean() < 0.05, (scheme, err.mean())


def test_pins_catch_mx_scale_one_exponent_high():
    def bad(x):  # X = 2^(floor(log2 amax) - 1): one exponent too high
        x = np.asarray(x, np.float64)
        _, ex = np.frexp(np.abs(x).max())  # amax = m 2^ex, m in [0.5, 1): floor(log2) = ex - 1
        X = 2.0 ** (ex - 2)
        return codec.e2m1_value(codec.e2m1_encode(x, X)) * X
    rng = np.random.default_rng(25)
    x = rng.standard_normal((4, 32))
    with pytest.raises(AssertionError):
        for i in range(4):
            assert list(bad(x[i])) == _mx_block_brute(x[i])


def _nvfp4_row_brute(row):
    """One-level NVFP4 value of a float32 row by exact rationals (the block rule at g = 1)."""
    out = []
    table = pins._fraction_e4m3_table()
    for b0 in range(0, len(row), 16):
        sc, codes = pins.expected_block(row[b0:b0 + 16], Fraction(1), table)
        for c in codes:
            out.append(float((-1 if c & 8 else 1) * GRID[c & 7] * table[sc]))
    return out


def _quantize_brute(row, scheme):
    if scheme == "mxfp4":
        return [v for j in range(0, len(row), 32) for v in _mx_block_brute(row[j:j + 32])]
    if scheme == "mxfp8":
        return [v for j in range(0, len(row), 32) for v in _mx8_block_brute(row[j:j + 32])]
    if scheme == "nvfp4":
        return _nvfp4_row_brute(row)
    return pins.expected_nvfp4_dual_row(row)


def check_prefill_a4q_paged(prefill_a4q, scheme, seed=26):
    """prefill_a4q on a paged, ragged, GQA (2 query heads per KV head), causal batch against
    Python loops: each query row quantized by the exhaustive / exact-rational quantizers above, K
    and V dequantized independently of the page table, scores and weights as Python floats,
    weights rounded to bf16 for the PV sum and the normaliser from the unrounded weights."""
    rng = np.random.default_rng(seed)
    d, hq, hkv, ps = 64, 4, 2, 16
    q_lens, kv_lens = [2, 5, 1], [3, 21, 17]
    pages = [(n + ps - 1) // ps for n in kv_lens]
    perm = rng.permutation(sum(pages) + 3)
    bt = np.zeros((3, max(pages)), np.int32)
    off = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[off:off + n]; off += n
    oc = cache.PagedCache(sum(pages) + 3, hkv, head_dim=d, page_size=ps)
    sm = 1 / math.sqrt(d)
    kd, vd, qs = [], [], []
    for b, (ql, kl) in enumerate(zip(q_lens, kv_lens)):
        k = (rng.standard_normal((kl, hkv, d)) * 2).astype(np.float32)
        v = rng.standard_normal((kl, hkv, d)).astype(np.float32)
        kb = (k.view(np.uint32) >> 16).astype(np.uint16)
        vb = (v.view(np.uint32) >> 16).astype(np.uint16)
        pos = np.arange(kl)
        oc.append(kb, vb, bt[b][pos // ps].astype(np.int64) * ps + pos % ps)
        rt = lambda bits: np.array([_nvfp4_row_brute(pins.bf16_value(r)) for r in bits.reshape(-1, d)]).reshape(kl, hkv, d)  # noqa: E731
        kd.append(rt(kb)); vd.append(rt(vb))
        qs.append((rng.standard_normal((ql, hq, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    qb = np.concatenate(qs)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    got = prefill_a4q(oc, qb, cu, kv_lens, bt, sm, scheme)
    for b, (ql, kl) in enumerate(zip(q_lens, kv_lens)):
        for h in range(hq):
            kvh = h // (hq // hkv)
            for i in range(ql):
                qv = _quantize_brute(pins.bf16_value(qs[b][i, h]), scheme)
                last = kl - ql + i
                z = [sm * math.fsum(qv[t] * kd[b][j, kvh, t] for t in range(d)) for j in range(last + 1)]
                zm = max(z)
                p = [math.exp(x - zm) for x in z]
                den = math.fsum(p)
                for t in range(d):
                    ref = math.fsum(_bf16(p[j]) * vd[b][j, kvh, t] for j in range(len(p))) / den
                    assert abs(got[cu[b] + i, h, t] - ref) < 1e-12, (scheme, b, h, i, t)


@pytest.mark.parametrize("scheme", a4q.SCHEMES)
def test_prefill_a4q_paged_ragged_vs_brute_force(scheme):
    check_prefill_a4q_paged(a4q.prefill_a4q, scheme)


def test_nvfp4_dual_vs_exact_rationals():
    pins.check_nvfp4_dual(a4q)


def test_pins_catch_prefill_a4q_top_left_mask():
    def top_left(oc, qb, cu, kv_lens, bt, sm, scheme):  # rows see keys 0..i (top-left alignment)
        o = np.full((int(cu[-1]), 4, 64), np.nan)
        for b in range(len(kv_lens)):
            q0, q1 = int(cu[b]), int(cu[b + 1])
            sub = a4q.prefill_a4q(oc, qb[q0:q1], np.array([0, q1 - q0], np.int32), [q1 - q0],
                                  bt[b:b + 1], sm, scheme)
            o[q0:q1] = sub
        return o
    with pytest.raises(AssertionError):
        check_prefill_a4q_paged(top_left, "mxfp4")


def test_pins_catch_dual_level_without_the_448():
    def bad(q, scheme):
        q32 = np.asarray(q, np.float32)
        amax = np.abs(q32).max(axis=-1, keepdims=True)
        g = (amax / np.float32(6.0)).astype(np.float32)
        g = np.where(g > 0, g, np.float32(1.0)).astype(np.float32)
        return a4q._nvfp4_values((q32 / g).astype(np.float32)) * g.astype(np.float64)
    import types
    with pytest.raises(AssertionError):
        pins.check_nvfp4_dual(types.SimpleNamespace(quantize_q=bad))


# ---- MXFP8 queries and the two-term E4M3 bridge of K (the GPU A4Q variant's scheme) --------

E4M3_POS = [f for f in pins._fraction_e4m3_table()]


def _mx8_block_brute(vals):
    """MXFP8 of one 32-value block by exhaustive search over the E4M3 values: X = 2^(e - 8)
    with e the integer 2^e <= amax < 2^(e+1); |v| / X goes to the nearest E4M3 magnitude (ties:
    the even code), beyond 448 to 448; sign kept."""
    fr = [Fraction(float(v)) for v in vals]
    amax = max(abs(v) for v in fr)
    if amax == 0:
        return [0.0] * len(vals)
    e = 0
    while Fraction(2) ** e > amax:
        e -= 1
    while Fraction(2) ** (e + 1) <= amax:
        e += 1
    X = Fraction(2) ** (e - 8)
    out = []
    for v in fr:
        r = abs(v) / X
        if r >= E4M3_POS[-1]:
            mag = E4M3_POS[-1]
        else:
            best = None
            for code, gv in enumerate(E4M3_POS):
                d = abs(r - gv)
                if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
                    best = (d, code, gv)
            mag = best[2]
        out.append(float((-1 if v < 0 else 1) * mag * X))
    return out


def test_mxfp8_against_exhaustive_search():
    rng = np.random.default_rng(41)
    x = rng.standard_normal((60, 64)) * np.exp(rng.uniform(-12, 12, (60, 1)))
    x[3, :32] = 0.0
    x[4, 5] = 2.0 ** 7 * 1.9375  # amax / X = 496: saturates to 448
    x[5, 9] = 512.0              # amax a power of two
    x = x.astype(np.float32).astype(np.float64)
    got = a4q.mxfp8_values(x)
    for i in range(x.shape[0]):
        for j in (0, 32):
            assert list(got[i, j:j + 32]) == _mx8_block_brute(x[i, j:j + 32]), (i, j)


def test_pins_catch_mxfp8_without_saturation_bound():
    def bad(x):  # X one exponent higher (amax / X in [128, 256)): no saturation, other codes
        x = np.asarray(x, np.float64)
        _, ex = np.frexp(np.abs(x).max())
        X = 2.0 ** (ex - 8)
        return codec.e4m3_value(codec.e4m3_encode_signed(x / X)) * X
    rng = np.random.default_rng(42)
    x = rng.standard_normal((4, 32))
    x[:, 0] = 1.9 * np.exp2(np.arange(4))  # amax / X = 486.4 under the rule: saturates to 448
    with pytest.raises(AssertionError):
        for i in range(4):
            assert list(bad(x[i])) == _mx8_block_brute(x[i])


def _bridge_brute(x_block, s_pair, terms=2):
    """The two-term bridge of one 32-value block by exact rationals: E from the larger scale,
    X = 2^(E - 5); hi, lo nearest-even E4M3 (searched exhaustively) of y and y - hi.  With
    terms=1 the value is X hi alone."""
    def fl(sv):
        if sv == 0:
            return -15
        e = 0
        while Fraction(2) ** e > sv:
            e -= 1
        while Fraction(2) ** (e + 1) <= sv:
            e += 1
        return e
    X = Fraction(2) ** (max(fl(Fraction(float(s_pair[0]))), fl(Fraction(float(s_pair[1])))) - 5)

    def near(r):
        a = abs(r)
        best = None
        for code, gv in enumerate(E4M3_POS):
            d = abs(a - gv)
            if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
                best = (d, gv)
        return (-1 if r < 0 else 1) * best[1]
    out = []
    for v in x_block:
        y = Fraction(float(v)) / X
        hi = near(y)
        lo = near(y - hi) if terms == 2 else 0
        out.append(float(X * (hi + lo)))
    return out


def _cache_blocks(seed, n, ratio_exp):
    """NVFP4 cache values of n 32-value blocks whose two 16-value halves differ in scale by up
    to 2^ratio_exp (both halves inside the E4M3 scale range), with their block scales."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 32)) * np.exp2(rng.uniform(-8 + ratio_exp / 2, 8 - ratio_exp / 2, (n, 1)))
    x[:, 16:] *= np.exp2(-rng.integers(0, ratio_exp + 1, (n, 1)))
    codes, sc = codec.quantize(x.astype(np.float32))
    return codec.dequantize(codec.pack(codes), sc), codec.e4m3_value(sc)


def test_k_bridge_is_exact_within_a_scale_ratio_of_2_to_the_8():
    xv, s = _cache_blocks(43, 3000, 8)
    hi, lo, e, br = a4q.k_bridge(xv, s)
    assert np.array_equal(br, xv)
    y = xv / np.repeat(np.exp2(e), 32, axis=-1)
    assert np.abs(y).max() < 384


def test_k_bridge_against_exact_rationals_on_wide_blocks():
    # first halves' scales near 2^7.4, second halves' 2^-3.3 .. 2^-7.3: 2^11 .. 2^15 apart, so
    # the low term of the small half is not always exact
    rng = np.random.default_rng(44)
    x = rng.standard_normal((60, 32))
    x[:, :16] *= 400.0
    x[:, 16:] *= np.exp2(-rng.uniform(2, 6, (60, 1)))
    codes, sc = codec.quantize(x.astype(np.float32))
    xv, s = codec.dequantize(codec.pack(codes), sc), codec.e4m3_value(sc)
    assert np.all(s > 0)
    _, _, _, br = a4q.k_bridge(xv, s)
    for i in range(xv.shape[0]):
        assert list(br[i]) == _bridge_brute(xv[i], s[i]), i
    assert not np.array_equal(br, xv)  # some values were rounded by the bridge


def test_pins_catch_k_bridge_without_the_low_term():
    def bad(x, s):
        hi, lo, e, br = a4q.k_bridge(x, s)
        X = np.repeat(np.exp2(e), 32, axis=-1)
        return hi, lo, e, X * codec.e4m3_value(hi)
    xv, s = _cache_blocks(45, 200, 4)
    with pytest.raises(AssertionError):
        assert np.array_equal(bad(xv, s)[3], xv)


# ---- the one-term form of K (X hi alone) ----------------------------------------------------

def test_k_one_term_against_exact_rationals():
    # ordinary blocks and blocks whose halves are 2^11 .. 2^15 apart (subnormal E4M3 terms)
    xv, s = _cache_blocks(46, 40, 6)
    rng = np.random.default_rng(47)
    x = rng.standard_normal((40, 32))
    x[:, :16] *= 400.0
    x[:, 16:] *= np.exp2(-rng.uniform(2, 6, (40, 1)))
    codes, sc = codec.quantize(x.astype(np.float32))
    xv = np.concatenate([xv, codec.dequantize(codec.pack(codes), sc)])
    s = np.concatenate([s, codec.e4m3_value(sc)])
    got = a4q.k_one_term(xv, s)
    for i in range(xv.shape[0]):
        assert list(got[i]) == _bridge_brute(xv[i], s[i], terms=1), i
    assert not np.array_equal(got, xv)


def test_k_one_term_error_bound():
    """|X hi - x| <= 2^-4 |x| in E4M3's normal range (|y| >= 2^-6) and <= 2^-10 X below it: half
    a unit in the last place of a 3-bit mantissa, or of the subnormal step 2^-9."""
    xv, s = _cache_blocks(48, 20000, 12)
    _, _, e, _ = a4q.k_bridge(xv, s)
    X = np.repeat(np.exp2(e), 32, axis=-1)
    err = np.abs(a4q.k_one_term(xv, s) - xv)
    normal = np.abs(xv / X) >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(xv[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10 * X[~normal])
    assert err.max() > 0 and (~normal).any()


def test_k_one_term_exact_for_power_of_two_scales_within_2_to_the_13():
    """Both halves' scales powers of two at most 2^13 apart: X e2m1 2^k values with at most 2
    significant bits, all inside E4M3's range, so X hi is the cache value itself."""
    rng = np.random.default_rng(49)
    n = 4000
    a0 = rng.integers(-9, 9, n)
    a1 = np.clip(a0 - rng.integers(0, 14, n), -9, 8)
    codes = rng.integers(0, 16, (n, 32)).astype(np.uint8)
    sv = np.stack([np.exp2(a0), np.exp2(a1)], axis=1).astype(np.float64)
    xv = codec.e2m1_value(codes) * np.repeat(sv, 16, axis=-1)
    assert np.array_equal(a4q.k_one_term(xv, sv), xv)
    # one step past the bound the smallest values fall off E4M3's subnormal grid
    sv2 = np.stack([np.full(n, 2.0 ** 5), np.full(n, 2.0 ** -9)], axis=1)
    xv2 = codec.e2m1_value(codes) * np.repeat(sv2, 16, axis=-1)
    assert not np.array_equal(a4q.k_one_term(xv2, sv2), xv2)


def test_pins_catch_k_one_term_rounded_toward_zero():
    def bad(x, s):  # E4M3 of y truncated instead of nearest-even
        _, _, e, _ = a4q.k_bridge(x, s)
        X = np.repeat(np.exp2(e), 32, axis=-1)
        y = x / X
        m, ex = np.frexp(np.abs(y))
        step = np.ldexp(1.0, np.maximum(ex - 4, -9))
        return np.sign(y) * np.floor(np.abs(y) / step) * step * X
    xv, s = _cache_blocks(50, 40, 6)
    with pytest.raises(AssertionError):
        got = bad(xv, s)
        for i in range(xv.shape[0]):
            assert list(got[i]) == _bridge_brute(xv[i], s[i], terms=1), i


def check_prefill_mx_paged(prefill_mx, q_format, seed=27, k_terms=2):
    """prefill_mx on a paged, ragged, GQA, causal batch against Python loops: queries quantized
    by the exhaustive MX searches above, K bridged (k_terms 2) or rounded to its one-term form
    (1) by exact rationals from independently quantized values, softmax and PV in Python
    floats."""
    rng = np.random.default_rng(seed)
    d, hq, hkv, ps = 64, 4, 2, 16
    q_lens, kv_lens = [3, 1, 4], [19, 5, 33]
    pages = [(n + ps - 1) // ps for n in kv_lens]
    perm = rng.permutation(sum(pages) + 2)
    bt = np.zeros((3, max(pages)), np.int32)
    off = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[off:off + n]; off += n
    oc = cache.PagedCache(sum(pages) + 2, hkv, head_dim=d, page_size=ps)
    sm = 1 / math.sqrt(d)
    kd, vd, qs = [], [], []
    table = pins._fraction_e4m3_table()
    for b, (ql, kl) in enumerate(zip(q_lens, kv_lens)):
        k = (rng.standard_normal((kl, hkv, d)) * 2).astype(np.float32)
        k[:, :, :16] *= 8  # the first 16-value block of every K row x8
        v = rng.standard_normal((kl, hkv, d)).astype(np.float32)
        kb = (k.view(np.uint32) >> 16).astype(np.uint16)
        vb = (v.view(np.uint32) >> 16).astype(np.uint16)
        pos = np.arange(kl)
        oc.append(kb, vb, bt[b][pos // ps].astype(np.int64) * ps + pos % ps)
        kk = np.zeros((kl, hkv, d))
        for t in range(kl):
            for h in range(hkv):
                row = pins.bf16_value(kb[t, h])
                vals, scs = [], []
                for b0 in range(0, d, 16):
                    sc, codes = pins.expected_block(row[b0:b0 + 16], Fraction(1), table)
                    scs.append(float(table[sc]))
                    vals += [float((-1 if c & 8 else 1) * GRID[c & 7] * table[sc]) for c in codes]
                for j in range(0, d, 32):
                    kk[t, h, j:j + 32] = _bridge_brute(vals[j:j + 32], scs[j // 16:j // 16 + 2],
                                                       terms=k_terms)
        kd.append(kk)
        vd.append(np.array([_nvfp4_row_brute(pins.bf16_value(r)) for r in vb.reshape(-1, d)]).reshape(kl, hkv, d))
        qs.append((rng.standard_normal((ql, hq, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    qb = np.concatenate(qs)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    got = prefill_mx(oc, qb, cu, kv_lens, bt, sm, q_format, k_terms=k_terms)
    quant = _mx8_block_brute if q_format == "mxfp8" else _mx_block_brute
    for b, (ql, kl) in enumerate(zip(q_lens, kv_lens)):
        for h in range(hq):
            kvh = h // (hq // hkv)
            for i in range(ql):
                row = pins.bf16_value(qs[b][i, h])
                qv = [v for j in range(0, d, 32) for v in quant(row[j:j + 32])]
                last = kl - ql + i
                z = [sm * math.fsum(qv[t] * kd[b][j, kvh, t] for t in range(d)) for j in range(last + 1)]
                zm = max(z)
                p = [math.exp(x - zm) for x in z]
                den = math.fsum(p)
                for t in range(d):
                    ref = math.fsum(p[j] * vd[b][j, kvh, t] for j in range(len(p))) / den
                    assert abs(got[cu[b] + i, h, t] - ref) < 1e-12, (q_format, b, h, i, t)


@pytest.mark.parametrize("k_terms", [2, 1])
@pytest.mark.parametrize("q_format", ["mxfp8", "mxfp4"])
def test_prefill_mx_paged_ragged_vs_brute_force(q_format, k_terms):
    check_prefill_mx_paged(a4q.prefill_mx, q_format, k_terms=k_terms)


def test_pins_catch_prefill_mx_one_term_with_the_bridged_k():
    def bad(oc, qb, cu, kv_lens, bt, sm, q_format, k_terms):  # k_terms ignored: exact K
        return a4q.prefill_mx(oc, qb, cu, kv_lens, bt, sm, q_format)
    with pytest.raises(AssertionError):
        check_prefill_mx_paged(bad, "mxfp8", k_terms=1)


def test_pins_catch_prefill_mx_with_unbridged_queries():
    def bad(oc, qb, cu, kv_lens, bt, sm, q_format, k_terms=2):  # queries left unquantized
        from oracle import attention
        return attention.prefill(oc, qb, cu, kv_lens, bt, sm)[0]
    with pytest.raises(AssertionError):
        check_prefill_mx_paged(bad, "mxfp8")
