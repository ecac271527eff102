"""Pins of the oracle's A4Q-style QK numerics (CPU only)."""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import a4q, cache, codec

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
