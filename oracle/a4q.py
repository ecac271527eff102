"""A4Q-style QK numerics, oracle side (test infrastructure; see the package docstring).

"NVFP4 KV cache A4Q prefill explained", section "Quantize Q instead of expanding K": the A4Q
kernel turns Q into block-scaled FP4 in the kernel for the QK product, feeds the packed K codes
and their stored block scales to that product unchanged, and does PV in BF16.  Section "Make
query accuracy a release gate" asks for the added error over varied sequence lengths, head
layouts, masking and outlier scales, with the scale scheme, block grouping and rounding
written down.  The pages leave those choices open; each scheme below is a reading, named by
what it does:

* ``nvfp4``       16 consecutive head-dim values per block; block scale
                  E4M3_RNE_sat(fl32(amax / 6)); elements E2M1 round-to-nearest-even, saturating
                  at 6 (the cache writer's own rule applied to each query row; one scale level).
* ``nvfp4_dual``  a float32 scale per (token, head) first, g = fl32(amax_row / (6 * 448)), so the
                  row's largest block scale lands at the top of the E4M3 range; y = fl32(q / g);
                  then the ``nvfp4`` rule on y; value g * s * e2m1 (two scale levels).
* ``mxfp4``       32 consecutive values per block with a power-of-two scale
                  X = 2^(floor(log2 amax) - 2) (the block's largest exponent minus E2M1's largest
                  exponent, 2); elements E2M1 round-to-nearest-even of v / X, saturating at 6
                  (the MX format; the one gfx950's block-scaled MFMA takes for its operands).
* ``mxfp8``       the same MX rule with E4M3 elements: X = 2^(floor(log2 amax) - 8) (E4M3's
                  largest exponent is 8), elements E4M3 round-to-nearest-even of v / X, saturating
                  at 448 (the block's largest element can lie in [256, 512) before saturation).

The attention is the oracle's plain definition with each query row replaced by its quantized
value (the QK product itself exact), K and V the cache's dequantized values, and the softmax
weights rounded to bf16 (nearest-even) as the PV operand; the normaliser sums the unrounded
weights (reading: only the PV operand is BF16).
"""
from __future__ import annotations

import numpy as np

from . import attention, codec
from .cache import PagedCache

SCHEMES = ("nvfp4", "nvfp4_dual", "mxfp4", "mxfp8")
MX_BLOCK = 32


def _nvfp4_values(y32: np.ndarray) -> np.ndarray:
    """Values g=1 NVFP4 quantization gives float32 rows y32 [..., D]: s * e2m1(code)."""
    codes, sc = codec.quantize(y32)
    return codec.dequantize(codec.pack(codes), sc)


def mxfp4_values(x: np.ndarray) -> np.ndarray:
    """MXFP4 quantization of float rows along the last axis (a multiple of 32 long): per block
    X = 2^(floor(log2 amax) - 2), element E2M1_RNE_sat(v / X); returns X * e2m1 in float64.
    A block of zeros stays zero."""
    x = np.asarray(x, dtype=np.float64)
    xb = x.reshape(*x.shape[:-1], x.shape[-1] // MX_BLOCK, MX_BLOCK)
    amax = np.abs(xb).max(axis=-1, keepdims=True)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    # floor(log2) of a float64 can be off by one next to a power of two: settle it exactly
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > amax, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= amax, e + 1, e)
    X = np.where(amax > 0, np.ldexp(1.0, (e - 2).astype(np.int64)), 0.0)
    codes = codec.e2m1_encode(xb, X)
    return (codec.e2m1_value(codes) * X).reshape(x.shape)


def _mx_shared_exponent(xb: np.ndarray) -> np.ndarray:
    """floor(log2 amax) of each block (last axis), exact; 0 for an all-zero block."""
    amax = np.abs(xb).max(axis=-1, keepdims=True)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    # floor(log2) of a float64 can be off by one next to a power of two: settle it exactly
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > amax, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= amax, e + 1, e)
    return np.where(amax > 0, e, 0.0).astype(np.int64)


def mxfp8_codes(x: np.ndarray):
    """MXFP8 (E4M3 elements) quantization of float rows along the last axis (a multiple of 32
    long): per block the E8M0 scale code c = floor(log2 amax) - 8 + 127 (clamped to 0..254; 127
    for an all-zero block) and element codes E4M3_RNE_sat(v / 2^(c - 127)), sign copied.
    Returns (element codes uint8 [..., D], scale codes int64 [..., D/32])."""
    x = np.asarray(x, dtype=np.float64)
    xb = x.reshape(*x.shape[:-1], x.shape[-1] // MX_BLOCK, MX_BLOCK)
    c = np.clip(_mx_shared_exponent(xb) - 8 + 127, 0, 254)
    y = xb / np.ldexp(1.0, c - 127)  # exact: a power of two
    codes = codec.e4m3_encode_signed(np.clip(y, -448.0, 448.0))
    return codes.reshape(x.shape), c[..., 0]


def mxfp8_values(x: np.ndarray) -> np.ndarray:
    """Value of the MXFP8 quantization of x: 2^(c - 127) * e4m3(code), float64."""
    codes, c = mxfp8_codes(x)
    x = np.asarray(x)
    vb = codec.e4m3_value(codes).reshape(*x.shape[:-1], x.shape[-1] // MX_BLOCK, MX_BLOCK)
    return (vb * np.ldexp(1.0, c - 127)[..., None]).reshape(x.shape)


def quantize_q(q: np.ndarray, scheme: str) -> np.ndarray:
    """Quantized value of float query rows q [..., D] (exact bf16 values) under ``scheme``."""
    q32 = np.asarray(q, dtype=np.float32)
    if scheme == "nvfp4":
        return _nvfp4_values(q32)
    if scheme == "nvfp4_dual":
        amax = np.abs(q32).max(axis=-1, keepdims=True)
        g = (amax / np.float32(codec.E2M1_MAX * 448.0)).astype(np.float32)
        g = np.where(g > 0, g, np.float32(1.0)).astype(np.float32)
        y = (q32 / g).astype(np.float32)
        return _nvfp4_values(y) * g.astype(np.float64)
    if scheme == "mxfp4":
        return mxfp4_values(q32)
    if scheme == "mxfp8":
        return mxfp8_values(q32)
    raise ValueError(f"unknown scheme {scheme!r}")


def _round_bf16(x: np.ndarray) -> np.ndarray:
    return codec.bf16_to_f32(codec.round_to_dtype(np.asarray(x, np.float32), "bf16")).astype(np.float64)


def attend_a4q(qh: np.ndarray, k: np.ndarray, v: np.ndarray, last_visible: np.ndarray,
               sm_scale: float) -> np.ndarray:
    """Rows of quantized queries qh [n][D] over k, v [m][D] (float64): scores exact, weights
    rounded to bf16 for the PV product, normaliser from the unrounded weights."""
    o = np.full((qh.shape[0], v.shape[1]), np.nan)
    cols = np.arange(k.shape[0])
    for r0 in range(0, qh.shape[0], 512):
        r1 = min(qh.shape[0], r0 + 512)
        z = sm_scale * (qh[r0:r1] @ k.T)
        z[cols[None, :] > np.asarray(last_visible[r0:r1])[:, None]] = -np.inf
        zmax = z.max(axis=1, initial=-np.inf)
        ok = np.isfinite(zmax)
        e = np.exp(z[ok] - zmax[ok, None])
        o[r0:r1][ok] = (_round_bf16(e) @ v) / e.sum(axis=1)[:, None]
    return o


def prefill_a4q(cache: PagedCache, q_bits: np.ndarray, cu_seqlens_q, kv_lens, block_table,
                sm_scale: float, scheme: str, causal: bool = True, rows=None) -> np.ndarray:
    """Causal paged prefill with A4Q-style QK (``scheme``); the arguments and the row selection
    follow ``attention.prefill``.  Returns o [total_q][Hq][D] in float64 (NaN where not
    evaluated)."""
    q = codec.bf16_to_f32(q_bits).astype(np.float64)
    total_q, hq, d = q.shape
    group = hq // cache.num_kv_heads
    o = np.full((total_q, hq, d), np.nan)
    want = np.ones(total_q, bool) if rows is None else np.isin(np.arange(total_q), rows)
    cu = np.asarray(cu_seqlens_q)
    for b in range(len(kv_lens)):
        q0, q1, kvl = int(cu[b]), int(cu[b + 1]), int(kv_lens[b])
        idx = np.nonzero(want[q0:q1])[0]
        if len(idx) == 0:
            continue
        kh, vh = cache.gather(block_table[b], kvl)
        last = (kvl - (q1 - q0) + idx) if causal else np.full(len(idx), kvl - 1)
        qq = quantize_q(q[q0 + idx], scheme)
        for h in range(hq):
            o[q0 + idx, h] = attend_a4q(qq[:, h], kh[:, h // group], vh[:, h // group], last, sm_scale)
    return o


# ---- the QK bridge for a block-scaled MFMA with power-of-two scales ------------------------
#
# A block-scaled matrix product that takes one power-of-two (E8M0) scale per 32 values cannot
# apply the cache's E4M3 scales per 16 values exactly, and no single FP8 value holds an NVFP4
# value (E2M1 code x E4M3 scale: up to 6 significant bits; E4M3 holds 4).  Reading used by the
# GPU variant: each 32-value block of a key (two 16-value scale blocks with scales s0, s1) gets
# X = 2^(E - 5), E = max(floor(log2 s0), floor(log2 s1)) with floor(log2 0) taken as -15; the
# values y = x / X (|y| < 384) are carried as two E4M3 terms, hi = E4M3_RNE(y) and
# lo = E4M3_RNE(y - hi); the product sees X (hi + lo).  That equals x whenever lo is exact in
# E4M3, which holds when the block's two scales lie within a factor 2^8 of each other.
#
# The one-term form keeps hi alone: the product sees X hi, one FP8 operand instead of two (half
# the matrix-core work of QK).  It rounds K to E4M3's 4 significant bits under the block's
# power-of-two scale: |X hi - x| <= 2^-4 |x| where |y| >= 2^-6 (E4M3's normal range), and at most
# half the subnormal step, 2^-10 X, below it.  It is an approximation beyond the pages' A4Q, whose
# product takes the cache's K exactly; where both 16-value block scales of a 32-value block are
# powers of two within 2^13 of each other every y has at most 2 significant bits inside E4M3's
# range and the one-term value is exact.

def k_bridge(x: np.ndarray, s: np.ndarray):
    """Two-term E4M3 form of cache values x [..., D] (float64, exact s * e2m1 values) whose
    16-value block scales are s [..., D/16].  Returns (hi codes, lo codes, scale exponent e
    [..., D/32] with X = 2^e, bridged values X (e4m3(hi) + e4m3(lo)))."""
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    with np.errstate(divide="ignore"):
        fl = np.where(s > 0, np.floor(np.log2(np.where(s > 0, s, 1.0))), -15.0)
    # E4M3 values are exact in float64; floor(log2) of them is exact (no rounding at powers of 2)
    fl = fl.reshape(*s.shape[:-1], s.shape[-1] // 2, 2).max(axis=-1).astype(np.int64)
    e = fl - 5
    X = np.repeat(np.ldexp(1.0, e), MX_BLOCK, axis=-1)
    y = x / X
    hi = codec.e4m3_encode_signed(y)
    lo = codec.e4m3_encode_signed(y - codec.e4m3_value(hi))
    bridged = X * (codec.e4m3_value(hi) + codec.e4m3_value(lo))
    return hi, lo, e, bridged


def k_one_term(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """One-term E4M3 form of cache values x [..., D] with 16-value block scales s [..., D/16]:
    X e4m3(hi), with X and hi as in ``k_bridge`` (float64)."""
    hi, _, e, _ = k_bridge(x, s)
    return np.repeat(np.ldexp(1.0, e), MX_BLOCK, axis=-1) * codec.e4m3_value(hi)


def gather_bridged_k(cache: PagedCache, block_table_row, n: int, k_terms: int = 2) -> np.ndarray:
    """K values of positions 0..n-1 of one sequence as the block-scaled product sees them:
    the two-term bridge (k_terms 2) or the one-term form (k_terms 1); float64 [n][H][D]."""
    if k_terms not in (1, 2):
        raise ValueError(f"k_terms must be 1 or 2, got {k_terms!r}")
    pos = np.arange(n)
    pages = np.asarray(block_table_row, dtype=np.int64)[pos // cache.page_size]
    kd, ks, _, _ = cache.token_rows(pages, pos % cache.page_size)
    x = codec.dequantize(kd, ks)
    s = codec.e4m3_value(ks)
    kv = k_bridge(x, s)[3] if k_terms == 2 else k_one_term(x, s)
    return kv * cache.k_global


def prefill_mx(cache: PagedCache, q_bits: np.ndarray, cu_seqlens_q, kv_lens, block_table,
               sm_scale: float, q_format: str, causal: bool = True, rows=None, k_terms: int = 2):
    """The A4Q-style prefill that gfx950's block-scaled MFMA computes: each query row quantized
    by ``q_format`` ("mxfp8" or "mxfp4", blocks of 32 consecutive head-dim values), K as its
    two-term E4M3 bridge (``k_terms`` 2) or its one-term form (1), QK exact on those values, and
    then the oracle's plain float64 attention (softmax and PV on the cache's V, unrounded).
    Other arguments as ``prefill_a4q``."""
    if q_format not in ("mxfp8", "mxfp4"):
        raise ValueError(f"q_format must be mxfp8 or mxfp4, got {q_format!r}")
    q = codec.bf16_to_f32(q_bits).astype(np.float64)
    total_q, hq, d = q.shape
    group = hq // cache.num_kv_heads
    o = np.full((total_q, hq, d), np.nan)
    want = np.ones(total_q, bool) if rows is None else np.isin(np.arange(total_q), rows)
    cu = np.asarray(cu_seqlens_q)
    for b in range(len(kv_lens)):
        q0, q1, kvl = int(cu[b]), int(cu[b + 1]), int(kv_lens[b])
        idx = np.nonzero(want[q0:q1])[0]
        if len(idx) == 0:
            continue
        kh = gather_bridged_k(cache, block_table[b], kvl, k_terms)
        _, vh = cache.gather(block_table[b], kvl)
        last = (kvl - (q1 - q0) + idx) if causal else np.full(len(idx), kvl - 1)
        qq = quantize_q(q[q0 + idx], q_format)
        for h in range(hq):
            o[q0 + idx, h] = attention.attend(qq[:, h], kh[:, h // group], vh[:, h // group], last,
                                              sm_scale)[0]
    return o
