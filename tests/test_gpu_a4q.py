"""GPU parity of the A4Q-style prefill (paged_prefill_nvfp4_a4q) against the oracle's prefill_mx:
queries quantized to MX blocks (MXFP8 or MXFP4), K through its two-term E4M3 bridge or its
one-term form (k_terms 1), float64 softmax and PV.  The bar is the stock path's (float32 output
max-abs 1e-2 / mean-abs 1e-3; bf16 beyond its rounding floor, and bit-equal to nearest-even
rounding of the float32 output).

The release-gate cases ("NVFP4 KV cache A4Q prefill explained", section "Make query accuracy a
release gate": lengths, head layouts, masks, outliers) also report the error the quantized query
adds against the stock oracle; that error is the measurement the gate asks for, not a bar."""
import numpy as np
import pytest
import torch

import attention_nvfp4_quantized_amd as A
import workload as W
from oracle import a4q
from oracle import attention as oattn
from gpu_cases import (LSE_ATOL, WORKERS, GpuPrefillCase, assert_attention_close,
                       assert_attention_close_bf16, attention_error, dev_bf16, oracle_cache, say)

pytestmark = pytest.mark.gpu

FORMATS = ["mxfp8", "mxfp4"]
FULL16K_ROWS = np.array([0, 1, 63, 64, 1000, 4095, 4096, 8191, 8192, 12345, 16319, 16320, 16383])


def _bf16_of(x32):
    b = np.ascontiguousarray(x32, np.float32).view(np.uint32)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _run(g, q_format, out_dtype, q=None, causal=True, num_splits=0, k_terms=2, return_lse=False):
    pc = g.pc
    o = A.prefill_a4q(g.cache, g.q if q is None else q, g.cu, g.kv, g.bt, pc.max_q_len,
                      pc.max_kv_len, pc.w.sm_scale, q_format=q_format, causal=causal,
                      out_dtype=out_dtype, num_splits=num_splits, k_terms=k_terms,
                      return_lse=return_lse)
    torch.cuda.synchronize()
    return o


def _ref(pc, oc, q_format, q_bits=None, causal=True, rows=None, k_terms=2):
    return a4q.prefill_mx(oc, pc.q_bits if q_bits is None else q_bits, pc.cu_seqlens_q, pc.kv_lens,
                          pc.layout.block_table, pc.w.sm_scale, q_format, causal=causal, rows=rows,
                          k_terms=k_terms)


def _check(name, g, ref, q_format, **kw):
    o32 = _run(g, q_format, torch.float32, **kw).cpu().numpy()
    o16 = _run(g, q_format, torch.bfloat16, **kw)
    what = f"{name} {q_format} k_terms={kw.get('k_terms', 2)}"
    assert_attention_close(o32, ref, f"{what} fp32")
    assert_attention_close_bf16(o16.float().cpu().numpy(), ref, f"{what} bf16")
    assert np.array_equal(o16.view(torch.int16).cpu().numpy().view(np.uint16), _bf16_of(o32))
    return o32


@pytest.mark.parametrize("k_terms", [2, 1])
@pytest.mark.parametrize("q_format", FORMATS)
@pytest.mark.parametrize("name", ["tiny", "tail128"])
def test_a4q_parity_all_rows(name, q_format, k_terms):
    say(f"[a4q] {name} {q_format} k_terms {k_terms}: every row")
    pc = W.prefill_case(W.get(name))
    g = GpuPrefillCase(pc)
    g.append()
    oc = oracle_cache(pc)
    _check(name, g, _ref(pc, oc, q_format, k_terms=k_terms), q_format, k_terms=k_terms)


@pytest.mark.parametrize("k_terms", [2, 1])
@pytest.mark.parametrize("q_format", FORMATS)
def test_a4q_parity_full16k_sampled_rows(q_format, k_terms):
    say(f"[a4q] full16k {q_format} k_terms {k_terms}: sampled rows")
    pc = W.prefill_case(W.get("full16k"))
    g = GpuPrefillCase(pc)
    g.append()
    oc = oracle_cache(pc)
    _check("full16k", g, _ref(pc, oc, q_format, rows=FULL16K_ROWS, k_terms=k_terms), q_format,
           k_terms=k_terms)


@pytest.mark.parametrize("k_terms", [2, 1])
@pytest.mark.parametrize("q_format", FORMATS)
@pytest.mark.parametrize("hq,hkv,splits,causal", [(32, 8, 0, True), (8, 8, 3, True), (64, 8, 0, False),
                                                  (16, 4, 2, False)])
def test_a4q_ragged_groups_splits_masks(q_format, hq, hkv, splits, causal, k_terms):
    say(f"[a4q] ragged batch, Hq {hq} Hkv {hkv} splits {splits} causal {causal} {q_format} "
        f"k_terms {k_terms}")
    w = W.custom("a4q", [70, 41, 5, 1], [70, 300, 1000, 33], hq, hkv, 3401 + hq, k_outlier_channels=6)
    pc = W.prefill_case(w)
    g = GpuPrefillCase(pc)
    g.append()
    oc = oracle_cache(pc)
    _check("ragged", g, _ref(pc, oc, q_format, causal=causal, k_terms=k_terms), q_format,
           causal=causal, num_splits=splits, k_terms=k_terms)


@pytest.mark.parametrize("q_format", FORMATS)
def test_a4q_one_term_k_values_through_single_key_scores(q_format):
    """Sequences of one key and one query row, each query head a one-hot row (16 at one head-dim
    index, exact in both MX formats): the log-sum-exp of a single score is the score itself (up
    to the library's log-sum-exp bar: the weight exp(0) = 1 may be rounded down to 1 - 2^-11), so
    it carries 16 sm_scale times one K value as the product saw it.  Every such value must be the
    oracle's nearest-even one-term E4M3 value: where the one-term form rounds, another rounding
    would move the score by far more than that bar.  K rows hold outliers and small halves, so
    subnormal terms and halfway cases occur."""
    say(f"[a4q] one-term K values through single-key scores, {q_format}")
    batch, hq, hkv = 512, 8, 1
    w = W.custom("a4q1key", [1] * batch, [1] * batch, hq, hkv, 3471)
    pc = W.prefill_case(w)
    rng = np.random.default_rng(3472)
    k = W.bf16_bits_to_f32(pc.k_bits).copy()
    k[:, :, ::32] *= 8.0
    for j in range(16, 128, 32):
        k[:, :, j:j + 16] *= np.exp2(-rng.uniform(0, 12, (k.shape[0], 1, 1))).astype(np.float32)
    pc.k_bits = W.f32_to_bf16_bits(k.astype(np.float32))
    dims = rng.integers(0, 128, (batch, hq))
    q = np.zeros((batch, hq, 128), np.float32)
    q[np.arange(batch)[:, None], np.arange(hq)[None, :], dims] = 16.0
    pc.q_bits = W.f32_to_bf16_bits(q)
    g = GpuPrefillCase(pc)
    g.append()
    oc = oracle_cache(pc)
    _, lse = _run(g, q_format, torch.float32, k_terms=1, return_lse=True)
    lse = lse.cpu().numpy().astype(np.float64)
    want = np.empty((batch, hq))
    exact = np.empty((batch, hq))
    for b in range(batch):
        k1 = a4q.gather_bridged_k(oc, pc.layout.block_table[b], 1, k_terms=1)[0, 0]
        k2 = a4q.gather_bridged_k(oc, pc.layout.block_table[b], 1, k_terms=2)[0, 0]
        want[b] = 16.0 * pc.w.sm_scale * k1[dims[b]]
        exact[b] = 16.0 * pc.w.sm_scale * k2[dims[b]]
    tol = 1e-5 * np.abs(want) + LSE_ATOL
    assert (np.abs(want - exact) > 2 * tol).sum() >= 200  # many scores tell the roundings apart
    bad = np.abs(lse - want) > tol
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} scores differ; first at "
                           f"{np.argwhere(bad)[0]}: {lse[bad][0]} vs {want[bad][0]}")
    o2, lse2 = _run(g, q_format, torch.float32, k_terms=2, return_lse=True)
    assert np.all(np.abs(lse2.cpu().numpy() - exact) <= 1e-5 * np.abs(exact) + LSE_ATOL)


def test_a4q_bridge_rounds_the_low_term_as_specified():
    """Keys whose 32-value blocks hold a large and a small 16-value half (scales 2^9 .. 2^15
    apart): the bridge's low term rounds; the kernel matches the oracle's bridged K."""
    say("[a4q] K blocks with widely different half scales")
    w = W.custom("a4qwide", [40, 9], [300, 129], 8, 2, 3451)
    pc = W.prefill_case(w)
    k = W.bf16_bits_to_f32(pc.k_bits).copy()
    rng = np.random.default_rng(3452)
    k[:, :, 0::32] *= 300.0  # one large value at the head of every 32-value block
    for j in range(16, 128, 32):
        k[:, :, j:j + 16] *= np.exp2(-rng.uniform(1, 5, (k.shape[0], k.shape[1], 1))).astype(np.float32)
    pc.k_bits = W.f32_to_bf16_bits(k.astype(np.float32))
    g = GpuPrefillCase(pc)
    g.append()
    oc = oracle_cache(pc)
    # the case does exercise the low term's rounding
    kd, ks, _, _ = oc.token_rows(np.arange(oc.num_pages), np.zeros(oc.num_pages, np.int64))
    from oracle import codec
    x = codec.dequantize(kd, ks)
    assert not np.array_equal(a4q.k_bridge(x, codec.e4m3_value(ks))[3], x)
    for q_format in FORMATS:
        _check("wide K blocks", g, _ref(pc, oc, q_format), q_format)


def _gate_cases():
    tiny = W.prefill_case(W.get("tiny"))
    t128 = W.prefill_case(W.get("tail128"))
    t16 = W.prefill_case(W.get("tail16"))
    yield "tiny, causal", tiny, None, True, None
    yield "tail128, causal", t128, None, True, None
    yield "tail128, no mask", t128, None, False, None
    yield "tail128, Q outlier channels x8", t128, W.scale_channels(t128.q_bits, 77, 4, 8.0), True, None
    yield "tail16, every row", t16, None, True, None


def test_a4q_release_gate_cases():
    """Each gate case: the kernel meets the bar against the A4Q scheme; its error against the
    stock oracle (float64 attention with the bf16 query) is reported next to the scheme's own."""
    for name, pc, q_bits, causal, rows in _gate_cases():
        g = GpuPrefillCase(pc)
        g.append()
        oc = oracle_cache(pc)
        stock, _ = oattn.prefill(oc, pc.q_bits if q_bits is None else q_bits, pc.cu_seqlens_q,
                                 pc.kv_lens, pc.layout.block_table, pc.w.sm_scale, causal=causal,
                                 rows=rows, workers=WORKERS)
        q = None if q_bits is None else dev_bf16(q_bits)
        for q_format in FORMATS:
            for k_terms in (2, 1):
                ref = _ref(pc, oc, q_format, q_bits=q_bits, causal=causal, rows=rows, k_terms=k_terms)
                o32 = _run(g, q_format, torch.float32, q=q, causal=causal, k_terms=k_terms).cpu().numpy()
                what = f"gate {name} {q_format} k_terms={k_terms}"
                assert_attention_close(o32, ref, f"{what} vs scheme")
                km, kmean = attention_error(o32, stock)
                sm, smean = attention_error(ref, stock)
                say(f"  {what}: kernel vs stock max {km:.3e} mean {kmean:.3e}; "
                    f"scheme vs stock max {sm:.3e} mean {smean:.3e}")
