"""Pins of the oracle's paged attention (CPU only): brute force, a library special
case, closed forms and invariances."""
import math

import numpy as np
import pytest
import torch

import workload as W
from oracle import attention, cache, codec
import pins


def _case(q_lens, kv_lens, hq, hkv, seed, k_out=0):
    w = W.custom("t", q_lens, kv_lens, hq, hkv, seed, k_outlier_channels=k_out)
    pc = W.prefill_case(w)
    c = cache.PagedCache(pc.layout.num_pages, hkv)
    c.append(pc.k_bits, pc.v_bits, pc.slot_mapping)
    return w, pc, c


def test_bruteforce_tiny_ragged():
    pins.check_attention_bruteforce(codec, cache, attention)


def test_bruteforce_head_dim_128():
    pins.check_attention_bruteforce(codec, cache, attention, seed=11, head_dim=128)


def test_gather_follows_page_table():
    w, pc, c = _case([5, 40], [37, 40], 4, 2, 2001)
    for b in range(2):
        kh, vh = c.gather(pc.layout.block_table[b], pc.kv_lens[b])
        s0, s1 = pc.cu_seqlens_kv[b], pc.cu_seqlens_kv[b + 1]
        kc, ks = codec.quantize(codec.bf16_to_f32(pc.k_bits[s0:s1]))
        vc, vs = codec.quantize(codec.bf16_to_f32(pc.v_bits[s0:s1]))
        assert np.array_equal(kh, codec.dequantize(codec.pack(kc), ks))
        assert np.array_equal(vh, codec.dequantize(codec.pack(vc), vs))


def test_matches_torch_sdpa_float64():
    w, pc, c = _case([7, 64], [30, 64], 8, 2, 2002, k_out=3)
    o, lse = attention.prefill(c, pc.q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table,
                               w.sm_scale)
    for b in range(2):
        q0, q1 = pc.cu_seqlens_q[b], pc.cu_seqlens_q[b + 1]
        kh, vh = c.gather(pc.layout.block_table[b], pc.kv_lens[b])
        q = torch.from_numpy(codec.bf16_to_f32(pc.q_bits[q0:q1]).astype(np.float64)).transpose(0, 1)
        k = torch.from_numpy(np.repeat(kh, 4, axis=1)).transpose(0, 1)
        v = torch.from_numpy(np.repeat(vh, 4, axis=1)).transpose(0, 1)
        ql, kl = q1 - q0, pc.kv_lens[b]
        mask = torch.from_numpy(np.arange(kl)[None, :] <= (kl - ql + np.arange(ql))[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask,
                                                               scale=w.sm_scale)
        np.testing.assert_allclose(o[q0:q1], ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)


def test_causal_rows_ignore_future_tokens():
    w, pc, c = _case([48], [48], 4, 1, 2003)
    o, _ = attention.prefill(c, pc.q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table,
                             w.sm_scale)
    i = 20
    k2, v2 = pc.k_bits.copy(), pc.v_bits.copy()
    rng = np.random.default_rng(0)
    k2[i + 1:] = rng.integers(0, 0x3F80, size=k2[i + 1:].shape)
    v2[i + 1:] = rng.integers(0, 0x3F80, size=v2[i + 1:].shape)
    c2 = cache.PagedCache(pc.layout.num_pages, 1)
    c2.append(k2, v2, pc.slot_mapping)
    o2, _ = attention.prefill(c2, pc.q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table,
                              w.sm_scale)
    assert np.array_equal(o[: i + 1], o2[: i + 1])
    assert not np.array_equal(o[i + 1:], o2[i + 1:])


def test_prefix_consistency_and_decode_is_last_row():
    w, pc, c = _case([40], [40], 4, 1, 2004)
    o, lse = attention.prefill(c, pc.q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table,
                               w.sm_scale)
    n = 23
    o_n, _ = attention.prefill(c, pc.q_bits[:n], np.array([0, n]), [n], pc.layout.block_table,
                               w.sm_scale)
    np.testing.assert_allclose(o_n, o[:n], rtol=0, atol=1e-13)
    od, ld = attention.decode(c, pc.q_bits[n - 1:n], [n], pc.layout.block_table, w.sm_scale)
    np.testing.assert_allclose(od[0], o[n - 1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(ld[0], lse[n - 1], rtol=0, atol=1e-13)


def test_zero_query_gives_window_mean():
    w, pc, c = _case([16], [50], 4, 2, 2005)
    q0 = np.zeros_like(pc.q_bits)
    o, lse = attention.prefill(c, q0, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table, w.sm_scale)
    _, vh = c.gather(pc.layout.block_table[0], 50)
    for i in range(16):
        for h in range(4):
            np.testing.assert_allclose(o[i, h], vh[: 50 - 16 + i + 1, h // 2].mean(axis=0),
                                       rtol=0, atol=1e-14)
            assert abs(lse[i, h] - math.log(50 - 16 + i + 1)) < 1e-14


def test_peaked_query_selects_one_value():
    w, pc, c = _case([1], [33], 1, 1, 2006)
    kh, vh = c.gather(pc.layout.block_table[0], 33)
    j = 17
    q = np.zeros((1, 1, 128), np.float32)
    q[0, 0] = 64.0 * np.sign(kh[j, 0])  # exact bf16 values; <q, k_j> dominates every other key
    qb = (q.view(np.uint32) >> 16).astype(np.uint16)
    o, _ = attention.decode(c, qb, [33], pc.layout.block_table, 1.0)
    np.testing.assert_allclose(o[0, 0], vh[j, 0], rtol=0, atol=1e-9)


def test_gqa_equals_replicated_heads():
    w, pc, c = _case([12], [45], 8, 2, 2007)
    o, _ = attention.prefill(c, pc.q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table,
                             w.sm_scale)
    rep = cache.PagedCache(pc.layout.num_pages, 8)
    rep.append(np.repeat(pc.k_bits, 4, axis=1), np.repeat(pc.v_bits, 4, axis=1), pc.slot_mapping)
    o2, _ = attention.prefill(rep, pc.q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table,
                              w.sm_scale)
    assert np.array_equal(o, o2)


def test_page_permutation_invariance():
    w, pc, c = _case([9, 33], [70, 33], 4, 1, 2008)
    o, _ = attention.prefill(c, pc.q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table,
                             w.sm_scale)
    perm = np.random.default_rng(1).permutation(pc.layout.num_pages).astype(np.int32)
    bt2 = perm[pc.layout.block_table]
    slots2 = perm[pc.slot_mapping // 16].astype(np.int64) * 16 + pc.slot_mapping % 16
    c2 = cache.PagedCache(pc.layout.num_pages, 1)
    c2.append(pc.k_bits, pc.v_bits, slots2)
    o2, _ = attention.prefill(c2, pc.q_bits, pc.cu_seqlens_q, pc.kv_lens, bt2, w.sm_scale)
    assert np.array_equal(o, o2)


def test_negative_slots_are_skipped():
    w, pc, c = _case([4], [20], 4, 1, 2009)
    slots = pc.slot_mapping.copy(); slots[3] = -1
    c2 = cache.PagedCache(pc.layout.num_pages, 1)
    c2.append(pc.k_bits, pc.v_bits, slots)
    p, off = pc.slot_mapping[3] // 16, pc.slot_mapping[3] % 16
    assert np.all(c2.k_data[p, :, off] == 0) and np.all(c2.k_scale[p, :, off] == 0)
    assert np.array_equal(np.delete(c2.k_data.reshape(-1, 1, 64), pc.slot_mapping[3], axis=0),
                          np.delete(c.k_data.reshape(-1, 1, 64), pc.slot_mapping[3], axis=0))


# --- planted mistakes -----------------------------------------------------------------------

def test_pins_catch_top_left_causal_alignment(monkeypatch):
    real = attention.attend

    def shifted(q, k, v, last, sm):
        return real(q, k, v, np.asarray(last) - (np.asarray(last) - np.arange(len(last))).min(), sm)
    monkeypatch.setattr(attention, "attend", shifted)
    with pytest.raises(AssertionError):
        pins.check_attention_bruteforce(codec, cache, attention)


def test_pins_catch_missing_softmax_scale(monkeypatch):
    real = attention.attend
    monkeypatch.setattr(attention, "attend", lambda q, k, v, last, sm: real(q, k, v, last, 1.0))
    with pytest.raises(AssertionError):
        pins.check_attention_bruteforce(codec, cache, attention)


def test_pins_catch_wrong_gqa_head_map(monkeypatch):
    real_prefill = attention.prefill

    def bad(c, qb, *a, **kw):
        # query head h reads kv head h % Hkv instead of h // G
        qb2 = qb.copy()
        hq = qb.shape[1]
        g = hq // c.num_kv_heads
        order = [(h % c.num_kv_heads) * g + h // c.num_kv_heads for h in range(hq)]
        o, l = real_prefill(c, qb2[:, order], *a, **kw)
        inv = np.argsort(order)
        return o[:, inv], l[:, inv]
    monkeypatch.setattr(attention, "prefill", bad)
    with pytest.raises(AssertionError):
        pins.check_attention_bruteforce(codec, cache, attention)
