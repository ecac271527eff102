"""Caches larger than 4 GiB per plane: every entry point addresses pages near the top of a
600,000-page pool, where byte offsets exceed 32 bits.

The tokens of a small ragged batch are placed on pages N-1, N-4, N-7, ... of the large cache.
Each result is compared with the oracle, which holds the same tokens on a compact pool (its
arithmetic does not depend on page ids), and with the same call on a compact GPU cache, which
must give the same bits: the kernels' arithmetic does not depend on where a page lives.
"""
import numpy as np
import pytest
import torch

import attention_nvfp4_quantized_amd as A
import workload as W
from gpu_cases import assert_attention_close, dev, dev_bf16, oracle_cache, oracle_prefill, say
from oracle import attention as oattn

pytestmark = pytest.mark.gpu

BIG_PAGES = 600_000


def _case():
    return W.prefill_case(W.custom("large", [64, 200, 17], [1000, 3000, 17], 32, 8, seed=9100,
                                   k_outlier_channels=8))


def _remap(pages: np.ndarray) -> np.ndarray:
    return BIG_PAGES - 1 - 3 * np.asarray(pages, dtype=np.int64)


class _Placed:
    """The case's inputs with its pages moved to the top of the large pool."""

    def __init__(self, pc):
        lay = pc.layout
        assert 3 * lay.num_pages < BIG_PAGES
        self.bt_small = dev(lay.block_table)
        self.bt_big = dev(_remap(lay.block_table).astype(np.int32))
        self.slots_small = dev(pc.slot_mapping)
        big_slots = _remap(pc.slot_mapping // 16) * 16 + pc.slot_mapping % 16
        self.slots_big = dev(big_slots.astype(np.int64))
        self.used_small = np.unique(pc.slot_mapping // 16)
        self.used_big = _remap(self.used_small)
        self.k, self.v = dev_bf16(pc.k_bits), dev_bf16(pc.v_bits)
        self.q = dev_bf16(pc.q_bits)
        self.cu, self.kv = dev(pc.cu_seqlens_q), dev(pc.kv_lens)


def _planes_at(cache, pages):
    idx = torch.from_numpy(np.asarray(pages, dtype=np.int64)).to(cache.k_data.device)
    return [t.index_select(0, idx).cpu().numpy() for t in
            (cache.k_data, cache.k_scale, cache.v_data, cache.v_scale) if t is not None]


@pytest.mark.parametrize("kv_format", ["nvfp4", "fp8"])
def test_large_cache_append_prefill_decode_dequant(kv_format):
    pc = _case()
    w = pc.w
    say(f"[large cache] {kv_format}: {BIG_PAGES} pages x {w.num_kv_heads} heads, q {w.q_lens} "
        f"kv {w.kv_lens}")
    s = _Placed(pc)
    big = A.NVFP4KVCache(BIG_PAGES, w.num_kv_heads, kv_format=kv_format)
    small = A.NVFP4KVCache(pc.layout.num_pages, w.num_kv_heads, kv_format=kv_format)
    assert big.k_data.numel() > 2 ** 32
    A.append(big, s.k, s.v, s.slots_big)
    A.append(small, s.k, s.v, s.slots_small)
    torch.cuda.synchronize()

    oc = oracle_cache(pc, kv_format=kv_format)
    got = _planes_at(big, s.used_big)
    names = ("k_data", "v_data") if kv_format == "fp8" else ("k_data", "k_scale", "v_data", "v_scale")
    for name, g in zip(names, got):
        o = getattr(oc, name)[s.used_small]
        bad = np.argwhere(g != o)
        assert len(bad) == 0, f"{name}: {len(bad)} bytes differ at the top of the pool"

    for splits in (0, 3):
        o_big = A.prefill(big, s.q, s.cu, s.kv, s.bt_big, pc.max_q_len, pc.max_kv_len, w.sm_scale,
                          out_dtype=torch.float32, num_splits=splits)
        o_small = A.prefill(small, s.q, s.cu, s.kv, s.bt_small, pc.max_q_len, pc.max_kv_len,
                            w.sm_scale, out_dtype=torch.float32, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o_big, o_small), f"prefill, splits {splits}: large pool differs"
    ref, _ = oracle_prefill(pc, oc)
    assert_attention_close(o_big.cpu().numpy(), ref, f"prefill {kv_format} at the top of the pool")

    # decode: the last query row of each sequence over all of its keys
    last = pc.cu_seqlens_q[1:] - 1
    qd = s.q[torch.from_numpy(last.astype(np.int64)).cuda()].contiguous()
    d_big = A.decode(big, qd, s.kv, s.bt_big, pc.max_kv_len, w.sm_scale, out_dtype=torch.float32)
    d_small = A.decode(small, qd, s.kv, s.bt_small, pc.max_kv_len, w.sm_scale,
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(d_big, d_small), "decode: large pool differs"
    dref, _ = oattn.decode(oc, pc.q_bits[last], pc.kv_lens, pc.layout.block_table, w.sm_scale)
    assert_attention_close(d_big.cpu().numpy(), dref, f"decode {kv_format} at the top of the pool")

    # standalone dequantization of every appended slot
    kd, vd = A.dequant(big, s.slots_big, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rk, rv = oc.dequant_slots(pc.slot_mapping, "f32")
    assert np.array_equal(kd.cpu().numpy().view(np.uint32), np.asarray(rk, np.float32).view(np.uint32))
    assert np.array_equal(vd.cpu().numpy().view(np.uint32), np.asarray(rv, np.float32).view(np.uint32))
    del big, small
    torch.cuda.empty_cache()


def test_large_cache_repack_and_prefill_over_copy():
    """The fp16 copy of a 600,000-page pool (19.7 GB per plane): the repacked pages at the top
    of the pool are the oracle's bytes and the prefill over them equals the stock prefill."""
    pc = _case()
    w = pc.w
    say(f"[large cache] repack: {BIG_PAGES} pages x {w.num_kv_heads} heads")
    s = _Placed(pc)
    big = A.NVFP4KVCache(BIG_PAGES, w.num_kv_heads)
    A.append(big, s.k, s.v, s.slots_big)
    copy = A.NVFP4KVCache(BIG_PAGES, w.num_kv_heads, kv_format="f16")
    assert copy.k_data.numel() > 2 ** 34
    A.repack(big, copy, s.bt_big, s.kv, pc.max_kv_len)
    torch.cuda.synchronize()
    oc = oracle_cache(pc)
    rk, rv = oc.repack(pc.layout.block_table, pc.kv_lens)
    got = _planes_at(copy, s.used_big)
    for name, g, o in (("k", got[0], rk), ("v", got[1], rv)):
        g16 = np.ascontiguousarray(g).view(np.uint16)
        bad = np.argwhere(g16 != o[s.used_small])
        assert len(bad) == 0, f"repacked {name}: {len(bad)} values differ at the top of the pool"
    o_copy = A.prefill(copy, s.q, s.cu, s.kv, s.bt_big, pc.max_q_len, pc.max_kv_len, w.sm_scale,
                       out_dtype=torch.float32)
    o_stock = A.prefill(big, s.q, s.cu, s.kv, s.bt_big, pc.max_q_len, pc.max_kv_len, w.sm_scale,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o_copy, o_stock), "prefill over the large fp16 copy differs from the stock"
    del big, copy
    torch.cuda.empty_cache()
