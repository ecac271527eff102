"""GPU edge cases and invariances of the HIP path (each against the oracle or an exact property)."""
import numpy as np
import pytest
import torch

import attention_nvfp4_quantized_amd as A
import workload as W
from oracle import attention as oattn
from oracle import cache as ocache
from oracle import codec as ocodec
from gpu_cases import (DEV, LSE_ATOL, GpuPrefillCase, assert_attention_close, assert_cache_equal, dev, dev_bf16,
                       oracle_cache, oracle_prefill, say)

pytestmark = pytest.mark.gpu


def _case(q_lens, kv_lens, hq=32, hkv=8, seed=3001, k_out=0, **kw):
    w = W.custom("case", q_lens, kv_lens, hq, hkv, seed, k_outlier_channels=k_out, **kw)
    return W.prefill_case(w)


def _exhaustive_blocks(values: np.ndarray) -> np.ndarray:
    """Blocks holding every finite value under every nonzero E4M3 scale (amax = 6 s places the
    scale exactly), every positive amax, and the special cases."""
    blocks = []
    for c in range(1, 127):
        s = float(ocodec.e4m3_value(c))
        amax = np.float32(6.0 * s)
        pool = values[np.abs(values) <= amax]
        n = (len(pool) + 14) // 15
        blk = np.zeros((n, 16), np.float32)
        flat = np.zeros(n * 15, np.float32); flat[: len(pool)] = pool
        blk[:, 1:] = flat.reshape(n, 15)
        blk[:, 0] = amax
        blocks.append(blk)
    amaxes = values[values > 0]
    one = np.zeros((len(amaxes), 16), np.float32); one[:, 7] = amaxes; one[:, 8] = -amaxes / 3
    blocks.append(one)
    special = np.zeros((4, 16), np.float32)
    special[1] = -0.0
    special[2, ::2] = 2.0 ** -20
    special[3] = np.float32(6.375); special[3, 1::2] = -5.0
    blocks.append(special)
    x = np.concatenate(blocks)
    pad = (-len(x)) % 8
    return np.concatenate([x, np.zeros((pad, 16), np.float32)])


@pytest.mark.parametrize("input_dtype", ["bf16", "fp16"])
def test_codec_exhaustive_through_append(input_dtype):
    say(f"[codec] every finite {input_dtype} value under every E4M3 scale, and every {input_dtype} amax")
    if input_dtype == "bf16":
        vals = W.bf16_bits_to_f32(np.arange(65536, dtype=np.uint16))
    else:
        vals = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float32)
    x = _exhaustive_blocks(vals[np.isfinite(vals)])
    if input_dtype == "bf16":
        bits = W.f32_to_bf16_bits(x).reshape(-1, 1, 128)  # both sides read these bit patterns
        to_dev = dev_bf16
    else:
        bits = x.astype(np.float16).view(np.uint16).reshape(-1, 1, 128)  # both sides read these bit patterns
        to_dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(DEV).view(torch.float16)
    t = bits.shape[0]
    pages = (t + 15) // 16
    slots = np.random.default_rng(0).permutation(pages * 16)[:t].astype(np.int64)
    cache = A.NVFP4KVCache(pages, 1)
    A.append(cache, to_dev(bits), to_dev(bits[::-1].copy()), dev(slots))
    torch.cuda.synchronize()
    oc = ocache.PagedCache(pages, 1)
    oc.append(bits, bits[::-1].copy(), slots, input_dtype=input_dtype)
    got = [t_.cpu().numpy() for t_ in (cache.k_data, cache.k_scale, cache.v_data, cache.v_scale)]
    say(f"  {x.size} values in {t} tokens")
    assert_cache_equal(got, oc)


@pytest.mark.parametrize("gk,gv", [(1.0, 1.0), (1.5, 0.75)])
def test_dequant_bit_exact(gk, gv):
    say(f"[dequant] bf16 / fp16 / f32 rows of random slots, k_global {gk}, v_global {gv}")
    pc = _case([70, 41], [70, 41], 8, 4, 3010, k_out=4)
    g = GpuPrefillCase(pc, k_global=gk, v_global=gv)
    g.append()
    oc = oracle_cache(pc, k_global=gk, v_global=gv)
    rng = np.random.default_rng(3)
    slots = rng.permutation(pc.slot_mapping)[:97].copy()
    slots[[0, 50, 96]] = -1
    for name, dt in (("bf16", torch.bfloat16), ("fp16", torch.float16), ("f32", torch.float32)):
        k, v = A.dequant(g.cache, dev(slots), out_dtype=dt)
        torch.cuda.synchronize()
        ok, ov = oc.dequant_slots(slots, name)
        for got, exp, what in ((k, ok, "k"), (v, ov, "v")):
            gh = got.cpu().view(torch.int16).numpy().view(np.uint16) if name != "f32" else got.cpu().numpy()
            if name == "f32":
                assert np.array_equal(gh.view(np.uint32), np.asarray(exp, np.float32).view(np.uint32)), (name, what)
            else:
                bad = np.argwhere(gh != exp)
                assert len(bad) == 0, f"{name} {what}: {len(bad)} differ, first {bad[0].tolist()}"


def test_append_global_scales_and_skipped_slots():
    say("[append] k_global 1.5, v_global 0.75, some slots < 0")
    pc = _case([5, 9], [70, 37], 8, 2, 3002, k_out=4)
    slots = pc.slot_mapping.copy()
    slots[[3, 40, 71]] = -1
    pc.slot_mapping = slots
    g = GpuPrefillCase(pc, k_global=1.5, v_global=0.75)
    g.append()
    torch.cuda.synchronize()
    oc = ocache.PagedCache(pc.layout.num_pages, 2, k_global=1.5, v_global=0.75)
    oc.append(pc.k_bits, pc.v_bits, slots)
    assert_cache_equal(g.cache_host(), oc)


def test_prefill_global_scales():
    say("[prefill] k_global 1.5, v_global 0.75")
    pc = _case([64, 33], [64, 200], 16, 4, 3003)
    g = GpuPrefillCase(pc, k_global=1.5, v_global=0.75)
    g.append()
    o = g.prefill(torch.float32).cpu().numpy()
    ref, _ = oracle_prefill(pc, oracle_cache(pc, k_global=1.5, v_global=0.75))
    assert_attention_close(o, ref, "global scales")


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_ragged_batch(causal):
    say(f"[prefill] ragged batch causal={causal}")
    pc = _case([1, 17, 100, 1, 64], [1, 50, 300, 777, 64], seed=3004, k_out=10)
    g = GpuPrefillCase(pc)
    g.append()
    o, lse = g.prefill(torch.float32, causal=causal, return_lse=True)
    ref, ref_lse = oracle_prefill(pc, oracle_cache(pc), causal=causal)
    assert_attention_close(o.cpu().numpy(), ref, f"ragged causal={causal}")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=0, atol=LSE_ATOL)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (16, 2), (16, 1), (64, 2)])
def test_prefill_group_sizes(hq, hkv):
    say(f"[prefill] Hq={hq} Hkv={hkv}")
    pc = _case([40, 130], [90, 130], hq, hkv, 3005 + hq + hkv)
    g = GpuPrefillCase(pc)
    g.append()
    o = g.prefill(torch.float32).cpu().numpy()
    ref, _ = oracle_prefill(pc, oracle_cache(pc))
    assert_attention_close(o, ref, f"G={hq // hkv}")


@pytest.mark.parametrize("kv_format", ["nvfp4", "fp8"])
@pytest.mark.parametrize("q_max", [4, 5, 8, 9, 16, 17, 32, 33, 64, 65])
def test_prefill_kernel_boundaries(q_max, kv_format):
    """Query tiles on each side of the kernel choices at group size 4 (32 / 8 heads): up to 16
    columns (4 rows) the short-query kernel with one 16-column block, up to 32 with two, up to 64
    (16 rows) its four-wavefront shared-conversion form, 65-128 the four-wave tile kernel, above
    128 the 8-wave kernel; the longest sequence decides, the shorter one rides along."""
    say(f"[prefill] kernel boundary: max q_len {q_max} ({4 * q_max} columns), {kv_format}")
    pc = _case([q_max, max(1, q_max // 3)], [q_max + 700, q_max // 3 + 90], seed=3020 + q_max, k_out=10)
    g = GpuPrefillCase(pc, kv_format=kv_format)
    g.append()
    o, lse = g.prefill(torch.float32, return_lse=True)
    ref, ref_lse = oracle_prefill(pc, oracle_cache(pc, kv_format=kv_format))
    assert_attention_close(o.cpu().numpy(), ref, f"q_max={q_max} {kv_format}")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=0, atol=LSE_ATOL)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16])
def test_prefill_split_sweep(splits):
    say(f"[prefill] tails, num_splits={splits}")
    pc = _case([16, 7, 33], [3000, 1500, 4000], seed=3010)
    g = GpuPrefillCase(pc)
    g.append()
    o, lse = g.prefill(torch.float32, num_splits=splits, return_lse=True)
    ref, ref_lse = oracle_prefill(pc, oracle_cache(pc))
    assert_attention_close(o.cpu().numpy(), ref, f"splits={splits}")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=0, atol=LSE_ATOL)


def test_page_permutation_is_bitwise_invariant():
    say("[prefill/decode] permuted page pool")
    pc = _case([40, 100], [300, 100], seed=3011)
    g1 = GpuPrefillCase(pc)
    g1.append()
    o1 = g1.prefill(torch.float32).cpu().numpy()
    perm = np.random.default_rng(5).permutation(pc.layout.num_pages).astype(np.int32)
    pc2 = _case([40, 100], [300, 100], seed=3011)
    pc2.layout.block_table = perm[pc.layout.block_table]
    pc2.slot_mapping = perm[pc.slot_mapping // 16].astype(np.int64) * 16 + pc.slot_mapping % 16
    g2 = GpuPrefillCase(pc2)
    g2.append()
    o2 = g2.prefill(torch.float32).cpu().numpy()
    assert np.array_equal(o1, o2)
    q = dev_bf16(pc.q_bits[[39, 139]])
    d1 = A.decode(g1.cache, q, g1.kv, g1.bt, 300, pc.w.sm_scale, out_dtype=torch.float32)
    d2 = A.decode(g2.cache, q, g2.kv, g2.bt, 300, pc.w.sm_scale, out_dtype=torch.float32)
    assert torch.equal(d1, d2)


def test_future_tokens_leave_earlier_rows_bitwise_unchanged():
    say("[prefill] causal: perturb tokens after row 120")
    pc = _case([200], [200], seed=3012)
    g = GpuPrefillCase(pc)
    g.append()
    o1 = g.prefill(torch.float32).cpu().numpy()
    pc2 = _case([200], [200], seed=3012)
    rng = np.random.default_rng(1)
    pc2.k_bits[121:] = W.f32_to_bf16_bits(rng.standard_normal(pc2.k_bits[121:].shape).astype(np.float32))
    pc2.v_bits[121:] = W.f32_to_bf16_bits(rng.standard_normal(pc2.v_bits[121:].shape).astype(np.float32))
    g2 = GpuPrefillCase(pc2)
    g2.append()
    o2 = g2.prefill(torch.float32).cpu().numpy()
    assert np.array_equal(o1[:121], o2[:121])
    assert not np.array_equal(o1[121:], o2[121:])


def test_zero_query_gives_window_mean():
    say("[prefill] Q = 0 closed form")
    pc = _case([48], [300], 8, 2, 3013)
    g = GpuPrefillCase(pc)
    g.append()
    o = g.prefill(torch.float32, q=torch.zeros_like(g.q)).cpu().numpy()
    oc = oracle_cache(pc)
    _, vh = oc.gather(pc.layout.block_table[0], 300)
    ref = np.stack([np.stack([vh[: 300 - 48 + i + 1, h // 4].mean(axis=0) for h in range(8)])
                    for i in range(48)])
    assert_attention_close(o, ref, "window mean")


def test_decode_equals_last_prefill_row():
    say("[decode] decode at kv_len n vs prefill row n-1")
    pc = _case([1000, 77], [1000, 300], seed=3014)
    g = GpuPrefillCase(pc)
    g.append()
    o = g.prefill(torch.float32).cpu().numpy()
    rows = [999, 1000 + 76]
    q = dev_bf16(pc.q_bits[rows])
    kvl = dev(np.array([1000, 300], np.int32))
    d = A.decode(g.cache, q, kvl, g.bt, 1000, pc.w.sm_scale, out_dtype=torch.float32).cpu().numpy()
    assert_attention_close(d, o[rows], "decode vs prefill row", max_abs=2e-3, mean_abs=2e-4)


@pytest.mark.parametrize("hq,hkv,splits", [(32, 8, 0), (32, 8, 1), (32, 8, 5), (8, 8, 3),
                                           (64, 4, 0), (16, 16, 2)])
def test_decode_shapes_and_splits(hq, hkv, splits):
    say(f"[decode] Hq={hq} Hkv={hkv} splits={splits}")
    lens = [1, 15, 16, 17, 100, 1023, 4999, 2048]
    w = W.custom("dec", [1] * len(lens), lens, hq, hkv, 3020 + hq + splits)
    pc = W.prefill_case(w)  # one query per sequence = its last position
    g = GpuPrefillCase(pc)
    g.append()
    o, lse = A.decode(g.cache, g.q, g.kv, g.bt, max(lens), w.sm_scale, out_dtype=torch.float32,
                      return_lse=True, num_splits=splits)
    torch.cuda.synchronize()
    oc = oracle_cache(pc)
    ref, ref_lse = oattn.decode(oc, pc.q_bits, pc.kv_lens, pc.layout.block_table, w.sm_scale)
    assert_attention_close(o.cpu().numpy(), ref, f"decode G={hq // hkv} splits={splits}")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=0, atol=LSE_ATOL)


def test_runs_are_deterministic():
    say("[prefill/decode] repeated runs are bitwise identical")
    pc = _case([16, 16], [5000, 3000], seed=3030)
    g = GpuPrefillCase(pc)
    g.append()
    a = g.prefill(torch.float32)
    b = g.prefill(torch.float32)
    assert torch.equal(a, b)
    q = g.q[[15, 31]].contiguous()
    d1 = A.decode(g.cache, q, g.kv, g.bt, 5000, pc.w.sm_scale)
    d2 = A.decode(g.cache, q, g.kv, g.bt, 5000, pc.w.sm_scale)
    assert torch.equal(d1, d2)


def test_empty_inputs_are_no_ops():
    say("[edge] empty append / prefill / decode")
    cache = A.NVFP4KVCache(2, 8)
    e = torch.empty((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    A.append(cache, e, e, torch.empty(0, dtype=torch.int64, device="cuda"))
    q = torch.empty((0, 32, 128), dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(2, dtype=torch.int32, device="cuda")
    kv = torch.zeros(1, dtype=torch.int32, device="cuda")
    bt = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    out = A.prefill(cache, q, cu, kv, bt, 0, 0, 0.088)
    assert out.shape == (0, 32, 128)
    torch.cuda.synchronize()
    assert int(cache.k_data.abs().sum()) == 0
