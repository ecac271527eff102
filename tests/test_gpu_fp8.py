"""GPU parity of the FP8 (E4M3FN) control cache: the same append, prefill and decode entry points
over a descriptor with kv_format = FP8, against the oracle's FP8 cache.

Cache bytes are bit-exact; attention outputs meet the same max-abs 1e-2 / mean-abs 1e-3 bar as
the NVFP4 path (float32 output; bf16 beyond its rounding floor)."""
import numpy as np
import pytest
import torch

import attention_nvfp4_quantized_amd as A
import workload as W
from oracle import fp8cache as ofp8
from gpu_cases import (DEV, LSE_ATOL, DecodeRun, GpuPrefillCase, assert_attention_close,
                       assert_attention_close_bf16, assert_cache_equal, cache_planes, dev,
                       dev_bf16, oracle_cache, oracle_prefill, oracle_rows, say, spread_sequences)

pytestmark = pytest.mark.gpu

FULL16K_ROWS = np.array([0, 1, 63, 64, 4095, 4096, 8191, 8192, 16319, 16320, 16383])


def _dev16(bits, input_dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)
    return t.view(torch.bfloat16 if input_dtype == "bf16" else torch.float16)


@pytest.mark.parametrize("input_dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("gk,gv", [(1.0, 1.0), (1.5, 0.0625)])
def test_fp8_append_every_input_value(input_dtype, gk, gv):
    """Every 16-bit input pattern that is finite, in K (in order) and V (reversed), under unit
    and non-unit per-tensor scales: covers both signs of zero, subnormals, ties, and
    saturation past 448."""
    say(f"[fp8 append] every finite {input_dtype} value, k_global {gk}, v_global {gv}")
    pats = np.arange(65536, dtype=np.uint16)
    if input_dtype == "bf16":
        fin = np.isfinite(W.bf16_bits_to_f32(pats))
    else:
        fin = np.isfinite(pats.view(np.float16))
    pats = pats[fin]
    pats = np.concatenate([pats, np.zeros((-len(pats)) % 128, np.uint16)])
    bits = pats.reshape(-1, 1, 128)
    t = bits.shape[0]
    pages = (t + 15) // 16
    slots = np.random.default_rng(1).permutation(pages * 16)[:t].astype(np.int64)
    cache = A.NVFP4KVCache(pages, 1, k_global=gk, v_global=gv, kv_format="fp8")
    vb = bits[::-1].copy()
    A.append(cache, _dev16(bits, input_dtype), _dev16(vb, input_dtype), dev(slots))
    torch.cuda.synchronize()
    oc = ofp8.Fp8PagedCache(pages, 1, k_global=gk, v_global=gv)
    oc.append(bits, vb, slots, input_dtype=input_dtype)
    assert_cache_equal(cache_planes(cache), oc)


def _case(q_lens, kv_lens, hq=32, hkv=8, seed=3101, k_out=4, **kw):
    return W.prefill_case(W.custom("case", q_lens, kv_lens, hq, hkv, seed,
                                   k_outlier_channels=k_out, **kw))


@pytest.mark.parametrize("gk,gv", [(1.0, 1.0), (1.5, 0.75)])
def test_fp8_dequant_bit_exact(gk, gv):
    say(f"[fp8 dequant] bf16 / fp16 / f32 rows of random slots, k_global {gk}, v_global {gv}")
    pc = _case([70, 41], [70, 41], 8, 4)
    g = GpuPrefillCase(pc, k_global=gk, v_global=gv, kv_format="fp8")
    g.append()
    oc = oracle_cache(pc, k_global=gk, v_global=gv, kv_format="fp8")
    slots = np.random.default_rng(3).permutation(pc.slot_mapping)[:97].copy()
    slots[[0, 50, 96]] = -1
    for name, dt in (("bf16", torch.bfloat16), ("fp16", torch.float16), ("f32", torch.float32)):
        k, v = A.dequant(g.cache, dev(slots), out_dtype=dt)
        torch.cuda.synchronize()
        ok, ov = oc.dequant_slots(slots, name)
        for got, exp, what in ((k, ok, "k"), (v, ov, "v")):
            if name == "f32":
                gh, exp = got.cpu().numpy().view(np.uint32), np.asarray(exp, np.float32).view(np.uint32)
            else:
                gh = got.cpu().view(torch.int16).numpy().view(np.uint16)
            bad = np.argwhere(gh != exp)
            assert len(bad) == 0, f"{name} {what}: {len(bad)} differ, first {bad[0].tolist()}"


@pytest.mark.parametrize("name", ["tiny", "tail128"])
def test_fp8_prefill_parity_all_rows(name):
    w = W.get(name)
    say(f"[fp8 prefill] {name}")
    pc = W.prefill_case(w)
    g = GpuPrefillCase(pc, kv_format="fp8")
    g.append()
    torch.cuda.synchronize()
    oc = oracle_cache(pc, kv_format="fp8")
    assert_cache_equal(g.cache_host(), oc)
    o32, lse = g.prefill(torch.float32, return_lse=True)
    o16 = g.prefill(torch.bfloat16)
    ref, ref_lse = oracle_prefill(pc, oc)
    assert_attention_close(o32.cpu().numpy(), ref, f"fp8 {name} fp32")
    assert_attention_close_bf16(o16.float().cpu().numpy(), ref, f"fp8 {name} bf16")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=0, atol=LSE_ATOL)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (32, 8), (64, 8)])
def test_fp8_prefill_group_sizes_and_splits(hq, hkv):
    """Every prefill kernel width (query-head groups 1, 2, 4, 8) and a forced key split."""
    say(f"[fp8 prefill] Hq {hq}, Hkv {hkv}, q lens [70, 41], kv lens [70, 300]")
    pc = _case([70, 41], [70, 300], hq, hkv, seed=3102)
    g = GpuPrefillCase(pc, kv_format="fp8")
    g.append()
    ref, _ = oracle_prefill(pc, oracle_cache(pc, kv_format="fp8"))
    for splits in (0, 3):
        o = g.prefill(torch.float32, num_splits=splits).cpu().numpy()
        assert_attention_close(o, ref, f"fp8 Hq {hq} splits {splits}")


def test_fp8_prefill_full16k_sampled_rows():
    w = W.get("full16k")
    say("[fp8 prefill] full16k sampled rows")
    pc = W.prefill_case(w)
    g = GpuPrefillCase(pc, kv_format="fp8")
    g.append()
    o32 = g.prefill(torch.float32).cpu().numpy()
    ref, _ = oracle_prefill(pc, oracle_cache(pc, kv_format="fp8"), rows=FULL16K_ROWS)
    assert_attention_close(o32, ref, "fp8 full16k fp32")


def test_fp8_decode_parity_full_size():
    """The decode workload over the FP8 cache: all 64 sequences with their seeded K/V; the bytes
    of every step-appended slot, and both output types of four sequences spread over the length
    range at the first and last step."""
    w = W.get("decode")
    seqs = spread_sequences(w.kv_lens, 4)
    say(f"[fp8 decode] 64 sequences x 64 steps, oracle sequences {seqs}")
    run = DecodeRun(seqs, check_steps=(0, 63), kv_format="fp8")
    oc = run.oracle_cache()
    for name, got, e in zip(("k_data", "v_data"), run.step_rows, oracle_rows(oc, run.step_slots.reshape(-1))):
        assert np.array_equal(got, e), name
    refs = run.oracle(oc, (0, 63))
    for t in (0, 63):
        assert_attention_close(run.out[t], refs[t], f"fp8 decode step {t} fp32")
        assert_attention_close_bf16(run.out_bf16[t], refs[t], f"fp8 decode step {t} bf16")


def test_fp8_append_skipped_slots_and_global_scales():
    """Tokens with slot < 0 are not written (their rows stay zero), under non-unit scales."""
    say("[fp8 append] k_global 1.5, v_global 0.75, some slots < 0")
    pc = _case([5, 9], [70, 37], 8, 2, seed=3103)
    slots = pc.slot_mapping.copy()
    slots[[3, 40, 71, 106]] = -1
    pc.slot_mapping = slots
    g = GpuPrefillCase(pc, k_global=1.5, v_global=0.75, kv_format="fp8")
    g.append()
    torch.cuda.synchronize()
    assert_cache_equal(g.cache_host(), oracle_cache(pc, k_global=1.5, v_global=0.75, kv_format="fp8"))
