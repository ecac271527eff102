"""Seeded randomized GPU parity: many small prefill, A4Q-style prefill and decode problems with
random ragged lengths, group sizes, KV head counts, cache formats, query formats, K forms, masks,
key splits and output types, each against the oracle (cache bytes bit-exact; outputs within
max-abs 1e-2 / mean-abs 1e-3).

Every case prints its parameters before it runs, so a failure names its configuration."""
import numpy as np
import pytest
import torch

import attention_nvfp4_quantized_amd as A
import workload as W
from gpu_cases import (GpuPrefillCase, assert_attention_close, assert_attention_close_bf16,
                       assert_cache_equal, oracle_cache, oracle_prefill, say)
from oracle import a4q
from oracle import attention as oattn

pytestmark = pytest.mark.gpu

N_PREFILL = 64
N_DECODE = 32
N_A4Q = 24


def _prefill_config(i):
    rng = np.random.default_rng(5000 + i)
    batch = int(rng.integers(1, 5))
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 8, 16]))
    causal = bool(rng.integers(0, 4) > 0)
    q_lens = [int(x) for x in rng.integers(1, 200, size=batch)]
    kv_lens = [q + int(rng.integers(0, 700)) for q in q_lens]
    fmt = str(rng.choice(["nvfp4", "nvfp4", "fp8", "f16"]))
    splits = int(rng.choice([0, 0, 2, 5]))
    out = str(rng.choice(["f32", "bf16"]))
    return dict(batch=batch, hkv=hkv, hq=hkv * group, causal=causal, q_lens=q_lens,
                kv_lens=kv_lens, fmt=fmt, splits=splits, out=out, seed=6000 + i)


@pytest.mark.parametrize("i", range(N_PREFILL))
def test_prefill_random_configuration(i):
    c = _prefill_config(i)
    say(f"[fuzz prefill {i}] {c}")
    pc = W.prefill_case(W.custom("fuzz", c["q_lens"], c["kv_lens"], c["hq"], c["hkv"], c["seed"],
                                 k_outlier_channels=min(4, 128 * c["hkv"] // 8)))
    store = "fp8" if c["fmt"] == "fp8" else "nvfp4"
    g = GpuPrefillCase(pc, kv_format=store)
    g.append()
    torch.cuda.synchronize()
    oc = oracle_cache(pc, kv_format=store)
    assert_cache_equal(g.cache_host(), oc)
    cache = g.cache
    if c["fmt"] == "f16":
        cache = A.NVFP4KVCache(g.cache.num_pages, g.cache.num_kv_heads, kv_format="f16")
        A.repack(g.cache, cache, g.bt, g.kv, pc.max_kv_len)
    dt = torch.float32 if c["out"] == "f32" else torch.bfloat16
    o = A.prefill(cache, g.q, g.cu, g.kv, g.bt, pc.max_q_len, pc.max_kv_len, pc.w.sm_scale,
                  causal=c["causal"], out_dtype=dt, num_splits=c["splits"])
    torch.cuda.synchronize()
    ref, _ = oracle_prefill(pc, oc, causal=c["causal"])
    check = assert_attention_close if dt == torch.float32 else assert_attention_close_bf16
    check(o.float().cpu().numpy(), ref, f"fuzz {i}")


def _a4q_config(i):
    rng = np.random.default_rng(9000 + i)
    batch = int(rng.integers(1, 5))
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 8, 16]))
    q_lens = [int(x) for x in rng.integers(1, 160, size=batch)]
    kv_lens = [q + int(rng.integers(0, 600)) for q in q_lens]
    return dict(batch=batch, hkv=hkv, hq=hkv * group, causal=bool(rng.integers(0, 4) > 0),
                q_lens=q_lens, kv_lens=kv_lens, q_format=str(rng.choice(["mxfp8", "mxfp4"])),
                k_terms=int(rng.choice([1, 2])), splits=int(rng.choice([0, 0, 2, 5])),
                out=str(rng.choice(["f32", "bf16"])), seed=9500 + i)


@pytest.mark.parametrize("i", range(N_A4Q))
def test_a4q_prefill_random_configuration(i):
    """The A4Q-style prefill (NVFP4 cache) against the oracle's scheme of the same query format
    and K form."""
    c = _a4q_config(i)
    say(f"[fuzz a4q {i}] {c}")
    pc = W.prefill_case(W.custom("fuzza4q", c["q_lens"], c["kv_lens"], c["hq"], c["hkv"], c["seed"],
                                 k_outlier_channels=min(4, 128 * c["hkv"] // 8)))
    g = GpuPrefillCase(pc)
    g.append()
    oc = oracle_cache(pc)
    dt = torch.float32 if c["out"] == "f32" else torch.bfloat16
    o = A.prefill_a4q(g.cache, g.q, g.cu, g.kv, g.bt, pc.max_q_len, pc.max_kv_len, pc.w.sm_scale,
                      q_format=c["q_format"], causal=c["causal"], out_dtype=dt,
                      num_splits=c["splits"], k_terms=c["k_terms"])
    torch.cuda.synchronize()
    ref = a4q.prefill_mx(oc, pc.q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table,
                         pc.w.sm_scale, c["q_format"], causal=c["causal"], k_terms=c["k_terms"])
    check = assert_attention_close if dt == torch.float32 else assert_attention_close_bf16
    check(o.float().cpu().numpy(), ref, f"fuzz a4q {i}")


def _decode_config(i):
    rng = np.random.default_rng(7000 + i)
    batch = int(rng.integers(1, 9))
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 8, 16]))
    lens = [int(x) for x in rng.integers(1, 3000, size=batch)]
    fmt = str(rng.choice(["nvfp4", "fp8"]))
    splits = int(rng.choice([0, 0, 1, 3, 7]))
    return dict(batch=batch, hkv=hkv, hq=hkv * group, lens=lens, fmt=fmt, splits=splits,
                seed=8000 + i)


@pytest.mark.parametrize("i", range(N_DECODE))
def test_decode_random_configuration(i):
    """Decode over a cache filled by one append per sequence: the query of sequence b sees all
    of its kv_len keys."""
    c = _decode_config(i)
    say(f"[fuzz decode {i}] {c}")
    lens = c["lens"]
    pc = W.prefill_case(W.custom("fuzzdec", [1] * c["batch"], lens, c["hq"], c["hkv"], c["seed"]))
    g = GpuPrefillCase(pc, kv_format=c["fmt"])
    g.append()
    q = g.q  # one query row per sequence: [batch][Hq][128]
    o = A.decode(g.cache, q, g.kv, g.bt, max(lens), pc.w.sm_scale, out_dtype=torch.float32,
                 num_splits=c["splits"])
    torch.cuda.synchronize()
    oc = oracle_cache(pc, kv_format=c["fmt"])
    ref, _ = oattn.decode(oc, pc.q_bits, pc.kv_lens, pc.layout.block_table, pc.w.sm_scale)
    assert_attention_close(o.cpu().numpy(), ref, f"fuzz decode {i}")
