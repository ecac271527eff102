"""GPU parity: the HIP path against the oracle on the five seeded workloads.

Cache bytes and scales must be bit-exact; attention output (float32 and bf16) must be within
max-abs 1e-2 and mean-abs 1e-3 of the float64 oracle.  Large workloads run at full size in the
launch configuration the benchmark times, and are checked on sampled rows / sequences.
"""
import numpy as np
import pytest
import torch

import workload as W
from gpu_cases import (LSE_ATOL, DecodeRun, assert_attention_close_bf16, GpuPrefillCase,
                       assert_attention_close, assert_cache_equal, oracle_cache, oracle_prefill,
                       rows_of, say, seq_pages)

pytestmark = pytest.mark.gpu

FULL16K_ROWS = np.array([0, 1, 2, 15, 16, 31, 32, 63, 64, 65, 127, 128, 1000, 4095, 4096, 8191,
                         8192, 12345, 16255, 16256, 16319, 16320, 16382, 16383])


def _bf16_of(x32: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(x32, np.float32).view(np.uint32)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("name", ["tiny", "tail128", "full16k"])
def test_append_bit_exact(name):
    w = W.get(name)
    say(f"[append] {name}")
    pc = W.prefill_case(w)
    g = GpuPrefillCase(pc)
    g.append()
    torch.cuda.synchronize()
    assert_cache_equal(g.cache_host(), oracle_cache(pc))


def test_append_bit_exact_tail16_sampled_sequences():
    w = W.get("tail16")
    say("[append] tail16 (sequences 0 and 5)")
    pc = W.prefill_case(w)
    g = GpuPrefillCase(pc)
    g.append()
    torch.cuda.synchronize()
    seqs = [0, 5]
    pages = np.concatenate([seq_pages(pc.layout, b) for b in seqs])
    assert_cache_equal(g.cache_host(), oracle_cache(pc, seqs), pages=pages)


@pytest.mark.parametrize("name", ["tiny", "tail128"])
def test_prefill_parity_all_rows(name):
    w = W.get(name)
    say(f"[prefill] {name}")
    pc = W.prefill_case(w)
    g = GpuPrefillCase(pc)
    g.append()
    o32, lse = g.prefill(torch.float32, return_lse=True)
    o16 = g.prefill(torch.bfloat16)
    ref, ref_lse = oracle_prefill(pc, oracle_cache(pc))
    o32n = o32.cpu().numpy()
    assert_attention_close(o32n, ref, f"{name} fp32")
    assert_attention_close_bf16(o16.float().cpu().numpy(), ref, f"{name} bf16")
    assert np.array_equal(o16.view(torch.int16).cpu().numpy().view(np.uint16), _bf16_of(o32n))
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=0, atol=LSE_ATOL)


def _full_rows(n):
    """Sampled rows of an n-token full prefill: the first tiles, tile and page edges, the middle
    and the last rows."""
    r = FULL16K_ROWS[FULL16K_ROWS < n // 2]
    return np.unique(np.concatenate([r, [n // 2 - 1, n // 2, n - 65, n - 64, n - 2, n - 1]]))


@pytest.mark.parametrize("name", ["full8k", "full16k", "full32k"])
def test_prefill_parity_full_sampled_rows(name):
    w = W.get(name)
    say(f"[prefill] {name} sampled rows")
    pc = W.prefill_case(w)
    g = GpuPrefillCase(pc)
    g.append()
    o32 = g.prefill(torch.float32).cpu().numpy()
    o16 = g.prefill(torch.bfloat16).float().cpu().numpy()
    rows = FULL16K_ROWS if name == "full16k" else _full_rows(w.kv_lens[0])
    ref, _ = oracle_prefill(pc, oracle_cache(pc), rows=rows)
    assert_attention_close(o32, ref, f"{name} fp32")
    assert_attention_close_bf16(o16, ref, f"{name} bf16")


def test_prefill_parity_tail16_sampled_sequences():
    w = W.get("tail16")
    say("[prefill] tail16 sequences 0, 5")
    pc = W.prefill_case(w)
    g = GpuPrefillCase(pc)
    g.append()
    o32 = g.prefill(torch.float32).cpu().numpy()
    seqs = [0, 5]
    ref, _ = oracle_prefill(pc, oracle_cache(pc, seqs), rows=rows_of(pc, seqs))
    assert_attention_close(o32, ref, "tail16 fp32")


def test_decode_parity_full_size_sampled_sequences():
    w = W.get("decode")
    lens = np.asarray(w.kv_lens)
    sampled = [int(lens.argmin()), int(lens.argmax())]
    say(f"[decode] 64 steps, sampled sequences {sampled} (L = {lens[sampled].tolist()})")
    run = DecodeRun(sampled, check_steps=(0, 63))
    refs = run.oracle((0, 63), sampled)
    for t in (0, 63):
        assert_attention_close(run.out[t], refs[t], f"decode step {t}")
