"""GPU parity: the HIP path against the oracle on the five seeded workloads.

Cache bytes and scales must be bit-exact; attention output (float32 and bf16) must be within
max-abs 1e-2 and mean-abs 1e-3 of the float64 oracle.  Every workload runs at full size in the
launch configuration the benchmark times.  Compared in full: the cache bytes of the tiny,
tail128, full16k and tail16 appends, every row of the tiny, tail128, tail16 and full16k
prefills (float32, bf16 and the log-sum-exp), the bytes of all 64 x 64 slots the decode loop
appends, the whole caches and both output types of eight decode sequences spread over the
length range at the first and last step.  The full 8K / 32K prefills are checked on sampled
rows.
"""
import time

import numpy as np
import pytest
import torch

import workload as W
from oracle import attention as oattn
from gpu_cases import (WORKERS, LSE_ATOL, DecodeRun, GpuPrefillCase, assert_attention_close,
                       assert_attention_close_bf16, assert_cache_equal, oracle_cache,
                       oracle_prefill, oracle_rows, say, spread_sequences)

pytestmark = pytest.mark.gpu

FULL16K_ROWS = np.array([0, 1, 2, 15, 16, 31, 32, 63, 64, 65, 127, 128, 1000, 4095, 4096, 8191,
                         8192, 12345, 16255, 16256, 16319, 16320, 16382, 16383])


def _bf16_of(x32: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(x32, np.float32).view(np.uint32)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name", ["tiny", "tail128", "full16k", "tail16"])
def test_append_bit_exact(name):
    w = W.get(name)
    say(f"[append] {name}: every byte of the cache")
    pc = W.prefill_case(w)
    g = GpuPrefillCase(pc)
    g.append()
    torch.cuda.synchronize()
    assert_cache_equal(g.cache_host(), oracle_cache(pc))


@pytest.mark.parametrize("name", ["tiny", "tail128", "tail16"])
def test_prefill_parity_all_rows(name):
    w = W.get(name)
    say(f"[prefill] {name}: every row, float32 / bf16 / log-sum-exp")
    pc = W.prefill_case(w)
    g = GpuPrefillCase(pc)
    g.append()
    o32, lse = g.prefill(torch.float32, return_lse=True)
    o16 = g.prefill(torch.bfloat16)
    ref, ref_lse = oracle_prefill(pc, oracle_cache(pc))
    o32n = o32.cpu().numpy()
    assert_attention_close(o32n, ref, f"{name} fp32")
    assert_attention_close_bf16(o16.float().cpu().numpy(), ref, f"{name} bf16")
    assert np.array_equal(_bits(o16), _bf16_of(o32n))
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=0, atol=LSE_ATOL)


@pytest.fixture(scope="module")
def full16k():
    """The 16K causal prefill on the GPU (float32 with log-sum-exp, and the timed bf16 output)
    and the oracle over every row."""
    w = W.get("full16k")
    say("[prefill] full16k: GPU, then the oracle over all 16,384 rows x 32 heads")
    pc = W.prefill_case(w)
    g = GpuPrefillCase(pc)
    g.append()
    o32, lse = g.prefill(torch.float32, return_lse=True)
    o16 = g.prefill(torch.bfloat16)
    oc = oracle_cache(pc)
    ref = np.full((pc.total_q, w.num_qo_heads, 128), np.nan)
    ref_lse = np.full((pc.total_q, w.num_qo_heads), np.nan)
    t0 = time.perf_counter()
    for hk in range(w.num_kv_heads):  # one KV head's query heads at a time, with progress
        heads = list(range(hk * w.group, (hk + 1) * w.group))
        r, rl = oattn.prefill(oc, pc.q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table,
                              w.sm_scale, heads=heads, workers=WORKERS)
        ref[:, heads], ref_lse[:, heads] = r[:, heads], rl[:, heads]
        say(f"  oracle heads {heads[0]}-{heads[-1]} done ({time.perf_counter() - t0:.0f} s)")
    return dict(o32=o32.cpu().numpy(), lse=lse.cpu().numpy(), o16=_bits(o16), ref=ref,
                ref_lse=ref_lse)


def test_prefill_parity_full16k_every_row_fp32(full16k):
    assert not np.isnan(full16k["ref"]).any()
    assert_attention_close(full16k["o32"], full16k["ref"], "full16k fp32 (all rows)")
    np.testing.assert_allclose(full16k["lse"], full16k["ref_lse"], rtol=0, atol=LSE_ATOL)


def test_prefill_parity_full16k_every_row_bf16(full16k):
    o16 = (full16k["o16"].astype(np.uint32) << 16).view(np.float32)
    assert_attention_close_bf16(o16, full16k["ref"], "full16k bf16 (all rows)")
    assert np.array_equal(full16k["o16"], _bf16_of(full16k["o32"]))


def _full_rows(n):
    """Sampled rows of an n-token full prefill: the first tiles, tile and page edges, the middle
    and the last rows."""
    r = FULL16K_ROWS[FULL16K_ROWS < n // 2]
    return np.unique(np.concatenate([r, [n // 2 - 1, n // 2, n - 65, n - 64, n - 2, n - 1]]))


@pytest.mark.parametrize("name", ["full8k", "full32k"])
def test_prefill_parity_full_sampled_rows(name):
    w = W.get(name)
    say(f"[prefill] {name} sampled rows")
    pc = W.prefill_case(w)
    g = GpuPrefillCase(pc)
    g.append()
    o32 = g.prefill(torch.float32).cpu().numpy()
    o16 = g.prefill(torch.bfloat16).float().cpu().numpy()
    ref, _ = oracle_prefill(pc, oracle_cache(pc), rows=_full_rows(w.kv_lens[0]))
    assert_attention_close(o32, ref, f"{name} fp32")
    assert_attention_close_bf16(o16, ref, f"{name} bf16")


@pytest.fixture(scope="module")
def decode_run():
    w = W.get("decode")
    seqs = spread_sequences(w.kv_lens, 8)
    say(f"[decode] 64 sequences x 64 steps; oracle sequences {seqs} "
        f"(L = {np.asarray(w.kv_lens)[seqs].tolist()})")
    run = DecodeRun(seqs, check_steps=(0, 63))
    oc = run.oracle_cache()
    return run, oc


def test_decode_step_appends_bit_exact(decode_run):
    """Every slot the 64 steps append (one token of each of the 64 sequences per step)."""
    run, oc = decode_run
    exp = oracle_rows(oc, run.step_slots.reshape(-1))
    for name, got, e in zip(("k_data", "k_scale", "v_data", "v_scale"), run.step_rows, exp):
        bad = np.argwhere(got != e)
        assert len(bad) == 0, f"{name}: {len(bad)} bytes differ, first at {bad[0].tolist()}"


def test_decode_sequence_caches_bit_exact(decode_run):
    """The whole cache pages of the eight oracle sequences (their initial fill and their steps)."""
    run, oc = decode_run
    names = ("k_data", "k_scale", "v_data", "v_scale")
    for name, got in zip(names, run.seq_pages):
        e = getattr(oc, name)[run.oracle_pages]
        bad = np.argwhere(got != e)
        assert len(bad) == 0, f"{name}: {len(bad)} bytes differ, first at {bad[0].tolist()}"


def test_decode_parity_first_and_last_step(decode_run):
    run, oc = decode_run
    refs = run.oracle(oc, (0, 63))
    for t in (0, 63):
        assert_attention_close(run.out[t], refs[t], f"decode step {t} fp32")
        assert_attention_close_bf16(run.out_bf16[t], refs[t], f"decode step {t} bf16")
        got16 = run.out_bf16[t].astype(np.float32).view(np.uint32) >> 16
        assert np.array_equal(got16.astype(np.uint16), _bf16_of(run.out[t]))
