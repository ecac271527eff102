"""Helpers for the GPU tests: upload seeded workloads, run the HIP path through the binding,
and build the matching oracle cache.  Inputs come only from ``workload``; expected values only
from ``oracle``."""
from __future__ import annotations

import concurrent.futures as cf
import os
import sys

import numpy as np
import torch

import attention_nvfp4_quantized_amd as A
import workload as W
from oracle import attention as oattn
from oracle import cache as ocache
from oracle import fp8cache as ofp8

DEV = "cuda"
# host threads for the oracle's token and (sequence, head) maps
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))

# Output tolerance on attention (float32 output): the bar the path is held to.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3
# log-sum-exp: the kernels sum the rounded softmax weights (the same weights the PV product
# uses: fp16 rounded toward zero).  A weight in fp16's normal range (>= 2^-14) loses less than
# 2^-10 of itself; the largest weight of a row is >= 1, so the row sum S is >= 1 and the sum of
# the rounded weights lies within a relative 2^-10 of S, its log within 2^-10 (natural log;
# -ln(1 - 2^-10) < 2^-10 + 2^-20).  Weights below 2^-14 (fp16 subnormal) lose less than 2^-24
# each, absolute, a relative 2^-24 of S per key: at most 1/8 of 2^-10 even if every key of a
# 2,048-key row were that small (a score 14 below the row maximum in base 2), and the rows tested
# here have a few.  Plus float32 rounding of the scores, the maximum and the log: 5e-4.
LSE_ATOL = 2.0 ** -10 + 5e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


class GpuPrefillCase:
    def __init__(self, pc: W.PrefillCase, k_global=1.0, v_global=1.0, kv_format="nvfp4"):
        self.pc, self.w = pc, pc.w
        self.cache = A.NVFP4KVCache(pc.layout.num_pages, pc.w.num_kv_heads, k_global=k_global,
                                    v_global=v_global, kv_format=kv_format)
        self.k, self.v = dev_bf16(pc.k_bits), dev_bf16(pc.v_bits)
        self.slots = dev(pc.slot_mapping)
        self.q = dev_bf16(pc.q_bits)
        self.cu = dev(pc.cu_seqlens_q)
        self.kv = dev(pc.kv_lens)
        self.bt = dev(pc.layout.block_table)

    def append(self):
        A.append(self.cache, self.k, self.v, self.slots)

    def prefill(self, out_dtype=torch.float32, num_splits=0, causal=True, return_lse=False, q=None):
        r = A.prefill(self.cache, self.q if q is None else q, self.cu, self.kv, self.bt,
                      self.pc.max_q_len, self.pc.max_kv_len, self.w.sm_scale, causal=causal,
                      out_dtype=out_dtype, return_lse=return_lse, num_splits=num_splits)
        torch.cuda.synchronize()
        return r

    def cache_host(self):
        return cache_planes(self.cache)


def cache_planes(c: A.NVFP4KVCache):
    """The cache's byte planes on the host, in the order ``assert_cache_equal`` compares."""
    return [t.cpu().numpy() for t in (c.k_data, c.k_scale, c.v_data, c.v_scale) if t is not None]


def oracle_cache(pc: W.PrefillCase, seqs=None, k_global=1.0, v_global=1.0, kv_format="nvfp4"):
    """Oracle cache (NVFP4 or the FP8 control) holding the tokens of the given sequences (all
    by default)."""
    make = ofp8.Fp8PagedCache if kv_format == "fp8" else ocache.PagedCache
    c = make(pc.layout.num_pages, pc.w.num_kv_heads, k_global=k_global, v_global=v_global)
    seqs = range(pc.w.batch) if seqs is None else seqs
    for b in seqs:
        s0, s1 = pc.cu_seqlens_kv[b], pc.cu_seqlens_kv[b + 1]
        c.append(pc.k_bits[s0:s1], pc.v_bits[s0:s1], pc.slot_mapping[s0:s1], workers=WORKERS)
    return c


def seq_pages(layout: W.PageLayout, b: int) -> np.ndarray:
    return layout.block_table[b][: layout.pages_per_seq[b]]


def assert_cache_equal(gpu_planes, oc, pages=None):
    names = ("k_data", "v_data") if isinstance(oc, ofp8.Fp8PagedCache) else (
        "k_data", "k_scale", "v_data", "v_scale")
    assert len(gpu_planes) == len(names)
    for name, g in zip(names, gpu_planes):
        o = getattr(oc, name)
        if pages is not None:
            g, o = g[pages], o[pages]
        bad = np.argwhere(g != o)
        assert len(bad) == 0, f"{name}: {len(bad)} bytes differ, first at {bad[0].tolist()}"


def attention_error(gpu: np.ndarray, ref: np.ndarray):
    m = ~np.isnan(ref)
    d = np.abs(gpu.astype(np.float64)[m] - ref[m])
    return float(d.max(initial=0.0)), float(d.mean()) if d.size else 0.0


def assert_attention_close(gpu: np.ndarray, ref: np.ndarray, what: str, max_abs=MAX_ABS,
                           mean_abs=MEAN_ABS):
    assert np.isfinite(gpu[~np.isnan(ref)]).all(), f"{what}: non-finite output"
    mx, mean = attention_error(gpu, ref)
    say(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e} over {int((~np.isnan(ref)).sum())} values")
    assert mx <= max_abs and mean <= mean_abs, f"{what}: max-abs {mx:.3e}, mean-abs {mean:.3e}"


def _bf16_round(x: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(x, np.float32).view(np.uint32)
    return (((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)


def assert_attention_close_bf16(gpu: np.ndarray, ref: np.ndarray, what: str, max_abs=MAX_ABS,
                                mean_abs=MEAN_ABS):
    """bf16 outputs: a correctly rounded bf16 value sits up to half an ulp from the float64
    value (7.8e-3 for |o| in [2, 4)), so the max-abs bar applies to the error beyond that
    rounding floor |bf16(ref) - ref|; the mean-abs bar applies to the raw error.  The floor is
    reported, never hidden."""
    m = ~np.isnan(ref)
    g, r = gpu.astype(np.float64)[m], ref[m]
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - r)
    floor = np.abs(_bf16_round(r).astype(np.float64) - r)
    beyond = (err - floor).max(initial=0.0)
    say(f"  {what}: max-abs {err.max():.3e} (bf16 floor there {floor[err.argmax()]:.3e}, "
        f"beyond floor {beyond:.3e}) mean-abs {err.mean():.3e}")
    assert beyond <= max_abs and err.mean() <= mean_abs, (
        f"{what}: max-abs beyond the bf16 floor {beyond:.3e}, mean-abs {err.mean():.3e}")


def oracle_prefill(pc: W.PrefillCase, oc: ocache.PagedCache, rows=None, causal=True):
    return oattn.prefill(oc, pc.q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table,
                         pc.w.sm_scale, causal=causal, rows=rows, workers=WORKERS)


def rows_of(pc: W.PrefillCase, seqs) -> np.ndarray:
    return np.concatenate([np.arange(pc.cu_seqlens_q[b], pc.cu_seqlens_q[b + 1]) for b in seqs])


def spread_sequences(lens, n: int) -> list:
    """n sequence indices spread over the range of lengths (sorted-length quantiles)."""
    order = np.argsort(np.asarray(lens), kind="stable")
    return sorted({int(order[i]) for i in np.linspace(0, len(order) - 1, n).round().astype(int)})


class DecodeRun:
    """The decode workload at full size and in the launch configuration the benchmark times:
    64 sequences, each with its seeded K/V, 64 steps of (append one token per sequence, decode
    with bf16 output).  At the checked steps the decode is also run with float32 output.  Keeps
    the step tokens of every sequence and the whole K/V of ``oracle_seqs``; after the loop,
    ``step_rows`` holds the cache rows of every step-appended slot and ``seq_pages`` the cache
    pages of the oracle sequences, read back from the device."""

    def __init__(self, oracle_seqs, check_steps, kv_format="nvfp4"):
        self.w = W.get("decode")
        self.dc = W.decode_case(self.w)
        self.kv_format = kv_format
        self.oracle_seqs = list(oracle_seqs)
        lay, w = self.dc.layout, self.w
        steps = w.decode_steps
        self.cache = A.NVFP4KVCache(lay.num_pages, w.num_kv_heads, kv_format=kv_format)
        self.kv_bits = {}
        self.step_k = np.zeros((steps, w.batch, w.num_kv_heads, w.head_dim), np.uint16)
        self.step_v = np.zeros_like(self.step_k)

        def draw(b):
            return b, self.dc.seq_kv(b)

        with cf.ThreadPoolExecutor(WORKERS) as ex:
            for b0 in range(0, w.batch, WORKERS):  # a pool's worth at a time bounds host memory
                for b, (k, v) in ex.map(draw, range(b0, min(w.batch, b0 + WORKERS))):
                    n = int(self.dc.init_lens[b]) - 1
                    A.append(self.cache, dev_bf16(k[:n]), dev_bf16(v[:n]), dev(lay.slots(b, np.arange(n))))
                    self.step_k[:, b], self.step_v[:, b] = k[n:n + steps], v[n:n + steps]
                    if b in self.oracle_seqs:
                        self.kv_bits[b] = (k, v)
                torch.cuda.synchronize()
        q_all = self.dc.step_q()
        bt = dev(lay.block_table)
        self.out, self.out_bf16 = {}, {}
        max_kv = int(self.dc.init_lens.max()) + steps - 1
        self.step_slots = np.stack([self.dc.step_slots(t) for t in range(steps)])
        for t in range(steps):
            A.append(self.cache, dev_bf16(self.step_k[t]), dev_bf16(self.step_v[t]),
                     dev(self.step_slots[t]))
            q, lens = dev_bf16(q_all[t]), dev(self.dc.step_kv_lens(t))
            o16 = A.decode(self.cache, q, lens, bt, max_kv, w.sm_scale, out_dtype=torch.bfloat16)
            if t in check_steps:
                self.out_bf16[t] = o16.float().cpu().numpy()
                self.out[t] = A.decode(self.cache, q, lens, bt, max_kv, w.sm_scale,
                                       out_dtype=torch.float32).cpu().numpy()
        torch.cuda.synchronize()
        self.q_all = q_all
        flat = torch.from_numpy(self.step_slots.reshape(-1)).to(DEV)
        pg, off = flat // 16, flat % 16
        self.step_rows = [t[pg, :, off, :].cpu().numpy() for t in self._planes()]
        pages = np.concatenate([seq_pages_of(lay, b, int(self.dc.init_lens[b]) + steps - 1)
                                for b in self.oracle_seqs])
        self.oracle_pages = pages
        idx = torch.from_numpy(pages.astype(np.int64)).to(DEV)
        self.seq_pages = [t[idx].cpu().numpy() for t in self._planes()]

    def _planes(self):
        c = self.cache
        return [t for t in (c.k_data, c.k_scale, c.v_data, c.v_scale) if t is not None]

    def oracle_cache(self):
        """Oracle cache holding the whole K/V of the oracle sequences (every position up to the
        last step) and the step tokens of every sequence."""
        lay = self.dc.layout
        make = ofp8.Fp8PagedCache if self.kv_format == "fp8" else ocache.PagedCache
        oc = make(lay.num_pages, self.w.num_kv_heads)
        for b in self.oracle_seqs:
            k, v = self.kv_bits[b]
            n = int(self.dc.init_lens[b]) + self.w.decode_steps - 1
            oc.append(k[:n], v[:n], lay.slots(b, np.arange(n)), workers=WORKERS)
        oc.append(self.step_k.reshape(-1, *self.step_k.shape[2:]),
                  self.step_v.reshape(-1, *self.step_v.shape[2:]), self.step_slots.reshape(-1),
                  workers=WORKERS)
        return oc

    def oracle(self, oc, steps):
        """Oracle outputs of the oracle sequences at the given steps (a decode at step t reads
        the first L_b + t tokens of the cache)."""
        return {t: oattn.decode(oc, self.q_all[t], self.dc.step_kv_lens(t), self.dc.layout.block_table,
                                self.w.sm_scale, seqs=self.oracle_seqs, workers=WORKERS)[0]
                for t in steps}


def seq_pages_of(layout: W.PageLayout, b: int, n_tokens: int) -> np.ndarray:
    return layout.block_table[b][: (n_tokens + 15) // 16]


def oracle_rows(oc, slots: np.ndarray):
    """The oracle cache's rows of the given slots, in the order of ``DecodeRun.step_rows``."""
    pg, off = slots // 16, slots % 16
    names = ("k_data", "v_data") if isinstance(oc, ofp8.Fp8PagedCache) else (
        "k_data", "k_scale", "v_data", "v_scale")
    return [getattr(oc, n)[pg, :, off, :] for n in names]
