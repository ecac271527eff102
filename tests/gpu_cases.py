"""Helpers for the GPU tests: upload seeded workloads, run the HIP path through the binding,
and build the matching oracle cache.  Inputs come only from ``workload``; expected values only
from ``oracle``."""
from __future__ import annotations

import sys

import numpy as np
import torch

import attention_nvfp4_quantized_amd as A
import workload as W
from oracle import attention as oattn
from oracle import cache as ocache
from oracle import fp8cache as ofp8

DEV = "cuda"

# Output tolerance on attention (float32 output): the bar the path is held to.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3
# log-sum-exp: the kernels sum the rounded softmax weights (the same weights the PV product
# uses: fp16 rounded toward zero, relative error below 2^-10); each is within a relative 2^-9 of
# its float value, so the sum is too and its log is within 2^-9 absolute.  Plus float32
# rounding of the rest.
LSE_ATOL = 2.0 ** -9 + 5e-4


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
        c.append(pc.k_bits[s0:s1], pc.v_bits[s0:s1], pc.slot_mapping[s0:s1])
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
                         pc.w.sm_scale, causal=causal, rows=rows)


def rows_of(pc: W.PrefillCase, seqs) -> np.ndarray:
    return np.concatenate([np.arange(pc.cu_seqlens_q[b], pc.cu_seqlens_q[b + 1]) for b in seqs])


class DecodeRun:
    """The decode workload at full size: 64 sequences, 64 steps of (append 64 tokens, decode).

    Sampled sequences carry their seeded K/V; the others keep zero K/V, which changes none of
    the sampled outputs (sequences are independent) and none of the launch shapes."""

    def __init__(self, sampled, check_steps, kv_format="nvfp4"):
        self.w = W.get("decode")
        self.dc = W.decode_case(self.w)
        self.kv_format = kv_format
        lay, w = self.dc.layout, self.w
        self.cache = A.NVFP4KVCache(lay.num_pages, w.num_kv_heads, kv_format=kv_format)
        self.kv_bits = {b: self.dc.seq_kv(b) for b in sampled}
        for b, (k, v) in self.kv_bits.items():
            n = int(self.dc.init_lens[b]) - 1
            A.append(self.cache, dev_bf16(k[:n]), dev_bf16(v[:n]), dev(lay.slots(b, np.arange(n))))
        q_all = self.dc.step_q()
        bt = dev(lay.block_table)
        self.out = {}
        max_kv = int(self.dc.init_lens.max()) + w.decode_steps - 1
        zeros = np.zeros((w.batch, w.num_kv_heads, w.head_dim), np.uint16)
        for t in range(w.decode_steps):
            kb, vb = zeros.copy(), zeros.copy()
            for b, (k, v) in self.kv_bits.items():
                kb[b], vb[b] = k[int(self.dc.init_lens[b]) - 1 + t], v[int(self.dc.init_lens[b]) - 1 + t]
            A.append(self.cache, dev_bf16(kb), dev_bf16(vb), dev(self.dc.step_slots(t)))
            o = A.decode(self.cache, dev_bf16(q_all[t]), dev(self.dc.step_kv_lens(t)), bt, max_kv,
                         w.sm_scale, out_dtype=torch.float32)
            if t in check_steps:
                self.out[t] = o.cpu().numpy()
        torch.cuda.synchronize()
        self.q_all = q_all

    def oracle(self, steps, sampled):
        """Oracle outputs at the given steps; its cache holds every token up to the last step
        (a decode at step t reads only the first L_b + t of them)."""
        lay = self.dc.layout
        make = ofp8.Fp8PagedCache if self.kv_format == "fp8" else ocache.PagedCache
        oc = make(lay.num_pages, self.w.num_kv_heads)
        for b in sampled:
            k, v = self.kv_bits[b]
            n = int(self.dc.init_lens[b]) + max(steps)
            oc.append(k[:n], v[:n], lay.slots(b, np.arange(n)))
        return {t: oattn.decode(oc, self.q_all[t], self.dc.step_kv_lens(t), lay.block_table,
                                self.w.sm_scale, seqs=sampled)[0] for t in steps}
