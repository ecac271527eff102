"""Benchmark of the NVFP4 paged-KV attention path on one MI355X.

Headline step (timed K times after W warm-ups): append of the 16,384-token chunk into the NVFP4
cache followed by the causal paged prefill over it (32 query / 8 KV heads, head_dim 128, page
size 16, shuffled pages).  ``value`` is the prefill's algorithmic FLOP rate over the whole step.
The same run also times the 64-step decode loop (batch 64, 16K..32K cached tokens; each step
appends one token per sequence and decodes) and reports decode microseconds per call and HBM
GB/s, and times the CPU oracle on a bounded sample of the prefill workload.  The FP8 control
cache (one E4M3FN byte per value) is timed on the 16K prefill, the decode loop and the short
prefill shapes, with NVFP4 / FP8 time ratios; the dequantize-ahead repack (NVFP4 pages to an
fp16 copy, then the prefill over the copy) is timed on the short shapes against the stock
prefill.  The A4Q-style prefill (query quantized in the kernel, QK on the block-scaled MFMA) is
timed against the stock prefill at 16K and on the 4 x 128 over 2K tails.

Algorithmic work (nothing masked, padded or re-read is counted):
  prefill FLOP = 4 * head_dim * Hq * sum_b [q_b (kv_b - q_b) + q_b (q_b + 1) / 2]
  decode bytes = sum_b kv_len_b * Hkv * 144 (K and V: 64 packed + 8 scale bytes each;
                 FP8 control: 256)
                 + Q and O (2 bytes * Hq * head_dim each per sequence)
  append bytes = tokens * Hkv * (2 * 2 * head_dim read + 2 * 72 written)
Peaks: bf16 dense MFMA 2.5 PFLOP/s; HBM 8 TB/s (MI355X published figures).

Prints one JSON line.  Inputs are resident in HBM before any timed region starts.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workload as W  # noqa: E402

METRIC = "NVFP4-KV causal prefill TFLOP/s @16K; decode µs/call & HBM GB/s"
PEAK_MFMA_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0
PMC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_full16k_prefill_decode_b64.json")
PREFILL_KERNEL = "nvfp4_prefill_staggered_kernel<0>"  # the NVFP4 instantiation
PREFILL_SOURCES = ["prefill.hip", "prefill_common.hpp", "device_common.hpp", "kernel_params.hpp"]
DECODE_KERNEL = "nvfp4_decode_kernel<0>"
DECODE_SOURCES = ["decode.hip", "device_common.hpp", "kernel_params.hpp"]
CPU_TARGET_S = 12.0  # seconds of oracle work the timed CPU sample aims at


def prefill_flops(q_lens, kv_lens, hq, d=128) -> float:
    pairs = sum(q * (kv - q) + q * (q + 1) // 2 for q, kv in zip(q_lens, kv_lens))
    return 4.0 * d * hq * pairs


def source_hash(files) -> str:
    """Hash of the kernel sources with comments and whitespace removed, so that a change of
    code, not of commentary, marks the committed counters as stale."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "attention_nvfp4_quantized_amd", "csrc", f)) as fh:
            text = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(which: str):
    """HBM bytes per launch of the prefill ("prefill") or decode ("decode") kernel from the
    committed rocprofv3 counter summary, or None when that kernel's sources changed since the
    counters were taken."""
    if not os.path.exists(PMC_FILE):
        return None
    with open(PMC_FILE) as f:
        pmc = json.load(f)
    entry = pmc.get(which)
    sources = PREFILL_SOURCES if which == "prefill" else DECODE_SOURCES
    if not entry or entry.get("source_hash") != source_hash(sources):
        return None
    return entry["hbm_bytes_per_launch"]


def bf16_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def run_prefill(args, torch, A):
    pc = prefill_case("full16k")
    w = pc.w
    cache = A.NVFP4KVCache(pc.layout.num_pages, w.num_kv_heads)
    k, v = bf16_dev(pc.k_bits, torch), bf16_dev(pc.v_bits, torch)
    slots = torch.from_numpy(pc.slot_mapping).cuda()
    q = bf16_dev(pc.q_bits, torch)
    cu = torch.from_numpy(pc.cu_seqlens_q).cuda()
    kv = torch.from_numpy(pc.kv_lens).cuda()
    bt = torch.from_numpy(pc.layout.block_table).cuda()
    out = torch.empty((pc.total_q, w.num_qo_heads, 128), dtype=torch.bfloat16, device="cuda")
    ws_bytes = A.prefill_workspace_size(w.batch, pc.total_q, pc.max_q_len, pc.max_kv_len,
                                        w.num_qo_heads, w.num_kv_heads)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        A.append(cache, k, v, slots)
        if ev is not None:
            ev[1].record()
        A.prefill(cache, q, cu, kv, bt, pc.max_q_len, pc.max_kv_len, w.sm_scale, out=out,
                  workspace=ws)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    append_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    prefill_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    flops = prefill_flops(w.q_lens, w.kv_lens, w.num_qo_heads)
    ms_step = (t1 - t0) * 1e3 / args.steps
    append_bytes = pc.k_bits.shape[0] * w.num_kv_heads * (2 * 2 * 128 + 2 * 72)
    return dict(w=w, pc=pc, flops=flops, ms_step=ms_step, append_ms=append_ms,
                prefill_ms=prefill_ms, append_bytes=append_bytes)


# cache bytes per (token, KV head) read by attention, K and V together
KV_BYTES = {"nvfp4": 144, "fp8": 256}


def run_decode(args, torch, A, formats=("nvfp4",)):
    """The 64-step decode loop once per cache format (the same tokens in every cache); returns
    one result dict per format."""
    w = W.get("decode")
    dc = W.decode_case(w)
    lay = dc.layout
    caches = {f: A.NVFP4KVCache(lay.num_pages, w.num_kv_heads, kv_format=f) for f in formats}
    steps = w.decode_steps
    step_k = np.zeros((steps, w.batch, w.num_kv_heads, 128), np.uint16)
    step_v = np.zeros_like(step_k)

    def fill(b):
        kb, vb = dc.seq_kv(b)
        n = int(dc.init_lens[b]) - 1
        step_k[:, b], step_v[:, b] = kb[n:n + steps], vb[n:n + steps]
        return b, kb[:n], vb[:n], lay.slots(b, np.arange(n))

    workers = min(16, len(os.sched_getaffinity(0)))
    with cf.ThreadPoolExecutor(workers) as ex:
        for b, kb, vb, sl in ex.map(fill, range(w.batch)):
            kd, vd, sd = bf16_dev(kb, torch), bf16_dev(vb, torch), torch.from_numpy(sl).cuda()
            for cache in caches.values():
                A.append(cache, kd, vd, sd)
    torch.cuda.synchronize()
    qs = bf16_dev(dc.step_q(), torch)
    ks, vs = bf16_dev(step_k, torch), bf16_dev(step_v, torch)
    slots = torch.from_numpy(np.stack([dc.step_slots(t) for t in range(steps)])).cuda()
    lens_np = np.stack([dc.step_kv_lens(t) for t in range(steps)])
    lens = torch.from_numpy(lens_np).cuda()
    bt = torch.from_numpy(lay.block_table).cuda()
    max_kv = int(lens_np.max())
    out = torch.empty((w.batch, w.num_qo_heads, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(A.decode_workspace_size(w.batch, max_kv, w.num_qo_heads, w.num_kv_heads),
                     dtype=torch.uint8, device="cuda")

    def loop(cache, ev=None):
        for t in range(steps):
            if ev is not None:
                ev[t][0].record()
            A.append(cache, ks[t], vs[t], slots[t])
            if ev is not None:
                ev[t][1].record()
            A.decode(cache, qs[t], lens[t], bt, max_kv, w.sm_scale, out=out, workspace=ws)
            if ev is not None:
                ev[t][2].record()

    results = {}
    for fmt, cache in caches.items():
        # the warm-up pass rewrites the same step tokens, so the timed pass sees identical caches
        loop(cache)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        t0 = time.perf_counter()
        loop(cache, ev)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        results[fmt] = decode_result(w, fmt, lens_np, ev, t1 - t0)
    return results


def decode_result(w, fmt, lens_np, ev, loop_s):
    steps = len(ev)
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    app_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    bytes_per_step = (lens_np.sum(axis=1) * w.num_kv_heads * KV_BYTES[fmt]
                      + 2 * 2 * w.batch * w.num_qo_heads * 128).astype(np.float64)
    gbps = float(bytes_per_step.sum() / (dec_ms.sum() * 1e-3) / 1e9)
    append_bytes = w.batch * w.num_kv_heads * (2 * 2 * 128 + KV_BYTES[fmt])
    out = {
        "workload": "decode", "kv_format": fmt, "batch": w.batch, "steps": steps,
        "kv_len_min": int(lens_np.min()), "kv_len_max": int(lens_np.max()),
        "loop_ms": round(loop_s * 1e3, 3),
        "us_per_call": round(float(dec_ms.mean()) * 1e3, 2),
        "bytes_per_call": int(bytes_per_step.mean()),
        "GBps": round(gbps, 1),
        "append_us_per_call": round(float(app_ms.mean()) * 1e3, 2),
        "append_GBps": round(append_bytes / (app_ms.mean() * 1e-3) / 1e9, 1),
    }
    if fmt == "nvfp4":
        out["roofline"] = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                           "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                           "traffic": measured_traffic("decode"), "kernel": DECODE_KERNEL}
    else:
        out["hbm_frac"] = round(gbps / PEAK_HBM_GBPS, 4)
    return out


def make_flush(torch):
    """A 512 MB read between timed calls: it refills the L2s and the 256 MB MALL with clean lines
    of another buffer, so the timed call reads its cache from HBM.  (Writing such a buffer
    instead would leave up to a MALL of dirty lines that the timed call has to write back.)"""
    buf = torch.zeros(128 << 20, dtype=torch.float32, device="cuda")
    return lambda: buf.max()


def run_repack_prefill(name, torch, A, reps=20):
    """Dequantize-ahead repack on a short-query workload: median µs of the repack pass (every
    page the batch reads, NVFP4 -> fp16 copy), of the prefill over the copy, and of both
    together, with a 512 MB buffer read before each call (cold caches), against the stock
    prefill over the packed cache measured the same way."""
    pc = prefill_case(name)
    w = pc.w
    cache = A.NVFP4KVCache(pc.layout.num_pages, w.num_kv_heads)
    A.append(cache, bf16_dev(pc.k_bits, torch), bf16_dev(pc.v_bits, torch),
             torch.from_numpy(pc.slot_mapping).cuda())
    dst = A.NVFP4KVCache(pc.layout.num_pages, w.num_kv_heads, kv_format="f16")
    q = bf16_dev(pc.q_bits, torch)
    cu = torch.from_numpy(pc.cu_seqlens_q).cuda()
    kv = torch.from_numpy(pc.kv_lens).cuda()
    bt = torch.from_numpy(pc.layout.block_table).cuda()
    out = torch.empty((pc.total_q, w.num_qo_heads, 128), dtype=torch.bfloat16, device="cuda")
    ws_bytes = A.prefill_workspace_size(w.batch, pc.total_q, pc.max_q_len, pc.max_kv_len,
                                        w.num_qo_heads, w.num_kv_heads)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    flush = make_flush(torch)

    def prefill(c):
        A.prefill(c, q, cu, kv, bt, pc.max_q_len, pc.max_kv_len, w.sm_scale, out=out, workspace=ws)

    def both():
        A.repack(cache, dst, bt, kv, pc.max_kv_len)
        prefill(dst)
        prefill(cache)

    warm_up(both, torch)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(reps)]
    for i in range(reps):
        flush()
        ev[i][0].record()
        A.repack(cache, dst, bt, kv, pc.max_kv_len)
        ev[i][1].record()
        prefill(dst)
        ev[i][2].record()
        flush()
        ev[i][3].record()
        prefill(cache)
        ev[i][4].record()
    torch.cuda.synchronize()
    med = lambda a, b: float(np.median([e[a].elapsed_time(e[b]) for e in ev])) * 1e3  # noqa: E731
    rep, pre, tot, stock = med(0, 1), med(1, 2), med(0, 2), med(3, 4)
    return {"workload": name, "us_repack": round(rep, 2), "us_prefill_over_copy": round(pre, 2),
            "us_repack_plus_prefill": round(tot, 2), "us_stock_prefill": round(stock, 2),
            "ratio_repack_path_over_stock": round(tot / stock, 3)}


_CASES = {}


def warm_up(fn, torch, min_calls=20, min_seconds=0.25):
    """Untimed calls of `fn` until at least `min_calls` have run and at least `min_seconds` of
    GPU time have passed (the shader clock ramps over the first launches after an idle spell,
    such as the host-side input generation that precedes each leg)."""
    t0 = time.perf_counter()
    n = 0
    while n < min_calls or time.perf_counter() - t0 < min_seconds:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def prefill_case(name):
    """Seeded host inputs of a prefill workload, generated once per run."""
    if name not in _CASES:
        _CASES[name] = W.prefill_case(W.get(name))
    return _CASES[name]


def run_full_prefill(name, torch, A, reps=20, kv_format="nvfp4"):
    """Kernel time of the append and the causal prefill of a full-length single request (the
    pages' benchmark matrix asks for full 8K and 32K prefill next to the tail shapes)."""
    pc = prefill_case(name)
    w = pc.w
    cache = A.NVFP4KVCache(pc.layout.num_pages, w.num_kv_heads, kv_format=kv_format)
    k, v = bf16_dev(pc.k_bits, torch), bf16_dev(pc.v_bits, torch)
    slots = torch.from_numpy(pc.slot_mapping).cuda()
    q = bf16_dev(pc.q_bits, torch)
    cu = torch.from_numpy(pc.cu_seqlens_q).cuda()
    kv = torch.from_numpy(pc.kv_lens).cuda()
    bt = torch.from_numpy(pc.layout.block_table).cuda()
    out = torch.empty((pc.total_q, w.num_qo_heads, 128), dtype=torch.bfloat16, device="cuda")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]

    def step(e=None):
        if e: e[0].record()
        A.append(cache, k, v, slots)
        if e: e[1].record()
        A.prefill(cache, q, cu, kv, bt, pc.max_q_len, pc.max_kv_len, w.sm_scale, out=out)
        if e: e[2].record()

    warm_up(step, torch)
    for e in ev:
        step(e)
    torch.cuda.synchronize()
    pre = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    app = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    flops = prefill_flops(w.q_lens, w.kv_lens, w.num_qo_heads)
    return {"workload": name, "kv_format": kv_format, "q_len": int(w.q_lens[0]),
            "kv_len": int(w.kv_lens[0]), "prefill_ms": round(pre, 4), "TFLOPs": round(flops / (pre * 1e-3) / 1e12, 2),
            "mfma_frac": round(flops / (pre * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
            "append_us": round(app * 1e3, 2), "flop_per_call": flops}


def run_short_prefill(name, torch, A, reps=20, kv_format="nvfp4"):
    """Prefill-only timing of a short workload (tiny: 1 x 256 queries over 256 keys, 4 / 1 heads;
    tail128: 4 x 128 queries over 2,048 keys; tail16: 8 x 16 queries over 16,384 keys): median µs
    per call with a 512 MB buffer read
    between calls (flushing L2 and MALL, so the packed cache comes from HBM) and warm
    back-to-back, with algorithmic TFLOP/s and GB/s (Q + O + packed KV of every sequence)."""
    pc = prefill_case(name)
    w = pc.w
    cache = A.NVFP4KVCache(pc.layout.num_pages, w.num_kv_heads, kv_format=kv_format)
    A.append(cache, bf16_dev(pc.k_bits, torch), bf16_dev(pc.v_bits, torch),
             torch.from_numpy(pc.slot_mapping).cuda())
    q = bf16_dev(pc.q_bits, torch)
    cu = torch.from_numpy(pc.cu_seqlens_q).cuda()
    kv = torch.from_numpy(pc.kv_lens).cuda()
    bt = torch.from_numpy(pc.layout.block_table).cuda()
    out = torch.empty((pc.total_q, w.num_qo_heads, 128), dtype=torch.bfloat16, device="cuda")
    ws_bytes = A.prefill_workspace_size(w.batch, pc.total_q, pc.max_q_len, pc.max_kv_len,
                                        w.num_qo_heads, w.num_kv_heads)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    flush = make_flush(torch)

    def call():
        A.prefill(cache, q, cu, kv, bt, pc.max_q_len, pc.max_kv_len, w.sm_scale, out=out,
                  workspace=ws)

    warm_up(call, torch)
    times = {}
    for mode in ("flushed", "warm"):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for i in range(reps):
            if mode == "flushed":
                flush()
            ev[i][0].record()
            call()
            ev[i][1].record()
        torch.cuda.synchronize()
        times[mode] = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    flops = prefill_flops(w.q_lens, w.kv_lens, w.num_qo_heads)
    nbytes = float(sum(w.kv_lens) * w.num_kv_heads * KV_BYTES[kv_format]
                   + 2 * 2 * pc.total_q * w.num_qo_heads * 128)
    t = times["flushed"] * 1e-3
    return {"workload": name, "kv_format": kv_format, "batch": w.batch, "q_len": int(w.q_lens[0]), "kv_len": int(w.kv_lens[0]),
            "us_flushed": round(times["flushed"] * 1e3, 2), "us_warm": round(times["warm"] * 1e3, 2),
            "TFLOPs": round(flops / t / 1e12, 2), "mfma_frac": round(flops / t / 1e12 / PEAK_MFMA_TFLOPS, 4),
            "GBps": round(nbytes / t / 1e9, 1), "hbm_frac": round(nbytes / t / 1e9 / PEAK_HBM_GBPS, 4),
            "flop_per_call": flops, "bytes_per_call": int(nbytes)}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return None


def run_a4q(name, torch, A, reps=20):
    """The A4Q-style prefill (query quantized to MX blocks in the kernel, QK on the block-scaled
    MFMA; MXFP8 and MXFP4 queries; K exact as two E4M3 terms, or as one term with the "_k1"
    suffix) against the stock prefill on the same cache: median µs per call, with a 512 MB
    buffer read before each call for the short shape (cold caches) and back to back for the
    full one."""
    pc = prefill_case(name)
    w = pc.w
    cache = A.NVFP4KVCache(pc.layout.num_pages, w.num_kv_heads)
    A.append(cache, bf16_dev(pc.k_bits, torch), bf16_dev(pc.v_bits, torch),
             torch.from_numpy(pc.slot_mapping).cuda())
    q = bf16_dev(pc.q_bits, torch)
    cu = torch.from_numpy(pc.cu_seqlens_q).cuda()
    kv = torch.from_numpy(pc.kv_lens).cuda()
    bt = torch.from_numpy(pc.layout.block_table).cuda()
    out = torch.empty((pc.total_q, w.num_qo_heads, 128), dtype=torch.bfloat16, device="cuda")
    ws_bytes = max(A.prefill_workspace_size(w.batch, pc.total_q, pc.max_q_len, pc.max_kv_len,
                                            w.num_qo_heads, w.num_kv_heads),
                   A.prefill_a4q_workspace_size(w.batch, pc.total_q, pc.max_q_len, pc.max_kv_len,
                                                w.num_qo_heads, w.num_kv_heads))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    flush = make_flush(torch) if w.batch > 1 else None
    calls = {
        "stock": lambda: A.prefill(cache, q, cu, kv, bt, pc.max_q_len, pc.max_kv_len, w.sm_scale,
                                   out=out, workspace=ws),
        "a4q_mxfp8": lambda: A.prefill_a4q(cache, q, cu, kv, bt, pc.max_q_len, pc.max_kv_len,
                                           w.sm_scale, q_format="mxfp8", out=out, workspace=ws),
        "a4q_mxfp4": lambda: A.prefill_a4q(cache, q, cu, kv, bt, pc.max_q_len, pc.max_kv_len,
                                           w.sm_scale, q_format="mxfp4", out=out, workspace=ws),
        "a4q_mxfp8_k1": lambda: A.prefill_a4q(cache, q, cu, kv, bt, pc.max_q_len, pc.max_kv_len,
                                              w.sm_scale, q_format="mxfp8", out=out, workspace=ws,
                                              k_terms=1),
        "a4q_mxfp4_k1": lambda: A.prefill_a4q(cache, q, cu, kv, bt, pc.max_q_len, pc.max_kv_len,
                                              w.sm_scale, q_format="mxfp4", out=out, workspace=ws,
                                              k_terms=1),
    }
    res = {"workload": name, "mode": "flushed" if flush is not None else "warm"}
    for key, fn in calls.items():
        warm_up(fn, torch)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for e in ev:
            if flush is not None:
                flush()
            e[0].record()
            fn()
            e[1].record()
        torch.cuda.synchronize()
        res["us_" + key] = round(float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * 1e3, 2)
    for key in ("a4q_mxfp8", "a4q_mxfp4", "a4q_mxfp8_k1", "a4q_mxfp4_k1"):
        res["ratio_" + key + "_over_stock"] = round(res["us_" + key] / res["us_stock"], 3)
    flops = prefill_flops(w.q_lens, w.kv_lens, w.num_qo_heads)
    for key in ("a4q_mxfp8", "a4q_mxfp8_k1"):
        res["TFLOPs_" + key] = round(flops / (res["us_" + key] * 1e-6) / 1e12, 2)
    return res


def run_cpu_baseline(pc, target_s=CPU_TARGET_S):
    """The oracle, untuned, on a bounded sample of the 16K prefill: all 32 heads of query rows
    spread evenly over the sequence (their visible keys included), after the oracle's append of
    all 16,384 tokens (timed separately).  Two short untimed calls (32 and 96 rows) give the
    host's fixed cost per call and time per row; the timed call then takes as many rows as fill
    about `target_s` seconds, so the sample is about that long on any host."""
    from oracle import attention as oattn
    from oracle import cache as ocache
    blas_threads = _blas_threads()
    w = pc.w
    t0 = time.perf_counter()
    oc = ocache.PagedCache(pc.layout.num_pages, w.num_kv_heads)
    oc.append(pc.k_bits, pc.v_bits, pc.slot_mapping)
    t_append = time.perf_counter() - t0

    def spread(n):
        return np.unique(np.linspace(0, pc.total_q - 1, n).round().astype(np.int64))

    def run(rows):
        t = time.perf_counter()
        oattn.prefill(oc, pc.q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table,
                      w.sm_scale, rows=rows)
        return time.perf_counter() - t

    t32, t96 = run(spread(32)), run(spread(96))
    per_row = max((t96 - t32) / 64, 1e-6)
    fixed = max(t32 - 32 * per_row, 0.0)
    n = int(np.clip((target_s - fixed) / per_row, 96, pc.total_q))
    rows = spread(n)
    t_pre = run(rows)
    flops = 4.0 * 128 * w.num_qo_heads * float((rows + 1).sum())
    cores = len(os.sched_getaffinity(0))
    return {"value": round(flops / t_pre / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(blas_threads or cores), "host_cores": cores, "kind": "oracle",
            "sample": "oracle float64 prefill of %d evenly spaced query rows x 32 heads of the "
                      "16K causal prefill (%.3g algorithmic FLOP, %.1f s), after the oracle's "
                      "append of all 16,384 tokens (%.1f s, not in value)"
                      % (len(rows), flops, t_pre, t_append),
            "rows": int(len(rows)), "seconds": round(t_pre + t_append, 2)}


def run_cpu_phases():
    """The oracle, untuned and single-process as it stands, timed per phase beside the GPU legs:
    the whole tiny and tail128 workloads (append of every token, then the prefill of every row),
    one of the eight tail16 sequences (append of its 16,384 tokens, prefill of its 16 rows;
    x 8 for the batch, labelled extrapolated), and one decode step of two sequences of the
    decode workload (append of their step token, decode over 16K-32K keys; x 32 for the 64
    sequences and x 64 for the loop, labelled extrapolated; the fill of their caches is set-up,
    not timed)."""
    from oracle import attention as oattn
    from oracle import cache as ocache
    out = {"blas_threads": _blas_threads(), "host_cores": len(os.sched_getaffinity(0))}
    for name in ("tiny", "tail128"):
        pc = prefill_case(name)
        w = pc.w
        t0 = time.perf_counter()
        oc = ocache.PagedCache(pc.layout.num_pages, w.num_kv_heads)
        oc.append(pc.k_bits, pc.v_bits, pc.slot_mapping)
        t1 = time.perf_counter()
        oattn.prefill(oc, pc.q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table, w.sm_scale)
        t2 = time.perf_counter()
        out[name] = {"append_s": round(t1 - t0, 3), "prefill_s": round(t2 - t1, 3),
                     "total_s": round(t2 - t0, 3), "sample": "whole workload"}
    pc = prefill_case("tail16")
    w = pc.w
    s0, s1 = int(pc.cu_seqlens_kv[0]), int(pc.cu_seqlens_kv[1])
    t0 = time.perf_counter()
    oc = ocache.PagedCache(pc.layout.num_pages, w.num_kv_heads)
    oc.append(pc.k_bits[s0:s1], pc.v_bits[s0:s1], pc.slot_mapping[s0:s1])
    t1 = time.perf_counter()
    oattn.prefill(oc, pc.q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table, w.sm_scale,
                  rows=np.arange(int(pc.cu_seqlens_q[0]), int(pc.cu_seqlens_q[1])))
    t2 = time.perf_counter()
    out["tail16"] = {"append_s": round(t1 - t0, 3), "prefill_s": round(t2 - t1, 3),
                     "total_s_extrapolated": round(8 * (t2 - t0), 3),
                     "sample": "sequence 0 of 8 (16,384 tokens appended, 16 rows x 32 heads); "
                               "total x 8, extrapolated"}
    w = W.get("decode")
    dc = W.decode_case(w)
    lay = dc.layout
    seqs = [int(np.argmin(w.kv_lens)), int(np.argmax(w.kv_lens))]
    oc = ocache.PagedCache(lay.num_pages, w.num_kv_heads)
    step_k = np.zeros((w.batch, w.num_kv_heads, 128), np.uint16)
    step_v = np.zeros_like(step_k)
    for b in seqs:
        kb, vb = dc.seq_kv(b)
        n = int(dc.init_lens[b]) - 1
        oc.append(kb[:n], vb[:n], lay.slots(b, np.arange(n)), workers=min(16, out["host_cores"]))
        step_k[b], step_v[b] = kb[n], vb[n]
    slots = dc.step_slots(0)
    t0 = time.perf_counter()
    oc.append(step_k[seqs], step_v[seqs], slots[seqs])
    t1 = time.perf_counter()
    oattn.decode(oc, dc.step_q()[0], dc.step_kv_lens(0), lay.block_table, w.sm_scale, seqs=seqs)
    t2 = time.perf_counter()
    step = (t2 - t0) * w.batch / len(seqs)
    out["decode"] = {"append_s": round(t1 - t0, 4), "decode_s": round(t2 - t1, 4),
                     "kv_lens": [int(dc.step_kv_lens(0)[b]) for b in seqs],
                     "step_s_extrapolated": round(step, 3),
                     "loop_s_extrapolated": round(step * w.decode_steps, 2),
                     "sample": "step 0 of sequences %s (shortest and longest); x %d for the 64 "
                               "sequences and x 64 for the loop, extrapolated"
                               % (seqs, w.batch // len(seqs))}
    return out


def fp8_summary(line, fp8):
    """The FP8 (E4M3FN, one byte per value) control cache timed on the same workloads, and the
    NVFP4 / FP8 time ratios (above 1: NVFP4 slower)."""
    out = dict(fp8)
    pre = fp8["prefill_full16k"]
    out["ratio_nvfp4_over_fp8"] = {
        "prefill_full16k": round(line["roofline"]["kernel_ms"] / pre["prefill_ms"], 3),
        "append_16k": round(line["append"]["us_per_call"] / pre["append_us"], 3),
    }
    if "decode" in fp8:
        out["ratio_nvfp4_over_fp8"]["decode"] = round(
            line["decode"]["us_per_call"] / fp8["decode"]["us_per_call"], 3)
    for n, f in zip(line.get("short_prefill", []), fp8.get("short_prefill", [])):
        out["ratio_nvfp4_over_fp8"][n["workload"] + "_flushed"] = round(n["us_flushed"] / f["us_flushed"], 3)
    for n, f in zip(line.get("prefill_matrix", []), fp8.get("prefill_matrix", [])):
        out["ratio_nvfp4_over_fp8"][n["workload"]] = round(n["prefill_ms"] / f["prefill_ms"], 3)
    return out


def copy_calibration(torch, sizes=(1 << 30, 1 << 26)):
    """Plain device copies of known sizes, for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE: 1 GiB,
    and 64 MiB, about the bf16 K and V that the 16K append reads (each copy's grid size tells the
    launches apart)."""
    for nbytes in sizes:
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 3}))


def progress(msg):
    """One line per leg on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {time.strftime('%H:%M:%S')} {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-short", action="store_true",
                    help="skip the tiny / tail128 / tail16 prefill timings (stock; repacked for the tails)")
    ap.add_argument("--no-matrix", action="store_true", help="skip the full 8K / 32K prefill timings")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 control-cache timings")
    ap.add_argument("--no-a4q", action="store_true", help="skip the A4Q-style prefill timings")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path has no multi-GPU mode (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import attention_nvfp4_quantized_amd as A
    A.load_library()
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)
        return

    progress("full16k append + prefill")
    pre = run_prefill(args, torch, A)
    value = pre["flops"] / (pre["ms_step"] * 1e-3) / 1e12
    achieved = pre["flops"] / (pre["prefill_ms"] * 1e-3) / 1e12
    w = pre["w"]
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(pre["ms_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "dtype_detail": "fp16 MFMA with fp32 accumulation (exact fp16 cache values; bf16 Q in, bf16 O out)",
        "data": "synthetic (seeded N(0,1) bf16, K outlier channels x8)",
        "config": {"workload": "full16k causal prefill + append", "batch": 1, "q_len": 16384,
                   "kv_len": 16384, "num_qo_heads": w.num_qo_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": 128, "page_size": 16,
                   "cache": "NVFP4 (E2M1 + E4M3 per 16)", "seed": w.seed},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
                     "traffic": measured_traffic("prefill"), "kernel": PREFILL_KERNEL,
                     "kernel_ms": round(pre["prefill_ms"], 4), "flop_per_launch": pre["flops"]},
        "append": {"us_per_call": round(pre["append_ms"] * 1e3, 2), "tokens": 16384,
                   "GBps": round(pre["append_bytes"] / (pre["append_ms"] * 1e-3) / 1e9, 1)},
    }
    fp8 = {}
    progress("decode loop")
    if not args.no_decode:
        dec = run_decode(args, torch, A, ("nvfp4",) if args.no_fp8 else ("nvfp4", "fp8"))
        line["decode"] = dec["nvfp4"]
        if "fp8" in dec:
            fp8["decode"] = dec["fp8"]
    progress("short prefill legs")
    if not args.no_short:
        line["short_prefill"] = [run_short_prefill(n, torch, A) for n in ("tiny", "tail128", "tail16")]
        if not args.no_fp8:
            fp8["short_prefill"] = [run_short_prefill(n, torch, A, kv_format="fp8")
                                    for n in ("tiny", "tail128", "tail16")]
    progress("repack legs")
    if not args.no_short:
        line["repack"] = [run_repack_prefill(n, torch, A) for n in ("tail128", "tail16")]
    progress("A4Q legs")
    if not args.no_a4q:
        line["a4q"] = [run_a4q(n, torch, A) for n in ("full16k", "tail128")]
    progress("8K / 32K prefill legs")
    if not args.no_matrix:
        line["prefill_matrix"] = [run_full_prefill(n, torch, A) for n in ("full8k", "full32k")]
        if not args.no_fp8:
            fp8["prefill_matrix"] = [run_full_prefill(n, torch, A, kv_format="fp8")
                                     for n in ("full8k", "full32k")]
    progress("FP8 16K prefill leg")
    if not args.no_fp8:
        fp8["prefill_full16k"] = run_full_prefill("full16k", torch, A, kv_format="fp8")
        line["fp8_control"] = fp8_summary(line, fp8)
    progress("CPU oracle baseline")
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = run_cpu_baseline(pre["pc"])
        line["cpu_baseline"]["phases"] = run_cpu_phases()
    print(json.dumps(line))


if __name__ == "__main__":
    main()
