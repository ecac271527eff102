"""Added output error of A4Q-style QK (``oracle/a4q.py``) against the stock read path, on the
seeded workloads (test infrastructure; CPU only).

"NVFP4 KV cache A4Q prefill explained", section "Make query accuracy a release gate": the error
a quantized query adds to the attention output is to be measured against a high-precision
reference over varied sequence lengths, head layouts, masking and outlier scales.  Both sides read the same oracle NVFP4 cache; the reference is the oracle's
float64 attention with the bf16 queries as given.  Cases:

* tiny (q = kv = 256, 4/1 heads, 2 K outlier channels), causal;
* tail128 (4 x 128 queries over 2,048 keys, 32/8 heads, 20 K outlier channels x8), causal and
  non-causal;
* tail128 with Q outlier channels: 4 of every 128 query dims (seeded, per head) scaled x8
  before bf16 rounding, the query-side counterpart of the K outlier channels;
* tail16 (8 x 16 queries over 16,384 keys), sequences 0 and 5;
* full16k and full32k, 24 evenly spaced query rows.

Schemes: the pages' reading (``a4q.SCHEMES`` through ``prefill_a4q``: QK exact on the quantized
query, weights rounded to bf16 for PV) and the scheme of the GPU variant
(``prefill_mx`` with "mxfp8" / "mxfp4" queries: K through its two-term E4M3 bridge, float64
softmax and PV), listed as ``gpu:mxfp8`` and ``gpu:mxfp4``, and its one-term K form
(``k_terms=1``: K rounded to one E4M3 term under the block's power-of-two scale), listed as
``gpu:mxfp8:k1`` and ``gpu:mxfp4:k1``.

Run: ``python -m oracle.a4q_report`` (prints a markdown table).
"""
from __future__ import annotations

import time

import numpy as np

from . import a4q, attention, cache


def _cache_of(pc, seqs=None):
    oc = cache.PagedCache(pc.layout.num_pages, pc.w.num_kv_heads)
    for b in (range(pc.w.batch) if seqs is None else seqs):
        s0, s1 = pc.cu_seqlens_kv[b], pc.cu_seqlens_kv[b + 1]
        oc.append(pc.k_bits[s0:s1], pc.v_bits[s0:s1], pc.slot_mapping[s0:s1], workers=8)
    return oc


def cases():
    import workload as W
    tiny = W.prefill_case(W.get("tiny"))
    t128 = W.prefill_case(W.get("tail128"))
    t16 = W.prefill_case(W.get("tail16"))
    f16 = W.prefill_case(W.get("full16k"))
    f32 = W.prefill_case(W.get("full32k"))
    rows_t16 = np.concatenate([np.arange(t16.cu_seqlens_q[b], t16.cu_seqlens_q[b + 1]) for b in (0, 5)])
    yield "tiny, causal", tiny, tiny.q_bits, True, None, None
    yield "tail128, causal", t128, t128.q_bits, True, None, None
    yield "tail128, no mask", t128, t128.q_bits, False, None, None
    yield "tail128, Q outlier channels x8", t128, W.scale_channels(t128.q_bits, 77, 4, 8.0), True, None, None
    yield "tail16, sequences 0 and 5", t16, t16.q_bits, True, rows_t16, [0, 5]
    yield "full16k, 24 rows", f16, f16.q_bits, True, np.linspace(0, 16383, 24).astype(np.int64), None
    yield "full32k, 24 rows", f32, f32.q_bits, True, np.linspace(0, 32767, 24).astype(np.int64), None


def main():
    print("| case | scheme | max-abs | mean-abs | within 1e-2 / 1e-3 |")
    print("|---|---|---|---|---|")
    t0 = time.time()
    for name, pc, q_bits, causal, rows, seqs in cases():
        oc = _cache_of(pc, seqs)
        ref, _ = attention.prefill(oc, q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table,
                                   pc.w.sm_scale, causal=causal, rows=rows)
        m = ~np.isnan(ref)
        for scheme in a4q.SCHEMES + ("gpu:mxfp8", "gpu:mxfp4", "gpu:mxfp8:k1", "gpu:mxfp4:k1"):
            if scheme.startswith("gpu:"):
                fmt = scheme.split(":")[1]
                o = a4q.prefill_mx(oc, q_bits, pc.cu_seqlens_q, pc.kv_lens, pc.layout.block_table,
                                   pc.w.sm_scale, fmt, causal=causal, rows=rows,
                                   k_terms=1 if scheme.endswith(":k1") else 2)
            else:
                o = a4q.prefill_a4q(oc, q_bits, pc.cu_seqlens_q, pc.kv_lens,
                                    pc.layout.block_table, pc.w.sm_scale, scheme, causal=causal,
                                    rows=rows)
            err = np.abs(o[m] - ref[m])
            ok = "yes" if err.max() <= 1e-2 and err.mean() <= 1e-3 else "no"
            print(f"| {name} | {scheme} | {err.max():.3e} | {err.mean():.3e} | {ok} |", flush=True)
    print(f"\n({time.time() - t0:.0f} s)")


if __name__ == "__main__":
    main()
