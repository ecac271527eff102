"""Attention over the dequantized NVFP4 cache, oracle side (test infrastructure).

What is computed is the stock read path: the packed K and V are unpacked,
converted and scaled back to values, and attention runs with bf16 queries
("NVFP4 KV cache A4Q prefill explained", sections "NVFP4 KV cache A4Q
prefill explained" and "Why NVFP4 KV cache A4Q prefill exists"; "NVFP4 KV
cache prefill vs decode performance", section "Cold prefill can lose on
conversion cost").  Prefill writes the chunk's K/V into the cache and then
reads every key, the chunk's own included, from the cache; decode scans the
whole cache of a sequence for its single newest query, after that token's K/V
has been written ("NVFP4 KV
cache prefill vs decode performance", section "NVFP4 KV cache prefill vs
decode performance").

Plain definition, in float64 (queries are exact bf16 values):

    z_j = sm_scale * <q_i, k_j>         for the visible keys j
    p   = exp(z - max z) / sum exp(z - max z)
    o_i = sum_j p_j v_j,   lse_i = max z + log sum exp(z - max z)

Readings: a query row i of a sequence with q_len queries and kv_len keys sees
keys j <= kv_len - q_len + i (queries sit at the tail of the sequence); query
head h reads KV head h // (Hq / Hkv).  Rows are evaluated in chunks only to
bound memory; every row is computed on its own, so chunking does not change
any result.
"""
from __future__ import annotations

import concurrent.futures as cf
import contextlib

import numpy as np

from .cache import PagedCache
from .codec import bf16_to_f32

_ROW_CHUNK = 512


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, last_visible: np.ndarray,
           sm_scale: float):
    """q [n][D], k/v [m][D] float64; row i sees keys 0..last_visible[i].

    Returns (o [n][D], lse [n]).  A row that sees no key gives NaN.
    """
    n, m = q.shape[0], k.shape[0]
    o = np.full((n, v.shape[1]), np.nan)
    lse = np.full(n, np.nan)
    cols = np.arange(m)
    for r0 in range(0, n, _ROW_CHUNK):
        r1 = min(n, r0 + _ROW_CHUNK)
        z = sm_scale * (q[r0:r1] @ k.T)
        z[cols[None, :] > np.asarray(last_visible[r0:r1])[:, None]] = -np.inf
        zmax = z.max(axis=1, initial=-np.inf)
        ok = np.isfinite(zmax)
        e = np.exp(z[ok] - zmax[ok, None])
        den = e.sum(axis=1)
        o[r0:r1][ok] = (e @ v) / den[:, None]
        lse[r0:r1][ok] = zmax[ok] + np.log(den)
    return o, lse


def _run(tasks, workers: int):
    """Run independent tasks (callables), in a thread pool when workers > 1 (each task then
    uses one BLAS thread, so the pool does not oversubscribe the cores)."""
    if workers <= 1:
        for t in tasks:
            t()
        return
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1, user_api="blas")
    except ImportError:  # pragma: no cover
        limit = contextlib.nullcontext()
    with limit, cf.ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(t) for t in tasks]:
            f.result()


def prefill(cache: PagedCache, q_bits: np.ndarray, cu_seqlens_q, kv_lens, block_table,
            sm_scale: float, causal: bool = True, rows=None, heads=None, workers: int = 1):
    """Causal paged prefill.  q_bits: bf16 patterns [total_q][Hq][D].

    ``rows`` (optional) lists the query-token indices to evaluate, ``heads`` (optional) the
    query heads; the others are left NaN.  ``workers`` > 1 evaluates (sequence, head) pairs in
    that many threads.  Returns (o [total_q][Hq][D], lse [total_q][Hq]) in float64.
    """
    q = bf16_to_f32(q_bits).astype(np.float64)
    total_q, hq, d = q.shape
    group = hq // cache.num_kv_heads
    o = np.full((total_q, hq, d), np.nan)
    lse = np.full((total_q, hq), np.nan)
    want = np.ones(total_q, bool) if rows is None else np.isin(np.arange(total_q), rows)
    cu = np.asarray(cu_seqlens_q)
    tasks = []
    for b in range(len(kv_lens)):
        q0, q1, kvl = int(cu[b]), int(cu[b + 1]), int(kv_lens[b])
        idx = np.nonzero(want[q0:q1])[0]
        if len(idx) == 0:
            continue
        kh, vh = cache.gather(block_table[b], kvl)
        qlen = q1 - q0
        last = (kvl - qlen + idx) if causal else np.full(len(idx), kvl - 1)
        for h in (range(hq) if heads is None else heads):
            def task(rows_=q0 + idx, h=h, kh=kh, vh=vh, last=last):
                oh, lh = attend(q[rows_, h], kh[:, h // group], vh[:, h // group], last, sm_scale)
                o[rows_, h] = oh
                lse[rows_, h] = lh
            tasks.append(task)
    _run(tasks, workers)
    return o, lse


def decode(cache: PagedCache, q_bits: np.ndarray, kv_lens, block_table, sm_scale: float,
           seqs=None, workers: int = 1):
    """Single-token decode: q_bits [B][Hq][D]; query b sees all kv_lens[b] keys.

    ``seqs`` (optional) restricts the evaluation to those sequences; ``workers`` > 1 evaluates
    the sequences in that many threads.
    """
    q = bf16_to_f32(q_bits).astype(np.float64)
    bsz, hq, d = q.shape
    group = hq // cache.num_kv_heads
    o = np.full((bsz, hq, d), np.nan)
    lse = np.full((bsz, hq), np.nan)

    def one(b):
        kvl = int(kv_lens[b])
        kh, vh = cache.gather(block_table[b], kvl)
        for h in range(hq):
            oh, lh = attend(q[b, h][None, :], kh[:, h // group], vh[:, h // group],
                            np.array([kvl - 1]), sm_scale)
            o[b, h], lse[b, h] = oh[0], lh[0]

    _run([lambda b=b: one(b) for b in (range(bsz) if seqs is None else seqs)], workers)
    return o, lse
