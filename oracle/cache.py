"""Paged NVFP4 KV cache, oracle side (test infrastructure; see the package docstring).

The cache writer quantizes bf16 K/V vectors, chooses block scales, packs the
codes and stores each token's row at its slot in the page pool ("NVFP4 KV cache prefill vs
decode performance", section "NVFP4 stores 4.5 bits per value before
padding"; "NVFP4 KV cache vs NVFP4 weights", section "The cache quantizes
values during serving").  The block-scale plane is kept linear (row-major,
not swizzled), as the FP4 utility kernels of "NVFP4 KV cache A4Q prefill
explained", section "Preserve the capacity and decode case" use it.

Page layout (a reading; the pages fix no layout), per layer and for X in {K, V}:

* ``X_data [num_pages][num_kv_heads][page_size][head_dim / 2]`` uint8
* ``X_scale[num_pages][num_kv_heads][page_size][head_dim / 16]`` uint8

A slot is ``page * page_size + offset``; slots < 0 are skipped.  Slots within
one append call are assumed distinct.
"""
from __future__ import annotations

import concurrent.futures as cf

import numpy as np

from . import codec

_TOKENS_PER_TASK = 2048


def map_tokens(fn, bits: np.ndarray, workers: int):
    """fn over consecutive token chunks of ``bits`` (each token's result depends on that token
    alone), in a thread pool when ``workers`` > 1; the chunk results joined in token order."""
    if workers <= 1 or len(bits) <= _TOKENS_PER_TASK:
        return fn(bits)
    chunks = [bits[i:i + _TOKENS_PER_TASK] for i in range(0, len(bits), _TOKENS_PER_TASK)]
    with cf.ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(fn, chunks))
    if isinstance(parts[0], tuple):
        return tuple(np.concatenate([p[i] for p in parts]) for i in range(len(parts[0])))
    return np.concatenate(parts)


class PagedCache:
    def __init__(self, num_pages: int, num_kv_heads: int, head_dim: int = 128,
                 page_size: int = 16, k_global: float = 1.0, v_global: float = 1.0):
        shape_d = (num_pages, num_kv_heads, page_size, head_dim // 2)
        shape_s = (num_pages, num_kv_heads, page_size, head_dim // codec.BLOCK)
        self.k_data = np.zeros(shape_d, np.uint8)
        self.v_data = np.zeros(shape_d, np.uint8)
        self.k_scale = np.zeros(shape_s, np.uint8)
        self.v_scale = np.zeros(shape_s, np.uint8)
        self.num_pages, self.num_kv_heads = num_pages, num_kv_heads
        self.head_dim, self.page_size = head_dim, page_size
        self.k_global, self.v_global = float(k_global), float(v_global)

    def nbytes(self) -> int:
        return sum(a.nbytes for a in (self.k_data, self.v_data, self.k_scale, self.v_scale))

    def append(self, k_bits: np.ndarray, v_bits: np.ndarray, slot_mapping: np.ndarray,
               input_dtype: str = "bf16", workers: int = 1):
        """Quantize bf16 or fp16 K/V ``[T][num_kv_heads][head_dim]`` (bit patterns) and write
        them to their slots ("NVFP4 KV cache A4Q prefill explained", section "Preserve the
        capacity and decode case": the writer takes BF16 or FP16 input).  ``workers`` > 1
        quantizes chunks of tokens in that many threads (tokens are independent)."""
        slots = np.asarray(slot_mapping, dtype=np.int64)
        keep = slots >= 0
        page = slots[keep] // self.page_size
        off = slots[keep] % self.page_size

        for bits, data, scale, g in ((k_bits, self.k_data, self.k_scale, self.k_global),
                                     (v_bits, self.v_data, self.v_scale, self.v_global)):
            def one(chunk, g=g):
                codes, sc = codec.quantize(codec.input_to_f32(chunk, input_dtype), g)
                return codec.pack(codes), sc
            packed, sc = map_tokens(one, np.asarray(bits), workers)
            data[page, :, off, :] = packed[keep]
            scale[page, :, off, :] = sc[keep]

    def token_rows(self, pages: np.ndarray, offsets: np.ndarray):
        """Packed rows and scale codes of the given (page, offset) tokens:
        (k_data, k_scale, v_data, v_scale), each [n][num_kv_heads][...]."""
        return (self.k_data[pages, :, offsets, :], self.k_scale[pages, :, offsets, :],
                self.v_data[pages, :, offsets, :], self.v_scale[pages, :, offsets, :])

    def dequant_slots(self, slot_mapping: np.ndarray, out_dtype: str = "bf16"):
        """The standalone dequantization: rows of the given slots as g * s * e2m1(code),
        formed in float32 (s * e2m1 is exact there; the product with g rounds once) and rounded
        to nearest-even in the output type; slots < 0 give zero rows.  Returns (k, v), each
        [n][num_kv_heads][head_dim] (bit patterns for bf16 / fp16, float32 for f32)."""
        slots = np.asarray(slot_mapping, dtype=np.int64)
        keep = slots >= 0
        page = np.where(keep, slots // self.page_size, 0)
        off = np.where(keep, slots % self.page_size, 0)
        out = []
        for data, scale, g in ((self.k_data, self.k_scale, self.k_global),
                               (self.v_data, self.v_scale, self.v_global)):
            codes = codec.unpack(data[page, :, off, :])
            s = np.repeat(codec.e4m3_value(scale[page, :, off, :]), codec.BLOCK, axis=-1)
            x = (s * codec.e2m1_value(codes)).astype(np.float32) * np.float32(g)
            x = np.where(keep[:, None, None], x, np.float32(0)).astype(np.float32)
            out.append(codec.round_to_dtype(x, out_dtype))
        return out[0], out[1]

    def repack(self, block_table: np.ndarray, kv_lens):
        """Dequantize-ahead repack ("NVFP4 KV cache A4Q prefill explained", section "Compare A4Q
        with dequantize-ahead repacking": each NVFP4 tile is converted once to FP16 before
        attention uses it): every page holding keys 0..kv_lens[b]-1 of a sequence becomes
        fp16 s * e2m1(code) (exact; the per-tensor scale g is left to the reader, as for the
        packed cache).  Returns fp16 bit patterns (k, v), each [num_pages][num_kv_heads]
        [page_size][head_dim]; pages no sequence reaches stay zero."""
        bt = np.asarray(block_table, dtype=np.int64)
        out = []
        for data, scale in ((self.k_data, self.k_scale), (self.v_data, self.v_scale)):
            o = np.zeros(data.shape[:-1] + (data.shape[-1] * 2,), np.uint16)
            for b, n in enumerate(np.asarray(kv_lens, dtype=np.int64)):
                pages = bt[b, : (int(n) + self.page_size - 1) // self.page_size]
                x = codec.dequantize(data[pages], scale[pages])  # exact s * e2m1 in float64
                o[pages] = codec.round_to_dtype(x.astype(np.float32), "fp16")
            out.append(o)
        return out[0], out[1]

    def gather(self, block_table_row: np.ndarray, n: int):
        """Dequantized K and V of positions 0..n-1 of one sequence: float64 [n][H][D]."""
        pos = np.arange(n)
        pages = np.asarray(block_table_row, dtype=np.int64)[pos // self.page_size]
        kd, ks, vd, vs = self.token_rows(pages, pos % self.page_size)
        return (codec.dequantize(kd, ks, self.k_global), codec.dequantize(vd, vs, self.v_global))
