"""Paged FP8 (E4M3FN) KV cache, oracle side: the control format the pages compare NVFP4
against (test infrastructure; see the package docstring).

"NVFP4 KV cache prefill vs decode performance" and "NVFP4 KV cache A4Q prefill explained"
quote every result as NVFP4 against an FP8 KV cache.  Reading: one E4M3FN byte per value and
one per-tensor scale g per K or V (the writer stores E4M3(fl32(x / g)), the reader multiplies
by g), in the same paged layout as the NVFP4 cache without the block-scale plane:

* ``X_data [num_pages][num_kv_heads][page_size][head_dim]`` uint8

The interface mirrors ``cache.PagedCache``, so the attention oracle reads either cache.
"""
from __future__ import annotations

import numpy as np

from . import codec
from .cache import map_tokens


class Fp8PagedCache:
    def __init__(self, num_pages: int, num_kv_heads: int, head_dim: int = 128,
                 page_size: int = 16, k_global: float = 1.0, v_global: float = 1.0):
        shape = (num_pages, num_kv_heads, page_size, head_dim)
        self.k_data = np.zeros(shape, np.uint8)
        self.v_data = np.zeros(shape, np.uint8)
        self.num_pages, self.num_kv_heads = num_pages, num_kv_heads
        self.head_dim, self.page_size = head_dim, page_size
        self.k_global, self.v_global = float(k_global), float(v_global)

    def nbytes(self) -> int:
        return self.k_data.nbytes + self.v_data.nbytes

    def append(self, k_bits: np.ndarray, v_bits: np.ndarray, slot_mapping: np.ndarray,
               input_dtype: str = "bf16", workers: int = 1):
        """Quantize bf16 or fp16 K/V ``[T][num_kv_heads][head_dim]`` and write their slots
        (``workers`` > 1: chunks of tokens in that many threads)."""
        slots = np.asarray(slot_mapping, dtype=np.int64)
        keep = slots >= 0
        page = slots[keep] // self.page_size
        off = slots[keep] % self.page_size
        for bits, data, g in ((k_bits, self.k_data, self.k_global), (v_bits, self.v_data, self.v_global)):
            codes = map_tokens(lambda c, g=g: codec.quantize_fp8(codec.input_to_f32(c, input_dtype), g),
                               np.asarray(bits), workers)
            data[page, :, off, :] = codes[keep]

    def dequant_slots(self, slot_mapping: np.ndarray, out_dtype: str = "bf16"):
        """The standalone dequantization: rows of the given slots as g * e4m3(code), formed in
        float32 (e4m3(code) is exact there; the product with g rounds once) and rounded to
        nearest-even in the output type; slots < 0 give zero rows.  Returns (k, v), each
        [n][num_kv_heads][head_dim] (bit patterns for bf16 / fp16, float32 for f32)."""
        slots = np.asarray(slot_mapping, dtype=np.int64)
        keep = slots >= 0
        page = np.where(keep, slots // self.page_size, 0)
        off = np.where(keep, slots % self.page_size, 0)
        out = []
        for data, g in ((self.k_data, self.k_global), (self.v_data, self.v_global)):
            x = codec.e4m3_value(data[page, :, off, :]).astype(np.float32) * np.float32(g)
            x = np.where(keep[:, None, None], x, np.float32(0)).astype(np.float32)
            out.append(codec.round_to_dtype(x, out_dtype))
        return out[0], out[1]

    def gather(self, block_table_row: np.ndarray, n: int):
        """Dequantized K and V of positions 0..n-1 of one sequence: float64 [n][H][D]."""
        pos = np.arange(n)
        pages = np.asarray(block_table_row, dtype=np.int64)[pos // self.page_size]
        off = pos % self.page_size
        return (codec.dequantize_fp8(self.k_data[pages, :, off, :], self.k_global),
                codec.dequantize_fp8(self.v_data[pages, :, off, :], self.v_global))
