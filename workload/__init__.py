"""Seeded synthetic inputs for NVFP4 paged-KV attention.

This module is shared by the tests, the benchmark and the oracle's callers.
It holds none of the method's arithmetic: it draws Gaussian values, rounds the
draws to bfloat16 bit patterns (the input dtype of the cache writer), and does
page-table / slot bookkeeping.  Everything it returns is plain numpy.

The five workloads follow the shapes the pages benchmark:

* ``tiny``         batch 1, q = kv = 256, 4 query heads over 1 KV head, two K
                   outlier channels x8 (a small parity case);
* ``tail128``      batch 4, 128 query tokens over 2048 KV tokens, 32/8 heads,
                   2 % of K channels x8 (the shape of the repacking benchmark
                   in "NVFP4 KV cache A4Q prefill explained", section
                   "Compare A4Q with dequantize-ahead repacking");
* ``full16k``      one 16,384-token causal prefill, 32/8 heads, K outlier
                   channels x8 (the controlled 16K run in the same page,
                   section "Quantize Q instead of expanding K");
* ``tail16``       batch 8, 16 new query tokens over 16,384 cached tokens
                   (chunked-prefill tails, section "Compare A4Q with
                   dequantize-ahead repacking");
* ``decode``       batch 64, single-token decode over 16K..32K cached tokens
                   with one appended token per step, 64 steps ("NVFP4 KV cache
                   prefill vs decode performance", section "Decode can win on
                   fewer bytes read").

Seeds: ``seed = 1000 + index`` (index 1..5 in the order above).  A
``SeedSequence(seed)`` is spawned into ``batch + 4`` children: one per sequence
(its K, V and Q, drawn in that order), then the page permutation, the
decode-step queries, the K outlier channels and the decode lengths.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

PAGE_SIZE = 16
HEAD_DIM = 128


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs here are finite Gaussian
    draws, so NaN handling is not needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    name: str
    index: int
    batch: int
    q_lens: list
    kv_lens: list
    num_qo_heads: int
    num_kv_heads: int
    k_outlier_channels: int  # number of (kv head, dim) channels of K scaled x8
    head_dim: int = HEAD_DIM
    page_size: int = PAGE_SIZE
    decode_steps: int = 0  # > 0 only for the decode workload
    outlier_factor: float = 8.0
    k_global: float = 1.0
    v_global: float = 1.0

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def group(self) -> int:
        return self.num_qo_heads // self.num_kv_heads

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def describe(self) -> dict:
        d = dict(workload=self.name, batch=self.batch, num_qo_heads=self.num_qo_heads,
                 num_kv_heads=self.num_kv_heads, head_dim=self.head_dim,
                 page_size=self.page_size, seed=self.seed)
        if self.decode_steps:
            d.update(decode_steps=self.decode_steps, kv_len_min=min(self.kv_lens),
                     kv_len_max=max(self.kv_lens) + self.decode_steps - 1)
        else:
            d.update(q_len=self.q_lens[0] if len(set(self.q_lens)) == 1 else self.q_lens,
                     kv_len=self.kv_lens[0] if len(set(self.kv_lens)) == 1 else self.kv_lens)
        return d


def _child(seed: int, batch: int, k: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed).spawn(batch + 4)[k])


def _seq_rngs(seed: int, batch: int) -> list:
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(batch + 4)[:batch]]


def _perm_rng(seed, batch):
    return _child(seed, batch, batch)


def _step_rng(seed, batch):
    return _child(seed, batch, batch + 1)


def _outlier_rng(seed, batch):
    return _child(seed, batch, batch + 2)


def _length_rng(seed, batch):
    return _child(seed, batch, batch + 3)


def decode_lengths(seed: int, batch: int, kv_max: int, steps: int, kv_min: int) -> list:
    """Initial decode lengths L_b, uniform over {kv_min, ..., kv_max - steps + 1}.

    Step t (0-based) attends over L_b + t tokens, so every decode call sees a
    KV length in [kv_min, kv_max].
    """
    rng = _length_rng(seed, batch)
    return [int(x) for x in rng.integers(kv_min, kv_max - steps + 2, size=batch)]


def get(name_or_index) -> Workload:
    table = {
        "tiny": lambda: Workload("tiny", 1, 1, [256], [256], 4, 1, 2),
        "tail128": lambda: Workload("tail128", 2, 4, [128] * 4, [2048] * 4, 32, 8, 20),
        "full16k": lambda: Workload("full16k", 3, 1, [16384], [16384], 32, 8, 20),
        "tail16": lambda: Workload("tail16", 4, 8, [16] * 8, [16384] * 8, 32, 8, 0),
        "decode": lambda: _decode_workload(),
        "full8k": lambda: Workload("full8k", 6, 1, [8192], [8192], 32, 8, 20),
        "full32k": lambda: Workload("full32k", 7, 1, [32768], [32768], 32, 8, 20),
    }
    if isinstance(name_or_index, int):
        name_or_index = list(table)[name_or_index - 1]
    return table[name_or_index]()


def _decode_workload(batch: int = 64, steps: int = 64, kv_min: int = 16384,
                     kv_max: int = 32768) -> Workload:
    lens = decode_lengths(1005, batch, kv_max, steps, kv_min)
    return Workload("decode", 5, batch, [1] * batch, lens, 32, 8, 0, decode_steps=steps)


ALL = ("tiny", "tail128", "full16k", "tail16", "decode", "full8k", "full32k")


def custom(name: str, q_lens, kv_lens, num_qo_heads: int, num_kv_heads: int, seed: int,
           k_outlier_channels: int = 0, head_dim: int = HEAD_DIM, k_global: float = 1.0,
           v_global: float = 1.0) -> Workload:
    """A workload of arbitrary shape (tests use it for ragged and edge cases)."""
    w = Workload(name, seed - 1000, len(q_lens), list(q_lens), list(kv_lens), num_qo_heads,
                 num_kv_heads, k_outlier_channels, head_dim=head_dim, k_global=k_global,
                 v_global=v_global)
    return w


# ----------------------------------------------------------------------------------------
# Page tables and slot mapping
# ----------------------------------------------------------------------------------------

@dataclass
class PageLayout:
    num_pages: int
    block_table: np.ndarray  # int32 [B][max_pages]; padded with 0
    pages_per_seq: list = field(default_factory=list)

    def slots(self, b: int, positions: np.ndarray) -> np.ndarray:
        """Cache slot of each token position of sequence b: page * page_size + offset."""
        positions = np.asarray(positions, dtype=np.int64)
        pages = self.block_table[b][positions // PAGE_SIZE].astype(np.int64)
        return pages * PAGE_SIZE + positions % PAGE_SIZE


def page_layout(w: Workload, capacity_lens=None) -> PageLayout:
    """A seeded random permutation of the whole page pool, handed out per sequence."""
    lens = capacity_lens if capacity_lens is not None else w.kv_lens
    per_seq = [(int(n) + PAGE_SIZE - 1) // PAGE_SIZE for n in lens]
    total = sum(per_seq)
    rng = _perm_rng(w.seed, w.batch)
    perm = rng.permutation(total).astype(np.int32)
    maxp = max(per_seq) if per_seq else 0
    bt = np.zeros((w.batch, max(maxp, 1)), dtype=np.int32)
    off = 0
    for b, n in enumerate(per_seq):
        bt[b, :n] = perm[off:off + n]
        off += n
    return PageLayout(total, bt, per_seq)


def outlier_channels(w: Workload) -> np.ndarray:
    """Flat indices (kv_head * head_dim + dim) of the K channels scaled by 8."""
    if w.k_outlier_channels == 0:
        return np.zeros(0, dtype=np.int64)
    rng = _outlier_rng(w.seed, w.batch)
    return np.sort(rng.choice(w.num_kv_heads * w.head_dim, size=w.k_outlier_channels,
                              replace=False)).astype(np.int64)


def _draw_kv(rng: np.random.Generator, n: int, w: Workload, chans: np.ndarray):
    shape = (n, w.num_kv_heads, w.head_dim)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if len(chans):
        kf = k.reshape(n, -1)
        kf[:, chans] *= np.float32(w.outlier_factor)
    return f32_to_bf16_bits(k), f32_to_bf16_bits(v)


@dataclass
class PrefillCase:
    w: Workload
    layout: PageLayout
    k_bits: np.ndarray        # uint16 [T][Hkv][D]  (all kv tokens of all sequences)
    v_bits: np.ndarray
    slot_mapping: np.ndarray  # int64 [T]
    q_bits: np.ndarray        # uint16 [total_q][Hq][D]
    cu_seqlens_q: np.ndarray  # int32 [B+1]
    kv_lens: np.ndarray       # int32 [B]
    cu_seqlens_kv: np.ndarray  # int32 [B+1], token offsets into k_bits/v_bits

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def max_q_len(self) -> int:
        return int(np.diff(self.cu_seqlens_q).max(initial=0))

    @property
    def max_kv_len(self) -> int:
        return int(self.kv_lens.max(initial=0))


def prefill_case(w: Workload) -> PrefillCase:
    """Q for the last q_len positions of each sequence and K/V for all kv_len positions.

    The K/V of every position (the cached prefix and the new chunk alike) is
    appended to the cache before the prefill reads it.
    """
    assert not w.decode_steps
    layout = page_layout(w)
    chans = outlier_channels(w)
    rngs = _seq_rngs(w.seed, w.batch)
    ks, vs, qs, slots = [], [], [], []
    for b in range(w.batch):
        k, v = _draw_kv(rngs[b], w.kv_lens[b], w, chans)
        q = f32_to_bf16_bits(rngs[b].standard_normal((w.q_lens[b], w.num_qo_heads, w.head_dim),
                                                     dtype=np.float32))
        ks.append(k); vs.append(v); qs.append(q)
        slots.append(layout.slots(b, np.arange(w.kv_lens[b])))
    empty = np.zeros((0, w.num_kv_heads, w.head_dim), np.uint16)
    cu_q = np.zeros(w.batch + 1, np.int32); cu_q[1:] = np.cumsum(w.q_lens)
    cu_kv = np.zeros(w.batch + 1, np.int32); cu_kv[1:] = np.cumsum(w.kv_lens)
    return PrefillCase(
        w, layout,
        np.concatenate(ks) if ks else empty, np.concatenate(vs) if vs else empty,
        np.concatenate(slots).astype(np.int64) if slots else np.zeros(0, np.int64),
        np.concatenate(qs) if qs else np.zeros((0, w.num_qo_heads, w.head_dim), np.uint16),
        cu_q, np.asarray(w.kv_lens, np.int32), cu_kv)


@dataclass
class DecodeCase:
    """Decode workload: sequence b starts with L_b - 1 cached tokens; step t appends
    position L_b - 1 + t and decodes over L_b + t tokens."""
    w: Workload
    layout: PageLayout
    init_lens: np.ndarray  # L_b

    def seq_kv(self, b: int):
        """K/V bf16 bits of all positions 0 .. L_b + steps - 2 of sequence b."""
        rng = _seq_rngs(self.w.seed, self.w.batch)[b]
        return _draw_kv(rng, int(self.init_lens[b]) + self.w.decode_steps - 1, self.w,
                        np.zeros(0, np.int64))

    def seq_kv_initial(self, b: int):
        k, v = self.seq_kv(b)
        n = int(self.init_lens[b]) - 1
        return k[:n], v[:n]

    def step_q(self):
        """Queries of every step: uint16 [steps][B][Hq][D]."""
        rng = _step_rng(self.w.seed, self.w.batch)
        x = rng.standard_normal((self.w.decode_steps, self.w.batch, self.w.num_qo_heads,
                                 self.w.head_dim), dtype=np.float32)
        return f32_to_bf16_bits(x)

    def step_slots(self, t: int) -> np.ndarray:
        return np.array([self.layout.slots(b, [int(self.init_lens[b]) - 1 + t])[0]
                         for b in range(self.w.batch)], dtype=np.int64)

    def step_kv_lens(self, t: int) -> np.ndarray:
        return (self.init_lens + t).astype(np.int32)


def decode_case(w: Workload) -> DecodeCase:
    assert w.decode_steps
    lens = np.asarray(w.kv_lens, dtype=np.int64)
    layout = page_layout(w, capacity_lens=lens + w.decode_steps - 1)
    return DecodeCase(w, layout, lens.astype(np.int32))


# ----------------------------------------------------------------------------------------
# Stress transforms of seeded inputs (value-range edge cases; no method arithmetic)
# ----------------------------------------------------------------------------------------

def scale_channels(bits: np.ndarray, seed: int, per_head: int, factor: float) -> np.ndarray:
    """bf16 patterns [T][H][D] with `per_head` seeded channels of every head multiplied by
    `factor` (then rounded to bf16): outlier channels on the query side."""
    rng = np.random.default_rng(seed)
    x = bf16_bits_to_f32(bits).copy()
    for h in range(x.shape[1]):
        x[:, h, rng.choice(x.shape[2], per_head, replace=False)] *= np.float32(factor)
    return f32_to_bf16_bits(x)


def scale_tokens_pow2(bits: np.ndarray, seed: int, lo: int, hi: int) -> np.ndarray:
    """bf16 patterns [T][H][D] with every token multiplied by its own seeded power of two
    2^e, e uniform in [lo, hi] (exact in bf16 inside its range): a wide dynamic range of block
    scales across tokens."""
    rng = np.random.default_rng(seed)
    e = rng.integers(lo, hi + 1, size=bits.shape[0]).astype(np.float32)
    x = bf16_bits_to_f32(bits) * np.exp2(e)[:, None, None].astype(np.float32)
    return f32_to_bf16_bits(x.astype(np.float32))
