// Device-side pieces shared by the prefill kernels (stock and A4Q-style): the LDS tile layout,
// packed-tile loads and their dequantization into LDS, the score, softmax and PV stages of one
// 64-key tile, the work-item and query-column bookkeeping, the query load and the epilogue.
#pragma once

#include "device_common.hpp"
#include "kernel_params.hpp"

namespace nvfp4kv {

constexpr int kTileKeys = 64;
constexpr int kKStride = 272;  // LDS bytes per K row: 256 + 16 pad (conflict-free 16 B accesses)
constexpr int kVStride = 256;  // LDS bytes per V row, 16-byte slots swizzled by v_offset()
constexpr int kKTileBytes = kTileKeys * kKStride;
constexpr int kVTileBytes = kTileKeys * kVStride;
constexpr int kBufBytes = kKTileBytes + kVTileBytes;

// Byte offset of 16-byte slot `slot` (0..15, i.e. head-dim values 8*slot..8*slot+7) of V row
// `key` in a V tile.  The slot index is XORed with 5 * (key & 3): the 64-byte granule index and
// the slot within the granule are both XORed with key & 3.  Then the 16 lanes of a dequantized
// write (4 keys x 4 quarters, one slot each) hit 16 distinct slots, and the 4 keys of a
// transposing read (one 64-byte granule each) hit 4 distinct granules.
__device__ __forceinline__ int v_offset(int key, int slot) {
  return key * kVStride + 16 * (slot ^ (5 * (key & 3)));
}

template <int NW, int FMT>
struct TileRegs {
  static constexpr int kItems = 512 / (64 * NW);  // 32-value chunks per thread per tile
  // 16-byte words per chunk: NVFP4 16 packed bytes, FP8 32 bytes, fp16 64 bytes
  static constexpr int kWords = FMT == kFmtNvfp4 ? 1 : (FMT == kFmtFp8 ? 2 : 4);
  static constexpr int kRowStride = FMT == kFmtNvfp4 ? kRowBytes : kHeadDim * kWords / 2;
  u32x4 data[kItems][kWords];
  uint32_t scale[FMT == kFmtNvfp4 ? kItems : 1];  // NVFP4: the chunk's two scale bytes
  int32_t page[kItems];  // page ids of the next tile to load (same value in every lane)
};

// Chunk `it` of a tile (0..511): X = it / 256 (K or V), key = (it % 256) / 4, quarter = it % 4
// (32 head-dim values).  A wavefront's 64 chunks are the 16 keys of one page.

// Fetch the page ids of tile `kt` with vector loads (one word, the same in every lane; `vzero`
// is a zero the compiler cannot see as uniform, which keeps the loads off the scalar path, whose
// wait would also drain the LDS queue).  Pages past the sequence's last page are clamped to it.
template <int NW, int FMT>
__device__ __forceinline__ void fetch_pages(const int32_t* bt_row, int kv_len, int kt, int vzero,
                                            TileRegs<NW, FMT>& r) {
  const int last_page = (kv_len - 1) >> 4;
#pragma unroll
  for (int j = 0; j < TileRegs<NW, FMT>::kItems; ++j) {
    const int sub = ((threadIdx.x + 64 * NW * j) & 255) >> 6;  // page of the tile, wave-uniform
    r.page[j] = bt_row[min(4 * kt + sub, last_page) + vzero];
  }
}

// Load the packed K and V chunks of tile `kt` that this thread dequantizes, using the page ids
// fetched for it, then fetch the page ids of tile `kt_next`.  Keys at or past kv_len are clamped
// to the last key: every load is unconditional and reads written cache bytes, and those keys are
// masked out of the softmax.
template <int NW, int FMT>
__device__ __forceinline__ void load_tile(const PrefillParams& p, const int32_t* bt_row, int hk,
                                          int kv_len, int kt, int kt_next, int vzero,
                                          TileRegs<NW, FMT>& r) {
  const int last = kv_len - 1;
#pragma unroll
  for (int j = 0; j < TileRegs<NW, FMT>::kItems; ++j) {
    const int it = threadIdx.x + 64 * NW * j;
    const int X = it >> 8;
    const int key = (it & 255) >> 2;
    const int qq = it & 3;
    const int page = uniform(r.page[j]);
    const int gkey = min(kt * kTileKeys + key, last);
    const int64_t row = ((int64_t)page * p.num_kv_heads + hk) * kPageSize + (gkey & 15);
    constexpr int kW = TileRegs<NW, FMT>::kWords;
    const uint8_t* dp = (X == 0 ? p.k_data : p.v_data) + row * TileRegs<NW, FMT>::kRowStride + 16 * kW * qq;
#pragma unroll
    for (int c = 0; c < kW; ++c) r.data[j][c] = *(const u32x4*)(dp + 16 * c);
    if constexpr (FMT == kFmtNvfp4) {
      const uint8_t* sp = (X == 0 ? p.k_scale : p.v_scale) + row * kScaleBytes + 2 * qq;
      r.scale[j] = *(const uint16_t*)sp;
    }
  }
  fetch_pages<NW, FMT>(bt_row, kv_len, kt_next, vzero, r);
}

// A zero held in a vector register that the compiler treats as lane-varying.
__device__ __forceinline__ int opaque_vzero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// Dequantize the loaded chunks to fp16 (exact) and write them to an LDS tile buffer.  The K / V
// choice is made with selects, not branches, so the tile stages stay one scheduling region.
template <int NW, int FMT>
__device__ __forceinline__ void store_tile(char* buf, const TileRegs<NW, FMT>& r) {
#pragma unroll
  for (int j = 0; j < TileRegs<NW, FMT>::kItems; ++j) {
    const int it = threadIdx.x + 64 * NW * j;
    const bool is_v = (it >> 8) != 0;
    const int key = (it & 255) >> 2;
    const int qq = it & 3;
    uint32_t o[16];
    if constexpr (FMT == kFmtNvfp4) {
      const f16x2 sc = e4m3_pair_h<false>(r.scale[j]);
      const f16x2 s0 = __builtin_shufflevector(sc, sc, 0, 0);
      const f16x2 s1 = __builtin_shufflevector(sc, sc, 1, 1);
      dequant8_h(r.data[j][0][0], s0, o + 0);
      dequant8_h(r.data[j][0][1], s0, o + 4);
      dequant8_h(r.data[j][0][2], s1, o + 8);
      dequant8_h(r.data[j][0][3], s1, o + 12);
    } else if constexpr (FMT == kFmtFp8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fp8x4_to_f16(r.data[j][0][i], o + 2 * i);
        fp8x4_to_f16(r.data[j][1][i], o + 8 + 2 * i);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[4 * c + i] = r.data[j][c][i];
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int off = is_v ? kKTileBytes + v_offset(key, 4 * qq + w) : key * kKStride + 64 * qq + 16 * w;
      *(u32x4*)(buf + off) = u32x4{o[4 * w], o[4 * w + 1], o[4 * w + 2], o[4 * w + 3]};
    }
  }
}

// S^T (64 keys x this wave's 32 columns) for the K tile in `buf`.  The K fragments of each
// k-step are read two k-steps ahead of their MFMAs; scheduling barriers keep that order (left
// alone, the compiler sinks every read next to its MFMA and each MFMA pair waits out a full
// LDS round trip).
__device__ __forceinline__ void tile_scores(const char* buf, int lane, const f16x8 (&qf)[8],
                                            f32x16& s0, f32x16& s1) {
  const char* kb = buf + (lane & 31) * kKStride + 16 * (lane >> 5);
  s0 = f32x16{};
  s1 = f32x16{};
  f16x8 a0[2], a1[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    a0[t] = *(const f16x8*)(kb + 32 * t);
    a1[t] = *(const f16x8*)(kb + 32 * kKStride + 32 * t);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    s0 = mfma32h(a0[t & 1], qf[t], s0);
    s1 = mfma32h(a1[t & 1], qf[t], s1);
    if (t + 2 < 8) {
      a0[t & 1] = *(const f16x8*)(kb + 32 * (t + 2));
      a1[t & 1] = *(const f16x8*)(kb + 32 * kKStride + 32 * (t + 2));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Causal / length mask on a tile whose keys start at k0: keys past the column's limit -> -inf.
__device__ __forceinline__ void tile_mask(f32x16& s0, f32x16& s1, int k0, int lim, int h32) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int key = k0 + 8 * (j >> 2) + 4 * h32 + (j & 3);
    if (key > lim) s0[j] = kNegInf;
    if (key + 32 > lim) s1[j] = kNegInf;
  }
}

// Running maximum (base 2) and lazy rescale: the reference maximum moves only when a tile's
// maximum exceeds it by more than 8, which keeps every weight <= 256.
__device__ __forceinline__ void tile_max_rescale(const f32x16& s0, const f32x16& s1, float cs,
                                                 float& m_used, float& l_part,
                                                 f32x16 (&acc_o)[4]) {
  float ma = fmaxf(s0[0], s0[1]);
  float mb = fmaxf(s1[0], s1[1]);
#pragma unroll
  for (int j = 2; j < 16; j += 2) {
    ma = fmaxf(fmaxf(ma, s0[j]), s0[j + 1]);
    mb = fmaxf(fmaxf(mb, s1[j]), s1[j + 1]);
  }
  const float mx = pair32_max(fmaxf(ma, mb)) * cs;
  if (wave_any(mx > m_used + 8.0f)) {
    const float m_new = fmaxf(m_used, mx);
    const float alpha = (m_new == kNegInf) ? 1.0f : fast_exp2(m_used - m_new);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc_o[i] *= alpha;
    l_part *= alpha;
    m_used = m_new;
  }
}

// Weights exp2(s * cs - m) as fp16 MFMA B operands (rounded toward zero, relative error below
// 2^-10); the row sum uses the same fp16 weights.
__device__ __forceinline__ void tile_probs(const f32x16& s0, const f32x16& s1, float cs,
                                           float m_used, f16x8 (&pb)[4], float& l_part) {
  const float mref = (m_used == kNegInf) ? 0.0f : m_used;
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    const f16x2 a = pack_f16x2_rtz(fast_exp2(fmaf(s0[j], cs, -mref)), fast_exp2(fmaf(s0[j + 1], cs, -mref)));
    const f16x2 b = pack_f16x2_rtz(fast_exp2(fmaf(s1[j], cs, -mref)), fast_exp2(fmaf(s1[j + 1], cs, -mref)));
    pb[j >> 3][j & 7] = a[0];
    pb[j >> 3][(j & 7) + 1] = a[1];
    pb[2 + (j >> 3)][j & 7] = b[0];
    pb[2 + (j >> 3)][(j & 7) + 1] = b[1];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) l_part = sum_f16x8(pb[u], l_part);
}

// O^T += V^T P^T: 4 head-dim blocks x (2 key blocks x 2 k-steps), for the V tile at `vtile`.
// The V^T operands come from the swizzled row-major V tile through transposing LDS reads: the
// lane reads 4 values of rows key0 and key0 + 8, with key0 = 16u + 4 h32 + t16/4, at head-dim
// offset 32 db + 16 (g16 & 1) + 4 (t16 & 3).
__device__ __forceinline__ void tile_pv_at(const char* vtile, int lane, const f16x8 (&pb)[4],
                                           f32x16 (&acc_o)[4]) {
  const int h32 = lane >> 5, g16 = lane >> 4, t16 = lane & 15;
  const int k4 = (t16 >> 2) & 3;  // key & 3 of every row this lane reads
  const int slot_lo = 2 * (g16 & 1) + ((t16 & 3) >> 1);
  const char* vb = vtile + (4 * h32 + (t16 >> 2)) * kVStride + 16 * (slot_lo ^ k4) + 8 * (t16 & 1);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const char* pa = vb + 16 * u * kVStride + 64 * (db ^ k4);
      const i16x4 lo = lds_read_tr16(pa);
      const i16x4 hi = lds_read_tr16(pa + 8 * kVStride);
      const f16x8 a = __builtin_bit_cast(
          f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc_o[db] = mfma32h(a, pb[u], acc_o[db]);
    }
  }
}

// The same for the V tile of a stock tile buffer (after its K tile).
__device__ __forceinline__ void tile_pv(const char* buf, int lane, const f16x8 (&pb)[4],
                                        f32x16 (&acc_o)[4]) {
  tile_pv_at(buf + kKTileBytes, lane, pb, acc_o);
}

// ---- work item and column bookkeeping shared by both kernels ------------------------------

struct PrefillItem {
  int split, b, hk, q_start, q_len, kv_len, pos0, pos_last, shift, t_begin, t_end;
};

// Work item of this workgroup: XCD-major so one KV head's items share an XCD; query tiles
// longest first.  Returns false if the workgroup has no rows.
__device__ __forceinline__ bool prefill_item(const PrefillParams& p, int cols, PrefillItem& w) {
  const int wg = blockIdx.x;
  const int item = (wg & 7) * p.items_per_xcd + (wg >> 3);
  if (item >= p.total_items) return false;
  w.split = item % p.num_splits;
  int r = item / p.num_splits;
  const int qt = p.q_tiles - 1 - (r % p.q_tiles);
  r /= p.q_tiles;
  w.b = r % p.batch;
  w.hk = r / p.batch;
  const int rows_per_tile = cols / p.group;
  w.q_start = p.cu_q[w.b];
  w.q_len = p.cu_q[w.b + 1] - w.q_start;
  w.kv_len = p.kv_lens[w.b];  // read with cu_q, not after the test below
  w.pos0 = qt * rows_per_tile;
  if (w.pos0 >= w.q_len) return false;
  w.pos_last = min(w.q_len, w.pos0 + rows_per_tile) - 1;
  w.shift = p.causal ? w.kv_len - w.q_len : 0;  // row i sees keys <= i + shift
  const int lim_tile = p.causal ? w.shift + w.pos_last : w.kv_len - 1;
  const int n_keys = max(0, min(w.kv_len, lim_tile + 1));
  const int n_tiles = (n_keys + kTileKeys - 1) / kTileKeys;
  const int per_split = (n_tiles + p.num_splits - 1) / p.num_splits;
  w.t_begin = w.split * per_split;
  w.t_end = min(n_tiles, w.t_begin + per_split);
  return true;
}

// This lane's query column (position, head) and the key limits of the lane and its wavefront.
struct PrefillCols {
  int h32, pos, head, lim, wlim_max, wlim_min;
  bool valid;
};

__device__ __forceinline__ PrefillCols prefill_cols(const PrefillParams& p, const PrefillItem& w,
                                                    int wave, int lane) {
  PrefillCols c;
  const int G = p.group;
  c.h32 = lane >> 5;
  const int col = 32 * wave + (lane & 31);
  c.pos = w.pos0 + col / G;
  c.head = w.hk * G + col % G;
  c.valid = c.pos <= w.pos_last;
  c.lim = c.valid ? (p.causal ? w.shift + c.pos : w.kv_len - 1) : -1;
  const int wpos_first = w.pos0 + (32 * wave) / G;
  const int wpos_last = w.pos0 + (32 * wave + 31) / G;
  const bool active = wpos_first <= w.pos_last;
  c.wlim_max = !active ? -1 : (p.causal ? w.shift + min(wpos_last, w.pos_last) : w.kv_len - 1);
  c.wlim_min = (!active || wpos_last > w.pos_last) ? -1
                                                   : (p.causal ? w.shift + wpos_first : w.kv_len - 1);
  return c;
}

// Q^T operand of this lane's column as fp16: 8 k-steps of 16 head-dim values (zero for padding
// lanes).  The column is scaled by 2^sh, chosen from its largest |q| (over the lane pair l, l^32)
// so that the largest lands in [2^15, 2^16): every bf16 element within a factor 2^32 of the
// largest converts exactly, and smaller ones are below float32 accumulation precision relative
// to it.  Returns score_scale * 2^-sh, which turns this column's MFMA scores into base-2 logits.
__device__ __forceinline__ float load_q(const PrefillParams& p, const PrefillItem& w,
                                        const PrefillCols& c, f16x8 (&qf)[8]) {
  const uint16_t* qp = p.q + ((int64_t)(w.q_start + (c.valid ? c.pos : 0)) * p.num_qo_heads + c.head) *
                                 kHeadDim + 8 * c.h32;
  // A padding lane reads the item's first row (it exists: an item starts inside its sequence)
  // and zeroes what it read, so the eight loads issue together with no branch between them.
  u32x4 raw[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) raw[t] = *(const u32x4*)(qp + 16 * t);
  float amax = 0.0f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (!c.valid) raw[t] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      amax = fmaxf(amax, fmaxf(fabsf(__builtin_bit_cast(float, raw[t][i] << 16)),
                               fabsf(__builtin_bit_cast(float, raw[t][i] & 0xFFFF0000u))));
  }
  amax = pair32_max(amax);
  const int sh = amax > 0.0f ? min(100, max(-100, 16 - __builtin_amdgcn_frexp_expf(amax))) : 0;
  const float up = __builtin_ldexpf(1.0f, sh);
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2 h = pack_f16x2_rtz(__builtin_bit_cast(float, raw[t][i] << 16) * up,
                                     __builtin_bit_cast(float, raw[t][i] & 0xFFFF0000u) * up);
      qf[t][2 * i] = h[0];
      qf[t][2 * i + 1] = h[1];
    }
  return p.score_scale * __builtin_ldexpf(1.0f, -sh);
}

// Normalise and store this lane's half of its column: O (bf16 or fp32) and the log-sum-exp,
// or, in split mode, the slice's normalised partial (fp16, nearest-even: before the per-tensor
// V scale it is a weighted mean of cache values, |x| <= 6 * 448, well inside fp16's range) and
// its base-2 log-sum-exp.
__device__ __forceinline__ void prefill_epilogue(const PrefillParams& p, const PrefillItem& w,
                                                 const PrefillCols& c, const f32x16 (&acc_o)[4],
                                                 float m_used, float l_part) {
  const float l_tot = pair32_sum(l_part);
  if (!c.valid) return;
  const int64_t orow = (int64_t)(w.q_start + c.pos) * p.num_qo_heads + c.head;
  const bool split_mode = p.num_splits > 1;
  const float inv = l_tot > 0.0f ? (split_mode ? 1.0f : p.out_scale) / l_tot : 0.0f;
  if (split_mode) {
    uint16_t* op = p.part_o + ((int64_t)w.split * p.total_q * p.num_qo_heads + orow) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d = 32 * db + 8 * jg + 4 * c.h32;
        *(u32x2*)(op + d) = u32x2{pack_f16x2_rne(acc_o[db][4 * jg] * inv, acc_o[db][4 * jg + 1] * inv),
                                  pack_f16x2_rne(acc_o[db][4 * jg + 2] * inv, acc_o[db][4 * jg + 3] * inv)};
      }
  } else if (p.out_f32) {
    float* op = (float*)p.out + orow * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d = 32 * db + 8 * jg + 4 * c.h32;
        *(f32x4*)(op + d) = f32x4{acc_o[db][4 * jg] * inv, acc_o[db][4 * jg + 1] * inv,
                                  acc_o[db][4 * jg + 2] * inv, acc_o[db][4 * jg + 3] * inv};
      }
  } else {
    uint16_t* op = (uint16_t*)p.out + orow * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d = 32 * db + 8 * jg + 4 * c.h32;
        *(u32x2*)(op + d) = u32x2{pack_bf16x2(acc_o[db][4 * jg] * inv, acc_o[db][4 * jg + 1] * inv),
                                  pack_bf16x2(acc_o[db][4 * jg + 2] * inv, acc_o[db][4 * jg + 3] * inv)};
      }
  }
  if (c.h32 != 0) return;
  const float lse2 = l_tot > 0.0f ? m_used + __log2f(l_tot) : kNegInf;
  if (split_mode)
    p.part_lse[(int64_t)w.split * p.total_q * p.num_qo_heads + orow] = lse2;
  else if (p.lse)
    p.lse[orow] = lse2 * kLn2;
}

}  // namespace nvfp4kv
