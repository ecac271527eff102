// Causal paged prefill over the NVFP4 KV cache for gfx950 (CDNA4).
//
// What is computed is the stock read path of "NVFP4 KV cache A4Q prefill explained" (section
// "Why NVFP4 KV cache A4Q prefill exists"): the packed K and V are unpacked, converted and
// scaled, and attention runs with bf16 queries.  The design is MI355X-first:
//
//  * A workgroup owns one KV head, one tile of query positions and (optionally) one slice of
//    the key range.  Its query "columns" are (position, head-of-group) pairs, so all query heads
//    that share the KV head use every dequantized KV tile: the unpack/scale work is paid once
//    per 64-key tile and amortised over 32 * waves columns.
//  * Each 64-key tile is loaded packed from HBM (72 B per key and head for each of K and V),
//    dequantized and written to LDS; the packed loads run two tiles ahead of their use.
//  * The tiles are fp16: every NVFP4 value (E2M1 code times E4M3 scale) is exact in fp16, and
//    the conversion is one fp4->fp16 convert plus one packed multiply per pair of values.  Q is
//    converted to fp16 once per workgroup with a per-column power-of-two scale (exact for every
//    element within 2^32 of the column's largest), folded into the softmax scale; the weights P
//    are fp16 too (relative error below 2^-10, finer than bf16).  K rows are padded to 272 B; V rows are 256 B with their
//    16-byte slots XOR-swizzled by key, so that both the dequantized writes and the transposing
//    reads are free of bank conflicts.
//  * Scores are computed transposed, S^T = K Q^T, with 32x32x16 fp16 MFMA: each lane then holds
//    16 keys of one query column per 32-key block, so the softmax row reduction is lane-local
//    plus one permlane32 swap, and P^T is already the B operand of O^T = V^T P^T.  V^T operands
//    come straight from the row-major V tile through the transposing LDS read.
//  * Online softmax in base 2 with the running maximum refreshed only when a tile's maximum
//    exceeds it by more than 8 (factor 256), which keeps P <= 256 and skips most rescales.
//  * Causal tile skipping: a workgroup walks only the keys its last row can see; waves whose
//    rows cannot see a tile skip its MFMAs; masks are applied only on tiles that need them.
//  * The workgroup -> work-item map sends all work of one KV head to one XCD (its L2 holds that
//    head's packed cache) and orders query tiles longest first.
//  * The kernels are templated on the cache format: NVFP4, the FP8 (E4M3FN) control cache, and
//    the fp16 copy the dequantize-ahead repack pass writes (stored to LDS without conversion).
#include "prefill_common.hpp"

namespace nvfp4kv {

// ---- narrow kernel: NW wavefronts of 32 columns, two LDS buffers ---------------------------
// Used for short query tiles, where the split-KV grid supplies the parallelism: NW = 4 (65..128
// columns); up to 64 columns go to the key-split kernel below, more than 128 to the 8-wave
// kernel.  It asks for two workgroups per CU (registers capped at 256: 232 for NVFP4, 246 for
// FP8, no spills; two tile buffers each fit the LDS twice), which the host's split count
// assumes; the fp16 (repacked) form would spill there and keeps one.
template <int NW, int FMT>
__global__ __launch_bounds__(64 * NW, FMT == kFmtF16 ? 1 : 2) void nvfp4_prefill_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kBufBytes];
  PrefillItem w;
  if (!prefill_item(p, 32 * NW, w)) return;
  const int lane = threadIdx.x & 63;
  const PrefillCols c = prefill_cols(p, w, uniform(threadIdx.x >> 6), lane);
  const int32_t* bt_row = p.block_table + (int64_t)w.b * p.bt_stride;
  const bool has_tiles = w.t_begin < w.t_end;
  const int vzero = opaque_vzero();
  const int t_last = w.t_end - 1;
  const int t0 = w.t_begin;
  // Three register sets in rotation: the packed loads of tile kt+4 are issued while tile kt is
  // consumed, so each tile's loads have three tiles of compute to arrive (these short-query
  // shapes are bound by memory latency).  The first three tiles' page ids are fetched before
  // the Q loads and their chunks loaded together.  Tile indices are clamped at t_last; writes
  // past the last tile land in a buffer that is not read again.
  TileRegs<NW, FMT> r0, r1, r2;
  if (has_tiles) {
    fetch_pages<NW, FMT>(bt_row, w.kv_len, t0, vzero, r0);
    fetch_pages<NW, FMT>(bt_row, w.kv_len, min(t0 + 1, t_last), vzero, r1);
    fetch_pages<NW, FMT>(bt_row, w.kv_len, min(t0 + 2, t_last), vzero, r2);
  }
  f16x8 qf[8];
  const float cs = load_q(p, w, c, qf);

  f32x16 acc_o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc_o[i] = f32x16{};
  float m_used = kNegInf;
  float l_part = 0.0f;

  if (has_tiles) {
    load_tile<NW, FMT>(p, bt_row, w.hk, w.kv_len, t0, min(t0 + 3, t_last), vzero, r0);
    load_tile<NW, FMT>(p, bt_row, w.hk, w.kv_len, min(t0 + 1, t_last), min(t0 + 4, t_last), vzero, r1);
    load_tile<NW, FMT>(p, bt_row, w.hk, w.kv_len, min(t0 + 2, t_last), min(t0 + 5, t_last), vzero, r2);
    store_tile<NW, FMT>(smem, r0);
    load_tile<NW, FMT>(p, bt_row, w.hk, w.kv_len, min(t0 + 3, t_last), min(t0 + 6, t_last), vzero, r0);
    __syncthreads();
    // One tile; register set R holds tile kt+1, which is written to the other buffer and then
    // reloaded with tile kt+4.
#define NVFP4KV_NARROW_STEP(KT, R)                                                                 \
  {                                                                                                \
    const int kt = (KT);                                                                           \
    char* buf = smem + ((kt - t0) & 1) * kBufBytes;                                                \
    const int k0 = kt * kTileKeys;                                                                 \
    if (k0 <= c.wlim_max) {                                                                        \
      f32x16 s0, s1;                                                                               \
      tile_scores(buf, lane, qf, s0, s1);                                                          \
      if (k0 + kTileKeys - 1 > c.wlim_min) tile_mask(s0, s1, k0, c.lim, c.h32);                    \
      tile_max_rescale(s0, s1, cs, m_used, l_part, acc_o);                                         \
      f16x8 pb[4];                                                                                 \
      tile_probs(s0, s1, cs, m_used, pb, l_part);                                                  \
      tile_pv(buf, lane, pb, acc_o);                                                               \
    }                                                                                              \
    store_tile<NW, FMT>(smem + ((kt + 1 - t0) & 1) * kBufBytes, R);                                     \
    load_tile<NW, FMT>(p, bt_row, w.hk, w.kv_len, min(kt + 4, t_last), min(kt + 7, t_last), vzero, R); \
    __syncthreads();                                                                               \
  }
    int kt3 = t0;
    for (; kt3 + 2 < w.t_end; kt3 += 3) {
      NVFP4KV_NARROW_STEP(kt3, r1)
      NVFP4KV_NARROW_STEP(kt3 + 1, r2)
      NVFP4KV_NARROW_STEP(kt3 + 2, r0)
    }
    if (kt3 < w.t_end) NVFP4KV_NARROW_STEP(kt3, r1)
    if (kt3 + 1 < w.t_end) NVFP4KV_NARROW_STEP(kt3 + 1, r2)
#undef NVFP4KV_NARROW_STEP
  }
  prefill_epilogue(p, w, c, acc_o, m_used, l_part);
}

// ---- key-split kernel: 2 column wavefronts x 2 key halves -----------------------------------
// For query tiles of at most 64 columns (short queries over long caches).  Four wavefronts load
// and dequantize every tile together; wavefront w covers column block w & 1 and keys
// 32 (w >> 1) .. 32 (w >> 1) + 31 of each tile, so each wavefront's per-tile chain (scores,
// softmax, PV) is half as long and two of them share each SIMD.  The two key halves of a column
// block are merged in LDS at the end (log-sum-exp of the two partial states).

// S^T for the 32 keys of one tile half (K rows 32 half .. 32 half + 31 of the tile in `buf`).
__device__ __forceinline__ void half_scores(const char* buf, int lane, int half,
                                            const f16x8 (&qf)[8], f32x16& s) {
  const char* kb = buf + (32 * half + (lane & 31)) * kKStride + 16 * (lane >> 5);
  s = f32x16{};
  f16x8 a[2];
  a[0] = *(const f16x8*)(kb);
  a[1] = *(const f16x8*)(kb + 32);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    s = mfma32h(a[t & 1], qf[t], s);
    if (t + 2 < 8) a[t & 1] = *(const f16x8*)(kb + 32 * (t + 2));
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Keys of the half starting at kh past the column's limit -> -inf.
__device__ __forceinline__ void half_mask(f32x16& s, int kh, int lim, int h32) {
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (kh + 8 * (j >> 2) + 4 * h32 + (j & 3) > lim) s[j] = kNegInf;
}

__device__ __forceinline__ void half_max_rescale(const f32x16& s, float cs, float& m_used,
                                                 float& l_part, f32x16 (&acc_o)[4]) {
  float m = fmaxf(s[0], s[1]);
#pragma unroll
  for (int j = 2; j < 16; j += 2) m = fmaxf(fmaxf(m, s[j]), s[j + 1]);
  const float mx = pair32_max(m) * cs;
  if (wave_any(mx > m_used + 8.0f)) {
    const float m_new = fmaxf(m_used, mx);
    const float alpha = (m_new == kNegInf) ? 1.0f : fast_exp2(m_used - m_new);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc_o[i] *= alpha;
    l_part *= alpha;
    m_used = m_new;
  }
}

__device__ __forceinline__ void half_probs(const f32x16& s, float cs, float m_used,
                                           f16x8 (&pb)[2], float& l_part) {
  const float mref = (m_used == kNegInf) ? 0.0f : m_used;
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    const f16x2 a = pack_f16x2_rtz(fast_exp2(fmaf(s[j], cs, -mref)), fast_exp2(fmaf(s[j + 1], cs, -mref)));
    pb[j >> 3][j & 7] = a[0];
    pb[j >> 3][(j & 7) + 1] = a[1];
  }
  l_part = sum_f16x8(pb[0], l_part);
  l_part = sum_f16x8(pb[1], l_part);
}

// O^T += V^T P^T over the 32 keys of one half (key blocks u = 2 half, 2 half + 1 of the tile).
__device__ __forceinline__ void half_pv(const char* buf, int lane, int half, const f16x8 (&pb)[2],
                                       f32x16 (&acc_o)[4]) {
  const int h32 = lane >> 5, g16 = lane >> 4, t16 = lane & 15;
  const int k4 = (t16 >> 2) & 3;
  const int slot_lo = 2 * (g16 & 1) + ((t16 & 3) >> 1);
  const char* vb = buf + kKTileBytes + (4 * h32 + (t16 >> 2)) * kVStride +
                   16 * (slot_lo ^ k4) + 8 * (t16 & 1);
#pragma unroll
  for (int uu = 0; uu < 2; ++uu) {
    const int u = 2 * half + uu;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const char* pa = vb + 16 * u * kVStride + 64 * (db ^ k4);
      const i16x4 lo = lds_read_tr16(pa);
      const i16x4 hi = lds_read_tr16(pa + 8 * kVStride);
      const f16x8 a = __builtin_bit_cast(
          f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc_o[db] = mfma32h(a, pb[uu], acc_o[db]);
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(256, 2) void nvfp4_prefill_ksplit_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kBufBytes];
  PrefillItem w;
  if (!prefill_item(p, 64, w)) return;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int half = wave >> 1;
  const PrefillCols c = prefill_cols(p, w, wave & 1, lane);
  const int32_t* bt_row = p.block_table + (int64_t)w.b * p.bt_stride;
  const bool has_tiles = w.t_begin < w.t_end;
  const int vzero = opaque_vzero();
  const int t_last = w.t_end - 1;
  const int t0 = w.t_begin;
  // the first three tiles' page ids go out before the Q loads (as in the narrow kernel)
  TileRegs<4, FMT> r0, r1, r2;
  if (has_tiles) {
    fetch_pages<4, FMT>(bt_row, w.kv_len, t0, vzero, r0);
    fetch_pages<4, FMT>(bt_row, w.kv_len, min(t0 + 1, t_last), vzero, r1);
    fetch_pages<4, FMT>(bt_row, w.kv_len, min(t0 + 2, t_last), vzero, r2);
  }
  f16x8 qf[8];
  const float cs = load_q(p, w, c, qf);

  f32x16 acc_o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc_o[i] = f32x16{};
  float m_used = kNegInf;
  float l_part = 0.0f;

  if (has_tiles) {
    load_tile<4, FMT>(p, bt_row, w.hk, w.kv_len, t0, min(t0 + 3, t_last), vzero, r0);
    load_tile<4, FMT>(p, bt_row, w.hk, w.kv_len, min(t0 + 1, t_last), min(t0 + 4, t_last), vzero, r1);
    load_tile<4, FMT>(p, bt_row, w.hk, w.kv_len, min(t0 + 2, t_last), min(t0 + 5, t_last), vzero, r2);
    store_tile<4, FMT>(smem, r0);
    load_tile<4, FMT>(p, bt_row, w.hk, w.kv_len, min(t0 + 3, t_last), min(t0 + 6, t_last), vzero, r0);
    __syncthreads();
#define NVFP4KV_KSPLIT_STEP(KT, R)                                                                 \
  {                                                                                                \
    const int kt = (KT);                                                                           \
    char* buf = smem + ((kt - t0) & 1) * kBufBytes;                                                \
    const int kh = kt * kTileKeys + 32 * half;                                                     \
    if (kh <= c.wlim_max) {                                                                        \
      f32x16 sh;                                                                                   \
      half_scores(buf, lane, half, qf, sh);                                                        \
      if (kh + 31 > c.wlim_min) half_mask(sh, kh, c.lim, c.h32);                                   \
      half_max_rescale(sh, cs, m_used, l_part, acc_o);                                             \
      f16x8 pb[2];                                                                                 \
      half_probs(sh, cs, m_used, pb, l_part);                                                      \
      half_pv(buf, lane, half, pb, acc_o);                                                         \
    }                                                                                              \
    store_tile<4, FMT>(smem + ((kt + 1 - t0) & 1) * kBufBytes, R);                                 \
    load_tile<4, FMT>(p, bt_row, w.hk, w.kv_len, min(kt + 4, t_last), min(kt + 7, t_last), vzero, R); \
    __syncthreads();                                                                               \
  }
    int kt3 = t0;
    for (; kt3 + 2 < w.t_end; kt3 += 3) {
      NVFP4KV_KSPLIT_STEP(kt3, r1)
      NVFP4KV_KSPLIT_STEP(kt3 + 1, r2)
      NVFP4KV_KSPLIT_STEP(kt3 + 2, r0)
    }
    if (kt3 < w.t_end) NVFP4KV_KSPLIT_STEP(kt3, r1)
    if (kt3 + 1 < w.t_end) NVFP4KV_KSPLIT_STEP(kt3 + 1, r2)
#undef NVFP4KV_KSPLIT_STEP
  }

  // merge the two key halves of each column block: half 1 hands its state over through LDS
  // (16 KB of partial O and 512 B of (m, l) per column wavefront, inside the first tile buffer)
  __syncthreads();
  float* xo = (float*)smem + (wave & 1) * (64 * 64 + 2 * 64);
  if (half == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) xo[(16 * i + j) * 64 + lane] = acc_o[i][j];
    xo[64 * 64 + lane] = m_used;
    xo[64 * 64 + 64 + lane] = l_part;
  }
  __syncthreads();
  if (half == 1) return;
  const float m1 = xo[64 * 64 + lane];
  const float l1 = xo[64 * 64 + 64 + lane];
  const float M = fmaxf(m_used, m1);
  const float a0 = (m_used == kNegInf) ? 0.0f : fast_exp2(m_used - M);
  const float a1 = (m1 == kNegInf) ? 0.0f : fast_exp2(m1 - M);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc_o[i][j] = acc_o[i][j] * a0 + xo[(16 * i + j) * 64 + lane] * a1;
  l_part = l_part * a0 + l1 * a1;
  m_used = M;
  prefill_epilogue(p, w, c, acc_o, m_used, l_part);
}

// ---- staggered kernel: 8 wavefronts, two anti-phased groups --------------------------------
//
// Two wavefronts share each SIMD (waves w and w+4).  Per 64-key tile a wavefront spends about as
// long in MFMA work (QK, PV) as in VALU work (softmax, dequantization), so the two groups run
// the same stages in opposite phase:
//   group 0 (waves 0-3):  QK(kt)      | softmax(kt) | PV(kt)        | dequant(kt+2)
//   group 1 (waves 4-7):  softmax(kt) | PV(kt)      | dequant(kt+2) | QK(kt+1)
// i.e. MFMA-VALU-MFMA-VALU against VALU-MFMA-VALU-MFMA, so one wavefront of a SIMD feeds the
// matrix core while the other uses the vector ALU.  Group 1 computes the next tile's scores
// before the tile barrier, so tiles are dequantized two ahead into a third LDS buffer.
constexpr int kStagWaves = 8;

template <int FMT>
__global__ __launch_bounds__(64 * kStagWaves) void nvfp4_prefill_staggered_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) char smem[3 * kBufBytes];
  PrefillItem w;
  if (!prefill_item(p, 32 * kStagWaves, w)) return;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const bool ahead = wave >= 4;  // group 1 scores the next tile before each barrier
  const PrefillCols c = prefill_cols(p, w, wave, lane);
  const int32_t* bt_row = p.block_table + (int64_t)w.b * p.bt_stride;
  const bool has_tiles = w.t_begin < w.t_end;
  const int vzero = opaque_vzero();
  const int t_last = w.t_end - 1;
  const int t0 = w.t_begin;
  // Two register sets take turns: the packed loads of tile kt+4 are issued while tile kt is
  // consumed, two tiles ahead of their dequantization.  The first two tiles' page ids are
  // fetched before the Q loads and their chunks loaded together.  Tile indices are clamped at
  // t_last.
  TileRegs<kStagWaves, FMT> ra, rb;
  if (has_tiles) {
    fetch_pages<kStagWaves, FMT>(bt_row, w.kv_len, t0, vzero, ra);
    fetch_pages<kStagWaves, FMT>(bt_row, w.kv_len, min(t0 + 1, t_last), vzero, rb);
  }
  f16x8 qf[8];
  const float cs = load_q(p, w, c, qf);

  f32x16 acc_o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc_o[i] = f32x16{};
  float m_used = kNegInf;
  float l_part = 0.0f;

  if (has_tiles) {
    load_tile<kStagWaves, FMT>(p, bt_row, w.hk, w.kv_len, t0, min(t0 + 2, t_last), vzero, ra);
    load_tile<kStagWaves, FMT>(p, bt_row, w.hk, w.kv_len, min(t0 + 1, t_last), min(t0 + 3, t_last), vzero, rb);
    store_tile<kStagWaves, FMT>(smem, ra);
    store_tile<kStagWaves, FMT>(smem + kBufBytes, rb);
    __syncthreads();
    load_tile<kStagWaves, FMT>(p, bt_row, w.hk, w.kv_len, min(t0 + 2, t_last), min(t0 + 4, t_last), vzero, ra);
    load_tile<kStagWaves, FMT>(p, bt_row, w.hk, w.kv_len, min(t0 + 3, t_last), min(t0 + 5, t_last), vzero, rb);

    f32x16 s0 = f32x16{}, s1 = f32x16{};
    if (ahead && t0 * kTileKeys <= c.wlim_max) tile_scores(smem, lane, qf, s0, s1);
    int bi = 0;  // buffer holding tile kt
    // One tile, with register set R holding tile kt+2.  (A macro rather than a lambda: a lambda
    // capturing the kernel arguments by reference makes the compiler re-load them from memory.)
#define NVFP4KV_STAG_STEP(KT, R)                                                                   \
  {                                                                                                \
    const int kt = (KT);                                                                           \
    char* bcur = smem + bi * kBufBytes;                                                            \
    char* bnext = smem + (bi == 2 ? 0 : bi + 1) * kBufBytes;                                       \
    char* bfill = smem + (bi == 0 ? 2 : bi - 1) * kBufBytes; /* receives tile kt+2 */              \
    const int k0 = kt * kTileKeys;                                                                 \
    if (k0 <= c.wlim_max) {                                                                        \
      if (!ahead) tile_scores(bcur, lane, qf, s0, s1);                                             \
      if (k0 + kTileKeys - 1 > c.wlim_min) tile_mask(s0, s1, k0, c.lim, c.h32);                    \
      tile_max_rescale(s0, s1, cs, m_used, l_part, acc_o);                                         \
      f16x8 pb[4];                                                                                 \
      tile_probs(s0, s1, cs, m_used, pb, l_part);                                                  \
      tile_pv(bcur, lane, pb, acc_o);                                                              \
    }                                                                                              \
    /* unconditional, so every step has the same loads in flight; past the last tile the */      \
    /* writes land in a buffer that is not read again */                                           \
    store_tile<kStagWaves, FMT>(bfill, R);                                                              \
    load_tile<kStagWaves, FMT>(p, bt_row, w.hk, w.kv_len, min(kt + 4, t_last), min(kt + 6, t_last),    \
                          vzero, R);                                                               \
    if (ahead && kt + 1 < w.t_end && k0 + kTileKeys <= c.wlim_max)                                 \
      tile_scores(bnext, lane, qf, s0, s1);                                                        \
    __syncthreads();                                                                               \
    bi = bi == 2 ? 0 : bi + 1;                                                                     \
  }
    // Both halves of the unrolled loop are unconditional, so the loads of the two register sets
    // are always in flight in the same order and the compiler's wait counts stay partial.
    int kt2 = t0;
    for (; kt2 + 1 < w.t_end; kt2 += 2) {
      NVFP4KV_STAG_STEP(kt2, ra)
      NVFP4KV_STAG_STEP(kt2 + 1, rb)
    }
    if (kt2 < w.t_end) NVFP4KV_STAG_STEP(kt2, ra)
#undef NVFP4KV_STAG_STEP
  }
  prefill_epilogue(p, w, c, acc_o, m_used, l_part);
}

template <int FMT>
hipError_t launch_prefill_fmt(const PrefillParams& p, int waves, hipStream_t stream) {
  const dim3 grid((unsigned)(8 * p.items_per_xcd));
  switch (waves) {
    case 8: hipLaunchKernelGGL(nvfp4_prefill_staggered_kernel<FMT>, grid, dim3(512), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((nvfp4_prefill_kernel<4, FMT>), grid, dim3(256), 0, stream, p); break;
    case 2:  // up to 64 columns: two column wavefronts, each tile's keys split between two more
      hipLaunchKernelGGL(nvfp4_prefill_ksplit_kernel<FMT>, grid, dim3(256), 0, stream, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, int waves, hipStream_t stream) {
  switch (p.format) {
    case kFmtNvfp4: return launch_prefill_fmt<kFmtNvfp4>(p, waves, stream);
    case kFmtFp8: return launch_prefill_fmt<kFmtFp8>(p, waves, stream);
    case kFmtF16: return launch_prefill_fmt<kFmtF16>(p, waves, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nvfp4kv
