// A4Q-style causal paged prefill over the NVFP4 cache for gfx950: the query is quantized in the
// kernel and QK runs on the block-scaled low-precision MFMA ("NVFP4 KV cache A4Q prefill
// explained", section "Quantize Q instead of expanding K"); PV stays on the fp16 path of the stock
// kernel.  An opt-in variant: its added error is the query quantization alone, measured against
// the oracle (section "Make query accuracy a release gate").
//
// gfx950's block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) takes FP8 or FP4 operands with
// one power-of-two (E8M0) scale per 32 values of the reduction.  The pages' kernel feeds the
// cache's packed E2M1 K with its E4M3 scales per 16 values straight to an NVFP4 tensor-core
// product; here that cannot be exact: an E8M0 scale cannot hold E4M3 mantissas, and one FP8 value
// cannot hold an NVFP4 value (up to 6 significant bits).  So:
//
//  * Q: each column's 128 values are quantized once per workgroup in blocks of 32 consecutive
//    head-dim values, OCP MX rule: scale 2^(floor(log2 amax) - emax) (emax 8 for MXFP8 E4M3
//    elements, 2 for MXFP4 E2M1), elements rounded to nearest-even and saturated.
//  * K: each 32-value block of a key is carried exactly as X (hi + lo): X = 2^(E - 5) with E the
//    larger floor(log2) of the block's two E4M3 scales, hi = E4M3(y), lo = E4M3(y - hi) for
//    y = x / X (|y| < 384).  Both terms are FP8 operands of their own MFMA, under the same E8M0
//    scale; lo is exact whenever the two scales are within 2^8 of each other.
//  * QK is then two FP8 MFMAs per 32 keys x 32 columns x 64 head-dim values: the same matrix-core
//    time as the stock fp16 path, with more conversion work per tile.  The bridge is what gfx950
//    needs for an exact K; the A4Q saving of the pages' hardware does not carry over.
//  * The one-term form (template argument KT = 1) keeps hi alone: one FP8 MFMA per 64 values, half
//    the QK matrix-core time, at the cost of K rounded to E4M3's 4 significant bits under the
//    block's power-of-two scale (relative error at most 2^-4 per value in E4M3's normal range):
//    an approximation beyond the pages' A4Q, whose product takes K exactly.
//
// Operand layout of the 32x32x64 block-scaled MFMA (measured on the device): for lane l = r + 32h,
// an FP8 operand holds reduction index k = 16h + i in bytes i = 0..15 and k = 32 + 16h + (i - 16)
// in bytes 16..31; an FP4 operand holds k = 32h + j in nibble j (low nibble first) of bytes 0..15;
// lane r + 32b supplies the scale of k = 32b .. 32b + 31 for row / column r.
//
// The kernel is the 8-wave staggered kernel of the stock path (two anti-phased wavefront
// groups, three LDS tile buffers, packed loads two tiles ahead) with the K half of each tile
// buffer holding the hi and lo planes and the block exponents instead of an fp16 K tile.
#include "prefill_common.hpp"

namespace nvfp4kv {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(2))) short s16x2;

constexpr int kQfMxfp8 = 1;  // query formats (template argument QF)
constexpr int kQfMxfp4 = 2;

// A4Q tile buffer: K hi plane [64 keys][144 B] (128 FP8 values + 16 B pad: the 16-byte reads of
// 16 consecutive rows fall on distinct banks), K lo plane, the E8M0 code of each (key, 32-value
// block) [64][4 B], then the V tile of the stock layout.
constexpr int kQKStride = 144;
constexpr int kQKPlane = kTileKeys * kQKStride;
constexpr int kQScaleOff = 2 * kQKPlane;
constexpr int kQVOff = kQScaleOff + kTileKeys * 4;
constexpr int kQBufBytes = kQVOff + kVTileBytes;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// E8M0 code of the MX scale 2^(floor(log2 amax) - emax), clamped to the code range; 127 (1.0) for
// an all-zero block.
__device__ __forceinline__ int mx_scale_code(float amax, int emax) {
  if (!(amax > 0.0f)) return 127;
  const int fl = __builtin_amdgcn_frexp_expf(amax) - 1;  // amax = m 2^(fl + 1), m in [0.5, 1)
  return min(254, max(0, fl - emax + 127));
}

// This lane's query column quantized to MX blocks, as the B operands of the two 64-value k-steps
// (qb) with their E8M0 codes (qsc), laid out for the block-scaled MFMA.  Padding lanes read the
// item's first row and zero it.  Returns the base-2 score scale.
template <int QF>
__device__ __forceinline__ float load_q_mx(const PrefillParams& p, const PrefillItem& w,
                                           const PrefillCols& c, i32x8 (&qb)[2], int (&qsc)[2]) {
  const int h = c.h32;
  const uint16_t* qp = p.q + ((int64_t)(w.q_start + (c.valid ? c.pos : 0)) * p.num_qo_heads + c.head) * kHeadDim;
  if constexpr (QF == kQfMxfp8) {
    // groups g = 0..3: head-dim values 32 g + 16 h .. + 15; k-step ks takes groups 2 ks (bytes
    // 0-15) and 2 ks + 1 (bytes 16-31); block b = values 32 b .. 32 b + 31 is group b of both
    // lane halves
    u32x4 raw[4][2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      raw[g][0] = *(const u32x4*)(qp + 32 * g + 16 * h);
      raw[g][1] = *(const u32x4*)(qp + 32 * g + 16 * h + 8);
    }
    int code[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float amax = 0.0f;
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        if (!c.valid) raw[g][v] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(raw[g][v][i])), fabsf(bf16_hi(raw[g][v][i]))));
      }
      code[g] = mx_scale_code(pair32_max(amax), 8);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int g = 2 * ks + half;
        const int sh = 127 - code[g];
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            // four values -> four E4M3 bytes (x / X exact; clamped so the conversion never
            // leaves the finite range; nearest-even inside it)
            const float y0 = __builtin_amdgcn_fmed3f(__builtin_ldexpf(bf16_lo(raw[g][v][i]), sh), -448.0f, 448.0f);
            const float y1 = __builtin_amdgcn_fmed3f(__builtin_ldexpf(bf16_hi(raw[g][v][i]), sh), -448.0f, 448.0f);
            const float y2 = __builtin_amdgcn_fmed3f(__builtin_ldexpf(bf16_lo(raw[g][v][i + 1]), sh), -448.0f, 448.0f);
            const float y3 = __builtin_amdgcn_fmed3f(__builtin_ldexpf(bf16_hi(raw[g][v][i + 1]), sh), -448.0f, 448.0f);
            int o = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
            o = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, o, true);
            qb[ks][4 * half + 2 * v + i / 2] = o;
          }
      }
      qsc[ks] = code[2 * ks + h];
    }
  } else {
    // k-step ks: this lane holds head-dim values 64 ks + 32 h .. + 31, i.e. all of block
    // 2 ks + h, as 32 E2M1 codes (value j in nibble j of bytes 0-15)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 raw[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) raw[v] = *(const u32x4*)(qp + 64 * ks + 32 * h + 8 * v);
      float amax = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (!c.valid) raw[v] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(raw[v][i])), fabsf(bf16_hi(raw[v][i]))));
      }
      const int code = mx_scale_code(amax, 2);
      const int sh = 127 - code;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        uint32_t o = 0u;
        o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, __builtin_ldexpf(bf16_lo(raw[v][0]), sh),
                                                     __builtin_ldexpf(bf16_hi(raw[v][0]), sh), 1.0f, 0);
        o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, __builtin_ldexpf(bf16_lo(raw[v][1]), sh),
                                                     __builtin_ldexpf(bf16_hi(raw[v][1]), sh), 1.0f, 1);
        o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, __builtin_ldexpf(bf16_lo(raw[v][2]), sh),
                                                     __builtin_ldexpf(bf16_hi(raw[v][2]), sh), 1.0f, 2);
        o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, __builtin_ldexpf(bf16_lo(raw[v][3]), sh),
                                                     __builtin_ldexpf(bf16_hi(raw[v][3]), sh), 1.0f, 3);
        qb[ks][v] = (int)o;
        qb[ks][4 + v] = 0;
      }
      qsc[ks] = code;
    }
  }
  return p.score_scale;
}

// Dequantize the loaded chunks into an A4Q tile buffer: V chunks to the fp16 V tile (as the stock
// kernel), K chunks to their hi (and for KT = 2 lo) E4M3 bytes and the E8M0 code of their 32-value
// block.
template <int KT>
__device__ __forceinline__ void store_tile_a4q(char* buf, const TileRegs<8, kFmtNvfp4>& r) {
  const int it = threadIdx.x;  // one chunk per thread and tile
  const bool is_v = (it >> 8) != 0;
  const int key = (it & 255) >> 2;
  const int qq = it & 3;
  const f16x2 sc = e4m3_pair_h<false>(r.scale[0]);
  if (is_v) {
    const f16x2 s0 = __builtin_shufflevector(sc, sc, 0, 0);
    const f16x2 s1 = __builtin_shufflevector(sc, sc, 1, 1);
    uint32_t o[16];
    dequant8_h(r.data[0][0][0], s0, o + 0);
    dequant8_h(r.data[0][0][1], s0, o + 4);
    dequant8_h(r.data[0][0][2], s1, o + 8);
    dequant8_h(r.data[0][0][3], s1, o + 12);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      *(u32x4*)(buf + kQVOff + v_offset(key, 4 * qq + w)) = u32x4{o[4 * w], o[4 * w + 1], o[4 * w + 2], o[4 * w + 3]};
    return;
  }
  // E from the fp16 exponent fields of the two block scales (every nonzero E4M3 value is a
  // normal fp16 number; a zero scale counts as -15); y = code * (s * 2^(5 - E)), exact in fp16
  const uint32_t sb = __builtin_bit_cast(uint32_t, sc);
  const int E = max((int)((sb >> 10) & 31u), (int)((sb >> 26) & 31u)) - 15;
  const _Float16 mult = (_Float16)__builtin_ldexpf(1.0f, min(5 - E, 14));
  const f16x2 sa = sc * f16x2{mult, mult};
  uint32_t y[16];
  dequant8_h(r.data[0][0][0], __builtin_shufflevector(sa, sa, 0, 0), y + 0);
  dequant8_h(r.data[0][0][1], __builtin_shufflevector(sa, sa, 0, 0), y + 4);
  dequant8_h(r.data[0][0][2], __builtin_shufflevector(sa, sa, 1, 1), y + 8);
  dequant8_h(r.data[0][0][3], __builtin_shufflevector(sa, sa, 1, 1), y + 12);
  uint32_t hi[8], lo[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f16x2 ya = __builtin_bit_cast(f16x2, y[2 * i]);
    const f16x2 yb = __builtin_bit_cast(f16x2, y[2 * i + 1]);
    s16x2 t = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(s16x2{0, 0}, ya, 1.0f, false);
    t = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(t, yb, 1.0f, true);
    hi[i] = __builtin_bit_cast(uint32_t, t);
    if constexpr (KT == 1) continue;
    // y - hi is exact in fp16: y has at most 6 significant bits and hi is y rounded to 4
    const f16x2 la = ya - __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi[i], 1.0f, false);
    const f16x2 lb = yb - __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi[i], 1.0f, true);
    s16x2 u = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(s16x2{0, 0}, la, 1.0f, false);
    u = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(u, lb, 1.0f, true);
    lo[i] = __builtin_bit_cast(uint32_t, u);
  }
  char* row = buf + key * kQKStride + 32 * qq;
  *(u32x4*)(row) = u32x4{hi[0], hi[1], hi[2], hi[3]};
  *(u32x4*)(row + 16) = u32x4{hi[4], hi[5], hi[6], hi[7]};
  if constexpr (KT == 2) {
    *(u32x4*)(row + kQKPlane) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    *(u32x4*)(row + kQKPlane + 16) = u32x4{lo[4], lo[5], lo[6], lo[7]};
  }
  *(uint8_t*)(buf + kQScaleOff + 4 * key + qq) = (uint8_t)(E + 122);  // E8M0 code of 2^(E - 5)
}

// S^T (64 keys x this wave's 32 columns) from the hi and (KT = 2) lo planes: per 32-key block and
// 64-value k-step, one block-scaled MFMA for each plane (same E8M0 scale).
template <int QF, int KT>
__device__ __forceinline__ void tile_scores_a4q(const char* buf, int lane, const i32x8 (&qb)[2],
                                                const int (&qsc)[2], f32x16& s0, f32x16& s1) {
  const int r = lane & 31, h = lane >> 5;
  constexpr int kBFmt = QF == kQfMxfp8 ? 0 : 4;  // operand format of the query (B)
  s0 = f32x16{};
  s1 = f32x16{};
  const uint32_t e0 = *(const uint32_t*)(buf + kQScaleOff + 4 * r);
  const uint32_t e1 = *(const uint32_t*)(buf + kQScaleOff + 4 * (32 + r));
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    i32x8 a[2][KT];  // [key block][plane]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int pl = 0; pl < KT; ++pl) {
        const char* src = buf + pl * kQKPlane + (32 * kb + r) * kQKStride + 64 * ks + 16 * h;
        const u32x4 x0 = *(const u32x4*)(src);
        const u32x4 x1 = *(const u32x4*)(src + 32);
        a[kb][pl] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                          (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      }
    const int sk0 = (e0 >> (8 * (2 * ks + h))) & 0xFF;
    const int sk1 = (e1 >> (8 * (2 * ks + h))) & 0xFF;
    s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[0][0], qb[ks], s0, 0, kBFmt, 0, sk0, 0, qsc[ks]);
    s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[1][0], qb[ks], s1, 0, kBFmt, 0, sk1, 0, qsc[ks]);
    if constexpr (KT == 2) {
      s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[0][1], qb[ks], s0, 0, kBFmt, 0, sk0, 0, qsc[ks]);
      s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[1][1], qb[ks], s1, 0, kBFmt, 0, sk1, 0, qsc[ks]);
    }
  }
}

// The staggered 8-wave kernel of the stock path with A4Q tile buffers and scores.
template <int QF, int KT>
__global__ __launch_bounds__(512) void nvfp4_prefill_a4q_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) char smem[3 * kQBufBytes];
  PrefillItem w;
  if (!prefill_item(p, 256, w)) return;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const bool ahead = wave >= 4;  // group 1 scores the next tile before each barrier
  const PrefillCols c = prefill_cols(p, w, wave, lane);
  const int32_t* bt_row = p.block_table + (int64_t)w.b * p.bt_stride;
  const bool has_tiles = w.t_begin < w.t_end;
  const int vzero = opaque_vzero();
  const int t_last = w.t_end - 1;
  const int t0 = w.t_begin;
  TileRegs<8, kFmtNvfp4> ra, rb;
  if (has_tiles) {
    fetch_pages<8, kFmtNvfp4>(bt_row, w.kv_len, t0, vzero, ra);
    fetch_pages<8, kFmtNvfp4>(bt_row, w.kv_len, min(t0 + 1, t_last), vzero, rb);
  }
  i32x8 qb[2];
  int qsc[2];
  const float cs = load_q_mx<QF>(p, w, c, qb, qsc);

  f32x16 acc_o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc_o[i] = f32x16{};
  float m_used = kNegInf;
  float l_part = 0.0f;

  if (has_tiles) {
    load_tile<8, kFmtNvfp4>(p, bt_row, w.hk, w.kv_len, t0, min(t0 + 2, t_last), vzero, ra);
    load_tile<8, kFmtNvfp4>(p, bt_row, w.hk, w.kv_len, min(t0 + 1, t_last), min(t0 + 3, t_last), vzero, rb);
    store_tile_a4q<KT>(smem, ra);
    store_tile_a4q<KT>(smem + kQBufBytes, rb);
    __syncthreads();
    load_tile<8, kFmtNvfp4>(p, bt_row, w.hk, w.kv_len, min(t0 + 2, t_last), min(t0 + 4, t_last), vzero, ra);
    load_tile<8, kFmtNvfp4>(p, bt_row, w.hk, w.kv_len, min(t0 + 3, t_last), min(t0 + 5, t_last), vzero, rb);

    f32x16 s0 = f32x16{}, s1 = f32x16{};
    if (ahead && t0 * kTileKeys <= c.wlim_max) tile_scores_a4q<QF, KT>(smem, lane, qb, qsc, s0, s1);
    int bi = 0;  // buffer holding tile kt
#define NVFP4KV_A4Q_STEP(TILE, R)                                                                  \
  {                                                                                                \
    const int kt = (TILE);                                                                         \
    char* bcur = smem + bi * kQBufBytes;                                                           \
    char* bnext = smem + (bi == 2 ? 0 : bi + 1) * kQBufBytes;                                      \
    char* bfill = smem + (bi == 0 ? 2 : bi - 1) * kQBufBytes; /* receives tile kt+2 */             \
    const int k0 = kt * kTileKeys;                                                                 \
    if (k0 <= c.wlim_max) {                                                                        \
      if (!ahead) tile_scores_a4q<QF, KT>(bcur, lane, qb, qsc, s0, s1);                            \
      if (k0 + kTileKeys - 1 > c.wlim_min) tile_mask(s0, s1, k0, c.lim, c.h32);                    \
      tile_max_rescale(s0, s1, cs, m_used, l_part, acc_o);                                         \
      f16x8 pb[4];                                                                                 \
      tile_probs(s0, s1, cs, m_used, pb, l_part);                                                  \
      tile_pv_at(bcur + kQVOff, lane, pb, acc_o);                                                  \
    }                                                                                              \
    store_tile_a4q<KT>(bfill, R);                                                                  \
    load_tile<8, kFmtNvfp4>(p, bt_row, w.hk, w.kv_len, min(kt + 4, t_last), min(kt + 6, t_last),   \
                            vzero, R);                                                             \
    if (ahead && kt + 1 < w.t_end && k0 + kTileKeys <= c.wlim_max)                                 \
      tile_scores_a4q<QF, KT>(bnext, lane, qb, qsc, s0, s1);                                       \
    __syncthreads();                                                                               \
    bi = bi == 2 ? 0 : bi + 1;                                                                     \
  }
    int kt2 = t0;
    for (; kt2 + 1 < w.t_end; kt2 += 2) {
      NVFP4KV_A4Q_STEP(kt2, ra)
      NVFP4KV_A4Q_STEP(kt2 + 1, rb)
    }
    if (kt2 < w.t_end) NVFP4KV_A4Q_STEP(kt2, ra)
#undef NVFP4KV_A4Q_STEP
  }
  prefill_epilogue(p, w, c, acc_o, m_used, l_part);
}

hipError_t launch_prefill_a4q(const PrefillParams& p, int q_format, int k_terms, hipStream_t stream) {
  const dim3 grid((unsigned)(8 * p.items_per_xcd));
  if (p.format != kFmtNvfp4 || (k_terms != 1 && k_terms != 2)) return hipErrorInvalidValue;
  switch (2 * q_format + k_terms - 1) {
    case 0: hipLaunchKernelGGL((nvfp4_prefill_a4q_kernel<kQfMxfp8, 1>), grid, dim3(512), 0, stream, p); break;
    case 1: hipLaunchKernelGGL((nvfp4_prefill_a4q_kernel<kQfMxfp8, 2>), grid, dim3(512), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((nvfp4_prefill_a4q_kernel<kQfMxfp4, 1>), grid, dim3(512), 0, stream, p); break;
    case 3: hipLaunchKernelGGL((nvfp4_prefill_a4q_kernel<kQfMxfp4, 2>), grid, dim3(512), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nvfp4kv
