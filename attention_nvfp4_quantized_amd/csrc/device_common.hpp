// Device-side building blocks shared by the gfx950 kernels: vector types, MFMA wrappers,
// the NVFP4 read-side conversion and a few cross-lane helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4kv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kHeadDim = 128;
constexpr int kPageSize = 16;
constexpr int kRowBytes = kHeadDim / 2;      // packed bytes per (token, head)
constexpr int kScaleBytes = kHeadDim / 16;   // scale bytes per (token, head)

typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// D(32x32) += A(32x16) * B(16x32).  Lane l holds A[l%32][8(l/32)+i], B[8(l/32)+i][l%32],
// D[8(j/4)+4(l/32)+j%4][l%32] (j = 0..15).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// D(16x16) += A(16x32) * B(32x16).  Lane l holds A[l%16][8(l/16)+i], B[8(l/16)+i][l%16],
// D[4(l/16)+j][l%16] (j = 0..3).
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp16 forms of the same two MFMA shapes (operand layouts as above).
__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16h(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// E4M3FN scale byte SEL of `word` -> float (exact: the hardware conversion agrees with the
// format definition on all 256 codes).
template <int SEL>
__device__ __forceinline__ float e4m3_byte(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8(word, SEL);
}

// Two E2M1 codes (byte SEL of `word`) -> their values as floats, unscaled and exact.
// The conversion's own scale operand only applies a power of two, so block scales are applied
// by a separate exact multiply.
template <int SEL>
__device__ __forceinline__ f32x2 e2m1_pair(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Eight E2M1 codes in `word` (element 0 in the low nibble) times scale s -> four bf16x2 words.
// Every product has at most 6 significant bits, so the bf16 results are exact.
__device__ __forceinline__ void dequant8(uint32_t word, float s, uint32_t out[4]) {
  f32x2 a = e2m1_pair<0>(word);
  f32x2 b = e2m1_pair<1>(word);
  f32x2 c = e2m1_pair<2>(word);
  f32x2 d = e2m1_pair<3>(word);
  out[0] = pack_bf16x2(a[0] * s, a[1] * s);
  out[1] = pack_bf16x2(b[0] * s, b[1] * s);
  out[2] = pack_bf16x2(c[0] * s, c[1] * s);
  out[3] = pack_bf16x2(d[0] * s, d[1] * s);
}

// The values of lanes l and l^32, in some order, in every lane (v_permlane32_swap on x and a
// copy of x).  Written as inline assembly because the compiler's lowering of the builtin reads
// the first result register for both results.  The s_nop padding covers the VALU-write ->
// permlane-read and permlane-write -> VALU-read wait states.  All 64 lanes must be active.
__device__ __forceinline__ f32x2 pair32_values(float x) {
  float a = x, b;
  asm volatile(
      "s_nop 4\n\t"
      "v_mov_b32 %1, %0\n\t"
      "s_nop 4\n\t"
      "v_permlane32_swap_b32 %0, %1\n\t"
      "s_nop 4"
      : "+v"(a), "=&v"(b));
  return f32x2{a, b};
}
// fp16 read-side conversion.  Every NVFP4 value, E2M1 code times E4M3 scale, has at most 6
// significant bits (2 from the code, 4 from the scale) and a magnitude in [2^-10, 2688], so it
// is exact as a normal fp16 number (11 significant bits, normal from 2^-14).

// Scale bytes 2*HI and 2*HI+1 of `word` -> fp16 pair (exact).
template <bool HI>
__device__ __forceinline__ f16x2 e4m3_pair_h(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, HI);
}

// Eight E2M1 codes in `word` (element 0 in the low nibble) times the scale in both halves of
// s -> four f16x2 words: one conversion and one packed multiply per pair, both exact.
__device__ __forceinline__ void dequant8_h(uint32_t word, f16x2 s, uint32_t out[4]) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * s);
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * s);
  out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * s);
  out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * s);
}

// Four E4M3FN bytes -> four fp16 values (two words), exact (every E4M3 value is an fp16 value).
__device__ __forceinline__ void fp8x4_to_f16(uint32_t w, uint32_t out[2]) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

// Cache formats the attention kernels read (template argument FMT): NVFP4 (packed E2M1 codes
// plus E4M3 block scales), the FP8 E4M3FN control cache (one byte per value, per-tensor scale
// only), and the fp16 copy the dequantize-ahead repack pass writes (prefill only).
constexpr int kFmtNvfp4 = 0;
constexpr int kFmtFp8 = 1;
constexpr int kFmtF16 = 2;

// Two floats -> fp16 pair, rounded toward zero (relative error < 2^-10).
__device__ __forceinline__ f16x2 pack_f16x2_rtz(float lo, float hi) {
  return __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// Two floats -> fp16 pair, rounded to nearest even; lo in the low half.
__device__ __forceinline__ uint32_t pack_f16x2_rne(float lo, float hi) {
  const f16x2 h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

// acc + the sum of the eight fp16 values of v.
__device__ __forceinline__ float sum_f16x8(f16x8 v, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
  return acc;
}

// The values of lanes l and l^16, in some order, in every lane (v_permlane16_swap, as above).
__device__ __forceinline__ f32x2 pair16_values(float x) {
  float a = x, b;
  asm volatile(
      "s_nop 4\n\t"
      "v_mov_b32 %1, %0\n\t"
      "s_nop 4\n\t"
      "v_permlane16_swap_b32 %0, %1\n\t"
      "s_nop 4"
      : "+v"(a), "=&v"(b));
  return f32x2{a, b};
}
__device__ __forceinline__ float pair16_max(float x) {
  const f32x2 v = pair16_values(x);
  return fmaxf(v[0], v[1]);
}
__device__ __forceinline__ float pair16_sum(float x) {
  const f32x2 v = pair16_values(x);
  return v[0] + v[1];
}

// Reductions over the lane pair (l, l^32); both lanes get the same bits.
__device__ __forceinline__ float pair32_max(float x) {
  const f32x2 v = pair32_values(x);
  return fmaxf(v[0], v[1]);
}
__device__ __forceinline__ float pair32_sum(float x) {
  const f32x2 v = pair32_values(x);
  return v[0] + v[1];
}

// acc + the sum of the eight bf16 values of v (four bf16 pair dot products with (1, 1)).
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
  return acc;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Block of LDS data read with the gfx950 transposing load: within each group of 16 lanes, the
// lane at position t receives element t%4 of the 4-element rows supplied by lanes t/4 + 4k
// (k = 0..3).
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
}

__device__ __forceinline__ int wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

}  // namespace nvfp4kv
