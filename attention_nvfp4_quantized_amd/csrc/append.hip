// NVFP4 cache append for gfx950: quantize bf16 K/V, choose E4M3 block scales, pack E2M1 codes
// two per byte, and write each (token, KV head) row to its paged slot ("NVFP4 KV cache vs NVFP4
// weights", section "The cache quantizes values during serving"; "NVFP4 KV cache prefill vs
// decode performance", section "NVFP4 stores 4.5 bits per value before padding").
//
// A wavefront covers 16 consecutive tokens of one KV head (K or V): lane l owns the two 16-value
// blocks 2(l%4), 2(l%4)+1 of token l/4, reading 64 contiguous input bytes and writing 16 packed
// bytes and 2 scale bytes.  When the 16 tokens fill one page (consecutive slots, as a prefill
// chunk's are), the wavefront writes a whole 1 KiB page row of packed data and a whole 128-byte
// line of scales, so no cache line is partially written.  The kernel is bound by HBM traffic.
//
// Exactness: the block scale is E4M3 round-to-nearest-even of the correctly rounded float32
// quotient amax / 6 (saturating at 448), computed with integer operations on the float bits.
// Element codes are E2M1 round-to-nearest-even (saturating at 6) of the exact quotient y / s,
// where y is a float32 value: x itself for bf16 (8 significant bits) or fp16 (11) input at g = 1,
// fl32(x / g) (up to 24) otherwise.  The rounding midpoints t * s (t in {0.25, 0.75, 1.25, 1.75,
// 2.5, 3.5, 5}, s with a 4-bit significand m_s in [1, 2)) are float32 numbers of at most 7
// significant bits.  So either y = t * s exactly, or |y - t * s| >= ulp(y), which puts y / s
// more than half a float32 ulp of t away from t (by the factor 2 / m_s > 1): at least 2^-24
// relative.  The kernel forms q = y * fl32(1/s) (relative error below 2^-22), corrects it once
// with the residual y - q s (exact: it has at most 6 significant bits), which leaves an error
// below 2^-44 relative before the final float32 rounding.  A quotient off a midpoint therefore
// rounds to a float32 value on the same side of t, and an exact midpoint comes out as exactly t;
// the hardware conversion then rounds q to E2M1 (ties to even, saturating).  Zeros keep their
// sign; a zero scale gives signed zeros.
#include "device_common.hpp"
#include "kernel_params.hpp"

namespace nvfp4kv {

// E4M3FN code of a non-negative finite float: nearest, ties to even, saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_encode_rne(float q) {
  if (q >= 448.0f) return 0x7Eu;
  if (q < 0.015625f) {
    // below 2^-6 the representable values are the multiples of 2^-9 (code = multiple);
    // q * 512 is exact and rint rounds half to even.  A result of 8 is 2^-6 = code 0x08.
    return (uint32_t)__builtin_rintf(q * 512.0f);
  }
  const uint32_t b = __float_as_uint(q);
  const uint32_t e = ((b >> 23) & 0xFFu) - 120u;  // rebias 127 -> 7
  const uint32_t mant = b & 0x7FFFFFu;
  const uint32_t keep = mant >> 20;
  const uint32_t rem = mant & 0xFFFFFu;
  const uint32_t up = (rem > 0x80000u) | ((rem == 0x80000u) & (keep & 1u));
  const uint32_t code = (e << 3) + keep + up;  // a mantissa carry moves into the exponent
  return code > 0x7Eu ? 0x7Eu : code;
}

// Quantize one 16-value block held as 8 pairs of bf16 (or fp16) values: returns the E4M3
// scale code and the packed codes (element 2i in the low nibble of byte i).
template <bool UNIT_G, bool FP16_IN>
__device__ __forceinline__ uint32_t quantize_block(const uint32_t (&w)[8], float g, u32x2& packed) {
  float y[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (FP16_IN) {  // every binary16 value converts exactly
      const f16x2 h = __builtin_bit_cast(f16x2, w[i]);
      y[2 * i] = (float)h[0];
      y[2 * i + 1] = (float)h[1];
    } else {
      y[2 * i] = __uint_as_float(w[i] << 16);
      y[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  if (!UNIT_G) {
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = __fdiv_rn(y[i], g);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(y[i]));

  const uint32_t sc = e4m3_encode_rne(__fdiv_rn(amax, 6.0f));
  const float s = e4m3_byte<0>(sc);
  const float r = sc != 0 ? __fdiv_rn(1.0f, s) : 0.0f;
  float q[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    // residual written as -(q0 s - y): for y = -0 the result stays -0 (the code keeps its sign)
    const float q0 = y[i] * r;
    q[i] = __builtin_fmaf(-__builtin_fmaf(q0, s, -y[i]), r, q0);
  }
  uint32_t lo = 0u, hi = 0u;
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, q[0], q[1], 1.0f, 0);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, q[2], q[3], 1.0f, 1);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, q[4], q[5], 1.0f, 2);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, q[6], q[7], 1.0f, 3);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, q[8], q[9], 1.0f, 0);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, q[10], q[11], 1.0f, 1);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, q[12], q[13], 1.0f, 2);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, q[14], q[15], 1.0f, 3);
  packed = u32x2{lo, hi};
  return sc;
}

// Grid: x = groups of 64 tokens (4 wavefronts x 16), y = KV head * 2 + (0 for K, 1 for V).
template <bool UNIT_G, bool FP16_IN>
__global__ __launch_bounds__(256) void nvfp4_append_kernel(AppendParams p) {
  const int which = blockIdx.y & 1;
  const int h = blockIdx.y >> 1;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 6) * 16 + (lane >> 2);
  const int pair = lane & 3;  // blocks 2 * pair, 2 * pair + 1
  if (t >= p.num_tokens) return;
  // The slot only decides whether the results are stored: the input loads and the arithmetic
  // do not wait for it (an early exit would make every load wait behind the slot load).
  const int64_t slot = p.slots[t];

  const uint16_t* src = (which == 0 ? p.k + t * p.k_stride : p.v + t * p.v_stride) +
                        (int64_t)h * kHeadDim + 32 * pair;
  const u32x4 in0 = *(const u32x4*)(src);
  const u32x4 in1 = *(const u32x4*)(src + 8);
  const u32x4 in2 = *(const u32x4*)(src + 16);
  const u32x4 in3 = *(const u32x4*)(src + 24);
  const float g = which == 0 ? p.k_global : p.v_global;
  const uint32_t wa[8] = {in0[0], in0[1], in0[2], in0[3], in1[0], in1[1], in1[2], in1[3]};
  const uint32_t wb[8] = {in2[0], in2[1], in2[2], in2[3], in3[0], in3[1], in3[2], in3[3]};
  u32x2 pa, pb;
  const uint32_t sa = quantize_block<UNIT_G, FP16_IN>(wa, g, pa);
  const uint32_t sb = quantize_block<UNIT_G, FP16_IN>(wb, g, pb);

  if (slot < 0) return;
  const int64_t page = slot >> 4;
  const int64_t row = (page * p.num_kv_heads + h) * kPageSize + (slot & 15);
  uint8_t* data = (which == 0 ? p.k_data : p.v_data) + row * kRowBytes + 16 * pair;
  uint8_t* scale = (which == 0 ? p.k_scale : p.v_scale) + row * kScaleBytes + 2 * pair;
  *(u32x4*)data = u32x4{pa[0], pa[1], pb[0], pb[1]};
  *(uint16_t*)scale = (uint16_t)(sa | (sb << 8));
}

// FP8 control cache writer: each value becomes the E4M3FN byte of y = fl32(x / g), rounded to
// nearest with ties to even, sign copied, magnitudes saturating at 448.  The input is clamped to
// [-448, 448] first (the median keeps -0), so the hardware conversion never leaves the finite
// range; in range it rounds to nearest-even.  Same grid and lane map as the NVFP4 writer; a lane
// writes 32 bytes.
template <bool UNIT_G, bool FP16_IN>
__device__ __forceinline__ uint32_t fp8_encode4(uint32_t w0, uint32_t w1, float g) {
  float y[4];
  if (FP16_IN) {
    const f16x2 a = __builtin_bit_cast(f16x2, w0), b = __builtin_bit_cast(f16x2, w1);
    y[0] = (float)a[0]; y[1] = (float)a[1]; y[2] = (float)b[0]; y[3] = (float)b[1];
  } else {
    y[0] = __uint_as_float(w0 << 16); y[1] = __uint_as_float(w0 & 0xFFFF0000u);
    y[2] = __uint_as_float(w1 << 16); y[3] = __uint_as_float(w1 & 0xFFFF0000u);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!UNIT_G) y[i] = __fdiv_rn(y[i], g);
    y[i] = __builtin_amdgcn_fmed3f(y[i], -448.0f, 448.0f);
  }
  int o = 0;
  o = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], o, false);
  o = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], o, true);
  return (uint32_t)o;
}

template <bool UNIT_G, bool FP16_IN>
__global__ __launch_bounds__(256) void fp8_append_kernel(AppendParams p) {
  const int which = blockIdx.y & 1;
  const int h = blockIdx.y >> 1;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 6) * 16 + (lane >> 2);
  const int qq = lane & 3;  // values 32 qq .. 32 qq + 31
  if (t >= p.num_tokens) return;
  // The slot only decides whether the results are stored: the input loads and the arithmetic
  // do not wait for it (an early exit would make every load wait behind the slot load).
  const int64_t slot = p.slots[t];

  const uint16_t* src = (which == 0 ? p.k + t * p.k_stride : p.v + t * p.v_stride) +
                        (int64_t)h * kHeadDim + 32 * qq;
  u32x4 in[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) in[i] = *(const u32x4*)(src + 8 * i);
  const float g = which == 0 ? p.k_global : p.v_global;
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = fp8_encode4<UNIT_G, FP16_IN>(in[i][0], in[i][1], g);
    o[2 * i + 1] = fp8_encode4<UNIT_G, FP16_IN>(in[i][2], in[i][3], g);
  }
  if (slot < 0) return;
  const int64_t row = ((slot >> 4) * p.num_kv_heads + h) * kPageSize + (slot & 15);
  uint8_t* data = (which == 0 ? p.k_data : p.v_data) + row * kHeadDim + 32 * qq;
  *(u32x4*)data = u32x4{o[0], o[1], o[2], o[3]};
  *(u32x4*)(data + 16) = u32x4{o[4], o[5], o[6], o[7]};
}

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.num_tokens + 63) / 64), (unsigned)(2 * p.num_kv_heads));
  const bool unit = p.k_global == 1.0f && p.v_global == 1.0f;
  if (p.fp8) {
    if (p.fp16_in) {
      if (unit) hipLaunchKernelGGL((fp8_append_kernel<true, true>), grid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((fp8_append_kernel<false, true>), grid, dim3(256), 0, stream, p);
    } else {
      if (unit) hipLaunchKernelGGL((fp8_append_kernel<true, false>), grid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((fp8_append_kernel<false, false>), grid, dim3(256), 0, stream, p);
    }
    return hipGetLastError();
  }
  if (p.fp16_in) {
    if (unit) hipLaunchKernelGGL((nvfp4_append_kernel<true, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((nvfp4_append_kernel<false, true>), grid, dim3(256), 0, stream, p);
  } else {
    if (unit) hipLaunchKernelGGL((nvfp4_append_kernel<true, false>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((nvfp4_append_kernel<false, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace nvfp4kv
