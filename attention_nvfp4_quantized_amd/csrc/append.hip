// NVFP4 cache append for gfx950: quantize bf16 K/V, choose E4M3 block scales, pack E2M1 codes
// two per byte, and write each (token, KV head) row to its paged slot ("NVFP4 KV cache vs NVFP4
// weights", section "The cache quantizes values during serving"; "NVFP4 KV cache prefill vs
// decode performance", section "NVFP4 stores 4.5 bits per value before padding").
//
// A wavefront covers 16 consecutive tokens of one KV head (K or V) in four passes; in each pass
// 16 lanes read one whole 256-byte input row (16 bytes each, so every load instruction reads
// whole rows), a 16-value block spans two neighbouring lanes (its maximum taken across the pair),
// and the row's 64 packed bytes and 8 scale bytes are stored by contiguous lanes.  When the 16
// tokens fill one page (consecutive slots, as a prefill chunk's are), the wavefront writes a
// whole 1 KiB page row of packed data and a whole 128-byte line of scales.  The kernel is bound
// by HBM traffic.
//
// Exactness: the block scale is E4M3 round-to-nearest-even of the correctly rounded float32
// quotient amax / 6 (saturating at 448), computed with integer operations on the float bits.
// Element codes are E2M1 round-to-nearest-even (saturating at 6) of the exact quotient y / s,
// where y is a float32 value: x itself for bf16 (8 significant bits) or fp16 (11) input at g = 1,
// fl32(x / g) (up to 24) otherwise.  The rounding midpoints t * s (t in {0.25, 0.75, 1.25, 1.75,
// 2.5, 3.5, 5}, s with a 4-bit significand m_s in [1, 2)) are float32 numbers of at most 7
// significant bits.  So either y = t * s exactly, or |y - t * s| >= ulp(y), which puts y / s
// more than half a float32 ulp of t away from t (by the factor 2 / m_s > 1): at least 2^-24
// relative.  The kernel forms q = y * r with r the hardware reciprocal of s (within one ulp, so
// q is within 2^-22 relative), corrects it once with the residual y - q s (exact: its bits span
// at most 7 places), which leaves an error below 2^-44 relative before the final float32
// rounding.  A quotient off a midpoint therefore rounds to a float32 value on the same side of
// t, and an exact midpoint comes out as exactly t; the hardware conversion then rounds q to E2M1
// (ties to even, saturating).  Zeros keep their sign; a zero scale gives signed zeros.
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

// fl32(a / 6) for a >= 0.  With unit global scales a is a bf16 or fp16 value, and the quotient
// estimate a * fl32(1/6) corrected once with its exact residual (two FMAs) is the correctly
// rounded quotient for every such value (checked exhaustively against exact rational
// arithmetic); other inputs take the IEEE division.
template <bool UNIT_G>
__device__ __forceinline__ float div6_rn(float a) {
  if constexpr (UNIT_G) {
    constexpr float kSixth = 1.0f / 6.0f;
    const float q0 = a * kSixth;
    return __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, a), kSixth, q0);
  } else {
    return __fdiv_rn(a, 6.0f);
  }
}

// The maximum of x over the lane pair (l, l ^ 1) (a DPP quad permutation [1, 0, 3, 2]).
__device__ __forceinline__ float pair1_max(float x) {
  const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false);
  return fmaxf(x, __int_as_float(y));
}

// Quantize this lane's half of a 16-value block (8 values as 4 pairs of bf16 or fp16; the other
// half is in lane l ^ 1): returns the block's E4M3 scale code (the same in both lanes) and the
// packed codes of the 8 values (value 2i in the low nibble of byte i).
template <bool UNIT_G, bool FP16_IN>
__device__ __forceinline__ uint32_t quantize_half_block(const u32x4 w, float g, uint32_t& packed) {
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (FP16_IN) {  // every binary16 value converts exactly
      // (the element is copied out first: a bit cast taken straight from a vector element has
      // been compiled as a cast of element 0)
      const uint32_t wi = w[i];
      const f16x2 h = __builtin_bit_cast(f16x2, wi);
      y[2 * i] = (float)h[0];
      y[2 * i + 1] = (float)h[1];
    } else {
      y[2 * i] = __uint_as_float(w[i] << 16);
      y[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  if (!UNIT_G) {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = __fdiv_rn(y[i], g);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[i]));
  amax = pair1_max(amax);

  const uint32_t sc = e4m3_encode_rne(div6_rn<UNIT_G>(amax));
  const float s = e4m3_byte<0>(sc);
  const float r = sc != 0 ? __builtin_amdgcn_rcpf(s) : 0.0f;
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // residual written as -(q0 s - y): for y = -0 the result stays -0 (the code keeps its sign)
    const float q0 = y[i] * r;
    q[i] = __builtin_fmaf(-__builtin_fmaf(q0, s, -y[i]), r, q0);
  }
  uint32_t o = 0u;
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, q[0], q[1], 1.0f, 0);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, q[2], q[3], 1.0f, 1);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, q[4], q[5], 1.0f, 2);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, q[6], q[7], 1.0f, 3);
  packed = o;
  return sc;
}

// Grid: x = groups of 64 tokens (4 wavefronts x 16), y = KV head * 2 + (0 for K, 1 for V).
// A wavefront handles 16 consecutive tokens of one KV head in 4 passes of 4 tokens: in each pass
// the 16 lanes of row r hold token 4 i + r, lane c of the row its bytes 16 c .. 16 c + 15 (values
// 8 c .. 8 c + 7, half of block c / 2).  Every load instruction reads four whole 256-byte input
// rows, and the row's 64 packed bytes and 8 scale bytes are stored by contiguous lanes.
template <bool UNIT_G, bool FP16_IN>
__global__ __launch_bounds__(256) void nvfp4_append_kernel(AppendParams p) {
  const int which = blockIdx.y & 1;
  const int h = blockIdx.y >> 1;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int64_t t_base = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 6) * 16 + (lane >> 4);
  const uint16_t* in = which == 0 ? p.k : p.v;
  const int64_t stride = which == 0 ? p.k_stride : p.v_stride;
  const float g = which == 0 ? p.k_global : p.v_global;
  // Loads first, for all four passes: the slots only decide whether results are stored.
  u32x4 w[4];
  int64_t slot[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // a token past the end re-reads the last one and stores nothing (no branches around loads)
    const int64_t t = min(t_base + 4 * i, (int64_t)p.num_tokens - 1);
    w[i] = *(const u32x4*)(in + t * stride + (int64_t)h * kHeadDim + 8 * c);
    const int64_t sl = p.slots[t];
    slot[i] = t_base + 4 * i < p.num_tokens ? sl : -1;
  }
  uint8_t* data = which == 0 ? p.k_data : p.v_data;
  uint8_t* scale = which == 0 ? p.k_scale : p.v_scale;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t packed;
    const uint32_t sc = quantize_half_block<UNIT_G, FP16_IN>(w[i], g, packed);
    // scale bytes of blocks c/2 .. c/2 + 3 gathered into lanes c = 0 and 8 of the row
    const uint32_t s2 = sc | ((uint32_t)__shfl_down((int)sc, 2, 16) << 8);
    const uint32_t s4 = s2 | ((uint32_t)__shfl_down((int)s2, 4, 16) << 16);
    if (slot[i] >= 0) {
      const int64_t row = ((slot[i] >> 4) * p.num_kv_heads + h) * kPageSize + (slot[i] & 15);
      *(uint32_t*)(data + row * kRowBytes + 4 * c) = packed;
      if ((c & 7) == 0) *(uint32_t*)(scale + row * kScaleBytes + (c >> 1)) = s4;
    }
  }
}

// FP8 control cache writer: each value becomes the E4M3FN byte of y = fl32(x / g), rounded to
// nearest with ties to even, sign copied, magnitudes saturating at 448.  The input is clamped to
// [-448, 448] first (the median keeps -0), so the hardware conversion never leaves the finite
// range; in range it rounds to nearest-even.  Same grid and lane map as the NVFP4 writer; a lane
// writes the 8 bytes of its 8 values.
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
  const int c = lane & 15;
  const int64_t t_base = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 6) * 16 + (lane >> 4);
  const uint16_t* in = which == 0 ? p.k : p.v;
  const int64_t stride = which == 0 ? p.k_stride : p.v_stride;
  const float g = which == 0 ? p.k_global : p.v_global;
  u32x4 w[4];
  int64_t slot[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // a token past the end re-reads the last one and stores nothing (no branches around loads)
    const int64_t t = min(t_base + 4 * i, (int64_t)p.num_tokens - 1);
    w[i] = *(const u32x4*)(in + t * stride + (int64_t)h * kHeadDim + 8 * c);
    const int64_t sl = p.slots[t];
    slot[i] = t_base + 4 * i < p.num_tokens ? sl : -1;
  }
  uint8_t* data = which == 0 ? p.k_data : p.v_data;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x2 o = {fp8_encode4<UNIT_G, FP16_IN>(w[i][0], w[i][1], g),
                     fp8_encode4<UNIT_G, FP16_IN>(w[i][2], w[i][3], g)};
    if (slot[i] >= 0) {
      const int64_t row = ((slot[i] >> 4) * p.num_kv_heads + h) * kPageSize + (slot[i] & 15);
      *(u32x2*)(data + row * kHeadDim + 8 * c) = o;
    }
  }
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
