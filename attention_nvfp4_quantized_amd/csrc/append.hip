// NVFP4 cache append for gfx950: quantize bf16 K/V, choose E4M3 block scales, pack E2M1 codes
// two per byte, and write each (token, KV head) row to its paged slot ("NVFP4 KV cache vs NVFP4
// weights", section "The cache quantizes values during serving"; "NVFP4 KV cache prefill vs
// decode performance", section "NVFP4 stores 4.5 bits per value before padding").
//
// One thread owns one 16-value block: it reads 32 contiguous input bytes, writes 8 packed bytes
// and one scale byte.  Eight consecutive threads cover one 64-byte cache row, so both the loads
// and the stores are contiguous across a wavefront.  The kernel is bound by HBM traffic.
//
// Exactness: the block scale is E4M3 round-to-nearest-even of the correctly rounded float32
// quotient amax / 6 (saturating at 448), computed with integer operations on the float bits.
// Element codes come from comparing |y| with the products t * s for the rounding midpoints
// t in {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}; each product has at most 7 significant bits, so the
// comparisons are exact and ties resolve to the even code.  No reciprocal is used.
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

__device__ __forceinline__ uint32_t e2m1_magnitude(float a, float t1, float t2, float t3, float t4,
                                                   float t5, float t6, float t7) {
  return (uint32_t)(a > t1) + (uint32_t)(a >= t2) + (uint32_t)(a > t3) + (uint32_t)(a >= t4) +
         (uint32_t)(a > t5) + (uint32_t)(a >= t6) + (uint32_t)(a > t7);
}

template <bool UNIT_G>
__global__ __launch_bounds__(256) void nvfp4_append_kernel(AppendParams p) {
  const int which = blockIdx.y;  // 0 = K, 1 = V
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int H = p.num_kv_heads;
  const int64_t nblk = (int64_t)p.num_tokens * H * 8;
  if (idx >= nblk) return;
  const int blk = (int)(idx & 7);
  const int64_t th = idx >> 3;
  const int h = (int)(th % H);
  const int64_t t = th / H;
  const int64_t slot = p.slots[t];
  if (slot < 0) return;

  const uint16_t* src = (which == 0 ? p.k + t * p.k_stride : p.v + t * p.v_stride) +
                        (int64_t)h * kHeadDim + blk * 16;
  const u32x4 lo = *(const u32x4*)(src);
  const u32x4 hi = *(const u32x4*)(src + 8);
  const uint32_t w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  float y[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    y[2 * i] = __uint_as_float(w[i] << 16);
    y[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  if (!UNIT_G) {
    const float g = which == 0 ? p.k_global : p.v_global;
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = __fdiv_rn(y[i], g);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(y[i]));

  const uint32_t sc = e4m3_encode_rne(__fdiv_rn(amax, 6.0f));
  const float s = e4m3_byte<0>(sc);
  const float t1 = 0.25f * s, t2 = 0.75f * s, t3 = 1.25f * s, t4 = 1.75f * s;
  const float t5 = 2.5f * s, t6 = 3.5f * s, t7 = 5.0f * s;
  const uint32_t keep = sc != 0 ? 0x7u : 0x0u;  // a zero scale forces magnitude 0
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t sign = __float_as_uint(y[i]) >> 31;
    const uint32_t mag = e2m1_magnitude(fabsf(y[i]), t1, t2, t3, t4, t5, t6, t7) & keep;
    packed[i >> 3] |= ((sign << 3) | mag) << (4 * (i & 7));
  }

  const int64_t page = slot >> 4;
  const int64_t row = (page * H + h) * kPageSize + (slot & 15);
  uint8_t* data = (which == 0 ? p.k_data : p.v_data) + row * kRowBytes + blk * 8;
  uint8_t* scale = (which == 0 ? p.k_scale : p.v_scale) + row * kScaleBytes + blk;
  *(u32x2*)data = u32x2{packed[0], packed[1]};
  *scale = (uint8_t)sc;
}

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  const int64_t nblk = (int64_t)p.num_tokens * p.num_kv_heads * 8;
  const dim3 grid((unsigned)((nblk + 255) / 256), 2);
  if (p.k_global == 1.0f && p.v_global == 1.0f)
    hipLaunchKernelGGL(nvfp4_append_kernel<true>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(nvfp4_append_kernel<false>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace nvfp4kv
