// Standalone dequantization of NVFP4 cache rows for gfx950 ("NVFP4 KV cache A4Q prefill
// explained", section "Preserve the capacity and decode case": quantization and dequantization
// utilities over the linear block-scale layout).
//
// Grid: x = groups of 64 tokens (4 wavefronts x 16), y = KV head * 2 + (0 for K, 1 for V); lane l
// of a wavefront converts the 32 values (16 packed bytes, two scale bytes) of quarter l%4 of
// token l/4.  Each value is s * e2m1(code), exact in float32 (the fp4 conversion is exact and
// the E4M3 scale is applied by one exact multiply), times g (one float32 rounding), then rounded
// to nearest-even in the output type.  Slots < 0 give zero rows.  For the FP8 control cache a
// value is e4m3(code) times g, rounded the same way.
#include "device_common.hpp"
#include "kernel_params.hpp"

namespace nvfp4kv {

template <int OUT>  // 0 bf16, 1 f32, 2 f16
__global__ __launch_bounds__(256) void nvfp4_dequant_kernel(DequantParams p) {
  const int which = blockIdx.y & 1;
  const int h = blockIdx.y >> 1;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 6) * 16 + (lane >> 2);
  const int qq = lane & 3;
  if (t >= p.num_tokens) return;
  const int64_t slot = p.slots[t];
  float x[32];
  if (slot >= 0 && p.fp8) {
    // FP8 control cache: value = e4m3(code) * g (the conversion is exact)
    const int64_t row = ((slot >> 4) * p.num_kv_heads + h) * kPageSize + (slot & 15);
    const uint8_t* src = (which == 0 ? p.k_data : p.v_data) + row * kHeadDim + 32 * qq;
    const u32x4 d0 = *(const u32x4*)src, d1 = *(const u32x4*)(src + 16);
    const float g = which == 0 ? p.k_global : p.v_global;
    const uint32_t wd[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(wd[i], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(wd[i], true);
      x[4 * i] = lo[0] * g; x[4 * i + 1] = lo[1] * g;
      x[4 * i + 2] = hi[0] * g; x[4 * i + 3] = hi[1] * g;
    }
  } else if (slot >= 0) {
    const int64_t row = ((slot >> 4) * p.num_kv_heads + h) * kPageSize + (slot & 15);
    const u32x4 d = *(const u32x4*)((which == 0 ? p.k_data : p.v_data) + row * kRowBytes + 16 * qq);
    const uint32_t sw = *(const uint16_t*)((which == 0 ? p.k_scale : p.v_scale) + row * kScaleBytes + 2 * qq);
    const float g = which == 0 ? p.k_global : p.v_global;
    const float s0 = e4m3_byte<0>(sw), s1 = e4m3_byte<1>(sw);
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      const float s = wd < 2 ? s0 : s1;
      const f32x2 a = e2m1_pair<0>(d[wd]), b = e2m1_pair<1>(d[wd]);
      const f32x2 c = e2m1_pair<2>(d[wd]), e = e2m1_pair<3>(d[wd]);
      const float v8[8] = {a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
#pragma unroll
      for (int i = 0; i < 8; ++i) x[8 * wd + i] = (v8[i] * s) * g;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = 0.0f;
  }
  const int64_t off = ((int64_t)t * p.num_kv_heads + h) * kHeadDim + 32 * qq;
  void* out = which == 0 ? p.k_out : p.v_out;
  if (OUT == 1) {
    float* o = (float*)out + off;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(f32x4*)(o + 4 * i) = f32x4{x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]};
  } else {
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (OUT == 0) {
        w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
      } else {
        f16x2 hv;
        hv[0] = (_Float16)x[2 * i];
        hv[1] = (_Float16)x[2 * i + 1];
        w[i] = __builtin_bit_cast(uint32_t, hv);
      }
    }
    uint16_t* o = (uint16_t*)out + off;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4*)(o + 8 * i) = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
  }
}

// Dequantize-ahead repack ("NVFP4 KV cache A4Q prefill explained", section "Compare A4Q with
// dequantize-ahead repacking": convert each NVFP4 tile once, before the attention kernel uses it
// repeatedly): every page a sequence's keys occupy is converted to fp16 s * e2m1(code) (exact:
// at most 6 significant bits, magnitude in [2^-10, 2688]) into a paged fp16 copy with the same
// page ids.  The per-tensor scale g is not applied; the prefill over the copy applies it as it
// does over the packed cache.  Grid: x = groups of 4 pages of a sequence, y = sequence,
// z = KV head * 2 + (0 for K, 1 for V); a wavefront converts one page (lane l: quarter l%4 of
// row l/4, 16 packed bytes and 2 scale bytes in, 64 bytes out).  A page shared by several
// sequences is written with the same bytes by each.
__global__ __launch_bounds__(256) void nvfp4_repack_kernel(RepackParams p) {
  const int which = blockIdx.z & 1;
  const int h = blockIdx.z >> 1;
  const int b = blockIdx.y;
  const int pi = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int kv_len = p.kv_lens[b];
  if (pi * kPageSize >= kv_len) return;
  const int lane = threadIdx.x & 63;
  const int qq = lane & 3;
  const int64_t page = p.block_table[(int64_t)b * p.bt_stride + pi];
  const int64_t row = (page * p.num_kv_heads + h) * kPageSize + (lane >> 2);
  const u32x4 d = *(const u32x4*)((which == 0 ? p.k_data : p.v_data) + row * kRowBytes + 16 * qq);
  const uint32_t sw = *(const uint16_t*)((which == 0 ? p.k_scale : p.v_scale) + row * kScaleBytes + 2 * qq);
  const f16x2 sc = e4m3_pair_h<false>(sw);
  const f16x2 s0 = __builtin_shufflevector(sc, sc, 0, 0);
  const f16x2 s1 = __builtin_shufflevector(sc, sc, 1, 1);
  uint32_t o[16];
  dequant8_h(d[0], s0, o + 0);
  dequant8_h(d[1], s0, o + 4);
  dequant8_h(d[2], s1, o + 8);
  dequant8_h(d[3], s1, o + 12);
  uint16_t* dst = (which == 0 ? p.k_out : p.v_out) + row * kHeadDim + 32 * qq;
#pragma unroll
  for (int i = 0; i < 4; ++i) *(u32x4*)(dst + 8 * i) = u32x4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
}

hipError_t launch_repack(const RepackParams& p, int batch, int max_pages, hipStream_t stream) {
  const dim3 grid((unsigned)((max_pages + 3) / 4), (unsigned)batch, (unsigned)(2 * p.num_kv_heads));
  hipLaunchKernelGGL(nvfp4_repack_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_dequant(const DequantParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.num_tokens + 63) / 64), (unsigned)(2 * p.num_kv_heads));
  switch (p.out_dtype) {
    case 0: hipLaunchKernelGGL(nvfp4_dequant_kernel<0>, grid, dim3(256), 0, stream, p); break;
    case 1: hipLaunchKernelGGL(nvfp4_dequant_kernel<1>, grid, dim3(256), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(nvfp4_dequant_kernel<2>, grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nvfp4kv
