// Log-sum-exp merge of the key slices' partials for gfx950: the split prefill paths (tile and
// short-query kernels) and the split-KV decode write, per slice and output row, an fp16 partial
// output and a float32 log2-sum-exp; this kernel combines them into the output rows ("NVFP4 KV
// cache prefill vs decode performance", section "NVFP4 KV cache prefill vs decode performance":
// decode reads the whole cache per token, so it is split over keys).
#include "device_common.hpp"
#include "kernel_params.hpp"

namespace nvfp4kv {

// Log-sum-exp merge of split partials (fp16 values, float32 log-sum-exps): one wavefront per
// (query row, head); lane l owns head-dim values 2l and 2l+1.  Up to 8 slices (every split path
// here but long-key decode), all loads of the row, log-sum-exps and partials, are issued
// together before the maximum is known, so the row costs one memory round trip.  More slices:
// the lanes read the log-sum-exps in parallel and take their maximum across the wavefront, then
// the partials eight slices at a time with the eight loads issued together.  A partial of an
// empty slice is read but not used (it is not written); the weights and partials are
// accumulated in slice order either way.
__device__ __forceinline__ void merge_group(const MergeParams& p, int row, int lane, int s0, float mx,
                                            const float (&ls)[8], const f16x2 (&v)[8], float& wsum,
                                            float& o0, float& o1) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool use = s0 + j < p.num_splits && ls[j] != kNegInf;
    const float wgt = use ? fast_exp2(ls[j] - mx) : 0.0f;
    wsum += wgt;
    o0 = use ? fmaf(wgt, (float)v[j][0], o0) : o0;
    o1 = use ? fmaf(wgt, (float)v[j][1], o1) : o1;
  }
}

__global__ __launch_bounds__(256) void nvfp4_merge_kernel(MergeParams p) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int lane = threadIdx.x & 63;
  const int S = p.num_splits;
  float wsum = 0.0f, o0 = 0.0f, o1 = 0.0f;
  float mx = kNegInf;
  if (S <= 8) {
    float ls[8];
    f16x2 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t r = (int64_t)min(j, S - 1) * p.rows + row;
      ls[j] = p.part_lse[r];
      v[j] = *(const f16x2*)(p.part_o + r * kHeadDim + 2 * lane);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = j < S ? fmaxf(mx, ls[j]) : mx;
    if (mx != kNegInf) merge_group(p, row, lane, 0, mx, ls, v, wsum, o0, o1);
  } else {
    for (int s = lane; s < S; s += 64) mx = fmaxf(mx, p.part_lse[(int64_t)s * p.rows + row]);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
    if (mx != kNegInf) {
      for (int s0 = 0; s0 < S; s0 += 8) {
        float ls[8];
        f16x2 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int64_t r = (int64_t)min(s0 + j, S - 1) * p.rows + row;
          ls[j] = p.part_lse[r];
          v[j] = *(const f16x2*)(p.part_o + r * kHeadDim + 2 * lane);
        }
        merge_group(p, row, lane, s0, mx, ls, v, wsum, o0, o1);
      }
    }
  }
  const float inv = wsum > 0.0f ? p.out_scale / wsum : 0.0f;
  if (p.out_f32) {
    *(f32x2*)((float*)p.out + (int64_t)row * kHeadDim + 2 * lane) = f32x2{o0 * inv, o1 * inv};
  } else {
    *(uint32_t*)((uint16_t*)p.out + (int64_t)row * kHeadDim + 2 * lane) = pack_bf16x2(o0 * inv, o1 * inv);
  }
  if (p.lse && lane == 0) p.lse[row] = wsum > 0.0f ? (mx + __log2f(wsum)) * kLn2 : kNegInf;
}

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.rows + 3) / 4));
  hipLaunchKernelGGL(nvfp4_merge_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace nvfp4kv
