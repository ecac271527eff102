// Split-KV single-token paged decode over the NVFP4 KV cache for gfx950.
//
// Decode reads the whole growing cache for one query token per sequence and is bound by HBM
// bandwidth ("NVFP4 KV cache prefill vs decode performance", sections "NVFP4 KV cache prefill vs
// decode performance" and "Decode can win on fewer bytes read").  The kernel therefore spends as
// little as possible per cache byte:
//
//  * A workgroup (4 wavefronts) owns one (sequence, KV head, key slice).  Each wavefront walks a
//    contiguous quarter of the slice in steps of 32 tokens; all query heads of the group ride
//    along as MFMA columns, so each packed byte is read and converted exactly once.
//  * K goes from HBM straight into MFMA operand registers: lane l loads 16 bytes of one token
//    (32 head-dim values) and converts them, scaled, to fp16 (exact for every NVFP4 value: one
//    fp4->fp16 convert and one packed multiply per pair).  Q is fp16 with a per-column
//    power-of-two scale folded into the softmax scale.  The head-dim order inside each
//    32-wide k-step is permuted identically for K and Q, which leaves the dot products unchanged
//    and lets every lane use one 16-byte load.  Scores: S^T = K Q^T with 16x16x32 fp16 MFMA.
//  * V is converted the same way into a small per-wavefront LDS stage and read back with the
//    transposing LDS load as the A operand of O^T = V^T P^T; P^T needs no data movement.
//  * Online softmax in base 2 with lazy rescaling (refresh when the maximum grows by > 8).
//  * The four wavefronts are combined in LDS; one partial (o, log2-sum-exp) per (sequence, query
//    head, slice) goes to the workspace, and a merge kernel reduces the slices.
//  * The workgroup -> (KV head, sequence, slice) map keeps each KV head on one XCD.
//  * Loads run in a ring of register sets (two steps ahead for NVFP4, four for the FP8 control);
//    only a wavefront's last group of ring-depth steps can hold tokens past its range, and the
//    groups before it run without any per-token range selects or score masks.
//  * The same kernel reads the FP8 (E4M3FN) control cache (FMT = 1): 32 bytes per lane and
//    token, one conversion per pair of values and no block scales.
#include <mutex>

#include "device_common.hpp"
#include "kernel_params.hpp"

namespace nvfp4kv {

constexpr int kDecWaves = 4;
constexpr int kDecStep = 32;
constexpr int kDecVStride = 288;  // bytes per staged V row (256 + 32 pad for transposed reads)
constexpr int kDecStageBytes = kDecStep * kDecVStride;

// One lane's share of a 32-token step: 32 head-dim values of one token in each of two 16-token
// groups, for K and V (NVFP4: 16 packed bytes plus the dword holding two scale bytes; FP8: 32
// bytes).
template <int FMT>
struct DecodeRegs {
  u32x4 kd[2], vd[2];
  u32x4 kd2[FMT == kFmtFp8 ? 2 : 1], vd2[FMT == kFmtFp8 ? 2 : 1];
  uint32_t ks[FMT == kFmtNvfp4 ? 2 : 1], vs[FMT == kFmtNvfp4 ? 2 : 1];
};

// Page id of the wave-relative page index `pi` (uniform, < 128) from the two page-id registers.
__device__ __forceinline__ int page_at(int pt0, int pt1, int pi) {
  return __builtin_amdgcn_readlane(pi < 64 ? pt0 : pt1, pi & 63);
}

// Issue the loads of the 32 tokens starting at k (two 16-token groups, one page each).  Loads
// are unconditional: a group past the wave's range re-reads the range's last group (an L2 hit),
// and tokens past the range are zeroed at use time, so every step issues the same 8 loads and
// the wait counts stay exact.  Every cache byte is read once per call, so the NVFP4 loads are
// non-temporal (streaming): measured 340 -> 320 us per call of the decode workload, and a plain
// streaming-read kernel reaches 6.1 TB/s with such loads against 5.4 TB/s without.
template <int FMT>
__device__ __forceinline__ void decode_load(const DecodeParams& p, int hk, int wk0, int wk1,
                                            int pt0, int pt1, int k, int lane, DecodeRegs<FMT>& r) {
  const int last_group = (wk1 - 1) & ~15;
  const int q4 = lane >> 4;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int first = min(k + 16 * g, last_group);
    const int page = page_at(pt0, pt1, (first - wk0) >> 4);
    const int64_t row = ((int64_t)page * p.num_kv_heads + hk) * kPageSize + (lane & 15);
    if constexpr (FMT == kFmtNvfp4) {
      r.kd[g] = __builtin_nontemporal_load((const u32x4*)(p.k_data + row * kRowBytes + 16 * q4));
      r.vd[g] = __builtin_nontemporal_load((const u32x4*)(p.v_data + row * kRowBytes + 16 * q4));
      // the dword holding this lane's two scale bytes (shifted into place at use time)
      r.ks[g] = __builtin_nontemporal_load((const uint32_t*)(p.k_scale + row * kScaleBytes + 4 * (q4 >> 1)));
      r.vs[g] = __builtin_nontemporal_load((const uint32_t*)(p.v_scale + row * kScaleBytes + 4 * (q4 >> 1)));
    } else {
      const uint8_t* kp = p.k_data + row * kHeadDim + 32 * q4;
      const uint8_t* vp = p.v_data + row * kHeadDim + 32 * q4;
      // ordinary loads: each instruction covers every other 16 bytes of the rows, and as
      // streaming loads the second instruction fetched the lines again (FP8 decode 560 -> 720 us)
      r.kd[g] = *(const u32x4*)kp;
      r.kd2[g] = *(const u32x4*)(kp + 16);
      r.vd[g] = *(const u32x4*)vp;
      r.vd2[g] = *(const u32x4*)(vp + 16);
    }
  }
}

struct DecodeState {
  f32x4 acc_o[8];
  float m_used;
  float l_part;
};

// One 32-token step: scores, V staging, online softmax, PV.
template <int FMT, bool FULL>
__device__ __forceinline__ void decode_step(const DecodeRegs<FMT>& r, int k, int wk1, int lane,
                                            const f16x8 (&qf)[4], float cs, char* stage,
                                            DecodeState& st) {
  const int q4 = lane >> 4;
  const int t16 = lane & 15;
  f32x4 sc[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const bool ok = FULL || k + 16 * g + t16 < wk1;  // this lane's token is in range
    f32x4 a = f32x4{};
    if constexpr (FMT == kFmtNvfp4) {
      const uint32_t ksw = ok ? r.ks[g] >> (16 * (q4 & 1)) : 0u;
      const f16x2 sc2 = e4m3_pair_h<false>(ksw);
      const f16x2 s0 = __builtin_shufflevector(sc2, sc2, 0, 0);
      const f16x2 s1 = __builtin_shufflevector(sc2, sc2, 1, 1);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        uint32_t o4[4];
        dequant8_h(r.kd[g][kk], kk < 2 ? s0 : s1, o4);
        a = mfma16h(__builtin_bit_cast(f16x8, u32x4{o4[0], o4[1], o4[2], o4[3]}), qf[kk], a);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint32_t w0 = ok ? (kk < 2 ? r.kd[g][2 * kk] : r.kd2[g][2 * kk - 4]) : 0u;
        const uint32_t w1 = ok ? (kk < 2 ? r.kd[g][2 * kk + 1] : r.kd2[g][2 * kk - 3]) : 0u;
        uint32_t o4[4];
        fp8x4_to_f16(w0, o4);
        fp8x4_to_f16(w1, o4 + 2);
        a = mfma16h(__builtin_bit_cast(f16x8, u32x4{o4[0], o4[1], o4[2], o4[3]}), qf[kk], a);
      }
    }
    sc[g] = a;
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const bool ok = FULL || k + 16 * g + t16 < wk1;
    uint32_t o[16];
    if constexpr (FMT == kFmtNvfp4) {
      const uint32_t vsw = ok ? r.vs[g] >> (16 * (q4 & 1)) : 0u;
      const f16x2 sc2 = e4m3_pair_h<false>(vsw);
      const f16x2 s0 = __builtin_shufflevector(sc2, sc2, 0, 0);
      const f16x2 s1 = __builtin_shufflevector(sc2, sc2, 1, 1);
      dequant8_h(r.vd[g][0], s0, o + 0);
      dequant8_h(r.vd[g][1], s0, o + 4);
      dequant8_h(r.vd[g][2], s1, o + 8);
      dequant8_h(r.vd[g][3], s1, o + 12);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fp8x4_to_f16(ok ? r.vd[g][i] : 0u, o + 2 * i);
        fp8x4_to_f16(ok ? r.vd2[g][i] : 0u, o + 8 + 2 * i);
      }
    }
    char* dst = stage + (16 * g + t16) * kDecVStride + 64 * q4;
    *(u32x4*)(dst + 0) = u32x4{o[0], o[1], o[2], o[3]};
    *(u32x4*)(dst + 16) = u32x4{o[4], o[5], o[6], o[7]};
    *(u32x4*)(dst + 32) = u32x4{o[8], o[9], o[10], o[11]};
    *(u32x4*)(dst + 48) = u32x4{o[12], o[13], o[14], o[15]};
  }
  if constexpr (!FULL) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (k + 16 * g + 4 * q4 + j >= wk1) sc[g][j] = kNegInf;
  }
  float mx = kNegInf;
#pragma unroll
  for (int j = 0; j < 4; ++j) mx = fmaxf(mx, fmaxf(sc[0][j], sc[1][j]));
  // the column maximum (across the four lanes holding the column) is only needed when some
  // lane's own maximum exceeds the reference by more than 8
  mx *= cs;
  if (wave_any(mx > st.m_used + 8.0f)) {
    const float m_new = fmaxf(st.m_used, pair32_max(pair16_max(mx)));
    const float alpha = (m_new == kNegInf) ? 1.0f : fast_exp2(st.m_used - m_new);
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc_o[i] *= alpha;
    st.l_part *= alpha;
    st.m_used = m_new;
  }
  const float mref = (st.m_used == kNegInf) ? 0.0f : st.m_used;
  // fp16 weights (rounded toward zero, relative error below 2^-10); the row sum uses the same
  // rounded weights as the PV product
  f16x8 pb;
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const f16x2 e = pack_f16x2_rtz(fast_exp2(fmaf(sc[g][j], cs, -mref)),
                                     fast_exp2(fmaf(sc[g][j + 1], cs, -mref)));
      pb[4 * g + j] = e[0];
      pb[4 * g + j + 1] = e[1];
    }
  st.l_part = sum_f16x8(pb, st.l_part);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const char* lo_row = stage + (4 * q4 + (t16 >> 2)) * kDecVStride + 8 * (t16 & 3);
  const char* hi_row = lo_row + 16 * kDecVStride;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const i16x4 lo = lds_read_tr16(lo_row + 32 * mb);
    const i16x4 hi = lds_read_tr16(hi_row + 32 * mb);
    const f16x8 a = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    st.acc_o[mb] = mfma16h(a, pb, st.acc_o[mb]);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Register sets of loads in rotation (kRing - 1 steps in flight while one is consumed) and
// workgroups per CU for each cache format.  NVFP4: three sets at three workgroups, i.e. three
// wavefronts per SIMD (150 registers).  FP8, whose sets are twice the size: five sets at two
// workgroups (236 registers).  Measured against deeper rings and other occupancies, these were
// the fastest of the shapes that do not spill.
template <int FMT>
struct DecodeShape;
template <>
struct DecodeShape<kFmtNvfp4> {
  static constexpr int kRing = 3, kBlocks = 3;
};
template <>
struct DecodeShape<kFmtFp8> {
  static constexpr int kRing = 5, kBlocks = 2;
};

template <int FMT>
__global__ __launch_bounds__(256, DecodeShape<FMT>::kBlocks) void nvfp4_decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kDecWaves * kDecStageBytes];
  __shared__ float red_m[kDecWaves][16];
  __shared__ float red_l[kDecWaves][16];

  const int wg = blockIdx.x;
  const int ipx = (p.num_kv_heads * p.batch * p.num_splits + 7) / 8;
  const int item = (wg & 7) * ipx + (wg >> 3);
  if (item >= p.num_kv_heads * p.batch * p.num_splits) return;
  const int split = item % p.num_splits;
  const int b = (item / p.num_splits) % p.batch;
  const int hk = item / (p.num_splits * p.batch);

  const int G = p.group;
  const int Hq = p.num_qo_heads;
  const int kv_len = p.kv_lens[b];
  const int key_begin = split * p.chunk;
  const int64_t prow0 = ((int64_t)split * p.batch + b) * Hq + hk * G;  // first partial row
  if (key_begin >= kv_len) {
    if (threadIdx.x < G) p.part_lse[prow0 + threadIdx.x] = kNegInf;
    return;
  }

  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int col = lane & 15;
  const int q4 = lane >> 4;
  const bool colv = col < G;

  // Q^T operand of this lane's column as fp16, scaled by 2^sh chosen from the column's largest
  // |q| (over the four lanes holding the column) so that the largest lands in [2^15, 2^16):
  // every bf16 element within a factor 2^32 of it converts exactly.  2^-sh goes into cs.
  f16x8 qf[4];
  float cs;
  {
    const uint16_t* qp = p.q + ((int64_t)b * Hq + hk * G + (colv ? col : 0)) * kHeadDim + 32 * q4;
    // A padding lane reads column 0 (always present) and zeroes it: no branch between the loads.
    u32x4 raw[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) raw[ks] = *(const u32x4*)(qp + 8 * ks);
    float amax = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (!colv) raw[ks] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        amax = fmaxf(amax, fmaxf(fabsf(__builtin_bit_cast(float, raw[ks][i] << 16)),
                                 fabsf(__builtin_bit_cast(float, raw[ks][i] & 0xFFFF0000u))));
    }
    amax = pair32_max(pair16_max(amax));
    const int sh = amax > 0.0f ? min(100, max(-100, 16 - __builtin_amdgcn_frexp_expf(amax))) : 0;
    const float up = __builtin_ldexpf(1.0f, sh);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f16x2 h = pack_f16x2_rtz(__builtin_bit_cast(float, raw[ks][i] << 16) * up,
                                       __builtin_bit_cast(float, raw[ks][i] & 0xFFFF0000u) * up);
        qf[ks][2 * i] = h[0];
        qf[ks][2 * i + 1] = h[1];
      }
    cs = p.score_scale * __builtin_ldexpf(1.0f, -sh);
  }

  const int per_wave = p.chunk / kDecWaves;  // <= 2048: 128 page ids, two per lane
  const int wk0 = key_begin + w * per_wave;
  const int wk1 = min(kv_len, wk0 + per_wave);
  const int32_t* bt_row = p.block_table + (int64_t)b * p.bt_stride;
  char* stage = smem + w * kDecStageBytes;

  DecodeState st;
#pragma unroll
  for (int i = 0; i < 8; ++i) st.acc_o[i] = f32x4{};
  st.m_used = kNegInf;
  st.l_part = 0.0f;

  if (wk0 < wk1) {
    const int seq_pages = (kv_len + 15) >> 4;
    const int pb0 = (wk0 >> 4) + lane;
    const int pt0_ld = pb0 < seq_pages ? bt_row[pb0] : 0;
    const int pt1_ld = pb0 + 64 < seq_pages ? bt_row[pb0 + 64] : 0;
    // Copy the page ids through a register move the compiler cannot see into: the loop then
    // reads plain registers instead of load results it would re-wait for on every iteration.
    int pt0, pt1;
    asm volatile("v_mov_b32 %0, %1" : "=v"(pt0) : "v"(pt0_ld));
    asm volatile("v_mov_b32 %0, %1" : "=v"(pt1) : "v"(pt1_ld));
    // register sets in rotation: the loads of kRing - 1 32-token steps are in flight while
    // the next one is consumed
    constexpr int R = DecodeShape<FMT>::kRing;
    DecodeRegs<FMT> r[R];
#pragma unroll
    for (int i = 0; i < R - 1; ++i) decode_load(p, hk, wk0, wk1, pt0, pt1, wk0 + i * kDecStep, lane, r[i]);
    // groups of R steps wholly inside [wk0, wk1) skip every range check; the last group masks
    // the keys past wk1
    int k = wk0;
    for (; k + R * kDecStep <= wk1; k += R * kDecStep) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        decode_load(p, hk, wk0, wk1, pt0, pt1, k + (i + R - 1) * kDecStep, lane, r[(i + R - 1) % R]);
        __builtin_amdgcn_sched_barrier(0);
        decode_step<FMT, true>(r[i], k + i * kDecStep, wk1, lane, qf, cs, stage, st);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (k < wk1) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        decode_load(p, hk, wk0, wk1, pt0, pt1, k + (i + R - 1) * kDecStep, lane, r[(i + R - 1) % R]);
        __builtin_amdgcn_sched_barrier(0);
        decode_step<FMT, false>(r[i], k + i * kDecStep, wk1, lane, qf, cs, stage, st);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- combine the four wavefronts in LDS
  const float l_tot = pair32_sum(pair16_sum(st.l_part));
  __syncthreads();  // every wavefront is done with its V stage
  float* red_o = (float*)smem;  // [wave][16 columns][128]
  if (q4 == 0) {
    red_m[w][col] = st.m_used;
    red_l[w][col] = l_tot;
  }
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
    *(f32x4*)(red_o + (w * 16 + col) * kHeadDim + 16 * mb + 4 * q4) = st.acc_o[mb];
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += 256) {
    const int c = idx >> 7;
    const int d = idx & 127;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) M = fmaxf(M, red_m[ww][c]);
    float L = 0.0f, o = 0.0f;
    if (M != kNegInf) {
#pragma unroll
      for (int ww = 0; ww < kDecWaves; ++ww) {
        const float mw = red_m[ww][c];
        const float wt = mw == kNegInf ? 0.0f : fast_exp2(mw - M);
        L = fmaf(wt, red_l[ww][c], L);
        o = fmaf(wt, red_o[(ww * 16 + c) * kHeadDim + d], o);
      }
    }
    // fp16, nearest-even: a weighted mean of cache values before the per-tensor V scale
    p.part_o[(prow0 + c) * kHeadDim + d] = __builtin_bit_cast(uint16_t, (_Float16)(L > 0.0f ? o / L : 0.0f));
    if (d == 0) p.part_lse[prow0 + c] = L > 0.0f ? M + __log2f(L) : kNegInf;
  }
}

// ---- static scratch of the allocation-free decode entry point ----------------------------
// One array per GPU, held from code-object load until the process ends.  Host code never uses
// the array's name as an address (on the host it names a stand-in, not device memory): the
// device address of the current GPU's copy comes from hipGetSymbolAddress, looked up once per
// device with that device current, and is what the kernels receive.  The decode writes every
// partial and log-sum-exp the merge uses before the merge reads it, so nothing in the array
// has to start at zero; calls that overlap on one GPU share the array and race.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (addr == nullptr) return hipErrorInvalidSymbol;
    per_device[dev] = addr;
  }
  *ptr = per_device[dev];
  *bytes = kDecodeScratchBytes;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  const int items = p.num_kv_heads * p.batch * p.num_splits;
  const dim3 grid((unsigned)(8 * ((items + 7) / 8)));
  if (p.fp8)
    hipLaunchKernelGGL(nvfp4_decode_kernel<kFmtFp8>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(nvfp4_decode_kernel<kFmtNvfp4>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace nvfp4kv
