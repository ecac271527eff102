// Causal paged prefill for short query tiles over long caches (chunked-prefill tails, speculative
// chunks: "NVFP4 KV cache A4Q prefill explained", sections "Compare A4Q with dequantize-ahead
// repacking" and "Build the benchmark matrix"), for gfx950.
//
// When a sequence brings at most 64 query columns ((position, head-of-group) pairs) per KV head,
// each cache byte feeds few matrix products and the work is closer to decode than to full
// prefill: the time goes to reading and converting the cache.  So these kernels follow the
// decode kernel instead of the LDS-tiled prefill kernels:
//
//  * A workgroup owns one (sequence, KV head, key slice), walked in 32-key steps.
//  * Packed K and V of the next steps are loaded into a ring of register sets and converted to
//    fp16 (exact for every cache value); K becomes 16x16x32 MFMA A operands directly (head-dim
//    order permuted identically in K and Q), V goes to an LDS stage read back transposed for
//    O^T = V^T P^T.
//  * Per query column: its Q as fp16 with a power-of-two scale (exact, as in the other kernels),
//    a base-2 online softmax with lazy rescaling, and fp16 weights rounded toward zero.  Every
//    converted K fragment and V^T fragment feeds one MFMA per 16-column block.
//  * Up to 32 columns (one or two blocks): four wavefronts, one per contiguous quarter of the
//    slice, each converting its own K and V with no workgroup barrier; the quarters are merged
//    in LDS at the end.
//  * 33 to 64 columns: the accumulators and Q operands of 64 columns do not fit one wavefront's
//    registers, and converting the cache once per 32 columns doubles the conversion work.  So
//    four wavefronts of 16 columns each share one conversion of every key: each converts a
//    quarter of the step's K and V into double-buffered LDS stages, with one workgroup barrier
//    per step, and at about 128 registers four such workgroups share a CU.
//  * Causal masking: query position i of a sequence sees keys <= kv_len - q_len + i, so steps
//    below kv_len - q_len + 1 are visible to every column and run without masks; only the steps
//    after that apply the per-column limit.
//  * One partial per (slice, row) goes to the split workspace; the merge kernel of the split
//    paths combines the slices.
#include "device_common.hpp"
#include "kernel_params.hpp"

namespace nvfp4kv {

constexpr int kTailQuarters = 4;
constexpr int kTailStep = 32;
constexpr int kTailVStride = 288;  // bytes per staged V row (256 + 32 pad for transposed reads)
constexpr int kTailVStage = kTailStep * kTailVStride;
constexpr int kTailKStage = kTailStep * kHeadDim * 2;  // converted K of a step, in lane order

// One lane's share of one cache plane (K or V) for a 32-key step: 32 head-dim values of one key
// in each of two 16-key groups (NVFP4: 16 packed bytes and the dword holding the two scale bytes;
// FP8: 32 bytes).
template <int FMT>
struct PlaneRegs {
  u32x4 d[2];
  u32x4 d2[FMT == kFmtFp8 ? 2 : 1];
  uint32_t s[FMT == kFmtNvfp4 ? 2 : 1];
};

// Page id of the wave-relative page index `pi` (uniform, < 128) from the two page-id registers.
__device__ __forceinline__ int tail_page(int pt0, int pt1, int pi) {
  return __builtin_amdgcn_readlane(pi < 64 ? pt0 : pt1, pi & 63);
}

// Loads of one plane for the 32 keys starting at k, unconditional: a group past the quarter's
// range re-reads its last group (an empty range reads its first page), and keys past the range
// are zeroed at use.  Each cache byte is read by one workgroup once, so the NVFP4 loads are
// non-temporal (streaming).
template <int FMT>
__device__ __forceinline__ void plane_load(const PrefillParams& p, const uint8_t* data,
                                           const uint8_t* scale, int hk, int wk0, int wk1, int pt0,
                                           int pt1, int k, int lane, PlaneRegs<FMT>& r) {
  const int last_group = max(wk0, (wk1 - 1) & ~15);
  const int q4 = lane >> 4;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int first = min(k + 16 * g, last_group);
    const int page = tail_page(pt0, pt1, (first - wk0) >> 4);
    const int64_t row = ((int64_t)page * p.num_kv_heads + hk) * kPageSize + (lane & 15);
    if constexpr (FMT == kFmtNvfp4) {
      r.d[g] = __builtin_nontemporal_load((const u32x4*)(data + row * kRowBytes + 16 * q4));
      r.s[g] = __builtin_nontemporal_load((const uint32_t*)(scale + row * kScaleBytes + 4 * (q4 >> 1)));
    } else {
      const uint8_t* dp = data + row * kHeadDim + 32 * q4;
      r.d[g] = *(const u32x4*)dp;  // ordinary loads: see group_load
      r.d2[g] = *(const u32x4*)(dp + 16);
    }
  }
}

// fp16 values of k-step kk (head-dim values 32 q4 + 8 kk .. + 7 of this lane's key) of group g;
// zero when the key is out of range (ok false).
template <int FMT>
__device__ __forceinline__ f16x8 plane_frag(const PlaneRegs<FMT>& r, int g, int kk, bool ok, int q4) {
  uint32_t o4[4];
  if constexpr (FMT == kFmtNvfp4) {
    const uint32_t sw = ok ? r.s[g] >> (16 * (q4 & 1)) : 0u;
    const f16x2 sc2 = e4m3_pair_h<false>(sw);
    const f16x2 s = kk < 2 ? __builtin_shufflevector(sc2, sc2, 0, 0) : __builtin_shufflevector(sc2, sc2, 1, 1);
    dequant8_h(r.d[g][kk], s, o4);
  } else {
    const uint32_t w0 = ok ? (kk < 2 ? r.d[g][2 * kk] : r.d2[g][2 * kk - 4]) : 0u;
    const uint32_t w1 = ok ? (kk < 2 ? r.d[g][2 * kk + 1] : r.d2[g][2 * kk - 3]) : 0u;
    fp8x4_to_f16(w0, o4);
    fp8x4_to_f16(w1, o4 + 2);
  }
  return __builtin_bit_cast(f16x8, u32x4{o4[0], o4[1], o4[2], o4[3]});
}

// V fragment (g, kk) of this lane into the transposed-read stage: row = key, 16 bytes at the
// lane's head-dim values.
__device__ __forceinline__ void stage_v(char* stage, int g, int kk, int lane, f16x8 v) {
  *(f16x8*)(stage + (16 * g + (lane & 15)) * kTailVStride + 64 * (lane >> 4) + 16 * kk) = v;
}

template <int NCB>
struct TailState {
  f32x4 acc_o[NCB][8];
  float m_used[NCB];
  f32x4 acc_l[NCB];  // column sums of the weights (every element holds the column's sum)
};

// Masks, online softmax and PV of one 32-key step, from the scores and the staged V.
template <int NCB, bool FULL>
__device__ __forceinline__ void softmax_pv(f32x4 (&sc)[NCB][2], int k, int wk1, int lane,
                                           const float (&cs)[NCB], const int (&lim)[NCB],
                                           const char* stage, TailState<NCB>& st) {
  const int q4 = lane >> 4;
  const int t16 = lane & 15;
  if constexpr (!FULL) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = k + 16 * g + 4 * q4 + j;
          if (key >= wk1 || key > lim[cb]) sc[cb][g][j] = kNegInf;
        }
  }
  // fp16 weights (rounded toward zero, relative error below 2^-10); each row sum uses the same
  // rounded weights as the PV product
  f16x8 pb[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    // the column maximum (across the four lanes holding the column) is only needed when some
    // lane's own maximum exceeds the reference by more than 8
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = fmaxf(mx, fmaxf(sc[cb][0][j], sc[cb][1][j]));
    mx *= cs[cb];
    if (wave_any(mx > st.m_used[cb] + 8.0f)) {
      const float m_new = fmaxf(st.m_used[cb], pair32_max(pair16_max(mx)));
      const float alpha = (m_new == kNegInf) ? 1.0f : fast_exp2(st.m_used[cb] - m_new);
#pragma unroll
      for (int i = 0; i < 8; ++i) st.acc_o[cb][i] *= alpha;
      st.acc_l[cb] *= alpha;
      st.m_used[cb] = m_new;
    }
    const float mref = (st.m_used[cb] == kNegInf) ? 0.0f : st.m_used[cb];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        const f16x2 e = pack_f16x2_rtz(fast_exp2(fmaf(sc[cb][g][j], cs[cb], -mref)),
                                       fast_exp2(fmaf(sc[cb][g][j + 1], cs[cb], -mref)));
        pb[cb][4 * g + j] = e[0];
        pb[cb][4 * g + j + 1] = e[1];
      }
  }
  // column sums on the matrix cores: a block of ones times P^T (the same rounded weights as PV)
  const f16x8 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f,
                      (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) st.acc_l[cb] = mfma16h(ones, pb[cb], st.acc_l[cb]);
  // V^T operand: the k order (keys) matches the weights' P^T layout above
  const char* lo_row = stage + (4 * q4 + (t16 >> 2)) * kTailVStride + 8 * (t16 & 3);
  const char* hi_row = lo_row + 16 * kTailVStride;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const i16x4 lo = lds_read_tr16(lo_row + 32 * mb);
    const i16x4 hi = lds_read_tr16(hi_row + 32 * mb);
    const f16x8 a = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) st.acc_o[cb][mb] = mfma16h(a, pb[cb], st.acc_o[cb][mb]);
  }
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One 32-key step of a wavefront that converts both planes itself (up to 32 columns).
template <int FMT, int NCB, bool FULL>
__device__ __forceinline__ void solo_step(const PlaneRegs<FMT>& rk, const PlaneRegs<FMT>& rv, int k,
                                          int wk1, int lane, const f16x8 (&qf)[NCB][4],
                                          const float (&cs)[NCB], const int (&lim)[NCB], char* stage,
                                          TailState<NCB>& st) {
  const int q4 = lane >> 4;
  const int t16 = lane & 15;
  f32x4 sc[NCB][2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const bool ok = FULL || k + 16 * g + t16 < wk1;  // this lane's key is in range
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) sc[cb][g] = f32x4{};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const f16x8 a = plane_frag(rk, g, kk, ok, q4);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) sc[cb][g] = mfma16h(a, qf[cb][kk], sc[cb][g]);
    }
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const bool ok = FULL || k + 16 * g + t16 < wk1;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) stage_v(stage, g, kk, lane, plane_frag(rv, g, kk, ok, q4));
  }
  wave_sync_lds();
  softmax_pv<NCB, FULL>(sc, k, wk1, lane, cs, lim, stage, st);
  wave_sync_lds();
}

// Register sets of loads in rotation and workgroups per CU for up to 32 columns (four
// wavefronts with NCB blocks each; NVFP4: 152 and 210 registers; FP8, whose sets are twice the
// size: 178 and 238).
template <int FMT, int NCB>
struct TailShape {
  static constexpr int kBlocks = NCB == 2 || FMT == kFmtFp8 ? 2 : 3;
  static constexpr int kRing = 3;
  static constexpr int kCols = 16 * NCB;  // columns per workgroup
  static constexpr int kStageBytes = kTailQuarters * kTailVStage;
  static constexpr int kRedBytes = kTailQuarters * kCols * (kHeadDim + 2) * 4;
  static constexpr int kSmem = kStageBytes > kRedBytes ? kStageBytes : kRedBytes;
};

template <int FMT, int NCB>
__global__ __launch_bounds__(256, (TailShape<FMT, NCB>::kBlocks)) void
nvfp4_prefill_tail_kernel(PrefillParams p) {
  using Shape = TailShape<FMT, NCB>;
  constexpr int kThreads = 256;
  constexpr int kCols = Shape::kCols;
  constexpr int kRowF = kHeadDim + 2;
  // LDS: the stages while walking; afterwards each quarter's (O, m, l) per column for the merge
  __shared__ __attribute__((aligned(16))) char smem[Shape::kSmem];
  __shared__ float coef[kTailQuarters][kCols];
  __shared__ float col_lse[kCols];

  const int wg = blockIdx.x;
  const int item = (wg & 7) * p.items_per_xcd + (wg >> 3);
  if (item >= p.total_items) return;
  // item = (hk * batch + b) * splits + split
  const int split = item % p.num_splits;
  const int b = (item / p.num_splits) % p.batch;
  const int hk = item / (p.num_splits * p.batch);
  const int G = p.group;
  const int Hq = p.num_qo_heads;
  const int q_start = p.cu_q[b];
  const int q_len = p.cu_q[b + 1] - q_start;
  const int kv_len = p.kv_lens[b];
  const int ncols = min(kCols, q_len * G);  // valid columns of this sequence
  const int key_begin = split * p.chunk;
  const int key_end = min(kv_len, key_begin + p.chunk);
  const int shift = p.causal ? kv_len - q_len : 0;  // position i sees keys <= shift + i
  const int64_t part0 = (int64_t)split * p.total_q * Hq;

  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int quarter = w;
  const int t16 = lane & 15;
  const int q4 = lane >> 4;

  if (ncols <= 0) return;  // no queries in this sequence
  if (key_begin >= key_end) {  // nothing in this slice: an empty partial per row
    for (int c = threadIdx.x; c < ncols; c += kThreads)
      p.part_lse[part0 + (int64_t)(q_start + c / G) * Hq + hk * G + c % G] = kNegInf;
    return;
  }

  // Q^T operands: column 16 cb + t16 holds head-dim values 32 q4 .. 32 q4 + 31 in this lane
  // (k-step kk: values 32 q4 + 8 kk .. + 7), scaled by a power of two chosen from the column's
  // largest |q| so that it lands in [2^15, 2^16) (every bf16 element within 2^32 of it exact).
  f16x8 qf[NCB][4];
  float cs[NCB];
  int lim[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int col = 16 * cb + t16;
    const bool colv = col < ncols;
    const int pos = colv ? col / G : 0;
    const uint16_t* qp = p.q + ((int64_t)(q_start + pos) * Hq + hk * G + (colv ? col % G : 0)) * kHeadDim + 32 * q4;
    u32x4 raw[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) raw[kk] = *(const u32x4*)(qp + 8 * kk);
    float amax = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (!colv) raw[kk] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        amax = fmaxf(amax, fmaxf(fabsf(__builtin_bit_cast(float, raw[kk][i] << 16)),
                                 fabsf(__builtin_bit_cast(float, raw[kk][i] & 0xFFFF0000u))));
    }
    amax = pair32_max(pair16_max(amax));
    const int sh = amax > 0.0f ? min(100, max(-100, 16 - __builtin_amdgcn_frexp_expf(amax))) : 0;
    const float up = __builtin_ldexpf(1.0f, sh);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f16x2 h = pack_f16x2_rtz(__builtin_bit_cast(float, raw[kk][i] << 16) * up,
                                       __builtin_bit_cast(float, raw[kk][i] & 0xFFFF0000u) * up);
        qf[cb][kk][2 * i] = h[0];
        qf[cb][kk][2 * i + 1] = h[1];
      }
    cs[cb] = p.score_scale * __builtin_ldexpf(1.0f, -sh);
    lim[cb] = colv ? (p.causal ? shift + pos : kv_len - 1) : -1;
  }

  const int per_quarter = p.chunk / kTailQuarters;  // <= 2048: 128 page ids, two per lane
  const int wk0 = key_begin + quarter * per_quarter;
  const int wk1 = min(key_end, wk0 + per_quarter);
  // keys below kv_len - q_len + 1 are visible to every column (all keys without the causal mask)
  const int wk_full = p.causal ? min(wk1, shift + 1) : wk1;
  const int32_t* bt_row = p.block_table + (int64_t)b * p.bt_stride;

  TailState<NCB> st;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc_o[cb][i] = f32x4{};
    st.m_used[cb] = kNegInf;
    st.acc_l[cb] = f32x4{};
  }

  constexpr int R = Shape::kRing;
  int pt0, pt1;
  {
    const int seq_pages = (kv_len + 15) >> 4;
    const int pb0 = (wk0 >> 4) + lane;
    const int pt0_ld = pb0 < seq_pages ? bt_row[pb0] : 0;
    const int pt1_ld = pb0 + 64 < seq_pages ? bt_row[pb0 + 64] : 0;
    // page ids through a register move the compiler cannot see into, so the loop reads plain
    // registers instead of re-waiting for the load results
    asm volatile("v_mov_b32 %0, %1" : "=v"(pt0) : "v"(pt0_ld));
    asm volatile("v_mov_b32 %0, %1" : "=v"(pt1) : "v"(pt1_ld));
  }

  if (wk0 < wk1) {
    char* stage = smem + quarter * kTailVStage;
    PlaneRegs<FMT> rk[R], rv[R];
#pragma unroll
    for (int i = 0; i < R - 1; ++i) {
      plane_load(p, p.k_data, p.k_scale, hk, wk0, wk1, pt0, pt1, wk0 + i * kTailStep, lane, rk[i]);
      plane_load(p, p.v_data, p.v_scale, hk, wk0, wk1, pt0, pt1, wk0 + i * kTailStep, lane, rv[i]);
    }
    int k = wk0;
    for (; k + R * kTailStep <= wk_full; k += R * kTailStep) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int nx = (i + R - 1) % R;
        plane_load(p, p.k_data, p.k_scale, hk, wk0, wk1, pt0, pt1, k + (i + R - 1) * kTailStep, lane, rk[nx]);
        plane_load(p, p.v_data, p.v_scale, hk, wk0, wk1, pt0, pt1, k + (i + R - 1) * kTailStep, lane, rv[nx]);
        __builtin_amdgcn_sched_barrier(0);
        solo_step<FMT, NCB, true>(rk[i], rv[i], k + i * kTailStep, wk1, lane, qf, cs, lim, stage, st);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    for (; k < wk1; k += R * kTailStep) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int nx = (i + R - 1) % R;
        plane_load(p, p.k_data, p.k_scale, hk, wk0, wk1, pt0, pt1, k + (i + R - 1) * kTailStep, lane, rk[nx]);
        plane_load(p, p.v_data, p.v_scale, hk, wk0, wk1, pt0, pt1, k + (i + R - 1) * kTailStep, lane, rv[nx]);
        __builtin_amdgcn_sched_barrier(0);
        solo_step<FMT, NCB, false>(rk[i], rv[i], k + i * kTailStep, wk1, lane, qf, cs, lim, stage, st);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- merge the quarters in LDS: [quarter][column][128 O values, m, l] as float32
  float l_tot[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) l_tot[cb] = st.acc_l[cb][0];
  __syncthreads();  // every wavefront is done with the stages
  float* red = (float*)smem;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    float* rw = red + (quarter * kCols + 16 * cb + t16) * kRowF;
    if (q4 == 0) {
      rw[kHeadDim] = st.m_used[cb];
      rw[kHeadDim + 1] = l_tot[cb];
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) rw[16 * mb + 4 * q4 + j] = st.acc_o[cb][mb][j];
  }
  __syncthreads();
  // per column: the quarters' weights (normalised by the column's total) and log2-sum-exp
  for (int c = threadIdx.x; c < ncols; c += kThreads) {
    float M = kNegInf;
#pragma unroll
    for (int qq = 0; qq < kTailQuarters; ++qq) M = fmaxf(M, red[(qq * kCols + c) * kRowF + kHeadDim]);
    float wt[kTailQuarters];
    float L = 0.0f;
#pragma unroll
    for (int qq = 0; qq < kTailQuarters; ++qq) {
      const float* rw = red + (qq * kCols + c) * kRowF;
      wt[qq] = (M == kNegInf || rw[kHeadDim] == kNegInf) ? 0.0f : fast_exp2(rw[kHeadDim] - M);
      L = fmaf(wt[qq], rw[kHeadDim + 1], L);
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
    for (int qq = 0; qq < kTailQuarters; ++qq) coef[qq][c] = wt[qq] * inv;
    col_lse[c] = L > 0.0f ? M + __log2f(L) : kNegInf;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < ncols * (kHeadDim / 2); idx += kThreads) {
    const int c = idx >> 6;
    const int d = 2 * (idx & 63);
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int qq = 0; qq < kTailQuarters; ++qq) {
      const float* rw = red + (qq * kCols + c) * kRowF + d;
      o0 = fmaf(coef[qq][c], rw[0], o0);
      o1 = fmaf(coef[qq][c], rw[1], o1);
    }
    const int64_t row = part0 + (int64_t)(q_start + c / G) * Hq + hk * G + c % G;
    // fp16, nearest-even: a weighted mean of cache values before the per-tensor V scale
    *(uint32_t*)(p.part_o + row * kHeadDim + d) = pack_f16x2_rne(o0, o1);
    if (d == 0) p.part_lse[row] = col_lse[c];
  }
}

// 33 to 64 columns: a workgroup of four wavefronts walks its key slice (at most 2048 keys) in
// 32-key steps, wavefront c owning columns 16 c .. 16 c + 15.  The step's four cache parts (K
// keys 0-15, K keys 16-31, V keys 0-15, V keys 16-31) are converted one per wavefront into
// double-buffered LDS stages (K in MFMA operand order, V for the transposed read), with one
// barrier per step; every wavefront then reads all of K and V^T.  Each wavefront writes its
// columns' partial directly.
constexpr int kQuadStage = 2 * kTailKStage + 2 * kTailVStage;

// One lane's share of one 16-key group of one plane: 32 head-dim values of one key.
template <int FMT>
struct GroupRegs {
  u32x4 d;
  u32x4 d2[1];  // FP8: the second 16 bytes
  uint32_t s;
};

// Load of the 16-key group starting at kg (unconditional, clamped as in plane_load).
template <int FMT>
__device__ __forceinline__ void group_load(const PrefillParams& p, const uint8_t* data,
                                           const uint8_t* scale, int hk, int wk0, int wk1, int pt0,
                                           int pt1, int kg, int lane, GroupRegs<FMT>& r) {
  const int last_group = max(wk0, (wk1 - 1) & ~15);
  const int q4 = lane >> 4;
  const int first = min(kg, last_group);
  const int page = tail_page(pt0, pt1, (first - wk0) >> 4);
  const int64_t row = ((int64_t)page * p.num_kv_heads + hk) * kPageSize + (lane & 15);
  if constexpr (FMT == kFmtNvfp4) {
    r.d = __builtin_nontemporal_load((const u32x4*)(data + row * kRowBytes + 16 * q4));
    r.s = __builtin_nontemporal_load((const uint32_t*)(scale + row * kScaleBytes + 4 * (q4 >> 1)));
  } else {
    const uint8_t* dp = data + row * kHeadDim + 32 * q4;
    // ordinary loads: each instruction covers every other 16 bytes of the rows, and as
    // streaming loads the second instruction would fetch the lines again
    r.d = *(const u32x4*)dp;
    r.d2[0] = *(const u32x4*)(dp + 16);
  }
}

// fp16 values of k-step kk of this lane's key in the group (zero when ok is false).
template <int FMT>
__device__ __forceinline__ f16x8 group_frag(const GroupRegs<FMT>& r, int kk, bool ok, int q4) {
  uint32_t o4[4];
  if constexpr (FMT == kFmtNvfp4) {
    const uint32_t sw = ok ? r.s >> (16 * (q4 & 1)) : 0u;
    const f16x2 sc2 = e4m3_pair_h<false>(sw);
    const f16x2 sv = kk < 2 ? __builtin_shufflevector(sc2, sc2, 0, 0) : __builtin_shufflevector(sc2, sc2, 1, 1);
    dequant8_h(r.d[kk], sv, o4);
  } else {
    const uint32_t w0 = ok ? (kk < 2 ? r.d[2 * kk] : r.d2[0][2 * kk - 4]) : 0u;
    const uint32_t w1 = ok ? (kk < 2 ? r.d[2 * kk + 1] : r.d2[0][2 * kk - 3]) : 0u;
    fp8x4_to_f16(w0, o4);
    fp8x4_to_f16(w1, o4 + 2);
  }
  return __builtin_bit_cast(f16x8, u32x4{o4[0], o4[1], o4[2], o4[3]});
}

template <int FMT>
struct QuadShape {
  static constexpr int kRing = 4;
};

template <int FMT, bool FULL>
__device__ __forceinline__ void quad_step(const GroupRegs<FMT>& r, int part, int k, int wk1, int lane,
                                          const f16x8 (&qf)[1][4], const float (&cs)[1],
                                          const int (&lim)[1], char* kst, char* vst,
                                          TailState<1>& st) {
  const int q4 = lane >> 4;
  const int t16 = lane & 15;
  const int pg = part & 1;  // key group of this wavefront's part
  {
    const bool ok = FULL || k + 16 * pg + t16 < wk1;
    f16x8 frag[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) frag[kk] = group_frag(r, kk, ok, q4);
    if (part < 2) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) *(f16x8*)(kst + ((4 * pg + kk) * 64 + lane) * 16) = frag[kk];
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) stage_v(vst, pg, kk, lane, frag[kk]);
    }
  }
  __syncthreads();
  f32x4 sc[1][2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    f16x8 kf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kf[kk] = *(const f16x8*)(kst + ((4 * g + kk) * 64 + lane) * 16);
    f32x4 a = f32x4{};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) a = mfma16h(kf[kk], qf[0][kk], a);
    sc[0][g] = a;
  }
  softmax_pv<1, FULL>(sc, k, wk1, lane, cs, lim, vst, st);
}

template <int FMT>
__global__ __launch_bounds__(256, 4) void nvfp4_prefill_tail_quad_kernel(PrefillParams p) {
  constexpr int R = QuadShape<FMT>::kRing;
  __shared__ __attribute__((aligned(16))) char smem[kQuadStage];

  const int wg = blockIdx.x;
  const int item = (wg & 7) * p.items_per_xcd + (wg >> 3);
  if (item >= p.total_items) return;
  // item = (hk * batch + b) * splits + split
  const int split = item % p.num_splits;
  const int b = (item / p.num_splits) % p.batch;
  const int hk = item / (p.num_splits * p.batch);
  const int G = p.group;
  const int Hq = p.num_qo_heads;
  const int q_start = p.cu_q[b];
  const int q_len = p.cu_q[b + 1] - q_start;
  const int kv_len = p.kv_lens[b];
  const int ncols = min(64, q_len * G);  // valid columns of this sequence
  const int key_begin = split * p.chunk;
  const int key_end = min(kv_len, key_begin + p.chunk);
  const int shift = p.causal ? kv_len - q_len : 0;  // position i sees keys <= shift + i
  const int64_t part0 = (int64_t)split * p.total_q * Hq;

  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int t16 = lane & 15;
  const int q4 = lane >> 4;

  if (ncols <= 0) return;  // no queries in this sequence
  if (key_begin >= key_end) {  // nothing in this slice: an empty partial per row
    for (int c = threadIdx.x; c < ncols; c += 256)
      p.part_lse[part0 + (int64_t)(q_start + c / G) * Hq + hk * G + c % G] = kNegInf;
    return;
  }

  // Q^T operand of column 16 w + t16 (see the other kernels): head-dim values 32 q4 + 8 kk .. + 7
  // in k-step kk, scaled by a power of two into [2^15, 2^16) (exact)
  f16x8 qf[1][4];
  float cs[1];
  int lim[1];
  const int col = 16 * w + t16;
  const bool colv = col < ncols;
  const int pos = colv ? col / G : 0;
  {
    const uint16_t* qp = p.q + ((int64_t)(q_start + pos) * Hq + hk * G + (colv ? col % G : 0)) * kHeadDim + 32 * q4;
    u32x4 raw[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) raw[kk] = *(const u32x4*)(qp + 8 * kk);
    float amax = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (!colv) raw[kk] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        amax = fmaxf(amax, fmaxf(fabsf(__builtin_bit_cast(float, raw[kk][i] << 16)),
                                 fabsf(__builtin_bit_cast(float, raw[kk][i] & 0xFFFF0000u))));
    }
    amax = pair32_max(pair16_max(amax));
    const int sh = amax > 0.0f ? min(100, max(-100, 16 - __builtin_amdgcn_frexp_expf(amax))) : 0;
    const float up = __builtin_ldexpf(1.0f, sh);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f16x2 h = pack_f16x2_rtz(__builtin_bit_cast(float, raw[kk][i] << 16) * up,
                                       __builtin_bit_cast(float, raw[kk][i] & 0xFFFF0000u) * up);
        qf[0][kk][2 * i] = h[0];
        qf[0][kk][2 * i + 1] = h[1];
      }
    cs[0] = p.score_scale * __builtin_ldexpf(1.0f, -sh);
    lim[0] = colv ? (p.causal ? shift + pos : kv_len - 1) : -1;
  }

  // the slice's keys, at most 2048 (128 page ids, two per lane)
  const int wk0 = key_begin;
  const int wk1 = key_end;
  const int wk_full = p.causal ? min(wk1, shift + 1) : wk1;  // keys visible to every column
  const int32_t* bt_row = p.block_table + (int64_t)b * p.bt_stride;
  int pt0, pt1;
  {
    const int seq_pages = (kv_len + 15) >> 4;
    const int pb0 = (wk0 >> 4) + lane;
    const int pt0_ld = pb0 < seq_pages ? bt_row[pb0] : 0;
    const int pt1_ld = pb0 + 64 < seq_pages ? bt_row[pb0 + 64] : 0;
    asm volatile("v_mov_b32 %0, %1" : "=v"(pt0) : "v"(pt0_ld));
    asm volatile("v_mov_b32 %0, %1" : "=v"(pt1) : "v"(pt1_ld));
  }

  TailState<1> st;
#pragma unroll
  for (int i = 0; i < 8; ++i) st.acc_o[0][i] = f32x4{};
  st.m_used[0] = kNegInf;
  st.acc_l[0] = f32x4{};

  // this wavefront's part: K (w < 2) or V, key group w & 1 of each step
  const int part = w;
  const uint8_t* data = part < 2 ? p.k_data : p.v_data;
  const uint8_t* scale = part < 2 ? p.k_scale : p.v_scale;
  const int goff = 16 * (part & 1);
  char* kst0 = smem;
  char* vst0 = smem + 2 * kTailKStage;
  GroupRegs<FMT> r[R];
#pragma unroll
  for (int i = 0; i < R - 1; ++i)
    group_load(p, data, scale, hk, wk0, wk1, pt0, pt1, wk0 + i * kTailStep + goff, lane, r[i]);
  int k = wk0;
  for (; k + R * kTailStep <= wk_full; k += R * kTailStep) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      group_load(p, data, scale, hk, wk0, wk1, pt0, pt1, k + (i + R - 1) * kTailStep + goff, lane, r[(i + R - 1) % R]);
      __builtin_amdgcn_sched_barrier(0);
      quad_step<FMT, true>(r[i], part, k + i * kTailStep, wk1, lane, qf, cs, lim,
                           kst0 + (i & 1) * kTailKStage, vst0 + (i & 1) * kTailVStage, st);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  for (; k < wk1; k += R * kTailStep) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      group_load(p, data, scale, hk, wk0, wk1, pt0, pt1, k + (i + R - 1) * kTailStep + goff, lane, r[(i + R - 1) % R]);
      __builtin_amdgcn_sched_barrier(0);
      quad_step<FMT, false>(r[i], part, k + i * kTailStep, wk1, lane, qf, cs, lim,
                            kst0 + (i & 1) * kTailKStage, vst0 + (i & 1) * kTailVStage, st);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // this wavefront's 16 columns: O / l as fp16 (nearest-even) and log2-sum-exp
  if (colv) {
    const float l_tot = st.acc_l[0][0];
    const int64_t row = part0 + (int64_t)(q_start + pos) * Hq + hk * G + col % G;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const f32x4 o = st.acc_o[0][mb];
      *(u32x2*)(p.part_o + row * kHeadDim + 16 * mb + 4 * q4) =
          u32x2{pack_f16x2_rne(o[0] * inv, o[1] * inv), pack_f16x2_rne(o[2] * inv, o[3] * inv)};
    }
    if (q4 == 0) p.part_lse[row] = l_tot > 0.0f ? st.m_used[0] + __log2f(l_tot) : kNegInf;
  }
}

template <int FMT>
hipError_t launch_tail_fmt(const PrefillParams& p, int ncb, hipStream_t stream) {
  const dim3 grid((unsigned)(8 * p.items_per_xcd));
  switch (ncb) {
    case 1: hipLaunchKernelGGL((nvfp4_prefill_tail_kernel<FMT, 1>), grid, dim3(256), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((nvfp4_prefill_tail_kernel<FMT, 2>), grid, dim3(256), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((nvfp4_prefill_tail_quad_kernel<FMT>), grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_tail(const PrefillParams& p, int ncb, hipStream_t stream) {
  switch (p.format) {
    case kFmtNvfp4: return launch_tail_fmt<kFmtNvfp4>(p, ncb, stream);
    case kFmtFp8: return launch_tail_fmt<kFmtFp8>(p, ncb, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nvfp4kv
