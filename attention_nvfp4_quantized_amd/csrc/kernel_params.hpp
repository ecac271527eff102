// Argument blocks passed from the C-ABI layer to the kernel launchers (host and device visible).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4kv {

struct AppendParams {
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_stride;  // elements between tokens
  int64_t v_stride;
  const int64_t* slots;
  uint8_t* k_data;
  uint8_t* k_scale;
  uint8_t* v_data;
  uint8_t* v_scale;
  float k_global;
  float v_global;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t fp16_in;  // input is IEEE binary16 (else bf16)
  int32_t fp8;      // FP8 E4M3FN cache (else NVFP4)
};

struct DequantParams {
  const int64_t* slots;
  const uint8_t* k_data;
  const uint8_t* k_scale;
  const uint8_t* v_data;
  const uint8_t* v_scale;
  float k_global;
  float v_global;
  void* k_out;
  void* v_out;
  int32_t out_dtype;  // 0 bf16, 1 f32, 2 f16
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t fp8;        // FP8 E4M3FN cache (else NVFP4)
};

struct PrefillParams {
  const uint8_t* k_data;
  const uint8_t* k_scale;
  const uint8_t* v_data;
  const uint8_t* v_scale;
  const uint16_t* q;
  const int32_t* cu_q;
  const int32_t* kv_lens;
  const int32_t* block_table;
  int32_t bt_stride;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t num_qo_heads;
  int32_t group;
  int32_t q_tiles;        // ceil(max_q_len / rows_per_tile)
  int32_t num_splits;
  int32_t causal;
  int32_t total_q;
  int32_t items_per_xcd;  // ceil(total_items / 8)
  int32_t total_items;    // num_kv_heads * batch * q_tiles * num_splits
  float score_scale;      // sm_scale * k_global * log2(e)
  float out_scale;        // v_global
  float* lse;             // optional [total_q][Hq] (natural log); unused in split mode
  void* out;              // [total_q][Hq][D]
  int32_t out_f32;
  uint16_t* part_o;       // split mode: fp16 [num_splits][total_q][Hq][D]
  float* part_lse;        // split mode: [num_splits][total_q][Hq] (log2 units)
  int32_t format;         // cache format: 0 NVFP4, 1 FP8 E4M3FN, 2 fp16 (repacked)
  int32_t chunk;          // short-query kernel: keys per split (multiple of 128)
};

struct RepackParams {
  const uint8_t* k_data;  // NVFP4 source planes
  const uint8_t* k_scale;
  const uint8_t* v_data;
  const uint8_t* v_scale;
  uint16_t* k_out;        // fp16 copy: [num_pages][num_kv_heads][16][128]
  uint16_t* v_out;
  const int32_t* block_table;
  const int32_t* kv_lens;
  int32_t bt_stride;
  int32_t num_kv_heads;
};

struct MergeParams {
  const uint16_t* part_o;  // fp16 [num_splits][rows][D]
  const float* part_lse;
  int32_t num_splits;
  int32_t rows;          // total_q * Hq
  float out_scale;
  void* out;
  int32_t out_f32;
  float* lse;
};

struct DecodeParams {
  const uint8_t* k_data;
  const uint8_t* k_scale;
  const uint8_t* v_data;
  const uint8_t* v_scale;
  const uint16_t* q;
  const int32_t* kv_lens;
  const int32_t* block_table;
  int32_t bt_stride;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t num_qo_heads;
  int32_t group;
  int32_t num_splits;
  int32_t chunk;          // keys per split (multiple of 64)
  float score_scale;
  uint16_t* part_o;       // fp16 [num_splits][batch][Hq][D]
  float* part_lse;        // [num_splits][batch][Hq]
  int32_t fp8;            // FP8 E4M3FN cache (else NVFP4)
};

// Static device scratch of the allocation-free decode entry point (bytes per GPU).
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;

// Address of this GPU's copy of the static decode scratch (the current device's), looked up
// once per device; *bytes receives its size.
hipError_t decode_scratch(void** ptr, size_t* bytes);

hipError_t launch_append(const AppendParams& p, hipStream_t stream);
hipError_t launch_dequant(const DequantParams& p, hipStream_t stream);
hipError_t launch_repack(const RepackParams& p, int batch, int max_pages, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, int waves, hipStream_t stream);
// A4Q-style prefill (8-wave kernel; NVFP4 cache only); q_format 0 = MXFP8, 1 = MXFP4 queries;
// k_terms 2 = K as its exact two-term E4M3 bridge, 1 = the one-term (hi only) form.
hipError_t launch_prefill_a4q(const PrefillParams& p, int q_format, int k_terms, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);
// Short-query prefill (up to 64 query columns per sequence and KV head; p.chunk keys per slice,
// at most 8192, or 2048 for ncb 4): ncb 1 or 2 column blocks of 16 per wavefront on key
// quarters, 4 = four wavefronts of 16 columns sharing each key's conversion; always writes split
// partials (p.part_o / p.part_lse) for launch_merge.
hipError_t launch_prefill_tail(const PrefillParams& p, int ncb, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

}  // namespace nvfp4kv
