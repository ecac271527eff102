// C ABI of the NVFP4 paged KV-cache attention library: argument validation, grid and split
// sizing, and kernel launches.  Nothing here allocates, frees or synchronizes.
#include "../../include/nvfp4kv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "kernel_params.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return NVFP4KV_OK;
}

int check_launch(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(NVFP4KV_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int check_cache(const nvfp4kv_cache_t* c) {
  if (!c) return fail(NVFP4KV_EINVAL, "cache descriptor is NULL");
  if (c->kv_format != NVFP4KV_FORMAT_NVFP4 && c->kv_format != NVFP4KV_FORMAT_FP8 &&
      c->kv_format != NVFP4KV_FORMAT_F16)
    return fail(NVFP4KV_EINVAL, "kv_format %d unknown", c->kv_format);
  const bool scales = c->kv_format == NVFP4KV_FORMAT_NVFP4;
  if (!c->k_data || !c->v_data || (scales && (!c->k_scale || !c->v_scale)))
    return fail(NVFP4KV_EINVAL, "cache plane pointer is NULL");
  if (c->head_dim != 128)
    return fail(NVFP4KV_EUNSUPPORTED, "head_dim %d unsupported (K and V head size must be 128)",
                c->head_dim);
  if (c->page_size != 16) return fail(NVFP4KV_EUNSUPPORTED, "page_size %d unsupported (16)", c->page_size);
  if (c->num_kv_heads < 1) return fail(NVFP4KV_EINVAL, "num_kv_heads must be >= 1");
  if (c->num_pages < 1) return fail(NVFP4KV_EINVAL, "num_pages must be >= 1");
  if (!(c->k_global > 0.0f) || !std::isfinite(c->k_global) || !(c->v_global > 0.0f) ||
      !std::isfinite(c->v_global))
    return fail(NVFP4KV_EINVAL, "global scales must be finite and > 0");
  if (c->kv_format == NVFP4KV_FORMAT_F16 && (((uintptr_t)c->k_data | (uintptr_t)c->v_data) & 15u))
    return fail(NVFP4KV_EINVAL, "fp16 cache planes must be 16-byte aligned");
  return NVFP4KV_OK;
}

// The fp16 (repacked) format is written by the repack pass and read by the prefill only.
int check_not_f16(const nvfp4kv_cache_t* c, const char* what) {
  if (c->kv_format == NVFP4KV_FORMAT_F16)
    return fail(NVFP4KV_EUNSUPPORTED, "%s does not take the fp16 (repacked) cache format", what);
  return NVFP4KV_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Workspace of the split paths, per (split, output row): the fp16 partial (128 values), then,
// after all partials, its float32 log-sum-exp.
constexpr size_t kPartRowBytes = 128 * sizeof(uint16_t) + sizeof(float);

constexpr int kDecodeChunkMin = 512;   // keys per decode slice, lower bound
constexpr int kDecodeChunkMax = 8192;  // keys per decode slice, upper bound

// Column wavefronts per prefill workgroup (query columns = rows x group of the longest
// sequence): 8 above 128 columns (the 8-wave kernel's 256-column tiles, the last one padded; from
// 129 columns on it beats the four-wave kernel), 4 for 65-128, else 2, which selects the
// key-split kernel (two column wavefronts, each tile's keys split between two more).  At 32
// columns or fewer the second column wavefront only pads, and the kernel still runs about twice
// as fast as one wavefront walking every key.
int prefill_waves(int max_q_len, int group) {
  const long cols = (long)max_q_len * group;
  if (cols > 128) return 8;
  if (cols > 64) return 4;
  return 2;
}

// Key slices per prefill work item.  Slicing buys parallelism when there are fewer work items
// than the GPU holds at once (256 CUs x workgroups per CU: one 8-wave workgroup, whose three
// tile buffers fill most of the LDS, or two narrow ones), but every extra slice writes and
// re-reads an fp16 partial of the whole output; so slice only up to that occupancy, and keep at
// least 8 tiles (512 keys) per slice.
int prefill_splits(int batch, int q_tiles, int num_kv_heads, int max_kv_len, int nw, int requested) {
  if (requested > 0) return requested;
  const long base = (long)batch * q_tiles * num_kv_heads;
  const long slots = 256L * (nw == 8 ? 1 : 2);
  if (base >= slots) return 1;
  const long want = (slots + base - 1) / base;
  const long cap = std::max(1, max_kv_len / 512);
  return (int)std::max(1L, std::min(want, cap));
}

// Key slices per (sequence, KV head) of a decode call.  The automatic count aims at about 512
// workgroups (two thirds of the 768 the GPU holds at once): measured on 1, 4, 16 and 64 sequences
// of 16K-32K keys, more slices only add workgroup set-up and merge work.  Long caches are sliced
// further by the per-slice key limit below.
int decode_splits(int batch, int num_kv_heads, int max_kv_len, int requested, int* chunk,
                  long target = 512, int chunk_max = kDecodeChunkMax) {
  int s = requested;
  if (s <= 0) {
    const long pairs = (long)batch * num_kv_heads;
    const long want = std::max(1L, (target + pairs - 1) / pairs);
    const long cap = std::max(1, (max_kv_len + kDecodeChunkMin - 1) / kDecodeChunkMin);
    s = (int)std::min(want, cap);
  }
  // slice length: a multiple of 4 waves x 32 tokens covering max_kv_len in s slices, and at
  // most 4 x 2048 keys (each wavefront keeps its slice's page ids in two registers)
  s = std::max(s, (max_kv_len + chunk_max - 1) / chunk_max);
  int c = (max_kv_len + s - 1) / s;
  c = ((c + 127) / 128) * 128;
  if (c < 128) c = 128;
  *chunk = c;
  return s;
}

bool group_ok(int g) { return g >= 1 && g <= 64 && (256 % g) == 0; }

// Prefill arguments checked and turned into kernel parameters (a4q = the A4Q-style kernel, which
// always runs the 8-wave kernel; otherwise up to 64 query columns per (sequence, KV head) take
// the short-query kernel on NVFP4 and FP8 caches); the workspace pointers are filled by
// launch_prefill_plan.
struct PrefillPlan {
  nvfp4kv::PrefillParams p;
  int nw;
  int ncb;  // > 0: the short-query kernel with this many column blocks
  bool empty;
  size_t workspace_bytes;
  void* out;
  float* lse;
};

// Short-query kernel for `cols` query columns per (sequence, KV head): 1 or 2 = four wavefronts
// on key quarters with that many 16-column blocks each, 4 = four wavefronts of 16 columns sharing
// one conversion of each key; 0 above 64 columns, where the tile kernels take over.
int tail_blocks(long cols) {
  if (cols > 64) return 0;
  return cols > 32 ? 4 : cols > 16 ? 2 : 1;
}

// Key slices per (sequence, KV head) of the short-query kernel, chosen like the decode's: about
// 1024 workgroups of at most 2048 keys for the 64-column kernel (four workgroups per CU), 512
// workgroups of at most 8192 keys (4 quarters x 2048) for the others; at least 512 keys per slice.
int tail_splits(int batch, int ncb, int num_kv_heads, int max_kv_len, int requested, int* chunk) {
  const int kv = std::max(max_kv_len, 1);
  if (ncb == 4) return decode_splits(batch, num_kv_heads, kv, requested, chunk, 1024, 2048);
  return decode_splits(batch, num_kv_heads, kv, requested, chunk, 512, 8192);
}

size_t prefill_workspace(int32_t batch, int32_t total_q, int32_t max_q_len, int32_t max_kv_len,
                         int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t num_splits, bool a4q) {
  if (batch <= 0 || total_q <= 0 || max_q_len <= 0 || num_kv_heads <= 0 || num_qo_heads <= 0 ||
      head_dim != 128 || num_qo_heads % num_kv_heads)
    return 0;
  const int g = num_qo_heads / num_kv_heads;
  if (!group_ok(g)) return 0;
  const int nw = a4q ? 8 : prefill_waves(max_q_len, g);
  const int q_tiles = (max_q_len + (32 * nw / g) - 1) / (32 * nw / g);
  const int s = prefill_splits(batch, q_tiles, num_kv_heads, max_kv_len, nw, num_splits);
  size_t bytes = s > 1 ? (size_t)s * total_q * num_qo_heads * kPartRowBytes : 0;
  // up to 64 columns the NVFP4 and FP8 caches take the short-query kernel, which always writes
  // slice partials; the fp16 (repacked) cache keeps the tile kernel: size for either
  if (const int ncb = a4q ? 0 : tail_blocks((long)max_q_len * g)) {
    int chunk = 0;
    const int st = tail_splits(batch, ncb, num_kv_heads, max_kv_len, num_splits, &chunk);
    bytes = std::max(bytes, (size_t)st * total_q * num_qo_heads * kPartRowBytes);
  }
  return bytes;
}

int plan_prefill(const nvfp4kv_cache_t* cache, const void* q, const int32_t* cu_seqlens_q,
                 const int32_t* kv_lens, const int32_t* block_table, int32_t block_table_stride,
                 int32_t batch, int32_t total_q, int32_t max_q_len, int32_t max_kv_len,
                 int32_t num_qo_heads, float sm_scale, int32_t causal, void* out, int32_t out_dtype,
                 float* lse, int32_t num_splits, bool a4q, PrefillPlan* plan) {
  plan->empty = false;
  if (int e = check_cache(cache)) return e;
  if (batch < 0 || total_q < 0 || max_q_len < 0 || max_kv_len < 0)
    return fail(NVFP4KV_EINVAL, "negative size");
  if (batch == 0 || total_q == 0 || max_q_len == 0) {
    plan->empty = true;
    return ok();
  }
  if (!q || !cu_seqlens_q || !kv_lens || !block_table || !out)
    return fail(NVFP4KV_EINVAL, "q, cu_seqlens_q, kv_lens, block_table or out is NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(NVFP4KV_EINVAL, "q/out must be 16-byte aligned");
  if (num_qo_heads < 1 || num_qo_heads % cache->num_kv_heads)
    return fail(NVFP4KV_EINVAL, "num_qo_heads %d is not a multiple of num_kv_heads %d", num_qo_heads,
                cache->num_kv_heads);
  const int g = num_qo_heads / cache->num_kv_heads;
  if (!group_ok(g)) return fail(NVFP4KV_EUNSUPPORTED, "query group size %d unsupported", g);
  // output rows (token, head) are indexed in 32 bits, with room for the merge grid's rounding
  if ((long)total_q * num_qo_heads > (1L << 30))
    return fail(NVFP4KV_EINVAL, "total_q x num_qo_heads = %ld rows: too large for one launch",
                (long)total_q * num_qo_heads);
  if (block_table_stride < (max_kv_len + 15) / 16)
    return fail(NVFP4KV_EINVAL, "block_table_stride %d too small for max_kv_len %d",
                block_table_stride, max_kv_len);
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale)) return fail(NVFP4KV_EINVAL, "sm_scale must be > 0");
  if (out_dtype != NVFP4KV_OUT_BF16 && out_dtype != NVFP4KV_OUT_F32)
    return fail(NVFP4KV_EINVAL, "out_dtype %d unknown", out_dtype);
  if (num_splits < 0) return fail(NVFP4KV_EINVAL, "num_splits < 0");

  const int nw = a4q ? 8 : prefill_waves(max_q_len, g);
  const int ncb = (a4q || cache->kv_format == NVFP4KV_FORMAT_F16) ? 0 : tail_blocks((long)max_q_len * g);
  const int rows = 32 * nw / g;
  const int q_tiles = ncb ? 1 : (max_q_len + rows - 1) / rows;
  int chunk = 0;
  const int s = ncb ? tail_splits(batch, ncb, cache->num_kv_heads, max_kv_len, num_splits, &chunk)
                    : prefill_splits(batch, q_tiles, cache->num_kv_heads, max_kv_len, nw, num_splits);
  const long items = (long)cache->num_kv_heads * batch * q_tiles * s;
  if (items > (1L << 30)) return fail(NVFP4KV_EINVAL, "problem too large for one launch");

  nvfp4kv::PrefillParams& p = plan->p;
  p = nvfp4kv::PrefillParams{};
  p.format = cache->kv_format;
  p.k_data = cache->k_data;
  p.k_scale = cache->k_scale;
  p.v_data = cache->v_data;
  p.v_scale = cache->v_scale;
  p.q = (const uint16_t*)q;
  p.cu_q = cu_seqlens_q;
  p.kv_lens = kv_lens;
  p.block_table = block_table;
  p.bt_stride = block_table_stride;
  p.batch = batch;
  p.num_kv_heads = cache->num_kv_heads;
  p.num_qo_heads = num_qo_heads;
  p.group = g;
  p.q_tiles = q_tiles;
  p.num_splits = s;
  p.causal = causal ? 1 : 0;
  p.total_q = total_q;
  p.total_items = (int)items;
  p.items_per_xcd = (int)((items + 7) / 8);
  p.score_scale = sm_scale * cache->k_global * 1.4426950408889634f;
  p.out_scale = cache->v_global;
  p.out_f32 = out_dtype == NVFP4KV_OUT_F32;
  p.chunk = chunk;
  plan->nw = nw;
  plan->ncb = ncb;
  plan->out = out;
  plan->lse = lse;
  plan->workspace_bytes = (s > 1 || ncb) ? (size_t)s * total_q * num_qo_heads * kPartRowBytes : 0;
  return NVFP4KV_OK;
}

// Launch the prefill (stock kernels for q_format < 0, else the A4Q-style kernel) and, with key
// splits, the merge of the partials kept in `ws`.
int launch_prefill_plan(PrefillPlan& plan, void* workspace, size_t workspace_bytes, int q_format,
                        hipStream_t st) {
  nvfp4kv::PrefillParams& p = plan.p;
  auto launch = [&]() {
    if (q_format >= 0)
      return nvfp4kv::launch_prefill_a4q(p, q_format & ~NVFP4KV_A4Q_K_ONE_TERM,
                                         (q_format & NVFP4KV_A4Q_K_ONE_TERM) ? 1 : 2, st);
    return plan.ncb ? nvfp4kv::launch_prefill_tail(p, plan.ncb, st) : nvfp4kv::launch_prefill(p, plan.nw, st);
  };
  if (p.num_splits > 1 || plan.ncb) {
    if (!workspace || workspace_bytes < plan.workspace_bytes)
      return fail(NVFP4KV_EWORKSPACE, "prefill needs %zu workspace bytes, got %zu", plan.workspace_bytes,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(NVFP4KV_EINVAL, "workspace must be 16-byte aligned");
    p.part_o = (uint16_t*)workspace;
    p.part_lse = (float*)(p.part_o + (size_t)p.num_splits * p.total_q * p.num_qo_heads * 128);
    p.lse = nullptr;
    p.out = nullptr;
    if (int e = check_launch(launch(), "prefill launch")) return e;
    nvfp4kv::MergeParams m{};
    m.part_o = p.part_o;
    m.part_lse = p.part_lse;
    m.num_splits = p.num_splits;
    m.rows = p.total_q * p.num_qo_heads;
    m.out_scale = p.out_scale;
    m.out = plan.out;
    m.out_f32 = p.out_f32;
    m.lse = plan.lse;
    return check_launch(nvfp4kv::launch_merge(m, st), "merge launch");
  }
  p.lse = plan.lse;
  p.out = plan.out;
  return check_launch(launch(), "prefill launch");
}

// Decode arguments checked and turned into kernel parameters; the workspace pointers are filled
// by launch_decode_plan.
struct DecodePlan {
  nvfp4kv::DecodeParams p;
  nvfp4kv::MergeParams m;
  size_t workspace_bytes;
};

int plan_decode(const nvfp4kv_cache_t* cache, const void* q, const int32_t* kv_lens,
                const int32_t* block_table, int32_t block_table_stride, int32_t batch,
                int32_t max_kv_len, int32_t num_qo_heads, float sm_scale, void* out,
                int32_t out_dtype, float* lse, int32_t num_splits, DecodePlan* plan) {
  if (int e = check_cache(cache)) return e;
  if (int e = check_not_f16(cache, "paged_decode_nvfp4")) return e;
  if (batch < 0 || max_kv_len < 0) return fail(NVFP4KV_EINVAL, "negative size");
  if (batch == 0) return ok();
  if (!q || !kv_lens || !block_table || !out)
    return fail(NVFP4KV_EINVAL, "q, kv_lens, block_table or out is NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(NVFP4KV_EINVAL, "q/out must be 16-byte aligned");
  if (num_qo_heads < 1 || num_qo_heads % cache->num_kv_heads)
    return fail(NVFP4KV_EINVAL, "num_qo_heads %d is not a multiple of num_kv_heads %d", num_qo_heads,
                cache->num_kv_heads);
  const int g = num_qo_heads / cache->num_kv_heads;
  if (g > 16) return fail(NVFP4KV_EUNSUPPORTED, "decode supports query groups of at most 16 (got %d)", g);
  if ((long)batch * num_qo_heads > (1L << 30))
    return fail(NVFP4KV_EINVAL, "batch x num_qo_heads = %ld rows: too large for one launch",
                (long)batch * num_qo_heads);
  if (max_kv_len < 1) return fail(NVFP4KV_EINVAL, "max_kv_len must be >= 1");
  if (block_table_stride < (max_kv_len + 15) / 16)
    return fail(NVFP4KV_EINVAL, "block_table_stride %d too small for max_kv_len %d",
                block_table_stride, max_kv_len);
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale)) return fail(NVFP4KV_EINVAL, "sm_scale must be > 0");
  if (out_dtype != NVFP4KV_OUT_BF16 && out_dtype != NVFP4KV_OUT_F32)
    return fail(NVFP4KV_EINVAL, "out_dtype %d unknown", out_dtype);
  if (num_splits < 0) return fail(NVFP4KV_EINVAL, "num_splits < 0");
  int chunk = 0;
  const int s = decode_splits(batch, cache->num_kv_heads, max_kv_len, num_splits, &chunk);
  const long items = (long)cache->num_kv_heads * batch * s;
  if (items > (1L << 30)) return fail(NVFP4KV_EINVAL, "problem too large for one launch");

  nvfp4kv::DecodeParams& p = plan->p;
  p = nvfp4kv::DecodeParams{};
  p.fp8 = cache->kv_format == NVFP4KV_FORMAT_FP8;
  p.k_data = cache->k_data;
  p.k_scale = cache->k_scale;
  p.v_data = cache->v_data;
  p.v_scale = cache->v_scale;
  p.q = (const uint16_t*)q;
  p.kv_lens = kv_lens;
  p.block_table = block_table;
  p.bt_stride = block_table_stride;
  p.batch = batch;
  p.num_kv_heads = cache->num_kv_heads;
  p.num_qo_heads = num_qo_heads;
  p.group = g;
  p.num_splits = s;
  p.chunk = chunk;
  p.score_scale = sm_scale * cache->k_global * 1.4426950408889634f;
  nvfp4kv::MergeParams& m = plan->m;
  m = nvfp4kv::MergeParams{};
  m.num_splits = s;
  m.rows = batch * num_qo_heads;
  m.out_scale = cache->v_global;
  m.out = out;
  m.out_f32 = out_dtype == NVFP4KV_OUT_F32;
  m.lse = lse;
  plan->workspace_bytes = (size_t)s * batch * num_qo_heads * kPartRowBytes;
  return NVFP4KV_OK;
}

// Launch the split kernel and the merge with the partials in `ws` (fp16 partials, then the
// float32 log-sum-exps).
int launch_decode_plan(DecodePlan& plan, void* ws, hipStream_t st) {
  plan.p.part_o = (uint16_t*)ws;
  plan.p.part_lse = (float*)(plan.p.part_o + (size_t)plan.p.num_splits * plan.p.batch *
                                                 plan.p.num_qo_heads * 128);
  plan.m.part_o = plan.p.part_o;
  plan.m.part_lse = plan.p.part_lse;
  if (int e = check_launch(nvfp4kv::launch_decode(plan.p, st), "decode launch")) return e;
  return check_launch(nvfp4kv::launch_merge(plan.m, st), "merge launch");
}

}  // namespace

extern "C" {

const char* nvfp4kv_last_error(void) { return g_last_error.c_str(); }

int32_t nvfp4kv_version(void) { return 100; }

int nvfp4_kv_append(const nvfp4kv_cache_t* cache, const void* k, const void* v,
                    int64_t k_token_stride, int64_t v_token_stride, int32_t input_dtype,
                    const int64_t* slot_mapping, int32_t num_tokens, void* stream) {
  if (int e = check_cache(cache)) return e;
  if (int e = check_not_f16(cache, "nvfp4_kv_append")) return e;
  if (input_dtype != NVFP4KV_IN_BF16 && input_dtype != NVFP4KV_IN_F16)
    return fail(NVFP4KV_EINVAL, "input_dtype %d unknown", input_dtype);
  if (num_tokens < 0) return fail(NVFP4KV_EINVAL, "num_tokens < 0");
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping) return fail(NVFP4KV_EINVAL, "k, v or slot_mapping is NULL");
  const int64_t row = (int64_t)cache->num_kv_heads * cache->head_dim;
  if (k_token_stride < row || v_token_stride < row)
    return fail(NVFP4KV_EINVAL, "token stride smaller than num_kv_heads * head_dim");
  if ((k_token_stride % 8) || (v_token_stride % 8) || !aligned16(k) || !aligned16(v))
    return fail(NVFP4KV_EINVAL, "k/v must be 16-byte aligned with token strides a multiple of 8");
  nvfp4kv::AppendParams p{};
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.k_stride = k_token_stride;
  p.v_stride = v_token_stride;
  p.slots = slot_mapping;
  p.k_data = cache->k_data;
  p.k_scale = cache->k_scale;
  p.v_data = cache->v_data;
  p.v_scale = cache->v_scale;
  p.k_global = cache->k_global;
  p.v_global = cache->v_global;
  p.num_tokens = num_tokens;
  p.num_kv_heads = cache->num_kv_heads;
  p.fp16_in = input_dtype == NVFP4KV_IN_F16;
  p.fp8 = cache->kv_format == NVFP4KV_FORMAT_FP8;
  return check_launch(nvfp4kv::launch_append(p, (hipStream_t)stream), "append launch");
}

int nvfp4_kv_dequant(const nvfp4kv_cache_t* cache, const int64_t* slot_mapping,
                     int32_t num_tokens, void* k_out, void* v_out, int32_t out_dtype,
                     void* stream) {
  if (int e = check_cache(cache)) return e;
  if (int e = check_not_f16(cache, "nvfp4_kv_dequant")) return e;
  if (out_dtype != NVFP4KV_OUT_BF16 && out_dtype != NVFP4KV_OUT_F32 && out_dtype != NVFP4KV_OUT_F16)
    return fail(NVFP4KV_EINVAL, "out_dtype %d unknown", out_dtype);
  if (num_tokens < 0) return fail(NVFP4KV_EINVAL, "num_tokens < 0");
  if (num_tokens == 0) return ok();
  if (!slot_mapping || !k_out || !v_out) return fail(NVFP4KV_EINVAL, "slot_mapping, k_out or v_out is NULL");
  if (!aligned16(k_out) || !aligned16(v_out)) return fail(NVFP4KV_EINVAL, "k_out / v_out must be 16-byte aligned");
  nvfp4kv::DequantParams p{};
  p.slots = slot_mapping;
  p.k_data = cache->k_data;
  p.k_scale = cache->k_scale;
  p.v_data = cache->v_data;
  p.v_scale = cache->v_scale;
  p.k_global = cache->k_global;
  p.v_global = cache->v_global;
  p.k_out = k_out;
  p.v_out = v_out;
  p.out_dtype = out_dtype;
  p.num_tokens = num_tokens;
  p.num_kv_heads = cache->num_kv_heads;
  p.fp8 = cache->kv_format == NVFP4KV_FORMAT_FP8;
  return check_launch(nvfp4kv::launch_dequant(p, (hipStream_t)stream), "dequant launch");
}

int nvfp4_kv_repack(const nvfp4kv_cache_t* src, const nvfp4kv_cache_t* dst,
                    const int32_t* block_table, int32_t block_table_stride,
                    const int32_t* kv_lens, int32_t batch, int32_t max_kv_len, void* stream) {
  if (int e = check_cache(src)) return e;
  if (int e = check_cache(dst)) return e;
  if (src->kv_format != NVFP4KV_FORMAT_NVFP4)
    return fail(NVFP4KV_EUNSUPPORTED, "repack source must be an NVFP4 cache");
  if (dst->kv_format != NVFP4KV_FORMAT_F16)
    return fail(NVFP4KV_EINVAL, "repack destination must have kv_format NVFP4KV_FORMAT_F16");
  if (dst->num_pages != src->num_pages || dst->num_kv_heads != src->num_kv_heads ||
      dst->k_global != src->k_global || dst->v_global != src->v_global)
    return fail(NVFP4KV_EINVAL, "repack destination must match the source's pages, heads and global scales");
  if (batch < 0 || max_kv_len < 0) return fail(NVFP4KV_EINVAL, "negative size");
  if (batch > 65535) return fail(NVFP4KV_EINVAL, "batch %d above 65535", batch);
  if (batch == 0 || max_kv_len == 0) return ok();
  if (!block_table || !kv_lens) return fail(NVFP4KV_EINVAL, "block_table or kv_lens is NULL");
  const int max_pages = (max_kv_len + 15) / 16;
  if (block_table_stride < max_pages)
    return fail(NVFP4KV_EINVAL, "block_table_stride %d too small for max_kv_len %d",
                block_table_stride, max_kv_len);
  nvfp4kv::RepackParams p{};
  p.k_data = src->k_data;
  p.k_scale = src->k_scale;
  p.v_data = src->v_data;
  p.v_scale = src->v_scale;
  p.k_out = (uint16_t*)dst->k_data;
  p.v_out = (uint16_t*)dst->v_data;
  p.block_table = block_table;
  p.kv_lens = kv_lens;
  p.bt_stride = block_table_stride;
  p.num_kv_heads = src->num_kv_heads;
  return check_launch(nvfp4kv::launch_repack(p, batch, max_pages, (hipStream_t)stream),
                      "repack launch");
}

size_t paged_prefill_nvfp4_workspace_size(int32_t batch, int32_t total_q, int32_t max_q_len,
                                          int32_t max_kv_len, int32_t num_qo_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t num_splits) {
  return prefill_workspace(batch, total_q, max_q_len, max_kv_len, num_qo_heads, num_kv_heads,
                           head_dim, num_splits, false);
}

size_t paged_prefill_nvfp4_a4q_workspace_size(int32_t batch, int32_t total_q, int32_t max_q_len,
                                              int32_t max_kv_len, int32_t num_qo_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t num_splits) {
  return prefill_workspace(batch, total_q, max_q_len, max_kv_len, num_qo_heads, num_kv_heads,
                           head_dim, num_splits, true);
}

int paged_prefill_nvfp4(const nvfp4kv_cache_t* cache, const void* q, const int32_t* cu_seqlens_q,
                        const int32_t* kv_lens, const int32_t* block_table,
                        int32_t block_table_stride, int32_t batch, int32_t total_q,
                        int32_t max_q_len, int32_t max_kv_len, int32_t num_qo_heads,
                        float sm_scale, int32_t causal, void* out, int32_t out_dtype, float* lse,
                        int32_t num_splits, void* workspace, size_t workspace_bytes,
                        void* stream) {
  PrefillPlan plan;
  if (int e = plan_prefill(cache, q, cu_seqlens_q, kv_lens, block_table, block_table_stride, batch,
                           total_q, max_q_len, max_kv_len, num_qo_heads, sm_scale, causal, out,
                           out_dtype, lse, num_splits, false, &plan))
    return e;
  if (plan.empty) return ok();
  return launch_prefill_plan(plan, workspace, workspace_bytes, -1, (hipStream_t)stream);
}

int paged_prefill_nvfp4_a4q(const nvfp4kv_cache_t* cache, const void* q,
                            const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                            const int32_t* block_table, int32_t block_table_stride, int32_t batch,
                            int32_t total_q, int32_t max_q_len, int32_t max_kv_len,
                            int32_t num_qo_heads, float sm_scale, int32_t causal, void* out,
                            int32_t out_dtype, float* lse, int32_t q_format, int32_t num_splits,
                            void* workspace, size_t workspace_bytes, void* stream) {
  const int q_base = q_format & ~NVFP4KV_A4Q_K_ONE_TERM;
  if (q_base != NVFP4KV_A4Q_MXFP8 && q_base != NVFP4KV_A4Q_MXFP4)
    return fail(NVFP4KV_EINVAL, "q_format %d unknown", q_format);
  if (int e = check_cache(cache)) return e;
  if (cache->kv_format != NVFP4KV_FORMAT_NVFP4)
    return fail(NVFP4KV_EUNSUPPORTED, "the A4Q-style prefill reads NVFP4 caches only");
  PrefillPlan plan;
  if (int e = plan_prefill(cache, q, cu_seqlens_q, kv_lens, block_table, block_table_stride, batch,
                           total_q, max_q_len, max_kv_len, num_qo_heads, sm_scale, causal, out,
                           out_dtype, lse, num_splits, true, &plan))
    return e;
  if (plan.empty) return ok();
  return launch_prefill_plan(plan, workspace, workspace_bytes, q_format, (hipStream_t)stream);
}

size_t paged_decode_nvfp4_workspace_size(int32_t batch, int32_t max_kv_len, int32_t num_qo_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t num_splits) {
  if (batch <= 0 || max_kv_len <= 0 || num_kv_heads <= 0 || num_qo_heads <= 0 || head_dim != 128)
    return 0;
  int chunk = 0;
  const int s = decode_splits(batch, num_kv_heads, max_kv_len, num_splits, &chunk);
  return (size_t)s * batch * num_qo_heads * kPartRowBytes;
}

int paged_decode_nvfp4(const nvfp4kv_cache_t* cache, const void* q, const int32_t* kv_lens,
                       const int32_t* block_table, int32_t block_table_stride, int32_t batch,
                       int32_t max_kv_len, int32_t num_qo_heads, float sm_scale, void* out,
                       int32_t out_dtype, float* lse, int32_t num_splits, void* workspace,
                       size_t workspace_bytes, void* stream) {
  DecodePlan plan;
  if (int e = plan_decode(cache, q, kv_lens, block_table, block_table_stride, batch, max_kv_len,
                          num_qo_heads, sm_scale, out, out_dtype, lse, num_splits, &plan))
    return e;
  if (batch == 0) return ok();
  if (!workspace || workspace_bytes < plan.workspace_bytes)
    return fail(NVFP4KV_EWORKSPACE, "decode needs %zu workspace bytes, got %zu", plan.workspace_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(NVFP4KV_EINVAL, "workspace must be 16-byte aligned");
  return launch_decode_plan(plan, workspace, (hipStream_t)stream);
}

int paged_decode_nvfp4_noalloc(const nvfp4kv_cache_t* cache, const void* q,
                               const int32_t* kv_lens, const int32_t* block_table,
                               int32_t block_table_stride, int32_t batch, int32_t max_kv_len,
                               int32_t num_qo_heads, float sm_scale, void* out, int32_t out_dtype,
                               float* lse, int32_t num_splits, void* stream) {
  DecodePlan plan;
  if (int e = plan_decode(cache, q, kv_lens, block_table, block_table_stride, batch, max_kv_len,
                          num_qo_heads, sm_scale, out, out_dtype, lse, num_splits, &plan))
    return e;
  if (batch == 0) return ok();
  if (plan.workspace_bytes > nvfp4kv::kDecodeScratchBytes)
    return fail(NVFP4KV_EWORKSPACE,
                "decode of %d sequences x %d query heads in %d key splits needs %zu scratch bytes; "
                "the allocation-free entry point holds %zu per GPU (call paged_decode_nvfp4 with a "
                "workspace)",
                batch, num_qo_heads, plan.p.num_splits, plan.workspace_bytes,
                nvfp4kv::kDecodeScratchBytes);
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  if (hipError_t e = nvfp4kv::decode_scratch(&scratch, &scratch_bytes); e != hipSuccess)
    return fail(NVFP4KV_EHIP, "static decode scratch lookup: %s", hipGetErrorString(e));
  return launch_decode_plan(plan, scratch, (hipStream_t)stream);
}

}  // extern "C"
