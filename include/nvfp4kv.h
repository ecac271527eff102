/*
 * nvfp4kv.h -- C ABI of the NVFP4 paged KV-cache attention library for AMD MI355X (gfx950).
 *
 * The operations follow the three "fanout.sh" pages on NVFP4 KV caches:
 *   [A] "NVFP4 KV cache A4Q prefill explained"
 *   [B] "NVFP4 KV cache prefill vs decode performance"
 *   [C] "NVFP4 KV cache vs NVFP4 weights"
 *
 * Cache format ([B] "NVFP4 stores 4.5 bits per value before padding"; [C] "NVFP4 KV cache vs
 * NVFP4 weights"): every value is a 4-bit E2M1 code, two codes per byte, and every block of 16
 * consecutive head-dim values of one (token, KV head) carries one E4M3 (OCP "FN") scale byte:
 * 72 bits per 16 values.  A per-tensor scale g (k_global / v_global) maps values into the block
 * range: the writer quantizes x / g and the reader multiplies by g.
 *
 * Element code: sign bit 3 copied from the input, magnitude = round-to-nearest-even of |x/g| / s
 * on the grid {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating at 6.  Block scale: s = E4M3 round-to-
 * nearest-even of fl32(amax / 6), saturating at 448; a zero scale gives magnitude 0.  Byte i of a
 * row holds element 2i in its low nibble and element 2i+1 in its high nibble.
 *
 * Page layout (per layer; X in {K, V}; page_size 16, head_dim 128):
 *   X_data  : uint8 [num_pages][num_kv_heads][16][head_dim / 2]
 *   X_scale : uint8 [num_pages][num_kv_heads][16][head_dim / 16]     (linear, not swizzled)
 * A cache slot is page * 16 + offset.  Pages are reached through a block table
 * (int32 [batch][block_table_stride]: page ids of positions 0, 16, 32, ...).
 *
 * Conventions shared by every entry point:
 *   - All pointers except `cache` itself are device pointers owned by the caller; `cache` is a
 *     host pointer to a descriptor holding device pointers.  `stream` is a hipStream_t (NULL =
 *     the default stream).  Calls are asynchronous on `stream`.
 *   - The library never allocates, frees or synchronizes.  Entry points that need scratch memory
 *     take a caller-provided workspace and report its size through a *_workspace_size call;
 *     paged_decode_nvfp4_noalloc uses a static device array of the library instead.
 *   - Only the cache (append), `out`, `lse` and `workspace` (or that static array) are written.
 *   - Return value: 0 on success, otherwise a negative NVFP4KV_E* code; the message of the last
 *     failure on the calling thread is returned by nvfp4kv_last_error().  Unsupported shapes are
 *     rejected; there is no fallback path.
 *   - Device-side index contents are the caller's contract (checked only where the host knows
 *     them): slots and block-table entries must address allocated pages, kv_len >= q_len for
 *     causal prefill, slots within one append call must be distinct.
 */
#ifndef NVFP4KV_H
#define NVFP4KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4KV_OK 0
#define NVFP4KV_EINVAL (-1)       /* null pointer, bad size or inconsistent arguments */
#define NVFP4KV_EUNSUPPORTED (-2) /* head_dim != 128, page_size != 16, unsupported group size */
#define NVFP4KV_EWORKSPACE (-3)   /* workspace missing or smaller than the *_workspace_size */
#define NVFP4KV_EHIP (-4)         /* the HIP runtime reported an error at launch */

#define NVFP4KV_OUT_BF16 0
#define NVFP4KV_OUT_F32 1
#define NVFP4KV_OUT_F16 2 /* nvfp4_kv_dequant only */

#define NVFP4KV_IN_BF16 0 /* writer input types of nvfp4_kv_append */
#define NVFP4KV_IN_F16 1

#define NVFP4KV_FORMAT_NVFP4 0 /* nvfp4kv_cache_t.kv_format */
#define NVFP4KV_FORMAT_FP8 1
#define NVFP4KV_FORMAT_F16 2   /* fp16 copy written by nvfp4_kv_repack; read by prefill only */

/*
 * FP8 control format (kv_format = NVFP4KV_FORMAT_FP8): the pages quote every NVFP4 result against
 * an FP8 KV cache ([A] "Why NVFP4 KV cache A4Q prefill exists"; [B] "NVFP4 KV cache prefill vs
 * decode performance").  Each value is one E4M3FN byte under the per-tensor scale g: the writer
 * stores E4M3 round-to-nearest-even, saturating at 448, of fl32(x / g) with the sign bit copied,
 * the reader multiplies by g.  X_data is uint8 [num_pages][num_kv_heads][16][head_dim]; there is
 * no block-scale plane (k_scale / v_scale are ignored and may be NULL).  Every entry point below
 * accepts either format through the descriptor.
 */
typedef struct nvfp4kv_cache {
  uint8_t* k_data;  /* [num_pages][num_kv_heads][page_size][head_dim/2]  (FP8: [..][head_dim]) */
  uint8_t* k_scale; /* [num_pages][num_kv_heads][page_size][head_dim/16] (FP8: unused)         */
  uint8_t* v_data;
  uint8_t* v_scale;
  float k_global; /* per-tensor scales g (> 0, finite) */
  float v_global;
  int32_t num_pages;
  int32_t page_size;    /* must be 16 */
  int32_t num_kv_heads; /* >= 1 */
  int32_t head_dim;     /* must be 128; K and V head sizes are equal ([C] "The two controls are
                           independent in vLLM" notes the backend requires it) */
  int32_t kv_format;    /* NVFP4KV_FORMAT_NVFP4 (0), NVFP4KV_FORMAT_FP8 (1) or
                           NVFP4KV_FORMAT_F16 (2, see nvfp4_kv_repack) */
} nvfp4kv_cache_t;

/*
 * Cache append ([B] "NVFP4 stores 4.5 bits per value before padding", "Decode can win on fewer
 * bytes read"; [C] "The cache quantizes values during serving"; [A] "Preserve the capacity and
 * decode case": the writer quantizes BF16 or FP16 input): quantize K and V, choose the block
 * scales, pack, and write each token's row to its slot.
 *   k, v          [num_tokens][num_kv_heads][head_dim] of `input_dtype` (NVFP4KV_IN_BF16 or
 *                 NVFP4KV_IN_F16); heads and dims contiguous, tokens `k_token_stride` /
 *                 `v_token_stride` elements apart (>= num_kv_heads*head_dim, multiples of 8,
 *                 16-byte aligned base pointers).
 *   slot_mapping  int64 [num_tokens]; slot < 0 skips the token; slots must be distinct and
 *                 < num_pages * page_size.
 * Bytes written are bit-identical to the format definition above.  num_tokens == 0 is a no-op.
 */
int nvfp4_kv_append(const nvfp4kv_cache_t* cache, const void* k, const void* v,
                    int64_t k_token_stride, int64_t v_token_stride, int32_t input_dtype,
                    const int64_t* slot_mapping, int32_t num_tokens, void* stream);

/*
 * Standalone dequantization ([A] "Preserve the capacity and decode case": quantization and
 * dequantization utilities over the linear block-scale layout): the cache rows of the given
 * slots as values g * s * e2m1(code).  s * e2m1 is exact in float32; the product with g is one
 * float32 rounding, and the result is rounded to nearest-even in the output type (with g = 1
 * every value is exact in bf16 and fp16).
 *   slot_mapping  int64 [num_tokens]; slot < 0 gives a zero row.
 *   k_out, v_out  [num_tokens][num_kv_heads][head_dim], contiguous, of `out_dtype`
 *                 (NVFP4KV_OUT_BF16, NVFP4KV_OUT_F16 or NVFP4KV_OUT_F32), 16-byte aligned.
 * num_tokens == 0 is a no-op.
 */
int nvfp4_kv_dequant(const nvfp4kv_cache_t* cache, const int64_t* slot_mapping,
                     int32_t num_tokens, void* k_out, void* v_out, int32_t out_dtype,
                     void* stream);

/*
 * Dequantize-ahead repack ([A] "Compare A4Q with dequantize-ahead repacking": the NVFP4 data is
 * widened to 16-bit floats a single time, ahead of the matrix products that reuse it): convert
 * every page that holds keys 0 .. kv_lens[b]-1 of each sequence b into an fp16 copy, for a
 * prefill over that copy (paged_prefill_nvfp4 with `dst`).
 *   src           NVFP4 cache (kv_format NVFP4KV_FORMAT_NVFP4).
 *   dst           fp16 copy (kv_format NVFP4KV_FORMAT_F16): k_data / v_data are fp16
 *                 [num_pages][num_kv_heads][16][head_dim] (256-byte rows, 16-byte aligned),
 *                 scale planes unused (may be NULL); same num_pages, num_kv_heads and global
 *                 scales as `src`.  A page keeps its id: the same block table addresses both.
 *                 Values are s * e2m1(code), exact in fp16; g is not applied (the prefill applies
 *                 it, as over the packed cache).  Pages no sequence reaches are not written.
 *   block_table   int32 [batch][block_table_stride] (>= ceil(max_kv_len / 16)); kv_lens int32
 *                 [batch], each <= max_kv_len.
 * batch == 0 or max_kv_len == 0 is a no-op; batch must be <= 65535.  The fp16 format is read by
 * paged_prefill_nvfp4 only; the other entry points reject it (NVFP4KV_EUNSUPPORTED).
 */
int nvfp4_kv_repack(const nvfp4kv_cache_t* src, const nvfp4kv_cache_t* dst,
                    const int32_t* block_table, int32_t block_table_stride,
                    const int32_t* kv_lens, int32_t batch, int32_t max_kv_len, void* stream);

/*
 * Causal paged prefill over the NVFP4 cache with bf16 queries ([A] "Why NVFP4 KV cache A4Q
 * prefill exists": K and V are unpacked, converted and scaled before BF16 QK and PV; [B] "NVFP4
 * KV cache prefill vs decode performance").  Append the chunk's K/V first: every key is read
 * from the cache.
 *   q             bf16 [total_q][num_qo_heads][head_dim], sequence b owns rows
 *                 cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1.
 *   cu_seqlens_q  int32 [batch+1], kv_lens int32 [batch]; with causal != 0 query row i of a
 *                 sequence sees keys j <= kv_len - q_len + i (queries at the tail; requires
 *                 kv_len >= q_len); with causal == 0 every row sees all kv_len keys.
 *   block_table   int32 [batch][block_table_stride].
 *   max_q_len, max_kv_len  host-side upper bounds of the device lengths (size the grid).
 *   query head h reads KV head h / (num_qo_heads / num_kv_heads); the group size must divide
 *   256 and be <= 64.
 *   out           [total_q][num_qo_heads][head_dim], bf16 (out_dtype 0) or float32 (1).
 *   lse           optional float32 [total_q][num_qo_heads]: natural-log sum of exp of the scaled
 *                 scores (NULL to skip).  A row that sees no key gets out = 0, lse = -inf.
 *   num_splits    0 = choose automatically; n > 0 splits each row's key range into n parts
 *                 whose partial results are merged (needs workspace).
 *   workspace     device scratch of at least paged_prefill_nvfp4_workspace_size(...) bytes
 *                 (may be NULL when that size is 0).
 * total_q * num_qo_heads must not exceed 2^30 (NVFP4KV_EINVAL otherwise).
 */
size_t paged_prefill_nvfp4_workspace_size(int32_t batch, int32_t total_q, int32_t max_q_len,
                                          int32_t max_kv_len, int32_t num_qo_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t num_splits);
int paged_prefill_nvfp4(const nvfp4kv_cache_t* cache, const void* q, const int32_t* cu_seqlens_q,
                        const int32_t* kv_lens, const int32_t* block_table,
                        int32_t block_table_stride, int32_t batch, int32_t total_q,
                        int32_t max_q_len, int32_t max_kv_len, int32_t num_qo_heads,
                        float sm_scale, int32_t causal, void* out, int32_t out_dtype, float* lse,
                        int32_t num_splits, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * A4Q-style prefill ([A] "Quantize Q instead of expanding K": the query is quantized inside the
 * kernel and QK runs on a low-precision matrix product; "Make query accuracy a release gate": the
 * added error is measured against the oracle).  Same arguments, semantics and workspace rules as
 * paged_prefill_nvfp4 (its own *_workspace_size), plus:
 *   q_format  NVFP4KV_A4Q_MXFP8: each query row's 128 values in blocks of 32 consecutive values,
 *             scale 2^(floor(log2 amax) - 8) (E8M0), elements E4M3 nearest-even saturating at
 *             448; NVFP4KV_A4Q_MXFP4: the same with E2M1 elements and 2^(floor(log2 amax) - 2),
 *             saturating at 6.
 * K is fed to gfx950's block-scaled MFMA as two E4M3 terms per value under one power-of-two scale
 * per 32 values (exact when a key's two 16-value block scales in each 32-value block are within
 * 2^8 of each other); softmax and PV are those of paged_prefill_nvfp4.  NVFP4 caches only
 * (other formats: NVFP4KV_EUNSUPPORTED).  Every query-tile width runs the 8-wave kernel.
 * OR-ing NVFP4KV_A4Q_K_ONE_TERM into q_format keeps the first term alone: one MFMA instead of
 * two per 64 head-dim values, K rounded to nearest-even E4M3 (4 significant bits) under the
 * block's power-of-two scale, relative error at most 2^-4 per value where the value is at least
 * 2^-6 times that scale.  This is an extra approximation: the pages' A4Q product takes K
 * exactly.  Any other q_format: NVFP4KV_EINVAL.
 */
#define NVFP4KV_A4Q_MXFP8 0
#define NVFP4KV_A4Q_MXFP4 1
#define NVFP4KV_A4Q_K_ONE_TERM 0x10
size_t paged_prefill_nvfp4_a4q_workspace_size(int32_t batch, int32_t total_q, int32_t max_q_len,
                                              int32_t max_kv_len, int32_t num_qo_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t num_splits);
int paged_prefill_nvfp4_a4q(const nvfp4kv_cache_t* cache, const void* q,
                            const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                            const int32_t* block_table, int32_t block_table_stride, int32_t batch,
                            int32_t total_q, int32_t max_q_len, int32_t max_kv_len,
                            int32_t num_qo_heads, float sm_scale, int32_t causal, void* out,
                            int32_t out_dtype, float* lse, int32_t q_format, int32_t num_splits,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Single-token paged decode ([B] "Decode can win on fewer bytes read": each step scans the whole
 * cache of a sequence for its one new query, after that token's K/V has been written).  Split-KV: each (sequence, KV head, split)
 * computes a partial softmax over its slice of the cache; a merge combines the partials.
 *   q        bf16 [batch][num_qo_heads][head_dim]; query b sees all kv_lens[b] keys.
 *   out      [batch][num_qo_heads][head_dim] bf16 or float32; lse as for prefill.
 *   num_splits  0 = automatic, else the number of key-range splits per (sequence, KV head).
 * The query group size must be <= 16 and batch * num_qo_heads <= 2^30.
 */
size_t paged_decode_nvfp4_workspace_size(int32_t batch, int32_t max_kv_len, int32_t num_qo_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t num_splits);
int paged_decode_nvfp4(const nvfp4kv_cache_t* cache, const void* q, const int32_t* kv_lens,
                       const int32_t* block_table, int32_t block_table_stride, int32_t batch,
                       int32_t max_kv_len, int32_t num_qo_heads, float sm_scale, void* out,
                       int32_t out_dtype, float* lse, int32_t num_splits, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Allocation-free decode, for callers that cannot allocate or hand over scratch memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation.  The same
 * computation, kernels and results as paged_decode_nvfp4 (same arguments without the workspace);
 * the split partials go to a static device array of NVFP4KV_DECODE_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends.  Nothing is allocated or freed:
 * the array's device address is looked up on the first call on each device.
 *   - A call whose partials need more than NVFP4KV_DECODE_SCRATCH_BYTES (split count x batch x
 *     num_qo_heads x 260 bytes, as paged_decode_nvfp4_workspace_size reports) is rejected with
 *     NVFP4KV_EWORKSPACE before any device work.
 *   - Every call on a GPU uses that GPU's one array, which keeps the last call's contents
 *     (nothing in it has to start at zero).  Calls that overlap on one GPU (different streams
 *     or host threads, or in flight at the same time) race on the array: order them, e.g. on one
 *     stream.
 */
#define NVFP4KV_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
int paged_decode_nvfp4_noalloc(const nvfp4kv_cache_t* cache, const void* q,
                               const int32_t* kv_lens, const int32_t* block_table,
                               int32_t block_table_stride, int32_t batch, int32_t max_kv_len,
                               int32_t num_qo_heads, float sm_scale, void* out, int32_t out_dtype,
                               float* lse, int32_t num_splits, void* stream);

/* Message describing the last non-zero return on the calling thread ("" if none). */
const char* nvfp4kv_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t nvfp4kv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4KV_H */
