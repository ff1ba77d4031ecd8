/*
 * fp8ts.h - C ABI of the FP8-e4m3 top-k sparse attention library (libfp8ts.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * Three operations, in the order a sparse-attention layer calls them:
 *
 *   fp8_quantize     per-tensor e4m3 quantization of the queries and the index
 *                    query (stored value = x / scale, None = unit scale);
 *                    fp8_quantize_pair does both tensors in one launch.
 *   indexer_topk     lightning indexer: scores every 128-token KV block by the
 *                    maximum index logit over its visible tokens and writes the
 *                    top-k block ids of every (index head, query) in strictly
 *                    ascending order, -1 padded.
 *   sparse_attn_fwd  attention over only the selected KV tokens (token mode,
 *                    MLA-style) or blocks (block mode, paged GQA), with online
 *                    softmax, optional attention sink, bf16 output and fp32
 *                    max_logits / lse.
 *
 * and two producers upstream of them:
 *
 *   fp8_rope_quantize  rotary position embedding fused with the quantization
 *                      of Q or K (no-rope part ++ rotated rope part per row).
 *   fp8_cache_store    quantize new K / V / index-K rows (or MLA latent + rope
 *                      rows) and scatter them into the paged e4m3 caches.
 *   fp8_qknorm_rope_quantize  per-head RMS norm + RoPE + quantization of the
 *                      index query / index key, writing fp8 rows and/or
 *                      storing them into the paged index-K cache.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named as device pointers must point to device memory of the
 *   current HIP device; "host" pointers are read during the call only.
 * - Every fp8 tensor is OCP e4m3fn, passed as raw bytes (uint8_t).  No other
 *   fp8 format is accepted: the pages forbid e5m2 on this path (sglang PR 30971
 *   digest, implementation step 1: e5m2 must never reach the fp8 attention
 *   kernel).
 * - Optional per-tensor scales are host pointers to one float: NULL means
 *   "None", i.e. unit scale with the multiply skipped (sglang PR 30971 digest,
 *   implementation steps 3 and 4).  A given scale must be finite and > 0.
 * - Ownership: the caller owns every input, output and workspace buffer.  The
 *   library allocates nothing per call, keeps no output cache and never
 *   writes its inputs (sglang PR 25751 digest, review thread on output
 *   aliasing).  Outputs are written in full, so they may be uninitialised
 *   ("empty", sglang PR 25460 digest, implementation step 4).  Outputs must
 *   not alias inputs.
 * - Streams: all work is enqueued asynchronously on `stream` (0 = the null
 *   stream).  No call synchronises, copies between host and device or
 *   allocates, so calls may be captured into a HIP graph.
 * - Errors: arguments are validated on the host before anything is launched.
 *   On failure the call returns a non-zero status, launches nothing, and
 *   fp8ts_last_error() describes the failure (thread-local string, valid until
 *   the next failing call on the same thread).  HIP launch failures return
 *   FP8TS_EHIP.  Device-side values (index lists, block tables, sequence
 *   lengths) cannot be validated without a copy: out-of-range entries are
 *   ignored by the kernels (treated as absent) rather than dereferenced.
 */
#ifndef FP8TS_H
#define FP8TS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fp8ts_status {
  FP8TS_OK = 0,
  FP8TS_EINVAL = 1,      /* malformed argument (null pointer, bad size, bad scale, ...) */
  FP8TS_EUNSUPPORTED = 2,/* well-formed but outside what the kernels implement */
  FP8TS_EHIP = 3         /* the HIP runtime reported an error */
};

enum fp8ts_dtype { FP8TS_BF16 = 0, FP8TS_FP16 = 1 };

enum fp8ts_attn_mode {
  FP8TS_TOKEN_MODE = 0, /* per-query token indices into a flat KV array (MLA) */
  FP8TS_BLOCK_MODE = 1  /* per-(index head, query) block ids into paged K/V (GQA) */
};

/* Message describing the last failed call on this thread ("" if none). */
const char *fp8ts_last_error(void);

/* ABI version of this header (incremented on any signature change). */
int fp8ts_abi_version(void);

/*
 * fp8_quantize - y = e4m3(fl32(fl32(x) * fl32(1 / scale))), per tensor.
 *
 * Follows the quantize kernel of the sglang PR 25460 digest (code excerpt of
 * _fp8_quantize_kernel: widen to fp32, multiply by one reciprocal scale, cast)
 * with the storage convention of the sglang PR 30971 digest (_quant_q_fp8:
 * the fp8 tensor holds value / scale; None skips the operation).
 * Rounding is to nearest, ties to even; magnitudes above 448 (and +-inf)
 * saturate to +-448; NaN maps to 0x7F with its sign bit.
 *
 * x               device, `rows` rows of `cols` elements of dtype `x_dtype`
 *                 (FP8TS_BF16 or FP8TS_FP16); element (r, c) at x[r * x_row_stride + c]
 *                 (the 2-D view of any tensor whose leading dims flatten).
 * out             device, e4m3 bytes; element (r, c) at out[r * out_row_stride + c].
 * x_row_stride    in elements, >= cols.   out_row_stride in bytes, >= cols.
 * scale           host, NULL (None) or one finite float > 0.  The reciprocal
 *                 is computed once on the host in fp32: 1.0f / *scale.
 * rows == 0 or cols == 0 is a no-op.
 * Errors: FP8TS_EINVAL for null pointers, negative sizes, short strides, an
 * unknown dtype, a bad scale, or overlapping x / out.
 */
int fp8_quantize(const void *x, int32_t x_dtype, int64_t rows, int64_t cols,
                 int64_t x_row_stride, uint8_t *out, int64_t out_row_stride,
                 const float *scale, hipStream_t stream);

/*
 * fp8_quantize_pair - fp8_quantize of two contiguous tensors of one dtype,
 * each with its own scale, in one launch: the queries and the index query of
 * a sparse-attention layer, which the layer quantizes per tensor with their
 * own scales (sglang PR 30971 digest, implementation step 3) right before the
 * indexer and the attention.  Codes are those of two fp8_quantize calls.
 *
 * x0, x1          device, n0 / n1 elements of dtype x_dtype, contiguous,
 *                 16-byte aligned.
 * out0, out1      device e4m3, n0 / n1 bytes, contiguous, 8-byte aligned.
 * scale0, scale1  host, NULL (None) or one finite float > 0 each.
 * n0, n1          multiples of 8 (FP8TS_EUNSUPPORTED otherwise, as is a
 *                 misaligned pointer: use fp8_quantize); either may be 0.
 * Errors: FP8TS_EINVAL for null pointers, negative sizes, an unknown dtype, a
 * bad scale, or any output overlapping an input or the other output.
 */
int fp8_quantize_pair(const void *x0, uint8_t *out0, int64_t n0, const float *scale0, const void *x1,
                      uint8_t *out1, int64_t n1, const float *scale1, int32_t x_dtype, hipStream_t stream);

/*
 * fp8_rope_quantize - rotary position embedding fused with e4m3 quantization,
 * writing each head's no-rope part and rotated rope part as one fp8 row:
 *   out[n, h] = e4m3(x_nope[n, h] * inv) ++ e4m3(rope(x_pe[n, h], positions[n]) * inv)
 * with inv = fl32(1 / scale) (None: no multiply).
 *
 * This is the fused producer of the MLA prefill hook: rope and quantize Q or
 * K and emit contiguous fp8 rows the attention kernel reads directly, with a
 * rope part shared by all heads broadcast to every head (sglang PR 25460
 * digest, implementation step 2 and the _fused_rope_fp8_quantize excerpt).
 * RoPE is RoFormer's rotary embedding: the rope dims form pairs, pair i at
 * position p turns by the angle whose cosine and sine are
 * cos_sin_cache[p][i] and cos_sin_cache[p][rope_dim/2 + i]:
 *   (a, b) -> (fl32(fl32(a cos) - fl32(b sin)), fl32(fl32(b cos) + fl32(a sin)))
 * (every product rounded on its own; no fused multiply-add).  is_neox != 0
 * pairs dim i with dim i + rope_dim/2 (rotate-half); 0 pairs dims 2i, 2i+1.
 * Rounding, saturation and NaN as in fp8_quantize.
 *
 * x_nope          device or NULL (exactly when nope_dim == 0), dtype x_dtype;
 *                 (n, h, c) at x_nope[n * nope_token_stride + h * nope_head_stride + c].
 * x_pe            device, dtype x_dtype; (n, h, c) at
 *                 x_pe[n * pe_token_stride + h * pe_head_stride + c];
 *                 pe_head_stride 0 shares one rope head across all heads.
 * cos_sin_cache   device fp32 [max_position, rope_dim] (cosines, then sines).
 * positions       device int64 [num_tokens].  A position outside
 *                 [0, max_position) writes 0x7F (NaN) over that token's rope
 *                 bytes; its no-rope bytes are written as usual.
 * out             device e4m3; row (n, h) of nope_dim + rope_dim bytes at
 *                 out + n * out_token_stride + h * out_head_stride.
 * Strides are in elements of the source (bytes for out).
 * nope_dim a multiple of 8, rope_dim of 16; sources and cos_sin_cache 16-byte
 * aligned, out 8-byte aligned, every stride a multiple of 8
 * (FP8TS_EUNSUPPORTED otherwise).  num_tokens == 0 is a no-op.
 * Errors: FP8TS_EINVAL for null pointers, bad sizes, an odd rope_dim, a bad
 * scale, overlapping output rows, or an output overlapping an input.
 */
int fp8_rope_quantize(const void *x_nope, const void *x_pe, int32_t x_dtype, int64_t num_tokens,
                      int32_t num_heads, int32_t nope_dim, int32_t rope_dim,
                      int64_t nope_token_stride, int64_t nope_head_stride, int64_t pe_token_stride,
                      int64_t pe_head_stride, const float *cos_sin_cache, int64_t max_position,
                      const int64_t *positions, int32_t is_neox, uint8_t *out,
                      int64_t out_token_stride, int64_t out_head_stride, const float *scale,
                      hipStream_t stream);

/*
 * fp8_cache_store - quantize new key / value / index-key rows and write them
 * into a paged e4m3 cache: cache row = e4m3(fl32(fl32(x) * fl32(1 / scale))).
 *
 * The pools keep fp8 values as value / scale with None meaning unit scale and
 * no division (sglang PR 30971 digest, implementation step 4: the K/V,
 * index-K and fused setters default their scale to None).  A second source
 * fills the rest of each row, which is how the MLA prefill hook packs the
 * latent part and the rope part of a token into one fp8 cache row (sglang PR
 * 25460 digest, implementation step 2).  Rounding, saturation and NaN as in
 * fp8_quantize.
 *
 * Token n goes to slot s = slot_mapping[n]: page s / page_size, in-page
 * offset s % page_size.  Element c of head h lands at
 *   cache[((page * num_heads + h) * page_size + offset) * (dim + dim2) + c]
 * (x for c < dim, x2 for dim <= c < dim + dim2).  This covers the block-mode
 * K/V caches [pages, Hkv, page_size, 128], the single-head index-K cache
 * (num_heads 1) and the flat MLA KV array [S, 576] (num_heads 1,
 * page_size 1, x = latent 512, x2 = rope 64).
 *
 * x               device, dtype x_dtype; element (n, h, c) at
 *                 x[n * x_token_stride + h * x_head_stride + c] (strides in
 *                 elements; e.g. the K part of a fused QKV projection).
 * x2              device or NULL; same dtype; (n, h, c) at
 *                 x2[n * x2_token_stride + h * x2_head_stride + c].  NULL
 *                 exactly when dim2 == 0.
 * slot_mapping    device int64 [num_tokens].  Negative slots (padding) and
 *                 slots >= num_pages * page_size are skipped.  A slot may
 *                 appear at most once per call (otherwise which token's row
 *                 survives is unspecified).
 * cache           device e4m3 [num_pages, num_heads, page_size, dim + dim2];
 *                 bytes of slots not named are left unchanged (the cache is
 *                 both read-modify-written state and the output).
 * scale           host, NULL (None) or one finite float > 0.
 * num_tokens == 0 is a no-op.
 * Errors: FP8TS_EINVAL for null pointers, bad sizes, an unknown dtype, a bad
 * scale, source strides that overlap rows, or a cache overlapping a source.
 */
int fp8_cache_store(const void *x, const void *x2, int32_t x_dtype, int64_t num_tokens,
                    int32_t num_heads, int32_t dim, int32_t dim2, int64_t x_token_stride,
                    int64_t x_head_stride, int64_t x2_token_stride, int64_t x2_head_stride,
                    const int64_t *slot_mapping, uint8_t *cache, int64_t num_pages,
                    int32_t page_size, const float *scale, hipStream_t stream);

/*
 * fp8_qknorm_rope_quantize - per-head RMS normalisation, RoPE and e4m3
 * quantization of index queries or index keys, with an optional store of the
 * codes into a paged cache:
 *   y    = x * r * w,  r = 1 / sqrt(mean(x^2) + eps)   (over each head's head_dim values)
 *   code = e4m3(nope(y) * inv) ++ e4m3(rope(last rope_dim dims of y, positions[n]) * inv)
 * with inv = fl32(1 / scale) (None: no multiply).
 *
 * This is the fused qk-norm + RoPE + index-insert producer of the MiniMax
 * sparse layer, which emits the index query directly in fp8 when the index
 * cache is e4m3 (vLLM PR 45892 digest, implementation steps 3 and 5).  The
 * pages give no formula for the norm; the one above is RMS normalisation with
 * a learned per-dim weight.  Precision: the squares are summed in fp64 (each
 * square of a bf16 / fp16 value is exact there, so the sum is independent of
 * order unless a row's magnitudes span more than fp64 holds); then
 * r = fl32(1 / sqrt(fl64(sum / head_dim) + eps)) in fp64, y = fl32(fl32(x r) w).
 * RoPE, rounding, saturation and NaN as in fp8_rope_quantize (the no-rope
 * dims come first in the row, the rotated dims last).
 *
 * x               device, dtype x_dtype; (n, h, c) at x[n * x_token_stride + h * x_head_stride + c].
 * norm_weight     device fp32 [head_dim].   eps: host float >= 0.
 * cos_sin_cache, positions, is_neox: as in fp8_rope_quantize (rope_dim wide);
 *                 an invalid position writes 0x7F over the rope bytes.
 * out             device e4m3 or NULL; row (n, h) of head_dim bytes at
 *                 out + n * out_token_stride + h * out_head_stride.
 * slot_mapping    device int64 [num_tokens] or NULL; with it, row (n, h) is
 *                 also stored into cache [num_pages, num_heads, page_size,
 *                 head_dim] at page s / page_size, offset s % page_size,
 *                 s = slot_mapping[n]; negative or out-of-range slots store
 *                 nothing (as fp8_cache_store).  At least one of out and
 *                 slot_mapping must be given.
 * head_dim a multiple of 8 and at most 512; rope_dim a multiple of 16 (0 for
 * no rotation) and at most head_dim; x, norm_weight and cos_sin_cache 16-byte
 * aligned, out and cache 8-byte aligned, every stride a multiple of 8
 * (FP8TS_EUNSUPPORTED otherwise).  num_tokens == 0 is a no-op.
 * Errors: FP8TS_EINVAL for null pointers, bad sizes, a negative or non-finite
 * eps, a bad scale, overlapping output rows, or an output overlapping an input.
 */
int fp8_qknorm_rope_quantize(const void *x, int32_t x_dtype, int64_t num_tokens, int32_t num_heads,
                             int32_t head_dim, int32_t rope_dim, int64_t x_token_stride,
                             int64_t x_head_stride, const float *norm_weight, float eps,
                             const float *cos_sin_cache, int64_t max_position,
                             const int64_t *positions, int32_t is_neox, uint8_t *out,
                             int64_t out_token_stride, int64_t out_head_stride,
                             const int64_t *slot_mapping, uint8_t *cache, int64_t num_pages,
                             int32_t page_size, const float *scale, hipStream_t stream);

/*
 * indexer_topk - ascending top-k block ids of the lightning indexer.
 *
 * Defined by the vLLM PR 45892 digest (implementation steps 1-4 and the
 * _fmha_indexer_topk excerpt: one maximum score per 128-token tile, tile id =
 * block id, a [num_index_heads, tokens, topk] shared output buffer) and the
 * sglang PR 30971 digest (implementation step 2 and review thread 2: strictly
 * ascending ids, -1 padding when a row has no more than k blocks).
 *
 * For query i of sequence b (flattened token t = cu_seqlens_q[b] + i) the
 * position is p = seq_lens[b] - q_len_b + i; key j is visible iff j <= p.
 * With nb = p / page_size + 1 visible blocks:
 *   nb <= topk : ids = 0, 1, ..., nb-1, then -1 ...
 *   nb >  topk : the topk blocks with the largest
 *                S[h,t,blk] = max_{j in blk, j <= p} sm_scale*idx_q_scale*idx_k_scale*<iq[t,h], ik[j]>
 *                (ties to the lower id), written in ascending id order.
 *
 * idx_q           device e4m3 [total_q, num_heads, head_dim] contiguous.
 * idx_k           device e4m3 [num_pages, page_size, head_dim] contiguous (single head).
 * block_table     device int32 [batch, max_blocks]: logical block -> physical page.
 * cu_seqlens_q    device int32 [batch + 1], cu_seqlens_q[batch] == total_q.
 * seq_lens        device int32 [batch], keys of each sequence including this step.
 * max_q_len       host upper bound of the per-sequence query counts.
 * num_heads       1, 2, 4, 8 or 16.   head_dim must be 128.   page_size must be 128.
 * topk            1..64.
 * out_ids         device int32 [num_heads, total_q, topk].
 * workspace       device scratch of at least indexer_topk_workspace_size(...) bytes
 *                 (block scores), 256-byte aligned.
 * Errors: FP8TS_EINVAL for malformed arguments; FP8TS_EUNSUPPORTED for a head
 * dim / page size / head count / topk / max_blocks outside the ranges above.
 */
size_t indexer_topk_workspace_size(int32_t total_q, int32_t num_heads, int32_t max_blocks);

int indexer_topk(const uint8_t *idx_q, const uint8_t *idx_k, int64_t num_pages,
                 const int32_t *block_table, int32_t max_blocks,
                 const int32_t *cu_seqlens_q, const int32_t *seq_lens, int32_t batch,
                 int32_t total_q, int32_t max_q_len, int32_t num_heads, int32_t head_dim,
                 int32_t page_size, float sm_scale, const float *idx_q_scale,
                 const float *idx_k_scale, int32_t topk, int32_t *out_ids,
                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sparse_attn_fwd - attention over the selected keys only.
 *
 * Semantics (sglang PR 25751 digest, code excerpt of sparse_mla_q8kv8_prefill_fwd,
 * and sglang PR 30971 digest, summary and implementation step 3):
 *   s = sm_scale * q_scale                  (q_scale folded into sm_scale)
 *   z_j = s * k_scale * <q, k_j>            for every selected key j
 *   z_sink = s * attn_sink[h]               (k_scale never touches the sink)
 *   M = max(max_j z_j, z_sink);  L = sum_j e^(z_j - M) + e^(z_sink - M)
 *   out = v_scale * sum_j e^(z_j - M) v_j / L           (bf16; 0 when L == 0)
 *   lse = M + ln L (natural log, includes the sink; -inf when L == 0)
 *   max_logits = max_j z_j (keys only; -inf when no key is selected)
 *
 * q               device e4m3 [total_q, num_q_heads, head_dim_qk] contiguous.
 * mode            FP8TS_TOKEN_MODE:
 *                   k = KV rows [num_kv, head_dim_qk] (one KV head), v = NULL
 *                   (V = first head_dim_v columns of the same rows, MLA) or
 *                   [num_kv, head_dim_v]; indices int32 [total_q, topk] token
 *                   ids (entries outside [0, num_kv) are absent; list order is
 *                   irrelevant); topk_length NULL or int32 [total_q] (only the
 *                   first topk_length[t] entries count).  The list is the
 *                   mask; no causality.  head_dim_qk 576 and head_dim_v 512.
 *                 FP8TS_BLOCK_MODE:
 *                   k, v = paged caches [num_kv pages, num_kv_heads, page_size,
 *                   head_dim]; indices = int32 [num_idx_heads, total_q, topk]
 *                   block ids as written by indexer_topk (set semantics; -1
 *                   and ids outside [0, max_blocks) are absent); query head h
 *                   reads index head h / (Hq / Hidx) and KV head h / (Hq / Hkv);
 *                   key j of a selected block counts iff j <= p (causal; p as
 *                   in indexer_topk).  head_dim_qk = head_dim_v = 128,
 *                   page_size 128.
 * block_table, cu_seqlens_q, seq_lens, batch, max_q_len: as in indexer_topk
 *                 (block mode only; may be NULL / 0 in token mode).
 * attn_sink       device float [num_q_heads] or NULL.
 * out             device bf16 [total_q, num_q_heads, head_dim_v].
 * max_logits, lse device float [total_q, num_q_heads].
 * workspace       device scratch of sparse_attn_workspace_size(...) bytes
 *                 (may be 0 bytes / NULL when that size is 0): partial
 *                 results of split key lists (decode, small token-mode
 *                 workloads) and, for block-mode prefill over sequences of
 *                 several query tiles, one bf16 V^T tile (32 KB) per
 *                 block-table slot and KV head, converted once per call.
 * Errors: FP8TS_EINVAL for malformed arguments; FP8TS_EUNSUPPORTED for head
 * dims, page sizes or head counts outside the ranges above (a token-mode
 * head_dim_v other than 512 in particular, as the pages' MLA kernel rejects).
 */
size_t sparse_attn_workspace_size(int32_t mode, int32_t batch, int32_t total_q,
                                  int32_t max_q_len, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t num_idx_heads,
                                  int32_t head_dim_v, int32_t topk, int32_t max_blocks);

int sparse_attn_fwd(int32_t mode, const uint8_t *q, const uint8_t *k, const uint8_t *v,
                    int64_t num_kv, const int32_t *indices, int32_t topk,
                    const int32_t *topk_length, const int32_t *block_table,
                    int32_t max_blocks, const int32_t *cu_seqlens_q,
                    const int32_t *seq_lens, int32_t batch, int32_t total_q,
                    int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t num_idx_heads, int32_t head_dim_qk, int32_t head_dim_v,
                    int32_t page_size, float sm_scale, const float *q_scale,
                    const float *k_scale, const float *v_scale, const float *attn_sink,
                    uint16_t *out, float *max_logits, float *lse, void *workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * sparse_attn_fwd_noalloc - sparse_attn_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  Arguments, semantics, outputs and errors
 * are those of sparse_attn_fwd without the workspace: the split partials and
 * pre-converted V^T tiles go to a scratch array the library holds in device
 * memory, one per device, from the first call on that device until the
 * process ends.  The call allocates nothing (no hipMalloc / hipFree, no
 * allocating library routine); its only set-up, on the first call on a
 * device, looks up that device's scratch address.
 *
 * Limit: calls whose sparse_attn_workspace_size(...) exceeds
 * sparse_attn_noalloc_scratch_bytes() (32 MiB) return FP8TS_EUNSUPPORTED and
 * launch nothing.  Nothing in the scratch has to start at zero (every byte a
 * call reads was written earlier in the same call).
 * Concurrency: every call on one device uses that device's one scratch array,
 * so calls that overlap in time on one device (different streams, or host
 * threads without ordering) race; calls ordered on one stream do not.
 * Errors: as sparse_attn_fwd, plus FP8TS_EHIP when the scratch address cannot
 * be obtained on the current device.
 */
int sparse_attn_fwd_noalloc(int32_t mode, const uint8_t *q, const uint8_t *k, const uint8_t *v,
                            int64_t num_kv, const int32_t *indices, int32_t topk,
                            const int32_t *topk_length, const int32_t *block_table,
                            int32_t max_blocks, const int32_t *cu_seqlens_q,
                            const int32_t *seq_lens, int32_t batch, int32_t total_q,
                            int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t num_idx_heads, int32_t head_dim_qk, int32_t head_dim_v,
                            int32_t page_size, float sm_scale, const float *q_scale,
                            const float *k_scale, const float *v_scale, const float *attn_sink,
                            uint16_t *out, float *max_logits, float *lse, hipStream_t stream);

/* Bytes of the per-device scratch behind sparse_attn_fwd_noalloc. */
size_t sparse_attn_noalloc_scratch_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8TS_H */
