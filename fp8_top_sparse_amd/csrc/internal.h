// Host-side internals shared by the C-ABI entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fp8ts.h"

namespace fp8ts {

// Records a formatted message as the thread's last error and returns `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// Returns FP8TS_OK, or FP8TS_EHIP with a message if the last launch failed.
int check_launch(const char *what);

// ---- quantize
// n0 and n1 multiples of 8; contiguous, x 16-byte and out 8-byte aligned
int launch_quantize_pair(const void *x0, uint8_t *out0, int64_t n0, bool has0, float inv0, const void *x1,
                         uint8_t *out1, int64_t n1, bool has1, float inv1, int dtype, hipStream_t stream);
int launch_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int64_t x_stride,
                    uint8_t *out, int64_t out_stride, bool has_scale, float scale_inv,
                    hipStream_t stream);

// ---- paged cache store
struct StoreArgs {
  const uint16_t *x, *x2;        // [N, heads, dim] / [N, heads, dim2] (x2 may be null when dim2 == 0)
  int64_t x_ts, x_hs, x2_ts, x2_hs;  // token / head strides in elements
  const int64_t *slots;          // [N]
  uint8_t *cache;                // [num_slots / page_size, heads, page_size, dim + dim2]
  int64_t num_tokens, num_slots;
  int32_t heads, dim, dim2, page_size;
};
int launch_cache_store(const StoreArgs &a, int dtype, bool has_scale, float scale_inv,
                       hipStream_t stream);

// ---- RoPE + quantize
// Division by an invariant 32-bit integer as a multiply-high and two shifts
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, section 4): exact for every 32-bit n.
struct FastDiv {
  uint32_t m;
  int32_t s1, s2;
};
inline FastDiv make_fastdiv(uint32_t d) {   // d >= 1
  int l = 0;
  while ((1ull << l) < d) ++l;              // ceil(log2 d)
  FastDiv f;
  f.m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
  f.s1 = l > 0 ? 1 : 0;
  f.s2 = l > 0 ? l - 1 : 0;
  return f;
}

struct RopeArgs {
  const uint16_t *x_nope, *x_pe;     // [N, heads, nope] / [N, heads or 1, rope]
  int64_t nope_ts, nope_hs, pe_ts, pe_hs;  // strides in elements (pe_hs 0: shared rope head)
  const float *cos_sin;              // [max_position, rope]: cosines then sines
  const int64_t *positions;          // [N]
  uint8_t *out;                      // row (n, h) at out + n * out_ts + h * out_hs, nope + rope bytes
  int64_t out_ts, out_hs;
  int64_t num_tokens, max_position;
  int32_t heads, nope, rope;
  bool neox;
  FastDiv div_nope, div_rope, div_heads;   // by nope / 8, rope / 8, heads (set by the launcher)
  int32_t rows_per_wg;                     // (set by the launcher)
};
int launch_rope_quantize(const RopeArgs &a, int dtype, bool has_scale, float scale_inv,
                         hipStream_t stream);

struct NormRopeArgs {
  const uint16_t *x;                 // row (n, h) at x + n * x_ts + h * x_hs, dim elements
  int64_t x_ts, x_hs;
  const float *weight;               // [dim]
  float eps;
  const float *cos_sin;              // [max_position, rope]: cosines then sines
  const int64_t *positions;          // [N]
  uint8_t *out;                      // NULL or row (n, h) at out + n * out_ts + h * out_hs
  int64_t out_ts, out_hs;
  const int64_t *slot_mapping;       // NULL or [N]
  uint8_t *cache;                    // [num_pages, heads, page_size, dim]
  int64_t num_slots;                 // num_pages * page_size
  int32_t page_size;
  int64_t num_tokens, max_position;
  int32_t heads, dim, rope;
  int32_t lanes_per_row;             // dim / 8 rounded up to a power of two
  bool neox;
};
int launch_qknorm_rope_quantize(const NormRopeArgs &a, int dtype, bool has_scale, float scale_inv,
                                hipStream_t stream);

// ---- indexer
struct IndexerArgs {
  const uint8_t *idx_q;
  const uint8_t *idx_k;
  int64_t num_pages;
  const int32_t *block_table;
  int32_t max_blocks;
  const int32_t *cu_seqlens_q;
  const int32_t *seq_lens;
  int32_t batch, total_q, max_q_len, num_heads, topk;
  float sigma;  // sm_scale * idx_q_scale * idx_k_scale (> 0)
  int32_t *out_ids;
  float *scores;  // workspace [num_heads, total_q, max_blocks]
};
size_t indexer_workspace_bytes(int32_t total_q, int32_t num_heads, int32_t max_blocks);
int launch_indexer(const IndexerArgs &a, hipStream_t stream);

// ---- attention
struct AttnArgs {
  int32_t mode;
  const uint8_t *q, *k, *v;
  int64_t num_kv;
  int64_t k_row_stride, v_row_stride;  // token mode: bytes between KV rows
  const int32_t *indices;
  int32_t topk;
  const int32_t *topk_length;
  const int32_t *block_table;
  int32_t max_blocks;
  const int32_t *cu_seqlens_q, *seq_lens;
  int32_t batch, total_q, max_q_len;
  int32_t hq, hkv, hidx, dqk, dv;
  float key_scale_log2;   // sm * q_scale * k_scale * log2(e)
  float sink_scale_log2;  // sm * q_scale * log2(e)
  float v_scale;
  const float *sink;
  uint16_t *out;
  float *max_logits, *lse;
  void *workspace;
};
size_t attn_workspace_bytes(int32_t mode, int32_t batch, int32_t total_q, int32_t max_q_len,
                            int32_t hq, int32_t hkv, int32_t hidx, int32_t dv, int32_t topk,
                            int32_t max_blocks);
int launch_attention(const AttnArgs &a, hipStream_t stream);

}  // namespace fp8ts
