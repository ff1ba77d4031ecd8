// C-ABI entry points: argument validation on the host, scale normalisation
// (None -> unit, checked once at the launch boundary as the sglang PR 30971
// digest prescribes in implementation step 3), then stream-ordered launches.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "internal.h"

namespace fp8ts {

static thread_local char g_last_error[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FP8TS_EHIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return FP8TS_OK;
}

// Optional scale: NULL -> (false, 1); otherwise must be finite and > 0.
static int read_scale(const char *fn, const char *name, const float *s, bool *present, float *value) {
  *present = s != nullptr;
  *value = 1.0f;
  if (!s) return FP8TS_OK;
  const float v = *s;
  if (!std::isfinite(v) || !(v > 0.0f)) return fail(FP8TS_EINVAL, "%s: %s must be finite and > 0 (got %g)", fn, name, (double)v);
  *value = v;
  return FP8TS_OK;
}

static bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

}  // namespace fp8ts

using namespace fp8ts;

extern "C" {

const char *fp8ts_last_error(void) { return g_last_error; }

int fp8ts_abi_version(void) { return 1; }

int fp8_quantize(const void *x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t x_row_stride,
                 uint8_t *out, int64_t out_row_stride, const float *scale, hipStream_t stream) {
  const char *fn = "fp8_quantize";
  if (x_dtype != FP8TS_BF16 && x_dtype != FP8TS_FP16)
    return fail(FP8TS_EINVAL, "%s: x_dtype must be 0 (bf16) or 1 (fp16), got %d", fn, x_dtype);
  if (rows < 0 || cols < 0) return fail(FP8TS_EINVAL, "%s: negative shape (%lld, %lld)", fn, (long long)rows, (long long)cols);
  bool has = false;
  float sv = 1.0f;
  if (int st = read_scale(fn, "scale", scale, &has, &sv)) return st;
  if (rows == 0 || cols == 0) return FP8TS_OK;
  if (!x || !out) return fail(FP8TS_EINVAL, "%s: null tensor pointer", fn);
  if (x_row_stride < cols) return fail(FP8TS_EINVAL, "%s: x_row_stride %lld < cols %lld", fn, (long long)x_row_stride, (long long)cols);
  if (out_row_stride < cols) return fail(FP8TS_EINVAL, "%s: out_row_stride %lld < cols %lld", fn, (long long)out_row_stride, (long long)cols);
  const size_t xb = (size_t)((rows - 1) * x_row_stride + cols) * 2;
  const size_t ob = (size_t)((rows - 1) * out_row_stride + cols);
  if (overlaps(x, xb, out, ob)) return fail(FP8TS_EINVAL, "%s: out overlaps x", fn);
  const float inv = has ? 1.0f / sv : 1.0f;   // fp32 reciprocal, rounded once
  return launch_quantize(x, x_dtype, rows, cols, x_row_stride, out, out_row_stride, has, inv, stream);
}

int fp8_quantize_pair(const void *x0, uint8_t *out0, int64_t n0, const float *scale0, const void *x1,
                      uint8_t *out1, int64_t n1, const float *scale1, int32_t x_dtype, hipStream_t stream) {
  const char *fn = "fp8_quantize_pair";
  if (x_dtype != FP8TS_BF16 && x_dtype != FP8TS_FP16)
    return fail(FP8TS_EINVAL, "%s: x_dtype must be 0 (bf16) or 1 (fp16), got %d", fn, x_dtype);
  if (n0 < 0 || n1 < 0) return fail(FP8TS_EINVAL, "%s: negative size", fn);
  bool h0 = false, h1 = false;
  float v0 = 1.0f, v1 = 1.0f;
  if (int st = read_scale(fn, "scale0", scale0, &h0, &v0)) return st;
  if (int st = read_scale(fn, "scale1", scale1, &h1, &v1)) return st;
  if (n0 == 0 && n1 == 0) return FP8TS_OK;
  if ((n0 > 0 && (!x0 || !out0)) || (n1 > 0 && (!x1 || !out1))) return fail(FP8TS_EINVAL, "%s: null tensor pointer", fn);
  if (n0 % 8 || n1 % 8)
    return fail(FP8TS_EUNSUPPORTED, "%s: element counts must be multiples of 8 (got %lld, %lld)", fn, (long long)n0,
                (long long)n1);
  if ((n0 > 0 && ((uintptr_t)x0 % 16 || (uintptr_t)out0 % 8)) || (n1 > 0 && ((uintptr_t)x1 % 16 || (uintptr_t)out1 % 8)))
    return fail(FP8TS_EUNSUPPORTED, "%s: x needs 16-byte and out 8-byte alignment", fn);
  const size_t xb0 = (size_t)n0 * 2, xb1 = (size_t)n1 * 2, ob0 = (size_t)n0, ob1 = (size_t)n1;
  if (overlaps(out0, ob0, x0, xb0) || overlaps(out0, ob0, x1, xb1) || overlaps(out1, ob1, x0, xb0) ||
      overlaps(out1, ob1, x1, xb1) || overlaps(out0, ob0, out1, ob1))
    return fail(FP8TS_EINVAL, "%s: an output overlaps an input or the other output", fn);
  const float i0 = h0 ? 1.0f / v0 : 1.0f, i1 = h1 ? 1.0f / v1 : 1.0f;   // fp32 reciprocals, rounded once
  return launch_quantize_pair(x0, out0, n0, h0, i0, x1, out1, n1, h1, i1, x_dtype, stream);
}

int fp8_cache_store(const void *x, const void *x2, int32_t x_dtype, int64_t num_tokens,
                    int32_t num_heads, int32_t dim, int32_t dim2, int64_t x_token_stride,
                    int64_t x_head_stride, int64_t x2_token_stride, int64_t x2_head_stride,
                    const int64_t *slot_mapping, uint8_t *cache, int64_t num_pages,
                    int32_t page_size, const float *scale, hipStream_t stream) {
  const char *fn = "fp8_cache_store";
  if (x_dtype != FP8TS_BF16 && x_dtype != FP8TS_FP16)
    return fail(FP8TS_EINVAL, "%s: x_dtype must be 0 (bf16) or 1 (fp16), got %d", fn, x_dtype);
  if (num_tokens < 0 || num_pages < 0) return fail(FP8TS_EINVAL, "%s: negative size", fn);
  if (num_heads < 1 || dim < 1 || dim2 < 0 || page_size < 1)
    return fail(FP8TS_EINVAL, "%s: need num_heads >= 1, dim >= 1, dim2 >= 0, page_size >= 1 (got %d, %d, %d, %d)",
                fn, num_heads, dim, dim2, page_size);
  if ((dim2 > 0) != (x2 != nullptr)) return fail(FP8TS_EINVAL, "%s: x2 must be given exactly when dim2 > 0", fn);
  bool has = false;
  float sv = 1.0f;
  if (int st = read_scale(fn, "scale", scale, &has, &sv)) return st;
  if (num_tokens == 0) return FP8TS_OK;
  if (!x || !slot_mapping || !cache) return fail(FP8TS_EINVAL, "%s: null tensor pointer", fn);
  if (num_pages == 0) return fail(FP8TS_EINVAL, "%s: empty cache", fn);
  // every (token, head) row of a source must be a separate run of elements
  auto rows_ok = [&](int64_t ts, int64_t hs, int32_t d) {
    if (ts < 0 || hs < 0) return false;
    if (num_heads > 1 && hs < d) return false;
    return num_tokens == 1 || ts >= (int64_t)(num_heads - 1) * hs + d;
  };
  if (!rows_ok(x_token_stride, x_head_stride, dim))
    return fail(FP8TS_EINVAL, "%s: x strides (%lld, %lld) overlap rows of %d elements", fn,
                (long long)x_token_stride, (long long)x_head_stride, dim);
  if (dim2 > 0 && !rows_ok(x2_token_stride, x2_head_stride, dim2))
    return fail(FP8TS_EINVAL, "%s: x2 strides (%lld, %lld) overlap rows of %d elements", fn,
                (long long)x2_token_stride, (long long)x2_head_stride, dim2);
  const int64_t row = (int64_t)dim + dim2;
  // the kernel indexes chunks and slots in 32 bits
  if (num_tokens * num_heads * row >= ((int64_t)1 << 31) || num_pages * page_size >= ((int64_t)1 << 31))
    return fail(FP8TS_EUNSUPPORTED, "%s: more than 2^31 - 1 elements or slots in one call", fn);
  const size_t cb = (size_t)(num_pages * num_heads * page_size * row);
  const size_t xb = (size_t)((num_tokens - 1) * x_token_stride + (int64_t)(num_heads - 1) * x_head_stride + dim) * 2;
  if (overlaps(x, xb, cache, cb)) return fail(FP8TS_EINVAL, "%s: cache overlaps x", fn);
  if (dim2 > 0) {
    const size_t x2b = (size_t)((num_tokens - 1) * x2_token_stride + (int64_t)(num_heads - 1) * x2_head_stride + dim2) * 2;
    if (overlaps(x2, x2b, cache, cb)) return fail(FP8TS_EINVAL, "%s: cache overlaps x2", fn);
  }
  if (overlaps(slot_mapping, (size_t)num_tokens * 8, cache, cb)) return fail(FP8TS_EINVAL, "%s: cache overlaps slot_mapping", fn);
  StoreArgs a{};
  a.x = static_cast<const uint16_t *>(x);
  a.x2 = static_cast<const uint16_t *>(x2);
  a.x_ts = x_token_stride;
  a.x_hs = x_head_stride;
  a.x2_ts = x2_token_stride;
  a.x2_hs = x2_head_stride;
  a.slots = slot_mapping;
  a.cache = cache;
  a.num_tokens = num_tokens;
  a.num_slots = num_pages * page_size;
  a.heads = num_heads;
  a.dim = dim;
  a.dim2 = dim2;
  a.page_size = page_size;
  const float inv = has ? 1.0f / sv : 1.0f;   // fp32 reciprocal, rounded once
  return launch_cache_store(a, x_dtype, has, inv, stream);
}

int fp8_rope_quantize(const void *x_nope, const void *x_pe, int32_t x_dtype, int64_t num_tokens,
                      int32_t num_heads, int32_t nope_dim, int32_t rope_dim,
                      int64_t nope_token_stride, int64_t nope_head_stride, int64_t pe_token_stride,
                      int64_t pe_head_stride, const float *cos_sin_cache, int64_t max_position,
                      const int64_t *positions, int32_t is_neox, uint8_t *out,
                      int64_t out_token_stride, int64_t out_head_stride, const float *scale,
                      hipStream_t stream) {
  const char *fn = "fp8_rope_quantize";
  if (x_dtype != FP8TS_BF16 && x_dtype != FP8TS_FP16)
    return fail(FP8TS_EINVAL, "%s: x_dtype must be 0 (bf16) or 1 (fp16), got %d", fn, x_dtype);
  if (num_tokens < 0 || max_position < 0) return fail(FP8TS_EINVAL, "%s: negative size", fn);
  if (num_heads < 1 || nope_dim < 0 || rope_dim < 2 || rope_dim % 2)
    return fail(FP8TS_EINVAL, "%s: need num_heads >= 1, nope_dim >= 0 and an even rope_dim >= 2 (got %d, %d, %d)",
                fn, num_heads, nope_dim, rope_dim);
  if ((nope_dim > 0) != (x_nope != nullptr))
    return fail(FP8TS_EINVAL, "%s: x_nope must be given exactly when nope_dim > 0", fn);
  if (nope_dim % 8 || rope_dim % 16)
    return fail(FP8TS_EUNSUPPORTED, "%s: nope_dim must be a multiple of 8 and rope_dim of 16 (got %d, %d)", fn,
                nope_dim, rope_dim);
  bool has = false;
  float sv = 1.0f;
  if (int st = read_scale(fn, "scale", scale, &has, &sv)) return st;
  if (num_tokens == 0) return FP8TS_OK;
  if (!x_pe || !cos_sin_cache || !positions || !out) return fail(FP8TS_EINVAL, "%s: null tensor pointer", fn);
  if (max_position == 0) return fail(FP8TS_EINVAL, "%s: empty cos_sin_cache", fn);
  const int64_t row = (int64_t)nope_dim + rope_dim;
  if (num_tokens * num_heads * row >= ((int64_t)1 << 31))
    return fail(FP8TS_EUNSUPPORTED, "%s: more than 2^31 - 1 elements in one call", fn);
  // source rows may be read by several heads (a shared rope head has stride 0); output rows must not overlap
  if (out_head_stride < row && num_heads > 1) return fail(FP8TS_EINVAL, "%s: out_head_stride %lld < row %lld", fn, (long long)out_head_stride, (long long)row);
  if (num_tokens > 1 && out_token_stride < (int64_t)(num_heads - 1) * out_head_stride + row)
    return fail(FP8TS_EINVAL, "%s: out_token_stride %lld overlaps rows", fn, (long long)out_token_stride);
  if (nope_token_stride < 0 || nope_head_stride < 0 || pe_token_stride < 0 || pe_head_stride < 0 ||
      out_token_stride < 0 || out_head_stride < 0)
    return fail(FP8TS_EINVAL, "%s: negative stride", fn);
  const bool aligned =
      (uintptr_t)x_pe % 16 == 0 && pe_token_stride % 8 == 0 && pe_head_stride % 8 == 0 &&
      (uintptr_t)cos_sin_cache % 16 == 0 && (uintptr_t)out % 8 == 0 && out_token_stride % 8 == 0 &&
      out_head_stride % 8 == 0 &&
      (nope_dim == 0 || ((uintptr_t)x_nope % 16 == 0 && nope_token_stride % 8 == 0 && nope_head_stride % 8 == 0));
  if (!aligned)
    return fail(FP8TS_EUNSUPPORTED, "%s: sources and cos_sin_cache need 16-byte alignment, out 8-byte, and every stride a multiple of 8", fn);
  const size_t ob = (size_t)((num_tokens - 1) * out_token_stride + (int64_t)(num_heads - 1) * out_head_stride + row);
  const size_t pb = (size_t)((num_tokens - 1) * pe_token_stride + (int64_t)(num_heads - 1) * pe_head_stride + rope_dim) * 2;
  if (overlaps(out, ob, x_pe, pb)) return fail(FP8TS_EINVAL, "%s: out overlaps x_pe", fn);
  if (nope_dim > 0) {
    const size_t nb = (size_t)((num_tokens - 1) * nope_token_stride + (int64_t)(num_heads - 1) * nope_head_stride + nope_dim) * 2;
    if (overlaps(out, ob, x_nope, nb)) return fail(FP8TS_EINVAL, "%s: out overlaps x_nope", fn);
  }
  if (overlaps(out, ob, cos_sin_cache, (size_t)(max_position * rope_dim * 4)))
    return fail(FP8TS_EINVAL, "%s: out overlaps cos_sin_cache", fn);
  if (overlaps(out, ob, positions, (size_t)num_tokens * 8)) return fail(FP8TS_EINVAL, "%s: out overlaps positions", fn);
  RopeArgs a{};
  a.x_nope = static_cast<const uint16_t *>(x_nope);
  a.x_pe = static_cast<const uint16_t *>(x_pe);
  a.nope_ts = nope_token_stride;
  a.nope_hs = nope_head_stride;
  a.pe_ts = pe_token_stride;
  a.pe_hs = pe_head_stride;
  a.cos_sin = cos_sin_cache;
  a.positions = positions;
  a.out = out;
  a.out_ts = out_token_stride;
  a.out_hs = out_head_stride;
  a.num_tokens = num_tokens;
  a.max_position = max_position;
  a.heads = num_heads;
  a.nope = nope_dim;
  a.rope = rope_dim;
  a.neox = is_neox != 0;
  const float inv = has ? 1.0f / sv : 1.0f;   // fp32 reciprocal, rounded once
  return launch_rope_quantize(a, x_dtype, has, inv, stream);
}

int fp8_qknorm_rope_quantize(const void *x, int32_t x_dtype, int64_t num_tokens, int32_t num_heads,
                             int32_t head_dim, int32_t rope_dim, int64_t x_token_stride,
                             int64_t x_head_stride, const float *norm_weight, float eps,
                             const float *cos_sin_cache, int64_t max_position,
                             const int64_t *positions, int32_t is_neox, uint8_t *out,
                             int64_t out_token_stride, int64_t out_head_stride,
                             const int64_t *slot_mapping, uint8_t *cache, int64_t num_pages,
                             int32_t page_size, const float *scale, hipStream_t stream) {
  const char *fn = "fp8_qknorm_rope_quantize";
  if (x_dtype != FP8TS_BF16 && x_dtype != FP8TS_FP16)
    return fail(FP8TS_EINVAL, "%s: x_dtype must be 0 (bf16) or 1 (fp16), got %d", fn, x_dtype);
  if (num_tokens < 0 || max_position < 0 || num_pages < 0) return fail(FP8TS_EINVAL, "%s: negative size", fn);
  if (num_heads < 1 || head_dim < 1 || rope_dim < 0 || rope_dim % 2 || rope_dim > head_dim)
    return fail(FP8TS_EINVAL, "%s: need num_heads >= 1, head_dim >= 1 and an even rope_dim in [0, head_dim] (got %d, %d, %d)",
                fn, num_heads, head_dim, rope_dim);
  if (!std::isfinite(eps) || eps < 0.0f) return fail(FP8TS_EINVAL, "%s: eps must be finite and >= 0 (got %g)", fn, (double)eps);
  if (!out && !slot_mapping) return fail(FP8TS_EINVAL, "%s: neither out nor slot_mapping given", fn);
  if (slot_mapping && page_size < 1) return fail(FP8TS_EINVAL, "%s: page_size must be >= 1 (got %d)", fn, page_size);
  if (head_dim % 8 || head_dim > 512 || rope_dim % 16)
    return fail(FP8TS_EUNSUPPORTED, "%s: head_dim must be a multiple of 8 up to 512 and rope_dim a multiple of 16 (got %d, %d)",
                fn, head_dim, rope_dim);
  bool has = false;
  float sv = 1.0f;
  if (int st = read_scale(fn, "scale", scale, &has, &sv)) return st;
  if (num_tokens == 0) return FP8TS_OK;
  if (!x || !norm_weight || (rope_dim > 0 && (!cos_sin_cache || !positions)))
    return fail(FP8TS_EINVAL, "%s: null tensor pointer", fn);
  if (slot_mapping && !cache) return fail(FP8TS_EINVAL, "%s: slot_mapping given without a cache", fn);
  if (rope_dim > 0 && max_position == 0) return fail(FP8TS_EINVAL, "%s: empty cos_sin_cache", fn);
  if (slot_mapping && num_pages == 0) return fail(FP8TS_EINVAL, "%s: empty cache", fn);
  if (num_tokens * num_heads * head_dim >= ((int64_t)1 << 31))
    return fail(FP8TS_EUNSUPPORTED, "%s: more than 2^31 - 1 elements in one call", fn);
  if (x_token_stride < 0 || x_head_stride < 0 || out_token_stride < 0 || out_head_stride < 0)
    return fail(FP8TS_EINVAL, "%s: negative stride", fn);
  if (out) {
    if (out_head_stride < head_dim && num_heads > 1)
      return fail(FP8TS_EINVAL, "%s: out_head_stride %lld < head_dim %d", fn, (long long)out_head_stride, head_dim);
    if (num_tokens > 1 && out_token_stride < (int64_t)(num_heads - 1) * out_head_stride + head_dim)
      return fail(FP8TS_EINVAL, "%s: out_token_stride %lld overlaps rows", fn, (long long)out_token_stride);
  }
  const bool aligned =
      (uintptr_t)x % 16 == 0 && x_token_stride % 8 == 0 && x_head_stride % 8 == 0 &&
      (uintptr_t)norm_weight % 16 == 0 && (rope_dim == 0 || (uintptr_t)cos_sin_cache % 16 == 0) &&
      (!out || ((uintptr_t)out % 8 == 0 && out_token_stride % 8 == 0 && out_head_stride % 8 == 0)) &&
      (!slot_mapping || (uintptr_t)cache % 8 == 0);
  if (!aligned)
    return fail(FP8TS_EUNSUPPORTED, "%s: x, norm_weight and cos_sin_cache need 16-byte alignment, out and cache 8-byte, and every stride a multiple of 8", fn);
  const size_t xb = (size_t)((num_tokens - 1) * x_token_stride + (int64_t)(num_heads - 1) * x_head_stride + head_dim) * 2;
  const size_t cb = slot_mapping ? (size_t)(num_pages * page_size) * num_heads * head_dim : 0;
  struct { const void *p; size_t n; const char *name; } ins[] = {
      {x, xb, "x"}, {norm_weight, (size_t)head_dim * 4, "norm_weight"},
      {cos_sin_cache, rope_dim > 0 ? (size_t)(max_position * rope_dim * 4) : 0, "cos_sin_cache"},
      {positions, rope_dim > 0 ? (size_t)num_tokens * 8 : 0, "positions"},
      {slot_mapping, slot_mapping ? (size_t)num_tokens * 8 : 0, "slot_mapping"}};
  if (out) {
    const size_t ob = (size_t)((num_tokens - 1) * out_token_stride + (int64_t)(num_heads - 1) * out_head_stride + head_dim);
    for (const auto &in : ins)
      if (overlaps(out, ob, in.p, in.n)) return fail(FP8TS_EINVAL, "%s: out overlaps %s", fn, in.name);
    if (overlaps(out, ob, cache, cb)) return fail(FP8TS_EINVAL, "%s: out overlaps cache", fn);
  }
  if (slot_mapping)
    for (const auto &in : ins)
      if (overlaps(cache, cb, in.p, in.n)) return fail(FP8TS_EINVAL, "%s: cache overlaps %s", fn, in.name);
  NormRopeArgs a{};
  a.x = static_cast<const uint16_t *>(x);
  a.x_ts = x_token_stride;
  a.x_hs = x_head_stride;
  a.weight = norm_weight;
  a.eps = eps;
  a.cos_sin = cos_sin_cache;
  a.positions = positions;
  a.out = out;
  a.out_ts = out_token_stride;
  a.out_hs = out_head_stride;
  a.slot_mapping = slot_mapping;
  a.cache = cache;
  a.num_slots = slot_mapping ? num_pages * page_size : 0;
  a.page_size = slot_mapping ? page_size : 1;
  a.num_tokens = num_tokens;
  a.max_position = max_position;
  a.heads = num_heads;
  a.dim = head_dim;
  a.rope = rope_dim;
  a.lanes_per_row = 1;
  while (a.lanes_per_row * 8 < head_dim) a.lanes_per_row *= 2;
  a.neox = is_neox != 0;
  const float inv = has ? 1.0f / sv : 1.0f;   // fp32 reciprocal, rounded once
  return launch_qknorm_rope_quantize(a, x_dtype, has, inv, stream);
}

size_t indexer_topk_workspace_size(int32_t total_q, int32_t num_heads, int32_t max_blocks) {
  if (total_q <= 0 || num_heads <= 0 || max_blocks <= 0) return 0;
  return indexer_workspace_bytes(total_q, num_heads, max_blocks);
}

int indexer_topk(const uint8_t *idx_q, const uint8_t *idx_k, int64_t num_pages,
                 const int32_t *block_table, int32_t max_blocks, const int32_t *cu_seqlens_q,
                 const int32_t *seq_lens, int32_t batch, int32_t total_q, int32_t max_q_len,
                 int32_t num_heads, int32_t head_dim, int32_t page_size, float sm_scale,
                 const float *idx_q_scale, const float *idx_k_scale, int32_t topk, int32_t *out_ids,
                 void *workspace, size_t workspace_bytes, hipStream_t stream) {
  const char *fn = "indexer_topk";
  if (batch < 0 || total_q < 0 || max_q_len < 0 || num_pages < 0 || max_blocks < 0)
    return fail(FP8TS_EINVAL, "%s: negative size", fn);
  if (!(num_heads == 1 || num_heads == 2 || num_heads == 4 || num_heads == 8 || num_heads == 16))
    return fail(FP8TS_EUNSUPPORTED, "%s: num_heads must be 1, 2, 4, 8 or 16 (got %d)", fn, num_heads);
  if (head_dim != 128) return fail(FP8TS_EUNSUPPORTED, "%s: head_dim must be 128 (got %d)", fn, head_dim);
  if (page_size != 128) return fail(FP8TS_EUNSUPPORTED, "%s: page_size must be 128 (got %d)", fn, page_size);
  if (topk < 1 || topk > 64) return fail(FP8TS_EUNSUPPORTED, "%s: topk must be in [1, 64] (got %d)", fn, topk);
  if (max_blocks > 4096) return fail(FP8TS_EUNSUPPORTED, "%s: max_blocks %d exceeds 4096", fn, max_blocks);
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
    return fail(FP8TS_EINVAL, "%s: sm_scale must be finite and > 0 (got %g)", fn, (double)sm_scale);
  bool hq = false, hk = false;
  float sq = 1.0f, sk = 1.0f;
  if (int st = read_scale(fn, "idx_q_scale", idx_q_scale, &hq, &sq)) return st;
  if (int st = read_scale(fn, "idx_k_scale", idx_k_scale, &hk, &sk)) return st;
  if (total_q == 0) return FP8TS_OK;
  if (batch == 0 || max_q_len == 0) return fail(FP8TS_EINVAL, "%s: total_q > 0 needs batch > 0 and max_q_len > 0", fn);
  if (max_q_len > total_q) return fail(FP8TS_EINVAL, "%s: max_q_len %d > total_q %d", fn, max_q_len, total_q);
  if (!idx_q || !idx_k || !block_table || !cu_seqlens_q || !seq_lens || !out_ids)
    return fail(FP8TS_EINVAL, "%s: null tensor pointer", fn);
  if (max_blocks == 0 || num_pages == 0) return fail(FP8TS_EINVAL, "%s: empty KV cache / block table", fn);
  const size_t need = indexer_workspace_bytes(total_q, num_heads, max_blocks);
  if (!workspace || workspace_bytes < need)
    return fail(FP8TS_EINVAL, "%s: workspace needs %zu bytes, got %zu", fn, need, workspace ? workspace_bytes : 0);
  if ((uintptr_t)workspace % 256) return fail(FP8TS_EINVAL, "%s: workspace must be 256-byte aligned", fn);
  if (overlaps(out_ids, (size_t)num_heads * total_q * topk * 4, idx_q, (size_t)total_q * num_heads * 128))
    return fail(FP8TS_EINVAL, "%s: out_ids overlaps idx_q", fn);
  IndexerArgs a{};
  a.idx_q = idx_q;
  a.idx_k = idx_k;
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.cu_seqlens_q = cu_seqlens_q;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.num_heads = num_heads;
  a.topk = topk;
  a.sigma = (float)((double)sm_scale * sq * sk);
  a.out_ids = out_ids;
  a.scores = static_cast<float *>(workspace);
  return launch_indexer(a, stream);
}

size_t sparse_attn_workspace_size(int32_t mode, int32_t batch, int32_t total_q, int32_t max_q_len,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t num_idx_heads,
                                  int32_t head_dim_v, int32_t topk, int32_t max_blocks) {
  if (total_q <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || topk <= 0) return 0;
  if (mode == FP8TS_BLOCK_MODE && (num_idx_heads <= 0 || max_blocks <= 0 || max_q_len <= 0 || batch <= 0)) return 0;
  return attn_workspace_bytes(mode, batch, total_q, max_q_len, num_q_heads, num_kv_heads, num_idx_heads,
                              head_dim_v, topk, max_blocks);
}

}  // extern "C"

namespace fp8ts {

// Validation and argument set-up shared by the two attention entry points:
// everything but the workspace.  On success fills `a` (workspace unset) and
// the workspace size the call needs.
static int prepare_attention(const char *fn, int32_t mode, const uint8_t *q, const uint8_t *k, const uint8_t *v,
                             int64_t num_kv, const int32_t *indices, int32_t topk, const int32_t *topk_length,
                             const int32_t *block_table, int32_t max_blocks, const int32_t *cu_seqlens_q,
                             const int32_t *seq_lens, int32_t batch, int32_t total_q, int32_t max_q_len,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t num_idx_heads, int32_t head_dim_qk,
                             int32_t head_dim_v, int32_t page_size, float sm_scale, const float *q_scale,
                             const float *k_scale, const float *v_scale, const float *attn_sink, uint16_t *out,
                             float *max_logits, float *lse, AttnArgs &a, size_t &need) {
  if (mode != FP8TS_TOKEN_MODE && mode != FP8TS_BLOCK_MODE)
    return fail(FP8TS_EINVAL, "%s: mode must be 0 (token) or 1 (block), got %d", fn, mode);
  if (total_q < 0 || num_kv < 0 || topk < 0 || batch < 0 || max_q_len < 0 || max_blocks < 0)
    return fail(FP8TS_EINVAL, "%s: negative size", fn);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
    return fail(FP8TS_EINVAL, "%s: num_q_heads %d must be a positive multiple of num_kv_heads %d", fn,
                num_q_heads, num_kv_heads);
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
    return fail(FP8TS_EINVAL, "%s: sm_scale must be finite and > 0 (got %g)", fn, (double)sm_scale);
  bool hq = false, hk = false, hv = false;
  float sq = 1.0f, sk = 1.0f, sv = 1.0f;
  if (int st = read_scale(fn, "q_scale", q_scale, &hq, &sq)) return st;
  if (int st = read_scale(fn, "k_scale", k_scale, &hk, &sk)) return st;
  if (int st = read_scale(fn, "v_scale", v_scale, &hv, &sv)) return st;

  if (mode == FP8TS_TOKEN_MODE) {
    if (head_dim_v != 512)
      return fail(FP8TS_EUNSUPPORTED, "%s: token mode hard-codes d_v = 512 (got d_v=%d)", fn, head_dim_v);
    if (head_dim_qk != 576)
      return fail(FP8TS_EUNSUPPORTED, "%s: token mode needs head_dim_qk = 576 (got %d)", fn, head_dim_qk);
    if (num_kv_heads != 1) return fail(FP8TS_EUNSUPPORTED, "%s: token mode has one shared KV head (got %d)", fn, num_kv_heads);
    if (topk < 1) return fail(FP8TS_EINVAL, "%s: topk must be >= 1", fn);
  } else {
    if (head_dim_qk != 128 || head_dim_v != 128)
      return fail(FP8TS_EUNSUPPORTED, "%s: block mode needs head_dim_qk = head_dim_v = 128 (got %d, %d)", fn,
                  head_dim_qk, head_dim_v);
    if (page_size != 128) return fail(FP8TS_EUNSUPPORTED, "%s: page_size must be 128 (got %d)", fn, page_size);
    if (num_idx_heads <= 0 || num_q_heads % num_idx_heads)
      return fail(FP8TS_EINVAL, "%s: num_q_heads %d must be a positive multiple of num_idx_heads %d", fn,
                  num_q_heads, num_idx_heads);
    const int G = num_q_heads / num_kv_heads, gqi = num_q_heads / num_idx_heads;
    if (G % gqi && gqi % G)
      return fail(FP8TS_EUNSUPPORTED, "%s: index-head groups (%d q heads) must nest with kv-head groups (%d)", fn,
                  gqi, G);
    if (G > 256) return fail(FP8TS_EUNSUPPORTED, "%s: more than 256 q heads per kv head", fn);
    if (topk < 1 || topk > 64) return fail(FP8TS_EUNSUPPORTED, "%s: block mode topk must be in [1, 64] (got %d)", fn, topk);
    if (max_blocks > 4096) return fail(FP8TS_EUNSUPPORTED, "%s: max_blocks %d exceeds 4096", fn, max_blocks);
  }
  need = 0;
  if (total_q == 0) return FP8TS_OK;
  if (!q || !k || !indices || !out || !max_logits || !lse) return fail(FP8TS_EINVAL, "%s: null tensor pointer", fn);
  if (num_kv == 0) return fail(FP8TS_EINVAL, "%s: empty KV", fn);
  if (mode == FP8TS_BLOCK_MODE) {
    if (!v) return fail(FP8TS_EINVAL, "%s: block mode needs a V cache", fn);
    if (!block_table || !cu_seqlens_q || !seq_lens || batch == 0 || max_blocks == 0 || max_q_len == 0)
      return fail(FP8TS_EINVAL, "%s: block mode needs block_table, cu_seqlens_q, seq_lens, batch, max_blocks, max_q_len", fn);
    if (max_q_len > total_q) return fail(FP8TS_EINVAL, "%s: max_q_len %d > total_q %d", fn, max_q_len, total_q);
  }
  need = attn_workspace_bytes(mode, batch, total_q, max_q_len, num_q_heads, num_kv_heads, num_idx_heads,
                              head_dim_v, topk, max_blocks);
  const size_t ob = (size_t)total_q * num_q_heads * head_dim_v * 2;
  if (overlaps(out, ob, q, (size_t)total_q * num_q_heads * head_dim_qk))
    return fail(FP8TS_EINVAL, "%s: out overlaps q", fn);

  a = AttnArgs{};
  a.mode = mode;
  a.q = q;
  a.k = k;
  a.v = v ? v : k;
  a.num_kv = num_kv;
  a.k_row_stride = head_dim_qk;
  a.v_row_stride = v ? head_dim_v : head_dim_qk;
  a.indices = indices;
  a.topk = topk;
  a.topk_length = topk_length;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.cu_seqlens_q = cu_seqlens_q;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.hidx = mode == FP8TS_BLOCK_MODE ? num_idx_heads : 1;
  a.dqk = head_dim_qk;
  a.dv = head_dim_v;
  // q_scale folds into sm_scale; it reaches both the key logits and the sink,
  // k_scale only the key logits.  Products taken in double, rounded once.
  const double s = (double)sm_scale * (double)sq;
  a.key_scale_log2 = (float)(s * (double)sk * 1.4426950408889634);
  a.sink_scale_log2 = (float)(s * 1.4426950408889634);
  a.v_scale = sv;
  a.sink = attn_sink;
  a.out = out;
  a.max_logits = max_logits;
  a.lse = lse;
  return FP8TS_OK;
}


// The library's own scratch for callers that cannot allocate: one copy per
// device, held until the process ends.  Host code uses the address
// hipGetSymbolAddress returns on each device, never the symbol itself.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::once_flag g_scratch_once[kMaxDevices];
static void *g_scratch_ptr[kMaxDevices];
static hipError_t g_scratch_err[kMaxDevices];

// Device address of this device's scratch (looked up once per device, with
// that device current), or null with a message.
static void *device_scratch(const char *fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(FP8TS_EHIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(FP8TS_EUNSUPPORTED, "%s: device %d is beyond the %d devices the scratch table covers", fn, dev, kMaxDevices);
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void *ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  if (!g_scratch_ptr[dev]) {
    fail(FP8TS_EHIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
         hipGetErrorString(g_scratch_err[dev]));
    return nullptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace fp8ts

extern "C" {

int sparse_attn_fwd(int32_t mode, const uint8_t *q, const uint8_t *k, const uint8_t *v, int64_t num_kv,
                    const int32_t *indices, int32_t topk, const int32_t *topk_length,
                    const int32_t *block_table, int32_t max_blocks, const int32_t *cu_seqlens_q,
                    const int32_t *seq_lens, int32_t batch, int32_t total_q, int32_t max_q_len,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t num_idx_heads, int32_t head_dim_qk,
                    int32_t head_dim_v, int32_t page_size, float sm_scale, const float *q_scale,
                    const float *k_scale, const float *v_scale, const float *attn_sink, uint16_t *out,
                    float *max_logits, float *lse, void *workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  const char *fn = "sparse_attn_fwd";
  AttnArgs a;
  size_t need = 0;
  if (int st = prepare_attention(fn, mode, q, k, v, num_kv, indices, topk, topk_length, block_table, max_blocks,
                                 cu_seqlens_q, seq_lens, batch, total_q, max_q_len, num_q_heads, num_kv_heads,
                                 num_idx_heads, head_dim_qk, head_dim_v, page_size, sm_scale, q_scale, k_scale,
                                 v_scale, attn_sink, out, max_logits, lse, a, need))
    return st;
  if (total_q == 0) return FP8TS_OK;
  if (need && (!workspace || workspace_bytes < need))
    return fail(FP8TS_EINVAL, "%s: workspace needs %zu bytes, got %zu", fn, need, workspace ? workspace_bytes : 0);
  if (need && (uintptr_t)workspace % 256) return fail(FP8TS_EINVAL, "%s: workspace must be 256-byte aligned", fn);
  a.workspace = workspace;
  return launch_attention(a, stream);
}

int sparse_attn_fwd_noalloc(int32_t mode, const uint8_t *q, const uint8_t *k, const uint8_t *v, int64_t num_kv,
                            const int32_t *indices, int32_t topk, const int32_t *topk_length,
                            const int32_t *block_table, int32_t max_blocks, const int32_t *cu_seqlens_q,
                            const int32_t *seq_lens, int32_t batch, int32_t total_q, int32_t max_q_len,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t num_idx_heads, int32_t head_dim_qk,
                            int32_t head_dim_v, int32_t page_size, float sm_scale, const float *q_scale,
                            const float *k_scale, const float *v_scale, const float *attn_sink, uint16_t *out,
                            float *max_logits, float *lse, hipStream_t stream) {
  const char *fn = "sparse_attn_fwd_noalloc";
  AttnArgs a;
  size_t need = 0;
  if (int st = prepare_attention(fn, mode, q, k, v, num_kv, indices, topk, topk_length, block_table, max_blocks,
                                 cu_seqlens_q, seq_lens, batch, total_q, max_q_len, num_q_heads, num_kv_heads,
                                 num_idx_heads, head_dim_qk, head_dim_v, page_size, sm_scale, q_scale, k_scale,
                                 v_scale, attn_sink, out, max_logits, lse, a, need))
    return st;
  if (total_q == 0) return FP8TS_OK;
  if (need > kScratchBytes)
    return fail(FP8TS_EUNSUPPORTED, "%s: the call needs %zu bytes of scratch, more than the library's %zu; "
                "use sparse_attn_fwd with a workspace", fn, need, kScratchBytes);
  if (need) {
    a.workspace = device_scratch(fn);
    if (!a.workspace) return FP8TS_EHIP;
  }
  return launch_attention(a, stream);
}

size_t sparse_attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

}  // extern "C"
