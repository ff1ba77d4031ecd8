// Per-tensor e4m3 quantization: y = e4m3(fl32(x) * scale_inv).
//
// Semantics follow the sglang PR 25460 digest (code excerpt of the Triton
// fp8_quantize kernel: widen to fp32, multiply by one reciprocal scale, cast)
// and the sglang PR 30971 digest (implementation step 3: None skips the scale).
//
// HBM-bound: 2 (bf16/fp16) + 1 (e4m3) bytes per element.  Each thread moves
// 16-byte loads / 8-byte stores; the conversion uses the gfx950 packed
// fp32 -> OCP e4m3 instruction (round to nearest even) on values clamped to
// +-448, so overflow saturates instead of producing NaN, and NaN is passed
// through unclamped.
#include "device.h"
#include "internal.h"

namespace fp8ts {
namespace {

template <int DT>
__device__ __forceinline__ float widen(uint16_t h) {
  if constexpr (DT == FP8TS_BF16) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, h);
  }
}

__device__ __forceinline__ float sat448(float v) {
  float c = fminf(fmaxf(v, -448.0f), 448.0f);
  return __builtin_isnan(v) ? v : c;
}

// 1 if v is a NaN with a clear sign bit.
__device__ __forceinline__ uint32_t pos_nan(float v) {
  return (__builtin_bit_cast(uint32_t, v) - 0x7F800001u) < 0x007FFFFFu ? 1u : 0u;
}

// Encode two floats into two e4m3 bytes (low 16 bits of the result).  The
// converter writes 0xFF for every NaN; flipping the sign bit back for
// positive NaN keeps the input's sign (0x7F / 0xFF).
__device__ __forceinline__ uint32_t enc2(float a, float b) {
  const uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false) & 0xFFFFu;
  return r ^ ((pos_nan(a) << 7) | (pos_nan(b) << 15));
}

template <bool HAS_SCALE>
__device__ __forceinline__ float scaled(float v, float s) {
  if constexpr (HAS_SCALE) return v * s;
  return v;
}

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// 8 elements (16 bytes of 16-bit inputs) -> 8 bytes.
template <int DT, bool HAS_SCALE>
__device__ __forceinline__ v2u quant8(v4u w, float s) {
  uint32_t in[4] = {w[0], w[1], w[2], w[3]};
  uint32_t o[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float f0 = scaled<HAS_SCALE>(widen<DT>(in[2 * j] & 0xFFFF), s);
    float f1 = scaled<HAS_SCALE>(widen<DT>(in[2 * j] >> 16), s);
    float f2 = scaled<HAS_SCALE>(widen<DT>(in[2 * j + 1] & 0xFFFF), s);
    float f3 = scaled<HAS_SCALE>(widen<DT>(in[2 * j + 1] >> 16), s);
    o[j] = enc2(f0, f1) | (enc2(f2, f3) << 16);
  }
  return (v2u){o[0], o[1]};
}

template <int DT, bool HAS_SCALE>
__device__ __forceinline__ uint8_t quant1(uint16_t h, float s) {
  return (uint8_t)(enc2(scaled<HAS_SCALE>(widen<DT>(h), s), 0.0f) & 0xFF);
}

// Contiguous tensor viewed as n elements; vector part in chunks of 8.
template <int DT, bool HAS_SCALE>
__global__ __launch_bounds__(256) void quantize_flat_kernel(const uint16_t *__restrict__ x,
                                                             uint8_t *__restrict__ out, int64_t n,
                                                             float s) {
  const int64_t nvec = n >> 3;
  const v4u *xv = reinterpret_cast<const v4u *>(x);
  v2u *ov = reinterpret_cast<v2u *>(out);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // two independent 16-byte loads in flight per thread
  for (; i + stride < nvec; i += 2 * stride) {
    v4u a = __builtin_nontemporal_load(xv + i);
    v4u b = __builtin_nontemporal_load(xv + i + stride);
    __builtin_nontemporal_store(quant8<DT, HAS_SCALE>(a, s), ov + i);
    __builtin_nontemporal_store(quant8<DT, HAS_SCALE>(b, s), ov + i + stride);
  }
  if (i < nvec) ov[i] = quant8<DT, HAS_SCALE>(xv[i], s);
  // ragged tail (< 8 elements), handled by the first threads of the grid
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t e = (nvec << 3) + t;
  if (t < 8 && e < n) out[e] = quant1<DT, HAS_SCALE>(x[e], s);
}

// Two contiguous tensors of one dtype, each with its own scale, in one launch:
// chunk i < c0 belongs to the first, the rest to the second (a wave straddles
// the boundary at most once).  Same codes as two quantize_flat_kernel launches.
template <int DT, bool H0, bool H1>
__global__ __launch_bounds__(256) void quantize_pair_kernel(const uint16_t *__restrict__ x0,
                                                             uint8_t *__restrict__ o0, int64_t c0, float s0,
                                                             const uint16_t *__restrict__ x1,
                                                             uint8_t *__restrict__ o1, int64_t c1, float s1) {
  const v4u *xv0 = reinterpret_cast<const v4u *>(x0);
  const v4u *xv1 = reinterpret_cast<const v4u *>(x1);
  v2u *ov0 = reinterpret_cast<v2u *>(o0);
  v2u *ov1 = reinterpret_cast<v2u *>(o1);
  const int64_t total = c0 + c1;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += 2 * stride) {
    // two independent 16-byte loads in flight per thread
    const int64_t j = i + stride;
    const bool has_j = j < total;
    const v4u a = __builtin_nontemporal_load(i < c0 ? xv0 + i : xv1 + (i - c0));
    v4u b = {0u, 0u, 0u, 0u};
    if (has_j) b = __builtin_nontemporal_load(j < c0 ? xv0 + j : xv1 + (j - c0));
    if (i < c0) {
      __builtin_nontemporal_store(quant8<DT, H0>(a, s0), ov0 + i);
    } else {
      __builtin_nontemporal_store(quant8<DT, H1>(a, s1), ov1 + (i - c0));
    }
    if (has_j) {
      if (j < c0) {
        __builtin_nontemporal_store(quant8<DT, H0>(b, s0), ov0 + j);
      } else {
        __builtin_nontemporal_store(quant8<DT, H1>(b, s1), ov1 + (j - c0));
      }
    }
  }
}

template <int DT, bool H0, bool H1>
int launch_pair_typed(const uint16_t *x0, uint8_t *o0, int64_t c0, float s0, const uint16_t *x1, uint8_t *o1,
                      int64_t c1, float s1, hipStream_t stream) {
  int64_t blocks = (c0 + c1 + 255) / 256;
  blocks = blocks > 2048 ? (blocks + 1) / 2 : blocks;   // as the single-tensor launch
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((quantize_pair_kernel<DT, H0, H1>), dim3((unsigned)blocks), dim3(256), 0, stream, x0, o0, c0,
                     s0, x1, o1, c1, s1);
  return check_launch("fp8_quantize_pair");
}

template <int DT>
int launch_pair_dt(const uint16_t *x0, uint8_t *o0, int64_t c0, bool h0, float s0, const uint16_t *x1,
                   uint8_t *o1, int64_t c1, bool h1, float s1, hipStream_t stream) {
  if (h0) {
    return h1 ? launch_pair_typed<DT, true, true>(x0, o0, c0, s0, x1, o1, c1, s1, stream)
              : launch_pair_typed<DT, true, false>(x0, o0, c0, s0, x1, o1, c1, s1, stream);
  }
  return h1 ? launch_pair_typed<DT, false, true>(x0, o0, c0, s0, x1, o1, c1, s1, stream)
            : launch_pair_typed<DT, false, false>(x0, o0, c0, s0, x1, o1, c1, s1, stream);
}

// Row-strided 2-D view.  VEC: cols, both strides and both base pointers allow
// 8-element vectors.  grid.x walks column chunks, grid.y walks rows.
template <int DT, bool HAS_SCALE, bool VEC>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t *__restrict__ x,
                                                             uint8_t *__restrict__ out,
                                                             int64_t rows, int64_t cols,
                                                             int64_t xs, int64_t os, float s) {
  const int64_t per = VEC ? 8 : 1;
  const int64_t nchunk = (cols + per - 1) / per;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const uint16_t *xr = x + r * xs;
    uint8_t *orow = out + r * os;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunk;
         c += (int64_t)gridDim.x * blockDim.x) {
      if constexpr (VEC) {
        v4u w = *reinterpret_cast<const v4u *>(xr + c * 8);
        *reinterpret_cast<v2u *>(orow + c * 8) = quant8<DT, HAS_SCALE>(w, s);
      } else {
        orow[c] = quant1<DT, HAS_SCALE>(xr[c], s);
      }
    }
  }
}

template <int DT, bool HAS_SCALE>
int launch_typed(const uint16_t *x, int64_t rows, int64_t cols, int64_t xs, uint8_t *out,
                 int64_t os, float s, hipStream_t stream) {
  const bool contiguous = (xs == cols) && (os == cols);
  const bool aligned = ((uintptr_t)x % 16 == 0) && ((uintptr_t)out % 8 == 0);
  if (contiguous && aligned) {
    const int64_t n = rows * cols;
    const int64_t nvec = n >> 3;
    int64_t blocks = (nvec + 255) / 256;
    // enough waves to saturate HBM: 256 CUs x 8 workgroups, each thread two chunks
    blocks = blocks > 2048 ? (blocks + 1) / 2 : blocks;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL((quantize_flat_kernel<DT, HAS_SCALE>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, x, out, n, s);
    return check_launch("fp8_quantize");
  }
  const bool vec = (cols % 8 == 0) && (xs % 8 == 0) && (os % 8 == 0) &&
                   ((uintptr_t)x % 16 == 0) && ((uintptr_t)out % 8 == 0);
  const int64_t per = vec ? 8 : 1;
  const int64_t nchunk = (cols + per - 1) / per;
  int64_t gx = (nchunk + 255) / 256;
  if (gx > 1024) gx = 1024;
  int64_t gy = rows < 65535 ? rows : 65535;
  if (vec) {
    hipLaunchKernelGGL((quantize_rows_kernel<DT, HAS_SCALE, true>), dim3((unsigned)gx, (unsigned)gy),
                       dim3(256), 0, stream, x, out, rows, cols, xs, os, s);
  } else {
    hipLaunchKernelGGL((quantize_rows_kernel<DT, HAS_SCALE, false>), dim3((unsigned)gx, (unsigned)gy),
                       dim3(256), 0, stream, x, out, rows, cols, xs, os, s);
  }
  return check_launch("fp8_quantize");
}

// ---- paged cache store: quantize token rows and scatter them by slot.
//
// Token n, head h, element c of x (and c of x2, placed after x in the row)
// goes to cache[page][h][off][c] with page = slot / page_size and
// off = slot % page_size; slots < 0 or >= num_slots write nothing.  The
// pool stores value / scale like the queries (sglang PR 30971 digest,
// implementation step 4); the two-source row is the MLA latent + rope pack
// (sglang PR 25460 digest, implementation step 2).
//
// HBM-bound: 2 + 1 bytes per element plus one 8-byte slot per token.  One
// thread per 8-element chunk of a (token, head) row; a row's chunks are
// adjacent threads, so each cache row is written as one contiguous run.
// Index arithmetic is 32-bit (the host keeps chunk and slot counts below
// 2^31); only byte offsets into the cache are formed in 64 bits.  Each thread
// takes two chunks and issues both source loads before it reads either slot:
// the source address does not depend on the slot, so the two loads and the
// slot reads are all in flight together.
template <int DT, bool HAS_SCALE, bool VEC>
__global__ __launch_bounds__(256) void cache_store_kernel(StoreArgs a, float s) {
  constexpr uint32_t per = VEC ? 8 : 1;
  const uint32_t c1 = (uint32_t)a.dim / per;
  const uint32_t cpr = c1 + (uint32_t)a.dim2 / per;
  const uint32_t total = (uint32_t)a.num_tokens * (uint32_t)a.heads * cpr;
  const uint32_t stride = gridDim.x * blockDim.x;
  const int64_t row = a.dim + a.dim2;
  for (uint32_t g0 = blockIdx.x * blockDim.x + threadIdx.x; g0 < total; g0 += 2 * stride) {
    bool live[2];
    uint32_t n[2], h[2], col[2];
    v4u w[2];
    uint16_t e[2];
    int64_t slot[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      live[k] = k == 0 || g0 + stride < total;
      const uint32_t g = live[k] ? g0 + k * stride : g0;   // a dead second chunk re-reads the first, never stored
      const uint32_t r = g / cpr;
      const uint32_t c = g - r * cpr;
      n[k] = r / (uint32_t)a.heads;
      h[k] = r - n[k] * (uint32_t)a.heads;
      const uint16_t *src;
      if (c < c1) {
        src = a.x + (int64_t)n[k] * a.x_ts + (int64_t)h[k] * a.x_hs + c * per;
        col[k] = c * per;
      } else {
        src = a.x2 + (int64_t)n[k] * a.x2_ts + (int64_t)h[k] * a.x2_hs + (c - c1) * per;
        col[k] = a.dim + (c - c1) * per;
      }
      if constexpr (VEC) {
        w[k] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(src));
      } else {
        e[k] = *src;
      }
      slot[k] = a.slots[n[k]];
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (!live[k] || slot[k] < 0 || slot[k] >= a.num_slots) continue;
      const uint32_t page = (uint32_t)slot[k] / (uint32_t)a.page_size;
      const uint32_t off = (uint32_t)slot[k] - page * (uint32_t)a.page_size;
      uint8_t *dst = a.cache + (((int64_t)page * a.heads + h[k]) * a.page_size + off) * row + col[k];
      if constexpr (VEC) {
        *reinterpret_cast<v2u *>(dst) = quant8<DT, HAS_SCALE>(w[k], s);
      } else {
        *dst = quant1<DT, HAS_SCALE>(e[k], s);
      }
    }
  }
}

template <int DT, bool HAS_SCALE>
int launch_store_typed(const StoreArgs &a, float s, hipStream_t stream) {
  const bool vec = a.dim % 8 == 0 && a.dim2 % 8 == 0 && a.x_ts % 8 == 0 && a.x_hs % 8 == 0 &&
                   (uintptr_t)a.x % 16 == 0 && (uintptr_t)a.cache % 8 == 0 &&
                   (a.dim2 == 0 || (a.x2_ts % 8 == 0 && a.x2_hs % 8 == 0 && (uintptr_t)a.x2 % 16 == 0));
  const int64_t per = vec ? 8 : 1;
  const int64_t total = a.num_tokens * a.heads * ((a.dim + a.dim2) / per);
  int64_t blocks = (total + 511) / 512;      // two chunks per thread
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (vec) {
    hipLaunchKernelGGL((cache_store_kernel<DT, HAS_SCALE, true>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a, s);
  } else {
    hipLaunchKernelGGL((cache_store_kernel<DT, HAS_SCALE, false>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a, s);
  }
  return check_launch("fp8_cache_store");
}

// ---- RoPE fused with quantization.
//
// Row (n, h) of the output = e4m3(x_nope[n, h, :]) ++ e4m3(rope(x_pe[n, h, :]))
// with the rotary embedding of RoFormer at position positions[n]: the rope
// dims form pairs (a, b) -> (a cos - b sin, b cos + a sin), pairing dim i with
// i + R/2 (rotate-half, is_neox) or dims 2i and 2i+1 (interleaved); pair i
// reads cos_sin_cache[p][i] and cos_sin_cache[p][R/2 + i].  This is the
// fused rope + quantize producer of the MLA prefill hook (sglang PR 25460
// digest, implementation step 2 and the _fused_rope_fp8_quantize excerpt),
// with the quantize step's scale convention.  The rotation is plain fp32
// with each product rounded on its own (no fused multiply-add), so every
// code is decided by the same operations whatever the compiler schedules.
// A position outside [0, max_position) writes 0x7F (NaN) over the rope part.
//
// HBM-bound: 2 + 1 bytes per element (the cos/sin rows of a token are read
// once per head from cache).  One thread per 8-element output chunk.
template <bool NEOX>
__device__ __forceinline__ void rope8(const float *x, const float *p, const float *c,
                                      const float *sn, bool first_half, float *o) {
#pragma clang fp contract(off)
  if constexpr (NEOX) {
    // x: 8 consecutive dims of one half, p: the partner dims of the other half
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xc = x[e] * c[e];
      const float ps = p[e] * sn[e];
      o[e] = first_half ? xc - ps : xc + ps;
    }
  } else {
    // x: 4 interleaved pairs; c, sn: their 4 angles
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = x[2 * e], b = x[2 * e + 1];
      const float ac = a * c[e], bs = b * sn[e], bc = b * c[e], as = a * sn[e];
      o[2 * e] = ac - bs;
      o[2 * e + 1] = bc + as;
    }
  }
}

template <int DT>
__device__ __forceinline__ void widen8(v4u w, float *f) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = widen<DT>(w[j] & 0xFFFF);
    f[2 * j + 1] = widen<DT>(w[j] >> 16);
  }
}

template <bool HAS_SCALE>
__device__ __forceinline__ v2u encode8(const float *f, float s) {
  uint32_t o[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    o[j] = enc2(scaled<HAS_SCALE>(f[4 * j], s), scaled<HAS_SCALE>(f[4 * j + 1], s)) |
           (enc2(scaled<HAS_SCALE>(f[4 * j + 2], s), scaled<HAS_SCALE>(f[4 * j + 3], s)) << 16);
  }
  return (v2u){o[0], o[1]};
}

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, const FastDiv &f) {
  const uint32_t t = __umulhi(n, f.m);
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

template <int DT, bool HAS_SCALE, bool NEOX>
__global__ __launch_bounds__(256) void rope_quantize_kernel(RopeArgs a, float s) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  // Workgroup w takes rows [w R, w R + R) (row = token x head).  Its chunk
  // index space holds first the no-rope chunks of its rows (R x c1), then
  // their rope chunks (R x c2), so a wave runs one of the two paths (a
  // 576-wide row has 64 + 8 chunks; mixing them in one wave would pay for
  // both), and every workgroup carries its share of the rope chunks, whose
  // position and cos/sin loads then overlap other workgroups' streaming
  // instead of forming the tail of the grid.
  const uint32_t c1 = (uint32_t)a.nope / 8;
  const uint32_t c2 = (uint32_t)a.rope / 8;
  const uint32_t rows = (uint32_t)a.num_tokens * (uint32_t)a.heads;
  const uint32_t r0 = blockIdx.x * (uint32_t)a.rows_per_wg;
  const uint32_t nr = min((uint32_t)a.rows_per_wg, rows - r0);
  const uint32_t total_a = nr * c1;
  const uint32_t total = total_a + nr * c2;
  const uint32_t half = (uint32_t)a.rope / 2;
  const uint32_t stride = blockDim.x;
  // Two chunks per thread.  Source loads (and the rotate-half partner) do not
  // depend on the position, so they are issued first; only the cos/sin rows
  // wait for it.
  for (uint32_t g0 = threadIdx.x; g0 < total; g0 += 2 * stride) {
    bool live[2], rope[2];
    uint32_t n[2], j0[2];
    uint8_t *dst[2];
    v4u w[2], pw[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      live[k] = k == 0 || g0 + stride < total;
      const uint32_t g = live[k] ? g0 + k * stride : g0;   // a dead second chunk re-reads the first, never stored
      rope[k] = g >= total_a;
      const uint32_t gi = rope[k] ? g - total_a : g;
      const uint32_t cw = rope[k] ? c2 : c1;
      const uint32_t r = r0 + fastdiv(gi, rope[k] ? a.div_rope : a.div_nope);
      const uint32_t c = gi - (r - r0) * cw;
      n[k] = fastdiv(r, a.div_heads);
      const uint32_t h = r - n[k] * (uint32_t)a.heads;
      dst[k] = a.out + (int64_t)n[k] * a.out_ts + (int64_t)h * a.out_hs + (rope[k] ? a.nope : 0) + c * 8;
      j0[k] = c * 8;
      const uint16_t *pe = a.x_pe + (int64_t)n[k] * a.pe_ts + (int64_t)h * a.pe_hs;
      const uint16_t *src = rope[k] ? pe + j0[k] : a.x_nope + (int64_t)n[k] * a.nope_ts + (int64_t)h * a.nope_hs + j0[k];
      w[k] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(src));
      if (NEOX && rope[k]) {
        pw[k] = *reinterpret_cast<const v4u *>(pe + (j0[k] < half ? j0[k] + half : j0[k] - half));
      } else {
        pw[k] = w[k];
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (!live[k]) continue;
      if (!rope[k]) {
        *reinterpret_cast<v2u *>(dst[k]) = quant8<DT, HAS_SCALE>(w[k], s);
        continue;
      }
      const int64_t pos = a.positions[n[k]];
      if (pos < 0 || pos >= a.max_position) {
        *reinterpret_cast<v2u *>(dst[k]) = (v2u){0x7F7F7F7Fu, 0x7F7F7F7Fu};
        continue;
      }
      const float *cs = a.cos_sin + pos * a.rope;
      float x[8], o[8];
      widen8<DT>(w[k], x);
      if constexpr (NEOX) {
        const bool first = j0[k] < half;
        const uint32_t i0 = first ? j0[k] : j0[k] - half;   // angle index of the chunk's first dim
        float p[8], cv[8], sv[8];
        widen8<DT>(pw[k], p);
        const v4f ca = *reinterpret_cast<const v4f *>(cs + i0), cb = *reinterpret_cast<const v4f *>(cs + i0 + 4);
        const v4f sa = *reinterpret_cast<const v4f *>(cs + half + i0),
                  sb = *reinterpret_cast<const v4f *>(cs + half + i0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          cv[e] = ca[e];
          cv[e + 4] = cb[e];
          sv[e] = sa[e];
          sv[e + 4] = sb[e];
        }
        rope8<true>(x, p, cv, sv, first, o);
      } else {
        const uint32_t i0 = j0[k] / 2;
        const v4f ca = *reinterpret_cast<const v4f *>(cs + i0);
        const v4f sa = *reinterpret_cast<const v4f *>(cs + half + i0);
        float cv[4] = {ca[0], ca[1], ca[2], ca[3]}, sv[4] = {sa[0], sa[1], sa[2], sa[3]};
        rope8<false>(x, nullptr, cv, sv, false, o);
      }
      *reinterpret_cast<v2u *>(dst[k]) = encode8<HAS_SCALE>(o, s);
    }
  }
}

template <int DT, bool HAS_SCALE>
int launch_rope_typed(const RopeArgs &args, float s, hipStream_t stream) {
  RopeArgs a = args;
  a.div_nope = make_fastdiv(a.nope >= 8 ? (uint32_t)a.nope / 8 : 1u);
  a.div_rope = make_fastdiv((uint32_t)a.rope / 8);
  a.div_heads = make_fastdiv((uint32_t)a.heads);
  // about 2048 chunks (eight per thread) per workgroup
  const int64_t rows = a.num_tokens * a.heads;
  a.rows_per_wg = (int32_t)std::max<int64_t>(1, 2048 / ((a.nope + a.rope) / 8));
  const int64_t blocks = (rows + a.rows_per_wg - 1) / a.rows_per_wg;
  if (a.neox) {
    hipLaunchKernelGGL((rope_quantize_kernel<DT, HAS_SCALE, true>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a, s);
  } else {
    hipLaunchKernelGGL((rope_quantize_kernel<DT, HAS_SCALE, false>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a, s);
  }
  return check_launch("fp8_rope_quantize");
}

// Per-head RMS norm + RoPE + e4m3 (+ paged store) of index q / k rows.
// One group of `lpr` lanes per (token, head) row, 8 consecutive dims per lane
// (lpr = dim / 8 rounded up to a power of two, so a 128-dim row takes 16
// lanes and a wave holds four rows; dim <= 512).  Reductions and partner
// shuffles stay inside a group.
// The squares are summed in fp64, where each is exact, so the normaliser does
// not depend on the reduction order; r = fl32(1 / sqrt(ss / dim + eps)) in
// fp64; y = fl32(fl32(x r) w); then the rope_quantize rotation and encode.
// A rotate-half partner lives in another lane and comes by shuffle.
template <int DT, bool HAS_SCALE, bool NEOX>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(NormRopeArgs a, float s) {
#pragma clang fp contract(off)
  typedef float v4f __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int lpr = a.lanes_per_row;
  const int gl = lane & (lpr - 1);                       // lane within the row's group
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / lpr);   // the wave's first row
  const int64_t rows = a.num_tokens * a.heads;
  if (row0 >= rows) return;                              // whole wave
  const int64_t row = row0 + lane / lpr;
  const bool live = row < rows;
  const int64_t n = live ? row / a.heads : 0;
  const int h = live ? (int)(row - n * a.heads) : 0;
  const int j0 = 8 * gl;
  const bool act = live && j0 < a.dim;
  v4u w = {0u, 0u, 0u, 0u};
  if (act) w = *reinterpret_cast<const v4u *>(a.x + n * a.x_ts + (int64_t)h * a.x_hs + j0);
  // the position and its cos/sin rows do not depend on x: load them now, so
  // their two dependent round trips overlap the row's load and reduction
  const int nope = a.dim - a.rope, half = a.rope / 2;
  const bool rope = act && j0 >= nope;
  const bool first = j0 - nope < half;
  const int jr = j0 - nope;
  const int i0 = NEOX ? (first ? jr : jr - half) : jr / 2;
  bool pos_ok = false;
  v4f ca = {0.f, 0.f, 0.f, 0.f}, cb = ca, sa = ca, sb = ca;
  if (rope) {
    const int64_t pos = a.positions[n];
    pos_ok = pos >= 0 && pos < a.max_position;
    if (pos_ok) {
      const float *cs = a.cos_sin + pos * a.rope;
      ca = *reinterpret_cast<const v4f *>(cs + i0);
      sa = *reinterpret_cast<const v4f *>(cs + half + i0);
      if (NEOX) {
        cb = *reinterpret_cast<const v4f *>(cs + i0 + 4);
        sb = *reinterpret_cast<const v4f *>(cs + half + i0 + 4);
      }
    }
  }
  float x[8];
  widen8<DT>(w, x);
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += (double)x[e] * (double)x[e];
#pragma unroll
  for (int m = lpr >> 1; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  const double den = sqrt(ss / (double)a.dim + (double)a.eps);
  const float r = (float)(1.0 / den);
  float y[8];
  if (act) {
    const v4f w0 = *reinterpret_cast<const v4f *>(a.weight + j0);
    const v4f w1 = *reinterpret_cast<const v4f *>(a.weight + j0 + 4);
    const float wt[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (x[e] * r) * wt[e];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = 0.f;
  }
  float p[8];
  if constexpr (NEOX) {
    // every lane takes part in the shuffles; only rope lanes use the result
    const int src = rope ? (first ? lane + half / 8 : lane - half / 8) : lane;   // same group
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = __shfl(y[e], src);
  }
  if (!act) return;
  v2u code;
  if (!rope) {
    code = encode8<HAS_SCALE>(y, s);
  } else if (!pos_ok) {
    code = (v2u){0x7F7F7F7Fu, 0x7F7F7F7Fu};
  } else {
    float o[8];
    if constexpr (NEOX) {
      const float cv[8] = {ca[0], ca[1], ca[2], ca[3], cb[0], cb[1], cb[2], cb[3]};
      const float sv[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
      rope8<true>(y, p, cv, sv, first, o);
    } else {
      const float cv[4] = {ca[0], ca[1], ca[2], ca[3]}, sv[4] = {sa[0], sa[1], sa[2], sa[3]};
      rope8<false>(y, nullptr, cv, sv, false, o);
    }
    code = encode8<HAS_SCALE>(o, s);
  }
  if (a.out) *reinterpret_cast<v2u *>(a.out + n * a.out_ts + (int64_t)h * a.out_hs + j0) = code;
  if (a.slot_mapping) {
    const int64_t slot = a.slot_mapping[n];
    if (slot >= 0 && slot < a.num_slots) {
      const int64_t pg = slot / a.page_size, off = slot - pg * a.page_size;
      *reinterpret_cast<v2u *>(a.cache + ((pg * a.heads + h) * a.page_size + off) * a.dim + j0) = code;
    }
  }
}

template <int DT, bool HAS_SCALE>
int launch_qknorm_typed(const NormRopeArgs &a, float s, hipStream_t stream) {
  const int64_t per_block = 4 * (64 / a.lanes_per_row);     // rows per 256-thread block
  const int64_t blocks = (a.num_tokens * a.heads + per_block - 1) / per_block;
  if (a.neox) {
    hipLaunchKernelGGL((qknorm_rope_kernel<DT, HAS_SCALE, true>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       a, s);
  } else {
    hipLaunchKernelGGL((qknorm_rope_kernel<DT, HAS_SCALE, false>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       a, s);
  }
  return check_launch("fp8_qknorm_rope_quantize");
}

}  // namespace

int launch_rope_quantize(const RopeArgs &a, int dtype, bool has_scale, float scale_inv,
                         hipStream_t stream) {
  if (dtype == FP8TS_BF16) {
    return has_scale ? launch_rope_typed<FP8TS_BF16, true>(a, scale_inv, stream)
                     : launch_rope_typed<FP8TS_BF16, false>(a, 1.0f, stream);
  }
  return has_scale ? launch_rope_typed<FP8TS_FP16, true>(a, scale_inv, stream)
                   : launch_rope_typed<FP8TS_FP16, false>(a, 1.0f, stream);
}

int launch_qknorm_rope_quantize(const NormRopeArgs &a, int dtype, bool has_scale, float scale_inv,
                                hipStream_t stream) {
  if (dtype == FP8TS_BF16) {
    return has_scale ? launch_qknorm_typed<FP8TS_BF16, true>(a, scale_inv, stream)
                     : launch_qknorm_typed<FP8TS_BF16, false>(a, 1.0f, stream);
  }
  return has_scale ? launch_qknorm_typed<FP8TS_FP16, true>(a, scale_inv, stream)
                   : launch_qknorm_typed<FP8TS_FP16, false>(a, 1.0f, stream);
}

int launch_cache_store(const StoreArgs &a, int dtype, bool has_scale, float scale_inv,
                       hipStream_t stream) {
  if (dtype == FP8TS_BF16) {
    return has_scale ? launch_store_typed<FP8TS_BF16, true>(a, scale_inv, stream)
                     : launch_store_typed<FP8TS_BF16, false>(a, 1.0f, stream);
  }
  return has_scale ? launch_store_typed<FP8TS_FP16, true>(a, scale_inv, stream)
                   : launch_store_typed<FP8TS_FP16, false>(a, 1.0f, stream);
}

int launch_quantize_pair(const void *x0, uint8_t *out0, int64_t n0, bool has0, float inv0, const void *x1,
                         uint8_t *out1, int64_t n1, bool has1, float inv1, int dtype, hipStream_t stream) {
  const uint16_t *a = static_cast<const uint16_t *>(x0), *b = static_cast<const uint16_t *>(x1);
  if (dtype == FP8TS_BF16)
    return launch_pair_dt<FP8TS_BF16>(a, out0, n0 / 8, has0, inv0, b, out1, n1 / 8, has1, inv1, stream);
  return launch_pair_dt<FP8TS_FP16>(a, out0, n0 / 8, has0, inv0, b, out1, n1 / 8, has1, inv1, stream);
}

int launch_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int64_t x_stride,
                    uint8_t *out, int64_t out_stride, bool has_scale, float scale_inv,
                    hipStream_t stream) {
  const uint16_t *xp = static_cast<const uint16_t *>(x);
  if (dtype == FP8TS_BF16) {
    return has_scale ? launch_typed<FP8TS_BF16, true>(xp, rows, cols, x_stride, out, out_stride, scale_inv, stream)
                     : launch_typed<FP8TS_BF16, false>(xp, rows, cols, x_stride, out, out_stride, 1.0f, stream);
  }
  return has_scale ? launch_typed<FP8TS_FP16, true>(xp, rows, cols, x_stride, out, out_stride, scale_inv, stream)
                   : launch_typed<FP8TS_FP16, false>(xp, rows, cols, x_stride, out, out_stride, 1.0f, stream);
}

}  // namespace fp8ts
