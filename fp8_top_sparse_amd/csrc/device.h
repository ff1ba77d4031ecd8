// Device-side building blocks for gfx950 (CDNA4): MFMA wrappers, fp8/bf16
// conversions and wave64 helpers.  Everything here is written for 64-lane
// wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8ts {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- ids and workgroup votes
// Workgroup and thread index (x dimension) read from the registers the
// hardware loads at wave launch.  blockIdx / threadIdx and the
// __syncthreads_or/_count votes are device-library functions; the inliner
// leaves them out of very large kernels (it caps a function's basic-block
// count), and the result of a call is then taken to differ between lanes:
// every index derived from the workgroup id lands in vector registers, and a
// buffer resource built from one is rebuilt in a loop over the lanes' values
// around each load.
__device__ __forceinline__ int block_index() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int thread_index() { return (int)__builtin_amdgcn_workitem_id_x(); }

// Number of threads of the workgroup (WAVES waves of 64) whose predicate
// holds.  Every thread must call it; it is a workgroup barrier, and its
// result is the same in every thread.
template <int WAVES>
__device__ __forceinline__ int wg_count(bool p) {
  __shared__ int wave_count[WAVES];
  // the ballot needs every lane active: take it before the lane-0 branch
  const int n_wave = __builtin_popcountll(__builtin_amdgcn_ballot_w64(p));
  __syncthreads();   // readers of an earlier vote are done with wave_count
  if ((thread_index() & 63) == 0) wave_count[thread_index() >> 6] = n_wave;
  __syncthreads();
  int n = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) n += wave_count[w];
  return n;
}

// Whether the predicate holds in any thread of the workgroup (as wg_count).
template <int WAVES>
__device__ __forceinline__ bool wg_or(bool p) {
  return wg_count<WAVES>(p) != 0;
}

// ---------------------------------------------------------------- MFMA
// Operand layout used throughout (16x16 output tiles, wave64):
//   A (16 x K): lane l holds row (l % 16), K-slice (l / 16)
//   B (K x 16): lane l holds column (l % 16), the same K-slice (l / 16)
//   D (16 x 16): lane l, register i holds row 4 * (l / 16) + i, column l % 16
// The contraction index is permuted identically in A and B, so any consistent
// assignment of K elements to (lane group, byte) is a valid operand layout.

// D += A(16x128, e4m3) * B(128x16, e4m3); lane K-slice = 32 bytes.
// cbsz = blgp = 0 selects OCP e4m3 for both operands; E8M0 scales 127 = 1.0.
__device__ __forceinline__ v4f mfma_16x16x128_e4m3(const v8i &a, const v8i &b, const v4f &c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// D += A(16x32, e4m3) * B(32x16, e4m3); lane K-slice = 8 bytes.
__device__ __forceinline__ v4f mfma_16x16x32_e4m3(long a, long b, const v4f &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

// D += A(16x32, bf16) * B(32x16, bf16); lane K-slice = 8 bf16.
__device__ __forceinline__ v4f mfma_16x16x32_bf16(const v8bf &a, const v8bf &b, const v4f &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- conversions
// Two e4m3 bytes of `packed` (selected half: hi = bytes 2,3) -> two floats, exact.
__device__ __forceinline__ v2f e4m3x2_to_f32(int packed, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_fp8(packed, true)
            : __builtin_amdgcn_cvt_pk_f32_fp8(packed, false);
}

// Four e4m3 bytes -> four bf16 (exact: every e4m3 value is a bf16 value).
__device__ __forceinline__ v4bf e4m3x4_to_bf16(int packed) {
  v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(packed, false);
  v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(packed, true);
  v4bf r;
  r[0] = (__bf16)lo[0];
  r[1] = (__bf16)lo[1];
  r[2] = (__bf16)hi[0];
  r[3] = (__bf16)hi[1];
  return r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  v2bf r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------- wave64
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Butterfly over lanes l ^ mask (mask < 64) via ds_bpermute (no LDS storage used).
__device__ __forceinline__ float shfl_xor_f32(float v, int mask) {
  int src = (lane_id() ^ mask) << 2;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, v)));
}

// Max / sum over the four lane groups (l, l^16, l^32, l^48) that hold the same
// MFMA column.
__device__ __forceinline__ float group4_max(float v) {
  v = fmaxf(v, shfl_xor_f32(v, 16));
  v = fmaxf(v, shfl_xor_f32(v, 32));
  return v;
}
__device__ __forceinline__ float group4_sum(float v) {
  v += shfl_xor_f32(v, 16);
  v += shfl_xor_f32(v, 32);
  return v;
}

// Max over the four lane groups (l, l ^ 16, l ^ 32, l ^ 48) holding one MFMA
// column, with gfx950 row-swap permutes instead of LDS-routed shuffles.  The
// swaps are written as asm (with the two wait states they need on either
// side) so that the compiler cannot merge the two halves of a swap.
__device__ __forceinline__ float group4_max_swap(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  v = fmaxf(a, b);
  a = v;
  b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

// Workgroup barrier that orders LDS accesses only.  Unlike __syncthreads it
// does not wait for outstanding global loads, so a tile prefetch issued before
// it stays in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Operand order for a 128-key x 128-byte e4m3 tile in LDS: the 16x16x128 A
// operand (kt, hh) of lane l sits at 1024 * (2 * kt + hh) + 16 * l and holds
// key 16 kt + (l & 15), bytes 32 (l >> 4) + 16 hh .. + 15, so every operand
// fetch is one contiguous 1 KB wave read.  Staging chunk ch (0..1023, 16
// bytes) maps to (key, part) so that wave-instruction q = ch >> 6 covers
// bytes 64 (q & 1) .. + 63 of keys 16 (q >> 1) .. + 15: its 16-lane write
// groups land on 16 distinct bank groups.
__device__ __forceinline__ int k_chunk_key(int ch) { return 16 * (ch >> 7) + (ch & 15); }
__device__ __forceinline__ int k_chunk_part(int ch) { return 4 * ((ch >> 6) & 1) + ((ch >> 4) & 3); }

// Two 16-byte reads 1 KB apart (the two halves of a 32-byte K operand).
__device__ __forceinline__ v8i lds_read32x2(const uint8_t *p) {
  const v4i lo = *reinterpret_cast<const v4i *>(p);
  const v4i hi = *reinterpret_cast<const v4i *>(p + 1024);
  return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ int k_tile_offset(int key, int part) {
  return 1024 * (2 * (key >> 4) + (part & 1)) + 16 * (16 * (part >> 1) + (key & 15));
}

// Raw buffer resource over one 16 KB tile of 128 rows x 128 bytes (dword 3:
// 32-bit data format); reads past the tile return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_tile_rsrc(const uint8_t *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), (short)0, 128 * 128, 0x00020000);
}

}  // namespace fp8ts
