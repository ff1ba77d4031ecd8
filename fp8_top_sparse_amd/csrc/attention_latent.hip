// Token-sparse MLA prefill attention over the latent cache layout: every
// 576-byte e4m3 K row holds the row's V in its leading 512 bytes (the caller
// passes no separate V).  The kernel behind sparse_attn_fwd in token mode for
// q heads in groups of 128 when V is the leading part of K.
//
// Semantics: sglang PR 25751 digest, code excerpt of
// sparse_mla_q8kv8_prefill_fwd (each query token attends to the KV rows its
// index list names; V is the first 512 columns of the 576-wide latent rows;
// out bf16 [s_q, h_q, 512], max_logits and lse fp32 [s_q, h_q], optional
// attn_sink and topk_length), with the scale handling of sglang PR 30971
// digest, implementation step 3.
//
// Workgroup: one query token x 128 q heads, 8 waves x 16 heads, 128 keys per
// tile.  Only the K rows are staged: buffer-to-LDS DMA puts each tile's rows
// in QK operand order, and the PV operands are read out of the same bytes.
//  * S^T = K Q^T + C on 16x16x128 e4m3 MFMA (+ two 16x16x32 for the last
//    64 bytes), one 64-key half of the tile at a time; C holds minus the
//    row's reference maximum.
//  * P = exp2(ck S - e) with one power-of-two exponent e per row and half
//    (the half's row maximum lands in [2^7, 2^8)), split into two e4m3 codes,
//    hi = e4m3(P) and lo = e4m3(P - hi).  hi + lo carries P to about 2^-8
//    relative, finer than a bf16 P.
//  * O^T += V^T (hi + lo)^T as two scaled 16x16x128 e4m3 MFMAs sharing one
//    V^T operand: the B operand's E8M0 scale (127 + e) restores 2^e, V is
//    used as stored (e4m3, exact), so nothing is widened or rewritten.
//  * The V^T operand comes straight from the staged K rows through the gfx950
//    transposing LDS read (ds_read_b64_tr_b8: in a 16-lane group, byte j of
//    lane i is byte i mod 8 of the 8-byte row addressed by lane 2j + i/8).
//    Odd 16-key blocks sit 128 bytes further (mod 256) in LDS, so the 32
//    lanes of each half-wave read distinct banks.
#include "attn_common.h"

namespace fp8ts {
namespace {

constexpr int kDqk = 576, kDv = 512;
constexpr int kKT = 128;                         // keys per tile
constexpr int kNkb = kKT / 16;                   // 16-key blocks per tile
constexpr int kNkc = 4;                          // 128-byte slices of the first 512 bytes
constexpr int kNdt = kDv / 16;                   // 16-dim output tiles
constexpr int kWaves = 8, kThreads = 512;        // 16 q heads per wave
constexpr int kRowsPerWg = 16 * kWaves;
static_assert(kWaves == kNkb, "wave w stages key block w");
// LDS tile (one of two buffers):
//   main: key block kb at kKbStride kb; its operand (kc, hh) of lane l at
//         + 1024 (2 kc + hh) + 16 l: key 16 kb + (l & 15), bytes
//         128 kc + 32 (l >> 4) + 16 hh .. + 15.  Byte d of key 16 kb + r
//         therefore sits at kKbStride kb + 1024 (2 (d / 128) + (d / 16) % 2)
//         + 16 (16 ((d % 128) / 32) + r) + d % 16.
//   tail: at kMain + 1024 kb + 16 l: key 16 kb + (l & 15), bytes
//         512 + 16 (l >> 4) .. + 15.
constexpr int kKbStride = 8 * 1024 + 128;        // 128 B mod 256 between neighbouring blocks
constexpr int kMain = kNkb * kKbStride;
constexpr int kTileBytes = kMain + kNkb * 1024;
constexpr int kIdxOff = 2 * kTileBytes;          // the split's index list (int32)
// Output staging at the end (over the tile buffers): 16 bf16 rows of 1 KB per
// wave; the 32-byte pitch step puts the 16 rows of each 8-byte write on
// different banks.
constexpr int kOutPitch = kDv * 2 + 32;
static_assert(kWaves * 16 * kOutPitch <= 2 * kTileBytes, "output staging fits the tile buffers");

typedef __attribute__((address_space(3))) void lds_void;

#define sched_reads(N) __builtin_amdgcn_sched_group_barrier(0x100, N, 0)
template <int R, int N>
__device__ __forceinline__ void sched_mfma_then_reads() {
  if constexpr (R > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (N > 0) __builtin_amdgcn_sched_group_barrier(0x100, N, 0);
    sched_mfma_then_reads<R - 1, N>();
  }
}

// Offset of output tile dt's bytes (16 dt .. + 15) within a key row slot group.
__host__ __device__ constexpr int dt_offset(int dt) {
  return 1024 * (2 * (dt / 8) + (dt % 2)) + 256 * ((dt % 8) / 2);
}

typedef __attribute__((address_space(3))) v2i lds_v2i;

// The 32-byte V^T operand of output tile dt: lane l holds dim 16 dt + (l & 15),
// byte 4 kb + i = key 16 kb + 4 (l >> 4) + i, as the P operand.  Four
// transposing reads, 8 keys (two key blocks, 2 kKbStride apart) each.  The
// compiler cannot tell which LDS bytes the intrinsic reads, so it waits for
// every buffer-to-LDS load in flight before the first of them: the last part
// of the next tile's loads, issued just before, is in flight there.  Written
// as asm statements that wait for their own reads instead, the 32 waits
// measured slower (1.78-1.83 ms against 1.68-1.69 ms on the 4096-token
// prompt).
__device__ __forceinline__ v8i vt_operand(const uint8_t *base, int dt) {
  v2i r[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    r[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(base + 2 * kKbStride * q + dt_offset(dt)));
  return (v8i){r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
}

// D += A B with B's 32-element blocks scaled by 2^(sb - 127), A unscaled.
__device__ __forceinline__ v4f mfma_scaled_b(const v8i &a, const v8i &b, const v4f &c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_latent_kernel(AttnArgs a, Grid gr) {
  constexpr int kCols = 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int32_t *idx_s = reinterpret_cast<int32_t *>(smem + kIdxOff);
  const int tid = thread_index();
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int col = lane & 15;

  int bid = block_index();
  const int split = bid % gr.splits;
  bid /= gr.splits;
  const int hg = bid % gr.n_tiles;
  const int tok = bid / gr.n_tiles;

  bool row_ok[kCols];
  int row_t[kCols], row_h[kCols];
  row_h[0] = hg * kRowsPerWg + wave * 16 + col;
  row_ok[0] = row_h[0] < a.hq;
  row_t[0] = tok;

  // ---------------------------------------------------------------- index list
  int list_len = a.topk;
  if (a.topk_length) list_len = max(0, min(a.topk, a.topk_length[tok]));
  const int chunk = ((list_len + gr.splits - 1) / gr.splits + kKT - 1) / kKT * kKT;
  const int lo = min(list_len, split * chunk);
  const int hi = min(list_len, lo + chunk);
  const int n_iter = (hi - lo + kKT - 1) / kKT;
  // a list entry: ids outside [0, num_kv) and positions past the list end are -1
  auto list_id = [&](int j) {
    int id = -1;
    if (lo + j < hi) {
      id = a.indices[(int64_t)tok * a.topk + lo + j];
      if (id < 0 || id >= a.num_kv) id = -1;
    }
    return id;
  };

  // ---------------------------------------------------------------- staging
  // Wave w moves key block w of a tile: its 8 main operands and its tail, the
  // lanes of every load reading key 16 w + (l & 15).  An absent key (-1, i.e.
  // record 0xFFFFFFFF) reads zeros.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(a.k), (short)a.k_row_stride, (int)a.num_kv, 0x00020000);
  // Part q (0..2) of a tile's loads: operand slots 3 q .. 3 q + 2 of the
  // wave's key block (slot 8 is the tail).  The parts are issued at three
  // points of the previous tile, so that the eight waves' row gathers do not
  // all queue behind the barrier at once.
  auto dma_part = [&](int id, uint8_t *tb, int part) {
    uint8_t *blk = tb + kKbStride * wave_s;
    // the uniform part of each byte offset goes in soffset (an instruction
    // offset would move the LDS destination as well)
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int slot = 3 * part + j;   // operand (kc, hh) = (slot / 2, slot % 2)
      if (slot < 8)
        __builtin_amdgcn_struct_ptr_buffer_load_lds(rk, (lds_void *)(blk + 1024 * slot), 16, id, 32 * g,
                                                    128 * (slot / 2) + 16 * (slot % 2), 0, 0);
      else
        __builtin_amdgcn_struct_ptr_buffer_load_lds(rk, (lds_void *)(tb + kMain + 1024 * wave_s), 16, id, 16 * g,
                                                    512, 0, 0);
    }
  };
  auto staged_id = [&](int it) { return idx_s[it * kKT + 16 * wave_s + col]; };

  // the first tile's loads (ids read from global memory here) and the Q
  // operands are in flight while the list is staged
  if (n_iter > 0) {
    const int id0 = list_id(16 * wave_s + col);
    dma_part(id0, smem, 0);
    dma_part(id0, smem, 1);
    dma_part(id0, smem, 2);
  }

  // ---------------------------------------------------------------- Q operands
  v8i qb[kNkc];
  long qt[2];
  {
    const uint8_t *qrow = a.q + ((int64_t)tok * a.hq + (row_ok[0] ? row_h[0] : 0)) * kDqk;
#pragma unroll
    for (int kc = 0; kc < kNkc; ++kc)
      qb[kc] = row_ok[0] ? gload32(qrow + 128 * kc + 32 * g) : (v8i){0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
      qt[mm] = row_ok[0] ? *reinterpret_cast<const long *>(qrow + 512 + 32 * mm + 8 * g) : 0;
  }

  bool bad = false;
  for (int j = tid; j < n_iter * kKT; j += kThreads) {
    const int id = list_id(j);
    idx_s[j] = id;
    bad |= id < 0;
  }
  const bool all_valid = !wg_or<kWaves>(bad);

  // ---------------------------------------------------------------- state
  v4f o[kNdt][kCols];
  float negm[kCols];      // minus the reference maximum (raw dot units); 0 before the first key
  float mraw[kCols];      // exact running maximum (raw dot units)
  float lsum[kCols];
  bool started = false;   // the rows share one list: they start on the same tile
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
#pragma unroll
    for (int dt = 0; dt < kNdt; ++dt) o[dt][c] = (v4f){0.f, 0.f, 0.f, 0.f};
    negm[c] = 0.f;
    mraw[c] = -INFINITY;
    lsum[c] = 0.f;
  }
  const float ck = a.key_scale_log2;
  const int op_lane = 16 * lane;
  // transposing-read address of this lane: 8-byte row of key
  // 16 (2 q + j / 4) + 4 g + j % 4, dims 16 dt + 8 (l & 1) .. + 7, j = (l & 15) / 2
  const int tr_j = col >> 1;
  const int tr_lane = kKbStride * (tr_j >> 2) + 16 * (4 * g + (tr_j & 3)) + 8 * (lane & 1);

  for (int pass = 0; pass < 2; ++pass) {
    bool overflow = false;
    if (pass == 1 && n_iter > 0) {
      const int id0 = staged_id(0);
      dma_part(id0, smem, 0);
      dma_part(id0, smem, 1);
      dma_part(id0, smem, 2);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

    for (int it = 0; it < n_iter; ++it) {
      // tile it is in LDS (its DMA completed before this barrier's wait), and
      // every wave is done with tile it - 1
      lds_barrier();
      const uint8_t *tb = smem + (it & 1) * kTileBytes;
      const bool next = it + 1 < n_iter;
      uint8_t *nb = smem + ((it + 1) & 1) * kTileBytes;
      const int nid = next ? staged_id(it + 1) : -1;
      if (next) dma_part(nid, nb, 0);
      v4f cinit[kCols];
#pragma unroll
      for (int c = 0; c < kCols; ++c) cinit[c] = (v4f){negm[c], negm[c], negm[c], negm[c]};
      // P operands of the tile: dword kb, byte i = key 16 kb + 4 g + i.  The
      // two 64-key halves (dwords 0..3, 4..7) are scored separately, each with
      // its own exponent; bytes 0..15 of every lane take the E8M0 scale of
      // lane groups 0, 1 and bytes 16..31 that of groups 2, 3, so lanes with
      // g < 2 supply the first half's scale and the others the second's.
      v8i ph[kCols], pl[kCols];
      int e_half[2][kCols];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // ---- S^T = K Q^T + C for 64 keys: four independent chains; operand
        // reads run two MFMAs ahead
        v4f s[4][kCols];
#pragma unroll
        for (int kc = 0; kc < kNkc; ++kc)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const v8i ka = lds_read32x2(tb + op_lane + kKbStride * (4 * h + kb) + 1024 * (2 * kc));
#pragma unroll
            for (int c = 0; c < kCols; ++c)
              s[kb][c] = mfma_16x16x128_e4m3(ka, qb[kc], kc == 0 ? cinit[c] : s[kb][c]);
          }
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const long kta = *reinterpret_cast<const long *>(tb + kMain + 1024 * (4 * h + kb) +
                                                             256 * (2 * mm + (g >> 1)) + 16 * col + 8 * (g & 1));
#pragma unroll
            for (int c = 0; c < kCols; ++c) s[kb][c] = mfma_16x16x32_e4m3(kta, qt[mm], s[kb][c]);
          }
        sched_reads(4);                  // operands of MFMAs 0, 1
        sched_mfma_then_reads<14, 2>();  // MFMAs 0..13, each followed by the reads of MFMA + 2
        sched_mfma_then_reads<8, 1>();   // MFMAs 14..21 (tail operands: one read each)
        sched_mfma_then_reads<2, 0>();
        // ---- absent keys (ids out of range, positions past the list end)
        if (!all_valid) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const v4i id4 = *reinterpret_cast<const v4i *>(idx_s + it * kKT + 16 * (4 * h + kb) + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int c = 0; c < kCols; ++c)
                if (id4[i] < 0) s[kb][c][i] = -INFINITY;
          }
        }
        // ---- row maxima, reference on the first half with a key, overflow check
        float mx[kCols];
#pragma unroll
        for (int c = 0; c < kCols; ++c) {
          float m = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            m = fmaxf(fmaxf(m, fmaxf(s[kb][c][0], s[kb][c][1])), fmaxf(s[kb][c][2], s[kb][c][3]));
          mx[c] = group4_max_swap(m);
          mraw[c] = fmaxf(mraw[c], mx[c] - negm[c]);
        }
        if (h == 0 && next) dma_part(nid, nb, 1);
        if (!started) {
          // uniform: every row sees the same keys, so all rows have a finite
          // maximum on the same half tile
          if (mx[0] != -INFINITY) {
#pragma unroll
            for (int c = 0; c < kCols; ++c) {
              const float delta = mx[c];
#pragma unroll
              for (int kb = 0; kb < 4; ++kb) s[kb][c] -= delta;
              mx[c] -= delta;
              negm[c] -= delta;
              cinit[c] = (v4f){negm[c], negm[c], negm[c], negm[c]};
            }
            started = true;
          }
        }
#pragma unroll
        for (int c = 0; c < kCols; ++c) overflow |= mx[c] * ck > kHeadroom;
        // ---- probabilities as e4m3 hi + lo pairs, row sums
#pragma unroll
        for (int c = 0; c < kCols; ++c) {
          // the half's row maximum maps into [2^7, 2^8): every P below 448
          const int e = min((int)floorf(fmaxf(mx[c] * ck, -120.f)) - 7, 120);
          const float ne = (float)(-e);
          e_half[h][c] = e;
          float ls = 0.f;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              p[i] = __builtin_amdgcn_exp2f(fmaf(s[kb][c][i], ck, ne));
              ls += p[i];
            }
            int hw = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
            hw = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], hw, true);
            const v2f h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);
            const v2f h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
            int lw = __builtin_amdgcn_cvt_pk_fp8_f32(p[0] - h01[0], p[1] - h01[1], 0, false);
            lw = __builtin_amdgcn_cvt_pk_fp8_f32(p[2] - h23[0], p[3] - h23[1], lw, true);
            ph[c][4 * h + kb] = hw;
            pl[c][4 * h + kb] = lw;
          }
          lsum[c] += __builtin_ldexpf(ls, e);
        }
      }
      int sb[kCols];
#pragma unroll
      for (int c = 0; c < kCols; ++c) {
        const int e0 = e_half[0][c], e1 = e_half[1][c];
        sb[c] = 127 + e1 + (g < 2) * (e0 - e1);
      }
      // ---- O^T += V^T (hi + lo)^T: the lo product of tile dt - 1 follows the
      // hi product of tile dt, and the operand reads run one tile ahead
      if (next) dma_part(nid, nb, 2);
      const uint8_t *tr = tb + tr_lane;
      v8i va_prev, va_cur = vt_operand(tr, 0);
#pragma unroll
      for (int dt = 0; dt < kNdt; ++dt) {
        v8i va_next;
        if (dt + 1 < kNdt) va_next = vt_operand(tr, dt + 1);
#pragma unroll
        for (int c = 0; c < kCols; ++c) {
          o[dt][c] = mfma_scaled_b(va_cur, ph[c], o[dt][c], sb[c]);
          if (dt > 0) o[dt - 1][c] = mfma_scaled_b(va_prev, pl[c], o[dt - 1][c], sb[c]);
        }
        va_prev = va_cur;
        va_cur = va_next;
      }
#pragma unroll
      for (int c = 0; c < kCols; ++c) o[kNdt - 1][c] = mfma_scaled_b(va_prev, pl[c], o[kNdt - 1][c], sb[c]);
      // order: reads of tiles 0, 1; hi 0; then per dt = 1..30 the reads of
      // tile dt + 1, hi dt and lo dt - 1; then hi 31, lo 30, lo 31
      sched_reads(8);
      sched_mfma_then_reads<1, 0>();
#pragma unroll
      for (int dt = 1; dt < kNdt - 1; ++dt) {
        sched_reads(4);
        sched_mfma_then_reads<2, 0>();
      }
      sched_mfma_then_reads<3, 0>();
      // the DMA of tile it + 1 lands before the next barrier
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    }
    // rare second pass: restart from the exact row maxima seen in the first one
    if (pass == 1 || !wg_or<kWaves>(overflow)) break;
    started = mraw[0] != -INFINITY;
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
      negm[c] = started ? -mraw[c] : 0.f;
      lsum[c] = 0.f;
#pragma unroll
      for (int dt = 0; dt < kNdt; ++dt) o[dt][c] = (v4f){0.f, 0.f, 0.f, 0.f};
    }
  }

  float m_ref[kCols], m_true[kCols];
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
    m_ref[c] = started ? -negm[c] * ck : -INFINITY;
    m_true[c] = mraw[c] * ck;
  }
  if (gr.splits > 1) {
    attn_epilogue<kCols, kNdt>(a, gr, split, g, row_ok, row_t, row_h, o, m_ref, m_true, lsum);
    return;
  }
  // Final outputs: the wave's 16 bf16 rows go through LDS (the tile buffers
  // are free once every wave has left the loop), so that each store writes
  // one contiguous 1 KB row instead of 8 bytes of each of 16 rows.
  const float l_tot = group4_sum(lsum[0]);
  const int64_t rowidx = (int64_t)tok * a.hq + row_h[0];
  const bool has_sink = a.sink != nullptr;
  const float zs = has_sink && row_ok[0] ? a.sink_scale_log2 * a.sink[row_h[0]] : -INFINITY;
  const float M = fmaxf(m_ref[0], zs);
  float Lt = 0.f, fo = 0.f;
  if (M != -INFINITY) {
    const float wk = m_ref[0] == -INFINITY ? 0.f : exp2f(m_ref[0] - M);
    Lt = l_tot * wk + (has_sink ? exp2f(zs - M) : 0.f);
    fo = Lt > 0.f ? wk * a.v_scale / Lt : 0.f;
  }
  if (g == 0 && row_ok[0]) {
    a.lse[rowidx] = Lt > 0.f ? (M + log2f(Lt)) * kLn2 : -INFINITY;
    a.max_logits[rowidx] = m_true[0] * kLn2;
  }
  __syncthreads();
  uint8_t *ob = smem + wave * 16 * kOutPitch;
#pragma unroll
  for (int dt = 0; dt < kNdt; ++dt) {
    const v4f x = o[dt][0] * fo;
    *reinterpret_cast<uint2 *>(ob + col * kOutPitch + 32 * dt + 8 * g) =
        make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
  }
  // the wave reads back only what it wrote: its own LDS writes are visible
  // to it once they have completed
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  const int h0 = hg * kRowsPerWg + wave * 16;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const v4i v = *reinterpret_cast<const v4i *>(ob + r * kOutPitch + 16 * lane);
    if (h0 + r < a.hq)
      *reinterpret_cast<v4i *>(a.out + ((int64_t)tok * a.hq + h0 + r) * kDv + 8 * lane) = v;
  }
}

}  // namespace

size_t token_latent_lds(int topk, int splits) {
  const int chunk = ((topk + splits - 1) / splits + kKT - 1) / kKT * kKT;
  return (size_t)kIdxOff + 4 * (size_t)chunk;
}

bool token_latent_fits(const AttnArgs &a, int splits) {
  // V is the leading d_v bytes of each K row; the K row stride fits the
  // buffer resource's 14-bit stride field, and the cache stays below 2 GB
  // (larger caches take the unpipelined kernel)
  return a.dqk == kDqk && a.dv == kDv && a.v == a.k && a.v_row_stride == a.k_row_stride && a.num_kv > 0 &&
         a.k_row_stride >= kDqk && a.k_row_stride < 16384 && a.k_row_stride % 16 == 0 &&
         (int64_t)a.num_kv * a.k_row_stride < ((int64_t)1 << 31) && token_latent_lds(a.topk, splits) <= kMaxLds;
}

int launch_token_latent(const AttnArgs &a, const Grid &gr, int64_t nblocks, hipStream_t stream) {
  const size_t lds = token_latent_lds(a.topk, gr.splits);
  if (lds > kMaxLds) return fail(FP8TS_EUNSUPPORTED, "sparse_attn_fwd: index list needs %zu bytes of LDS", lds);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(attn_latent_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return fail(FP8TS_EHIP, "sparse_attn_fwd: LDS attribute: %s", hipGetErrorString(e));
  hipLaunchKernelGGL(attn_latent_kernel, dim3((unsigned)nblocks), dim3(kThreads), lds, stream, a, gr);
  return check_launch("sparse_attn_fwd (token MLA, latent rows)");
}

}  // namespace fp8ts
