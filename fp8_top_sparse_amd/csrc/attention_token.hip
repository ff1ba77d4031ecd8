// Token-sparse MLA prefill attention (d_qk = 576, d_v = 512, one KV head
// shared by every q head): the kernel behind sparse_attn_fwd in token mode
// when the q heads come in groups of 128.
//
// Semantics: sglang PR 25751 digest, code excerpt of
// sparse_mla_q8kv8_prefill_fwd (each query token attends to the KV rows its
// index list names; out bf16 [s_q, h_q, 512], max_logits and lse fp32
// [s_q, h_q], optional attn_sink and topk_length; ids outside [0, s_kv) and
// list positions past topk_length take no part), with the scale handling of
// sglang PR 30971 digest, implementation step 3.
//
// Workgroup: one query token x 128 q heads.  Each wave owns COLS 16-row
// column tiles, so one K or V^T operand read from LDS feeds COLS MFMAs: with
// d_v = 512 the PV product dominates, and at 16 rows per wave the operand
// reads alone would saturate the LDS.  The index list of the token (its split
// of it) is staged in LDS once; K/V rows are gathered 32 keys per tile through
// buffer resources over the whole caches, an absent key reading zeros.
//
// Per tile (32 keys), the same ingredients as the block kernels:
//  * S^T = K Q^T + C on 16x16x128 e4m3 MFMA (4 slices of 128 bytes) plus two
//    16x16x32 e4m3 MFMA for the last 64 bytes; C holds minus the row's
//    reference maximum, so p = exp2(ck * S).
//  * P stays in registers as the B operand of the 16x16x32 bf16 PV MFMA.
//  * K (e4m3) and V^T (bf16) tiles sit in LDS in MFMA operand order; tiles
//    are double-buffered, tile t+1 written from registers while tile t is
//    computed and tile t+2 is in flight from memory.
#include "attn_common.h"

namespace fp8ts {
namespace {

constexpr int kDqk = 576, kDv = 512;
constexpr int kKT = 32;                          // keys per tile
constexpr int kNkc = 4;                          // 128-byte slices of a K row
constexpr int kNdt = kDv / 16;                   // 16-dim output tiles
constexpr int kWaves = 8, kThreads = 512;        // 16 query rows per wave
constexpr int kRowsPerWg = 16 * kWaves;
// LDS: two K tiles, two V^T tiles, the split's index list.
//   K main: operand (kt, kc, hh) of lane l at 1024 * ((4 kt + kc) * 2 + hh) + 16 l:
//           key 16 kt + (l & 15), bytes 128 kc + 32 (l >> 4) + 16 hh .. + 15
//   K tail: at kKMain + 1024 kt + 16 l: key 16 kt + (l & 15), bytes
//           512 + 16 (l >> 4) .. + 15; operand (kt, mm) of lane l (8 bytes,
//           512 + 32 mm + 8 (l >> 4)) therefore sits at
//           kKMain + 1024 kt + 256 (2 mm + (g >> 1)) + 16 (l & 15) + 8 (g & 1)
//   V^T:    operand dt of lane l at kVtPitch dt + 16 l: dim 16 dt + (l & 15),
//           keys vt_key(l >> 4, 0..7) (bf16).  The 16 extra bytes per tile put
//           the 32 lanes of each staging write on 32 distinct 8-byte bank slots
//           with every write of a thread at one base address plus a constant.
// Every K byte arrives by LDS DMA (16 bytes per lane, the lane order being the
// LDS order above); V is widened and transposed from registers.
constexpr int kKMain = kKT * 512;
constexpr int kKBytes = kKMain + kKT * 64;
constexpr int kVtPitch = 1024 + 16;
constexpr int kVtBytes = kNdt * kVtPitch;
constexpr int kVtOff = 2 * kKBytes;
constexpr int kIdxOff = kVtOff + 2 * kVtBytes;   // the split's index list (int32)
constexpr int kVUnits = (kKT / 4) * (kDv / 4);   // 4-key x 4-dim units of a V tile
constexpr int V_PER = kVUnits / kThreads;
// K rows reach LDS through a structured buffer resource (record = one cache
// row): the hardware forms base + index * stride + offset and writes zeros
// for an index at or past the record count, so an absent key (stored as -1,
// i.e. index 0xFFFFFFFF) needs no address arithmetic.  V rows are gathered
// with byte offsets (indexed dword gathers measured slower); an absent key
// gets an offset past the end of the cache, which also reads zeros.
constexpr uint32_t kNoRow = 0x80000000u;

typedef __attribute__((address_space(3))) void lds_void;

// Byte offset of row id (stride < 2^24, id < 2^24: one 24-bit multiply).
__device__ __forceinline__ uint32_t row_offset(int id, uint32_t stride24) {
  return id < 0 ? kNoRow : ((uint32_t)id & 0xFFFFFFu) * stride24;
}

// Instruction-order constraints for the scheduler (LDS reads ahead of the
// MFMAs that consume them): N LDS reads; then R x (one MFMA, N LDS reads).
#define sched_reads(N) __builtin_amdgcn_sched_group_barrier(0x100, N, 0)
template <int R, int N>
__device__ __forceinline__ void sched_mfma_then_reads() {
  if constexpr (R > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (N > 0) __builtin_amdgcn_sched_group_barrier(0x100, N, 0);
    sched_mfma_then_reads<R - 1, N>();
  }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_token_kernel(AttnArgs a, Grid gr) {
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
  // ids outside [0, num_kv) and the positions past the list end become -1
  bool bad = false;
  for (int j = tid; j < n_iter * kKT; j += kThreads) {
    int id = -1;
    if (lo + j < hi) {
      id = a.indices[(int64_t)tok * a.topk + lo + j];
      if (id < 0 || id >= a.num_kv) id = -1;
    }
    idx_s[j] = id;
    bad |= id < 0;
  }
  const bool all_valid = !wg_or<kWaves>(bad);

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

  // ---------------------------------------------------------------- staging
  // K: wave w moves operands (kt, kc, hh) = (w >> 2, w & 3, 0..1) of the tile
  // and, when w & 3 == 0, the tail of key tile kt: its lanes all read key
  // 16 (w >> 2) + (l & 15).  V: the units of a thread cover dims 4 d4 .. + 3
  // of keys 16 jh + 4 cix + i.
  const uint32_t vs = (uint32_t)a.v_row_stride & 0xFFFFFFu;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int k_kt = wave_s >> 2, k_kc = wave_s & 3;
  const bool k_tail = k_kc == 0;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(a.k), (short)a.k_row_stride, (int)a.num_kv, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(a.v), (short)0, (int)((a.num_kv - 1) * a.v_row_stride + kDv), 0x00020000);
  const int jh = tid & 1, d4 = (tid >> 1) & 127;
  uint32_t vreg[V_PER][4];
  auto dma_k = [&](int it, uint8_t *kb) {
    const int id = idx_s[it * kKT + 16 * k_kt + col];
    uint8_t *slot = kb + 1024 * (2 * wave_s);
    __builtin_amdgcn_struct_ptr_buffer_load_lds(rk, (lds_void *)slot, 16, id, 128 * k_kc + 32 * g, 0, 0, 0);
    // (an instruction offset would move the LDS destination as well)
    __builtin_amdgcn_struct_ptr_buffer_load_lds(rk, (lds_void *)(slot + 1024), 16, id, 128 * k_kc + 32 * g + 16, 0, 0,
                                                0);
    if (k_tail)
      __builtin_amdgcn_struct_ptr_buffer_load_lds(rk, (lds_void *)(kb + kKMain + 1024 * k_kt), 16, id, 512 + 16 * g, 0,
                                                  0, 0);
  };
  auto load_v = [&](int it) {
    const int32_t *ids = idx_s + it * kKT;
#pragma unroll
    for (int j = 0; j < V_PER; ++j) {
      const int cix = (tid + j * kThreads) >> 8;
      const v4i vid = *reinterpret_cast<const v4i *>(ids + 16 * jh + 4 * cix);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vreg[j][i] = __builtin_amdgcn_raw_buffer_load_b32(rv, row_offset(vid[i], vs) + 4 * d4, 0, 0);
    }
  };
  auto store_v = [&](uint8_t *vt) {
#pragma unroll
    for (int j = 0; j < V_PER; ++j) {
      const int cix = (tid + j * kThreads) >> 8;
      const uint32_t *w = vreg[j];
      // 4x4 byte transpose: x[s] = byte s (dim 4 d4 + s) of keys 0..3
      const uint32_t t0 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);
      const uint32_t t1 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
      const uint32_t t2 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
      const uint32_t t3 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
      const uint32_t x[4] = {__builtin_amdgcn_perm(t2, t0, 0x05040100u), __builtin_amdgcn_perm(t2, t0, 0x07060302u),
                             __builtin_amdgcn_perm(t3, t1, 0x05040100u), __builtin_amdgcn_perm(t3, t1, 0x07060302u)};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const v2i pr = {(int)bf16x2_from_e4m3(x[s4], false), (int)bf16x2_from_e4m3(x[s4], true)};
        *reinterpret_cast<v2i *>(vt + kVtPitch * (d4 >> 2) + 16 * (16 * (cix & 3) + 4 * (d4 & 3) + s4) + 8 * jh) = pr;
      }
    }
  };

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

  for (int pass = 0; pass < 2; ++pass) {
    bool overflow = false;
    if (n_iter > 0) {
      dma_k(0, smem);
      load_v(0);
      store_v(smem + kVtOff);
    }
    if (n_iter > 1) load_v(1);
    // drain the prologue loads here, once: otherwise the wait-count analysis
    // makes the first MFMA of every tile wait for the in-flight prefetch
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

    for (int it = 0; it < n_iter; ++it) {
      // tile it is in LDS (its K DMA completed before the previous barrier's
      // wait), and every wave is done with tile it - 1
      lds_barrier();
      const uint8_t *kb = smem + (it & 1) * kKBytes;
      const uint8_t *vt = smem + kVtOff + (it & 1) * kVtBytes;
      // K of tile it + 1 by DMA and V^T of tile it + 1 from registers, into
      // the buffers of tile it - 1; V of tile it + 2 into registers
      if (it + 1 < n_iter) {
        dma_k(it + 1, smem + ((it + 1) & 1) * kKBytes);
        store_v(smem + kVtOff + ((it + 1) & 1) * kVtBytes);
        if (it + 2 < n_iter) load_v(it + 2);
      }
      v4f cinit[kCols];
#pragma unroll
      for (int c = 0; c < kCols; ++c) cinit[c] = (v4f){negm[c], negm[c], negm[c], negm[c]};
      // ---- S^T = K Q^T + C for 32 keys: two independent accumulation chains
      // (key tiles 0 and 1); operand reads run two MFMAs ahead
      v4f s[2][kCols];
#pragma unroll
      for (int kc = 0; kc < kNkc; ++kc)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const v8i ka = lds_read32x2(kb + op_lane + 1024 * (2 * (4 * kt + kc)));
#pragma unroll
          for (int c = 0; c < kCols; ++c) s[kt][c] = mfma_16x16x128_e4m3(ka, qb[kc], kc == 0 ? cinit[c] : s[kt][c]);
        }
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const long kta = *reinterpret_cast<const long *>(kb + kKMain + 1024 * kt + 256 * (2 * mm + (g >> 1)) +
                                                           16 * col + 8 * (g & 1));
#pragma unroll
          for (int c = 0; c < kCols; ++c) s[kt][c] = mfma_16x16x32_e4m3(kta, qt[mm], s[kt][c]);
        }
      sched_reads(4);                 // operands of MFMAs 0, 1
      sched_mfma_then_reads<6, 2>();  // MFMAs 0..5, each followed by the reads of MFMA + 2
      sched_mfma_then_reads<4, 1>();  // MFMAs 6..9 (tail operands: one read each)
      sched_mfma_then_reads<2, 0>();
      // ---- absent keys (ids out of range, positions past the list end)
      if (!all_valid) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const v4i id4 = *reinterpret_cast<const v4i *>(idx_s + it * kKT + 16 * kt + 4 * g);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < kCols; ++c)
              if (id4[i] < 0) s[kt][c][i] = -INFINITY;
        }
      }
      // ---- row maxima, reference on the first tile with a key, overflow check
      float mx[kCols];
#pragma unroll
      for (int c = 0; c < kCols; ++c) {
        const float m = fmaxf(fmaxf(fmaxf(s[0][c][0], s[0][c][1]), fmaxf(s[0][c][2], s[0][c][3])),
                              fmaxf(fmaxf(s[1][c][0], s[1][c][1]), fmaxf(s[1][c][2], s[1][c][3])));
        mx[c] = group4_max_swap(m);
        mraw[c] = fmaxf(mraw[c], mx[c] - negm[c]);
      }
      if (!started) {
        // uniform: every row sees the same keys, so all rows have a finite
        // maximum on the same tile
        if (mx[0] != -INFINITY) {
#pragma unroll
          for (int c = 0; c < kCols; ++c) {
            const float delta = mx[c];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) s[kt][c] -= delta;
            mx[c] -= delta;
            negm[c] -= delta;
          }
          started = true;
        }
      }
#pragma unroll
      for (int c = 0; c < kCols; ++c) overflow |= mx[c] * ck > kHeadroom;
      // ---- probabilities, row sums, bf16 B operands
      v8bf pb[kCols];
#pragma unroll
      for (int c = 0; c < kCols; ++c) {
        float p[2][4];
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[kt][i] = __builtin_amdgcn_exp2f(s[kt][c][i] * ck);
            ls += p[kt][i];
          }
        lsum[c] += ls;
        v8bf v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = (__bf16)p[0][i];
          v[4 + i] = (__bf16)p[1][i];
        }
        pb[c] = v;
      }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int dt = 0; dt < kNdt; ++dt) {
        const v8bf va = *reinterpret_cast<const v8bf *>(vt + op_lane + kVtPitch * dt);
#pragma unroll
        for (int c = 0; c < kCols; ++c) o[dt][c] = mfma_16x16x32_bf16(va, pb[c], o[dt][c]);
      }
      // V^T operand reads run six MFMAs ahead
      sched_reads(6);
      sched_mfma_then_reads<kNdt - 6, 1>();
      sched_mfma_then_reads<6, 0>();
      // the K DMA of tile it + 1 lands before the next barrier (the V loads
      // of tile it + 2 are waited for right after it anyway)
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
  attn_epilogue<kCols, kNdt>(a, gr, split, g, row_ok, row_t, row_h, o, m_ref, m_true, lsum);
}

}  // namespace

size_t token_mla_lds(int topk, int splits) {
  const int chunk = ((topk + splits - 1) / splits + kKT - 1) / kKT * kKT;
  return (size_t)kIdxOff + 4 * (size_t)chunk;
}

int token_mla_rows() { return kRowsPerWg; }

bool token_mla_fits(const AttnArgs &a) {
  // the K row stride fits the buffer resource's 14-bit stride field; V byte
  // offsets stay below kNoRow and its ids and stride fit the 24-bit multiply
  const int64_t lim = (int64_t)kNoRow - 4096;
  return a.dqk == kDqk && a.dv == kDv && a.num_kv > 0 && a.num_kv < (1 << 24) && a.k_row_stride >= kDqk &&
         a.k_row_stride < 16384 && a.k_row_stride % 16 == 0 && a.v_row_stride >= kDv &&
         a.v_row_stride < (1 << 24) && a.v_row_stride % 4 == 0 && (a.num_kv - 1) * a.v_row_stride + kDv < lim;
}

int launch_token_mla(const AttnArgs &a, const Grid &gr, int64_t nblocks, hipStream_t stream) {
  const size_t lds = token_mla_lds(a.topk, gr.splits);
  if (lds > kMaxLds) return fail(FP8TS_EUNSUPPORTED, "sparse_attn_fwd: index list needs %zu bytes of LDS", lds);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(attn_token_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return fail(FP8TS_EHIP, "sparse_attn_fwd: LDS attribute: %s", hipGetErrorString(e));
  hipLaunchKernelGGL(attn_token_kernel, dim3((unsigned)nblocks), dim3(kThreads), lds, stream,
                     a, gr);
  return check_launch("sparse_attn_fwd (token MLA)");
}

}  // namespace fp8ts
