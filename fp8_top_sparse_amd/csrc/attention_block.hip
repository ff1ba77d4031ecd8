// Block-sparse prefill attention for GQA (d_qk = d_v = 128, 128-token pages):
// the dense-tile kernel behind sparse_attn_fwd in block mode when every
// sequence has many query rows per KV head.
//
// Semantics: sglang PR 25751 digest (sparse attention forward: out bf16,
// max_logits and lse fp32 per (token, head), optional attn_sink) with block
// selection as in vLLM PR 45892 digest (each query token attends to the
// 128-token blocks its index head selected, causally masked), and the scale
// handling of sglang PR 30971 digest, implementation step 3 (q_scale folded
// into sm_scale, k_scale on the QK dot only, v_scale on the output).
//
// Workgroup: kRows query rows = a tile of consecutive tokens x the q heads of
// one KV head, split into 16-row column tiles over the waves.  The
// workgroup walks the ascending union of its rows' block lists; rows that did
// not select the current block get probability 0.
//
// Cost model this layout follows (gfx950, per SIMD): MFMA time and VALU time
// add up, a wave64 VOP1/VOP2 op issues in ~2 cycles, a VOP3 op in ~4, and
// v_exp_f32 in ~8.  So the softmax is kept to one VOP2 multiply, one exp, one
// max, one add and half a bf16 pack per score:
//  * S^T = K Q^T (+ C) on 16x16x128 e4m3 MFMA, where C holds minus the row's
//    reference maximum (raw dot units), so p = exp2(ck * S) needs no subtract.
//    The reference is the row's first tile maximum; a later tile maximum more
//    than kHeadroom (log2 units) above it makes the workgroup rerun once with
//    the exact maxima.
//  * P stays in registers: the S^T output layout of a 16-key tile pair is the
//    B-operand layout of the 16x16x32 bf16 PV MFMA.
//  * K (e4m3) and V^T (bf16, keys of every 32-key chunk in PV operand order)
//    are stored in LDS in MFMA operand order, so each operand fetch is one
//    contiguous 1 KB wave read.  The staging writes are spread over distinct
//    bank groups (K: 16 keys per write instruction; V: each thread's dims are
//    rotated with one v_alignbyte per loaded dword).
//  * K/V tiles are double-buffered in LDS (or single-buffered, so that two
//    128-row workgroups share a CU): tile t+1 is written from registers while
//    tile t is computed and tile t+2 is in flight from HBM.  Barriers order
//    LDS only, so the prefetch stays in flight across them.
//  * Prefill waves own 32 rows (two column tiles), so every operand read from
//    LDS feeds two MFMAs, and scheduling-group barriers place the operand
//    reads ahead of their MFMAs (two waves per SIMD leave room in registers
//    for reads in flight).
#include "attn_common.h"

namespace fp8ts {
namespace {

constexpr int kD = 128;
constexpr int kNdt = kD / 16;             // 16-dim output tiles
// K and V^T tiles are stored in MFMA operand order: every operand fetch is
// one contiguous 1 KB wave read (64 lanes x 16 bytes), which the LDS serves
// without bank conflicts (padded row layouts cost two passes per read).
//   K:   operand (kt, hh) of lane l at 1024 * (2 * kt + hh) + 16 * l: key
//        16 kt + (l & 15), bytes 32 (l >> 4) + 16 hh .. + 15
//   V^T: operand (dt, m) of lane l at 1024 * (4 * dt + m) + 16 * l: dim
//        16 dt + (l & 15), keys of chunk 4 m + (l >> 4) (bf16, order vt_key)
constexpr int kKBytes = kPage * kD;
constexpr int kVBytes = kD * kPage * 2;
constexpr int kBufBytes = kKBytes + kVBytes;
constexpr int kKChunks = kPage * kD / 16;           // 16-byte chunks of a K tile
constexpr int kVUnits = (kD / 4) * 16 * 2;          // 4-dim x 4-key units of a V tile

// Kernel configuration: WAVES waves split ROWS query rows into 16-row column
// tiles; BUFS K/V tile buffers in LDS (2: one barrier per tile; 1: two
// barriers per tile, and the workgroup is sized so that two share a CU).
// PRE: V^T tiles come pre-converted from the workspace (vt_pages_kernel), and
// both K and V^T are staged by buffer-to-LDS DMA, with no staging registers.
template <int WAVES, int ROWS, int BUFS, bool PRE = false>
struct Cfg {
  static constexpr bool kPre = PRE;
  static constexpr int kWaves = WAVES;
  static constexpr int kThreads = WAVES * 64;
  static constexpr int kRows = ROWS;
  static constexpr int kBufs = BUFS;
  static constexpr int kCols = ROWS / 16 / WAVES;
  static constexpr int kMetaOff = BUFS * kBufBytes;
  static constexpr int kWavesPerSimd = (BUFS == 1 ? 2 : 1) * WAVES / 4;
  static_assert(kCols * 16 * WAVES == ROWS, "tile");
  static_assert(kKChunks % kThreads == 0 && kVUnits % kThreads == 0, "staging");
};
// prefill with tiles converted in the kernel (short prompts): 256-row tiles,
// 8 waves of 32 rows (each K or V^T operand read feeds two MFMAs),
// double-buffered
using PrefillCfg = Cfg<8, 256, 2>;
// prefill from the pre-converted V^T pages: the same 256-row tile as 16 waves
// of 16 rows, four per SIMD.  A wave skips every block that none of its 16
// rows selected.  Against 8 waves of 32 rows (with the block and thread
// indices, votes and lane masks kept scalar in both): 32k top-64 prompt
// 2.64-2.84 ms against 2.85-2.91 ms, and the 8k prompt, whose rows select
// every causal block, 0.236-0.241 ms against 0.250-0.254 ms.
using PrefillPreCfg = Cfg<16, 256, 2, true>;
// decode: few rows per kv head, so small single-buffered workgroups that
// share a CU keep more pages in flight
using DecodeCfg = Cfg<4, 64, 1>;

// V staging unit u (0..1023) of a 128-key x 128-dim tile: 4 dims x 4 keys,
// half jh = u & 1 of V^T chunk cix = u >> 6, dims 4 d4 .. + 3 with
// d4 = (u >> 1) & 31.  Its raw dword i (e4m3 dims 4 d4 .. + 3 of one key) is
// at vt_unit_src(u, i) in the page.
__device__ __forceinline__ int vt_unit_src(int u, int i) {
  return vt_key(u >> 6, 4 * (u & 1) + i) * kD + 4 * ((u >> 1) & 31);
}

// Writes unit u (raw dwords w) widened to bf16 into the V^T tile vt.
__device__ __forceinline__ void vt_store_unit(uint8_t *vt, int u, const uint32_t (&v)[4]) {
  const int jh = u & 1, d4 = (u >> 1) & 31, cix = u >> 6;
  // rotate so that byte s of w[i] is dim 4 * d4 + ((s + rot) & 3): the 16
  // lanes sharing a write cycle then hit 16 distinct bank groups
  const int rot = (d4 >> 2) & 3;
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = __builtin_amdgcn_alignbyte(v[i], v[i], rot);
  // 4x4 byte transpose: x[s] = byte s of keys 0..3
  const uint32_t t0 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);
  const uint32_t t1 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
  const uint32_t t2 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
  const uint32_t x[4] = {__builtin_amdgcn_perm(t2, t0, 0x05040100u), __builtin_amdgcn_perm(t2, t0, 0x07060302u),
                         __builtin_amdgcn_perm(t3, t1, 0x05040100u), __builtin_amdgcn_perm(t3, t1, 0x07060302u)};
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    const int d = 4 * d4 + ((s4 + rot) & 3);
    const v2i pr = {(int)bf16x2_from_e4m3(x[s4], false), (int)bf16x2_from_e4m3(x[s4], true)};
    *reinterpret_cast<v2i *>(vt + 1024 * (4 * (d >> 4) + (cix >> 2)) + 16 * (16 * (cix & 3) + (d & 15)) + 8 * jh) = pr;
  }
}

// V^T of the page behind every (block-table slot, kv head), in the prefill
// kernel's LDS operand order (bf16, 32 KB each), so that the prefill tiles,
// which each visit a page many times over, stage it by DMA alone.  Slot
// (b * max_blocks + j) * hkv + kvh; slots without a valid page are skipped.
__global__ __launch_bounds__(256) void vt_pages_kernel(AttnArgs a, uint8_t *vt_pages) {
  __shared__ __attribute__((aligned(16))) uint8_t vt_s[kVBytes];
  const int slot = block_index();
  const int kvh = slot % a.hkv;
  // scalar copy of the workgroup's page: keeps the buffer resource scalar
  const int page = __builtin_amdgcn_readfirstlane(a.block_table[slot / a.hkv]);
  if (page < 0 || page >= a.num_kv) return;
  const int tid = thread_index();
  const __amdgpu_buffer_rsrc_t rv = make_tile_rsrc(a.v + ((int64_t)page * a.hkv + kvh) * kPage * kD);
#pragma unroll
  for (int j = 0; j < kVUnits / 256; ++j) {
    const int u = tid + 256 * j;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b32(rv, vt_unit_src(u, i), 0, 0);
    vt_store_unit(vt_s, u, w);
  }
  __syncthreads();
  v4i *dst = reinterpret_cast<v4i *>(vt_pages + (int64_t)slot * kVBytes);
  for (int i = tid; i < kVBytes / 16; i += 256) dst[i] = reinterpret_cast<const v4i *>(vt_s)[i];
}

typedef __attribute__((address_space(3))) void lds_void;

// Instruction-order constraints for the scheduler (LDS reads ahead of the
// MFMAs that consume them): N LDS reads, then R x (M MFMAs, N LDS reads).
template <int R, int M, int N>
__device__ __forceinline__ void sched_mfma_then_reads() {
  if constexpr (R > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
    if constexpr (N > 0) __builtin_amdgcn_sched_group_barrier(0x100, N, 0);
    sched_mfma_then_reads<R - 1, M, N>();
  }
}

template <class C>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(C::kWavesPerSimd)))
void attn_block_kernel(AttnArgs a, Grid gr) {
  constexpr int kThreads = C::kThreads, kCols = C::kCols, kBufs = C::kBufs, kMetaOff = C::kMetaOff;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = thread_index();
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int col = lane & 15;

  int bid = block_index();
  const int split = bid % gr.splits;
  bid /= gr.splits;
  BlockRows<kCols> br;
  if (!block_rows<kCols>(a, gr, bid, wave, col, br)) return;

  uint32_t *bits = reinterpret_cast<uint32_t *>(smem + kMetaOff);
  int32_t *ucount = reinterpret_cast<int32_t *>(bits + (gr.NL + 1) * gr.W);
  int32_t *ulist = ucount + 4;
  int32_t *plist = ulist + gr.W * 32;
  const int U = block_union<kThreads>(a, gr, br.kvh, br.cu0, br.q_len, br.seq_len, br.t0, bits, ucount, ulist);
  const int chunk = (U + gr.splits - 1) / gr.splits;
  const int lo = min(U, split * chunk);
  const int n_iter = min(U, lo + chunk) - lo;
  // physical page of every block this workgroup visits (-1: no such page)
  for (int i = tid; i < n_iter; i += kThreads) {
    const int page = a.block_table[(int64_t)br.b * a.max_blocks + ulist[lo + i]];
    plist[i] = (page >= 0 && page < a.num_kv) ? page : -1;
  }
  __syncthreads();

  // ---------------------------------------------------------------- Q operands
  v8i qb[kCols];
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
    const int64_t qr = br.row_ok[c] ? (int64_t)br.row_t[c] * a.hq + br.row_h[c] : 0;
    qb[c] = br.row_ok[c] ? gload32(a.q + qr * kD + 32 * g) : (v8i){0, 0, 0, 0, 0, 0, 0, 0};
  }

  // ---------------------------------------------------------------- staging
  // K: 16-byte chunks, row-major.  V: units of 4 dims x 4 keys (half of a
  // V^T chunk): unit u -> half jh = u & 1, dims 4 * d4 .. + 3 with
  // d4 = (u >> 1) & 31, chunk cix = u >> 6.
  constexpr int K_PER = kKChunks / kThreads;
  constexpr int V_PER = kVUnits / kThreads;
  const int64_t kv_head_stride = (int64_t)kPage * kD;
  const int kvh_s = __builtin_amdgcn_readfirstlane(br.kvh);
  v4i kreg[C::kPre ? 1 : K_PER];
  uint32_t vreg[C::kPre ? 1 : V_PER][4];
  // page ids are workgroup-uniform: each tile is read through buffer
  // resources (scalar base, 16 KB extent) with 32-bit lane offsets, so no
  // 64-bit per-lane address stays live across the loop
  auto load_tile = [&](int page) {
    page = __builtin_amdgcn_readfirstlane(page);
    if (page < 0) return;
    const int64_t off = ((int64_t)page * a.hkv + kvh_s) * kv_head_stride;
    const __amdgpu_buffer_rsrc_t rk = make_tile_rsrc(a.k + off);
    const __amdgpu_buffer_rsrc_t rv = make_tile_rsrc(a.v + off);
#pragma unroll
    for (int j = 0; j < K_PER; ++j)
      kreg[j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
          rk, k_chunk_key(tid + j * kThreads) * kD + 16 * k_chunk_part(tid + j * kThreads), 0, 0));
#pragma unroll
    for (int j = 0; j < V_PER; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vreg[j][i] = __builtin_amdgcn_raw_buffer_load_b32(rv, vt_unit_src(tid + j * kThreads, i), 0, 0);
    }
  };
  auto store_tile = [&](int page, uint8_t *buf) {
    if (__builtin_amdgcn_readfirstlane(page) < 0) return;
#pragma unroll
    for (int j = 0; j < K_PER; ++j) {
      const int ch = tid + j * kThreads;
      *reinterpret_cast<v4i *>(buf + k_tile_offset(k_chunk_key(ch), k_chunk_part(ch))) = kreg[j];
    }
#pragma unroll
    for (int j = 0; j < V_PER; ++j) vt_store_unit(buf + kKBytes, tid + j * kThreads, vreg[j]);
  };
  // PRE: tile it by DMA.  K operand slot s (kt = s >> 1, hh = s & 1) of lane
  // l holds key 16 kt + (l & 15), bytes 32 (l >> 4) + 16 hh; the V^T tile is
  // copied as it stands in the workspace.  16 + 32 wave-sized 1 KB slots.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  // the sequence is workgroup-uniform: read it into a scalar so that the
  // V^T buffer resource below is scalar too (a resource the compiler sees as
  // per-lane costs a loop over its distinct values around every load)
  const int b_s = __builtin_amdgcn_readfirstlane(br.b);
  auto dma_tile = [&](int page, int blk, uint8_t *buf) {
    if (page < 0) return;
    const __amdgpu_buffer_rsrc_t rk = make_tile_rsrc(a.k + ((int64_t)page * a.hkv + kvh_s) * kv_head_stride);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        gr.vt_pages + (((int64_t)b_s * a.max_blocks + blk) * a.hkv + kvh_s) * kVBytes, (short)0, kVBytes,
        0x00020000);
    constexpr int kW = kThreads / 64;
    static_assert(16 % kW == 0, "K slots per wave");
#pragma unroll
    for (int j = 0; j < 16 / kW; ++j) {
      const int s = wave_s + kW * j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(buf + 1024 * s), 16,
                                               (16 * (s >> 1) + col) * kD + 32 * g + 16 * (s & 1), 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 32 / kW; ++j) {
      const int s = wave_s + kW * j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(buf + kKBytes + 1024 * s), 16, 1024 * s + 16 * lane,
                                               0, 0, 0);
    }
  };

  // ---------------------------------------------------------------- state
  v4f o[kNdt][kCols];
  float negm[kCols];      // minus the reference maximum (raw dot units); 0 before the first tile
  float mraw[kCols];      // exact row maximum (raw dot units), set at the end of a pass
  float msh[kCols];       // this lane's running maximum of S (raw units minus the reference)
  float lsum[kCols];
  // Per-row flags are kept as wave lane masks (bit l: the row of lane l in
  // column tile c), so that testing and combining them is scalar work:
  // startm, rows that took their reference maximum.
  uint64_t startm[kCols];
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
#pragma unroll
    for (int dt = 0; dt < kNdt; ++dt) o[dt][c] = (v4f){0.f, 0.f, 0.f, 0.f};
    negm[c] = 0.f;
    mraw[c] = -INFINITY;
    msh[c] = -INFINITY;
    lsum[c] = 0.f;
    startm[c] = 0;
  }
  const float ck = a.key_scale_log2;
  const int op_lane = 16 * lane;                       // operand fetch offset of this lane
  // earliest position among the wave's rows: a half tile whose last key is at
  // or below it needs no causal mask in any row
  int wave_pmin = 0x7fffffff;
#pragma unroll
  for (int c = 0; c < kCols; ++c)
    if (br.row_ok[c]) wave_pmin = min(wave_pmin, br.row_p[c]);
  for (int off = 1; off < 64; off <<= 1) wave_pmin = min(wave_pmin, __shfl_xor(wave_pmin, off, 64));
  wave_pmin = __builtin_amdgcn_readfirstlane(wave_pmin);

  // metadata of the tile about to be computed, read one tile ahead; t_selm:
  // lane mask of the rows that selected the tile's block
  int t_blk = 0;
  uint64_t t_selm[kCols];
  auto fetch_meta = [&](int it) {
    t_blk = __builtin_amdgcn_readfirstlane(ulist[lo + it]);
    const bool has_page = __builtin_amdgcn_readfirstlane(plist[it]) >= 0;
#pragma unroll
    for (int c = 0; c < kCols; ++c)
      t_selm[c] = __builtin_amdgcn_ballot_w64(
          has_page && br.row_ok[c] && ((bits[br.row_li[c] * gr.W + (t_blk >> 5)] >> (t_blk & 31)) & 1u));
  };

  // PRE: the page and block of tile it + 1 are loaded from LDS during tile
  // it - 1 (m_page_v, m_blk_v: consumed a tile later, so their latency never
  // shows), and the selection words of tile it + 1 during tile it (m_word).
  int m_page_v = 0, m_blk_v = 0;
  uint32_t m_word[kCols];
  for (int pass = 0; pass < 2; ++pass) {
    if constexpr (C::kPre) {
      if (n_iter > 1) {
        m_page_v = plist[1];
        m_blk_v = ulist[lo + 1];
      }
    }
    if (n_iter > 0) {
      if constexpr (C::kPre) {
        dma_tile(__builtin_amdgcn_readfirstlane(plist[0]), __builtin_amdgcn_readfirstlane(ulist[lo]), smem);
      } else {
        load_tile(plist[0]);
        store_tile(plist[0], smem);
      }
      fetch_meta(0);
    }
    if (!C::kPre && n_iter > 1) load_tile(plist[1]);
    // drain the prologue loads here, once: otherwise the wait-count analysis
    // makes the first MFMA of every tile wait for the in-flight prefetch
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

    for (int it = 0; it < n_iter; ++it) {
      // tile it is in LDS (two buffers: and every wave is done with tile it - 1)
      lds_barrier();
      const uint8_t *kt_s = smem + (kBufs == 2 ? (it & 1) * kBufBytes : 0);
      const uint8_t *vt_s = kt_s + kKBytes;
      const int blk = t_blk;
      uint64_t selm[kCols];
      uint64_t any_sel = 0;
#pragma unroll
      for (int c = 0; c < kCols; ++c) {
        selm[c] = t_selm[c];
        any_sel |= selm[c];
      }
      // stage tile it + 1 (loaded during the previous tile) into the buffer
      // tile it - 1 used, and start loading tile it + 2: this VALU and LDS
      // work overlaps the previous tile's PV products still in the MFMA pipe
      int n_page = -1, n_blk = 0;   // PRE: tile it + 1
      if constexpr (C::kPre) {
        if (it + 1 < n_iter) {
          n_page = __builtin_amdgcn_readfirstlane(m_page_v);
          n_blk = __builtin_amdgcn_readfirstlane(m_blk_v);
          dma_tile(n_page, n_blk, smem + ((it + 1) & 1) * kBufBytes);
#pragma unroll
          for (int c = 0; c < kCols; ++c) m_word[c] = bits[br.row_li[c] * gr.W + (n_blk >> 5)];
          if (it + 2 < n_iter) {
            m_page_v = plist[it + 2];
            m_blk_v = ulist[lo + it + 2];
          }
        }
      }
      if (!C::kPre && kBufs == 2 && it + 1 < n_iter) {
        store_tile(plist[it + 1], smem + ((it + 1) & 1) * kBufBytes);
        if (it + 2 < n_iter) load_tile(plist[it + 2]);
      }
      if (any_sel) {
        const int key_base = blk * kPage;
        v4f cinit[kCols];
#pragma unroll
        for (int c = 0; c < kCols; ++c) {
          const float cv = __builtin_amdgcn_inverse_ballot_w64(selm[c]) ? negm[c] : -INFINITY;
          cinit[c] = (v4f){cv, cv, cv, cv};
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // ---- S^T = K Q^T + C for 64 keys
          v4f s[4][kCols];
          // The MFMA runs (QK here, PV below) issue at raised wave priority:
          // when both waves of a SIMD are ready, the one feeding the matrix
          // core goes first and the other's softmax VALU fills its gaps.  The
          // priority changes also keep the exps out of the PV stream
          // (8k prefill: 263.7 us against 271.2 us, four paired runs).  With
          // four 16-row waves per SIMD they no longer help (32k: 2.675 ms
          // without against 2.703 ms with, eight paired runs), so that
          // configuration leaves every wave at the base priority.
          constexpr int kMfmaPrio = C::kWaves == 16 ? 0 : 1;
          __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
            const v8i ka = lds_read32x2(kt_s + op_lane + 1024 * (2 * (4 * h + kt)));
#pragma unroll
            for (int c = 0; c < kCols; ++c) s[kt][c] = mfma_16x16x128_e4m3(ka, qb[c], cinit[c]);
          }
          // K operand reads (two LDS reads each) run two operands ahead
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          sched_mfma_then_reads<2, kCols, 2>();
          sched_mfma_then_reads<2, kCols, 0>();
          __builtin_amdgcn_s_setprio(0);
          // ---- causal mask, only where some row of the wave may need one
          const int kpos0 = key_base + 64 * h;
          if (kpos0 + 63 > wave_pmin) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int pos = kpos0 + kt * 16 + 4 * g + i;
#pragma unroll
                for (int c = 0; c < kCols; ++c)
                  if (pos > br.row_p[c]) s[kt][c][i] = -INFINITY;
              }
          }
          // ---- running maxima, first-block references.  msh: the lane's
          // running maximum of S, a chain of 3-input maxima over its 16 keys of
          // the half (rows that did not select the block hold -inf here, C
          // being -inf).  It needs no other lane: the row's four lane groups
          // are reduced after the key loop, where the overflow test also runs.
          // Only rows taking their reference gather their row maximum; a row
          // takes it in half 0 of the first block it selected (its running
          // maximum is then this half's), so half 1 never does.
          uint64_t need_start = 0;
#pragma unroll
          for (int c = 0; c < kCols; ++c) {
            float m = msh[c];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
              m = fmaxf(fmaxf(m, s[kt][c][0]), s[kt][c][1]);
              m = fmaxf(fmaxf(m, s[kt][c][2]), s[kt][c][3]);
            }
            msh[c] = m;
            if (h == 0) need_start |= selm[c] & ~startm[c];
          }
          if (need_start) {
#pragma unroll
            for (int c = 0; c < kCols; ++c) {
              const float row_max = group4_max_swap(msh[c]);   // every lane takes part
              const bool st = __builtin_amdgcn_inverse_ballot_w64(selm[c] & ~startm[c]);
              const float delta = st ? row_max : 0.f;
#pragma unroll
              for (int kt = 0; kt < 4; ++kt) s[kt][c] -= delta;
              msh[c] -= delta;
              negm[c] -= delta;
              startm[c] |= selm[c];
              const float cv = __builtin_amdgcn_inverse_ballot_w64(selm[c]) ? negm[c] : -INFINITY;
              cinit[c] = (v4f){cv, cv, cv, cv};
            }
          }
          // ---- probabilities, row sums, bf16 B operands
          v8bf pb[2][kCols];
#pragma unroll
          for (int c = 0; c < kCols; ++c) {
            float p[4][4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                p[kt][i] = __builtin_amdgcn_exp2f(s[kt][c][i] * ck);
                lsum[c] += p[kt][i];
              }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              v8bf v;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                v[i] = (__bf16)p[2 * m][i];
                v[4 + i] = (__bf16)p[2 * m + 1][i];
              }
              pb[m][c] = v;
            }
          }
          // ---- O^T += V^T P^T
          __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
          for (int m = 0; m < 2; ++m) {
#pragma unroll
            for (int dt = 0; dt < kNdt; ++dt) {
              const v8bf va = *reinterpret_cast<const v8bf *>(vt_s + op_lane + 1024 * (4 * dt + 2 * h + m));
#pragma unroll
              for (int c = 0; c < kCols; ++c) o[dt][c] = mfma_16x16x32_bf16(va, pb[m][c], o[dt][c]);
            }
          }
          // V^T operand reads run kPvAhead MFMA groups ahead (the DMA-staged
          // configuration has the registers for more reads in flight)
          constexpr int kPvAhead = C::kPre ? 4 : 2;
          __builtin_amdgcn_sched_group_barrier(0x100, kPvAhead, 0);
          sched_mfma_then_reads<2 * kNdt - kPvAhead, kCols, 1>();
          sched_mfma_then_reads<kPvAhead, kCols, 0>();
          __builtin_amdgcn_s_setprio(0);
        }
      }
      if (it + 1 < n_iter) {
        if constexpr (C::kPre) {
          t_blk = n_blk;
#pragma unroll
          for (int c = 0; c < kCols; ++c)
            t_selm[c] = __builtin_amdgcn_ballot_w64(n_page >= 0 && br.row_ok[c] && ((m_word[c] >> (n_blk & 31)) & 1u));
        } else {
          fetch_meta(it + 1);
        }
        if (kBufs == 1) {
          lds_barrier();     // every wave is done with tile it
          store_tile(plist[it + 1], smem);
          if (it + 2 < n_iter) load_tile(plist[it + 2]);
        }
      }
      // PRE: the DMA of tile it + 1 lands before the next barrier
      if constexpr (C::kPre) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    }
    // the exact row maxima (the lanes' running maxima over the row's four
    // lane groups, back in raw units); a probability past 2^kHeadroom means
    // the reference was too far below the maximum for fp32
    bool overflow = false;
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
      overflow |= msh[c] * ck > kHeadroom;
      mraw[c] = group4_max_swap(msh[c]) - negm[c];
      msh[c] = -INFINITY;
    }
    // rare second pass: restart from the exact row maxima seen in the first one
    if (pass == 1 || !wg_or<C::kWaves>(overflow)) break;
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
      startm[c] = __builtin_amdgcn_ballot_w64(mraw[c] != -INFINITY);
      negm[c] = mraw[c] != -INFINITY ? -mraw[c] : 0.f;
      lsum[c] = 0.f;
#pragma unroll
      for (int dt = 0; dt < kNdt; ++dt) o[dt][c] = (v4f){0.f, 0.f, 0.f, 0.f};
    }
  }

  float m_ref[kCols], m_true[kCols];
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
    m_ref[c] = __builtin_amdgcn_inverse_ballot_w64(startm[c]) ? -negm[c] * ck : -INFINITY;
    m_true[c] = mraw[c] * ck;
  }
  attn_epilogue<kCols, kNdt>(a, gr, split, g, br.row_ok, br.row_t, br.row_h, o, m_ref, m_true, lsum);
}

template <class C>
size_t block_lds(const Grid &gr) {
  return (size_t)C::kMetaOff + 4 * ((size_t)(gr.NL + 1) * gr.W + 4 + 2 * (size_t)gr.W * 32);
}

template <class C>
int launch_block(const AttnArgs &a, const Grid &gr, int64_t nblocks, hipStream_t stream, const char *what) {
  const size_t lds = block_lds<C>(gr);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(attn_block_kernel<C>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return fail(FP8TS_EHIP, "sparse_attn_fwd: LDS attribute: %s", hipGetErrorString(e));
  hipLaunchKernelGGL(attn_block_kernel<C>, dim3((unsigned)nblocks), dim3(C::kThreads), lds, stream, a, gr);
  return check_launch(what);
}

}  // namespace

size_t block_prefill_lds(const Grid &gr) { return block_lds<PrefillCfg>(gr); }
int block_prefill_rows() { return PrefillCfg::kRows; }
size_t vt_page_bytes() { return kVBytes; }
int launch_block_prefill(const AttnArgs &a, const Grid &gr, int64_t nblocks, hipStream_t stream) {
  if (!gr.vt_pages) return launch_block<PrefillCfg>(a, gr, nblocks, stream, "sparse_attn_fwd (block prefill)");
  const int64_t slots = (int64_t)a.batch * a.max_blocks * a.hkv;
  hipLaunchKernelGGL(vt_pages_kernel, dim3((unsigned)slots), dim3(256), 0, stream, a, gr.vt_pages);
  if (int st = check_launch("sparse_attn_fwd (V^T pages)")) return st;
  return launch_block<PrefillPreCfg>(a, gr, nblocks, stream, "sparse_attn_fwd (block prefill)");
}

size_t block_decode_lds(const Grid &gr) { return block_lds<DecodeCfg>(gr); }
int block_decode_rows() { return DecodeCfg::kRows; }
int launch_block_decode(const AttnArgs &a, const Grid &gr, int64_t nblocks, hipStream_t stream) {
  return launch_block<DecodeCfg>(a, gr, nblocks, stream, "sparse_attn_fwd (block decode)");
}

}  // namespace fp8ts
