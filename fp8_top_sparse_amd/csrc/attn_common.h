// Pieces shared by the sparse-attention kernels: tile bookkeeping, LDS
// layouts, V staging, block-list union and the output epilogue.
//
// Semantics (all kernels): sglang PR 25751 digest, code excerpt of
// sparse_mla_q8kv8_prefill_fwd (out bf16 [s_q, h_q, d_v], max_logits and lse
// fp32 [s_q, h_q], optional attn_sink and topk_length), and sglang PR 30971
// digest, summary and implementation step 3 (q_scale folded into sm_scale,
// reaching the QK dot and the sink logit; k_scale never touching the sink;
// v_scale on the output; None = unit).
#pragma once

#include "device.h"
#include "internal.h"

namespace fp8ts {

constexpr int kPage = 128;

// A row's probabilities are taken relative to a reference maximum fixed at its
// first non-empty tile.  A later tile maximum more than kHeadroom above it
// (log2 units) could overflow fp32, so the workgroup then reruns its key loop
// once with the exact row maxima it tracked.
constexpr float kHeadroom = 64.0f;

struct Grid {
  int n_tiles;     // query tiles per sequence (block) / head groups (token)
  int splits;      // key-list splits (1 = write final outputs directly)
  int G;           // block: q heads per kv head
  int TT;          // block: tokens per tile
  int gqi;         // block: q heads per index head
  int n_il;        // block: index heads per kv head tile
  int NL;          // block: lists per workgroup
  int W;           // block: 32-bit words per block bitmap
  float *part_o;   // [splits, T, Hq, DV]
  float *part_ml;  // [splits, T, Hq, 4] = (m_ref, l, m_true, -)
  uint8_t *vt_pages;  // block prefill: [batch * max_blocks * hkv] V^T tiles (bf16, LDS operand order), or null
};

__device__ __forceinline__ v8i lds_read32(const uint8_t *p) {
  const v4i *q = reinterpret_cast<const v4i *>(p);
  v4i lo = q[0], hi = q[1];
  return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ v8i gload32(const uint8_t *p) {
  const v4i *q = reinterpret_cast<const v4i *>(p);
  v4i lo = q[0], hi = q[1];
  return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Tile-relative key held in slot j (0..7) of 16-byte V^T chunk cix (0..15):
// chunk cix = 4 * m + g serves the PV MFMA of 32-key group m for lane group g,
// whose slots j < 4 are keys 4g + j of the even 16-key S^T tile and slots
// j >= 4 keys 4g + j - 4 of the odd one.
__device__ __forceinline__ int vt_key(int cix, int j) {
  return 32 * (cix >> 2) + 16 * (j >> 2) + 4 * (cix & 3) + (j & 3);
}

__device__ __forceinline__ uint32_t bf16x2_from_e4m3(uint32_t packed, bool hi) {
  return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed, 1.0f, true)
                                         : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed, 1.0f, false));
}

// V^T tile layout (bf16): row d holds the keys of dimension d.  Keys are
// grouped in 8-byte units of 4; the unit index is XOR-swizzled with the row's
// 16-dim group (d / 16), and the row pitch is 8 bytes past a multiple of 256,
// so that the staging writes (lanes spread over dim groups) and the MFMA
// operand reads (lanes spread over 16 consecutive rows) hit distinct banks.
__device__ __forceinline__ int vt_offset(int vpitch, int d, int key4) {
  return d * vpitch + 8 * (key4 ^ ((d >> 4) & 7));
}

// Write one 4-key x 16-dim unit of V (e4m3 rows w[0..3], 16 bytes each, keys
// 4*kg .. 4*kg+3) into V^T.
__device__ __forceinline__ void stage_v_regs(uint8_t *vt, int vpitch, int kg, int d0, const v4i *w) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {       // dword q covers dims d0 + 4q .. 4q + 3
    v4bf c0 = e4m3x4_to_bf16(w[0][q]);
    v4bf c1 = e4m3x4_to_bf16(w[1][q]);
    v4bf c2 = e4m3x4_to_bf16(w[2][q]);
    v4bf c3 = e4m3x4_to_bf16(w[3][q]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v4bf colv = {c0[j], c1[j], c2[j], c3[j]};
      *reinterpret_cast<v4bf *>(vt + vt_offset(vpitch, d0 + 4 * q + j, kg)) = colv;
    }
  }
}

// Block-mode workgroup tile: ROWS rows = TT tokens x G q heads of one kv head.
template <int COLS>
struct BlockRows {
  int b, kvh, cu0, q_len, seq_len, t0;
  int row_t[COLS], row_h[COLS], row_p[COLS], row_li[COLS];
  bool row_ok[COLS];
};

// Decodes the workgroup's (sequence, tile, kv head), fills the lane's row
// metadata for its COLS column tiles (rows (wave * COLS + c) * 16 + col), and
// returns false when the tile holds no query of its sequence (uniform).
template <int COLS>
__device__ __forceinline__ bool block_rows(const AttnArgs &a, const Grid &gr, int bid, int wave, int col,
                                           BlockRows<COLS> &r) {
  r.kvh = bid % a.hkv;
  bid /= a.hkv;
  r.b = bid % a.batch;
  const int tile = gr.n_tiles - 1 - bid / a.batch;      // heavy (late) tiles first
  // sequence range, clamped to [0, total_q) whatever the device metadata holds
  r.cu0 = min(max(a.cu_seqlens_q[r.b], 0), a.total_q);
  r.q_len = min(max(a.cu_seqlens_q[r.b + 1] - r.cu0, 0), a.total_q - r.cu0);
  r.seq_len = a.seq_lens[r.b];
  r.t0 = tile * gr.TT;
  if (r.t0 >= r.q_len) return false;
  const int gi_lo = (r.kvh * gr.G) / gr.gqi;
#pragma unroll
  for (int c = 0; c < COLS; ++c) {
    const int row = (wave * COLS + c) * 16 + col;
    const int tt = r.t0 + row / gr.G;
    const int h = r.kvh * gr.G + row % gr.G;
    // rows past TT * G (when G does not divide the tile) belong to no token
    r.row_ok[c] = (row / gr.G) < gr.TT && tt < r.q_len;
    r.row_t[c] = r.cu0 + tt;
    r.row_h[c] = h;
    r.row_p[c] = r.row_ok[c] ? r.seq_len - r.q_len + tt : -1;
    r.row_li[c] = r.row_ok[c] ? (row / gr.G) * gr.n_il + (h / gr.gqi - gi_lo) : 0;
  }
  return true;
}

// Builds, in LDS, one bitmap per (token, index head) list of the tile and the
// ascending union of all its block ids.  bits: [(NL + 1) * W] words, then the
// union count and the union list.  Ids outside [0, max_blocks) and blocks with
// no key visible to the list's token are dropped (set semantics).  Returns the
// union size.  Every thread of the workgroup must call it.
template <int NT>
__device__ __forceinline__ int block_union(const AttnArgs &a, const Grid &gr, int kvh, int cu0, int q_len,
                                           int seq_len, int t0, uint32_t *bits, int32_t *ucount,
                                           int32_t *ulist) {
  const int tid = thread_index(), lane = tid & 63, wave = tid >> 6;
  const int64_t T = a.total_q;
  uint32_t *ubits = bits + gr.NL * gr.W;
  const int gi_lo = (kvh * gr.G) / gr.gqi;
  for (int w = tid; w < (gr.NL + 1) * gr.W; w += NT) bits[w] = 0u;
  __syncthreads();
  const int nsel = gr.NL * a.topk;
  for (int e = tid; e < nsel; e += NT) {
    const int li = e / a.topk;
    const int j = e - li * a.topk;
    const int tt = t0 + li / gr.n_il;
    const int gi = gi_lo + li % gr.n_il;
    if (tt >= q_len) continue;
    const int p = seq_len - q_len + tt;
    const int id = a.indices[((int64_t)gi * T + cu0 + tt) * a.topk + j];
    if (id < 0 || id >= a.max_blocks || (int64_t)id * kPage > p) continue;
    atomicOr(&bits[li * gr.W + (id >> 5)], 1u << (id & 31));
    atomicOr(&ubits[id >> 5], 1u << (id & 31));
  }
  __syncthreads();
  // wave 0: exclusive scan of the union words' popcounts, then emit ids ascending
  if (wave == 0) {
    int running = 0;
    for (int w0 = 0; w0 < gr.W; w0 += 64) {
      const int w = w0 + lane;
      const uint32_t word = w < gr.W ? ubits[w] : 0u;
      const int cnt = __popc(word);
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
      }
      int pos = running + incl - cnt;
      uint32_t m = word;
      while (m) {
        const int bit = __ffs(m) - 1;
        ulist[pos++] = w * 32 + bit;
        m &= m - 1;
      }
      running += __shfl(incl, 63, 64);
    }
    if (lane == 0) ucount[0] = running;
  }
  __syncthreads();
  return ucount[0];
}

// Writes the lane's rows: final outputs (splits == 1) or split partials.
//   O relative to m_ref (log2 units), l_part = the lane's share of the row sum.
template <int COLS, int NDT>
__device__ __forceinline__ void attn_epilogue(const AttnArgs &a, const Grid &gr, int split, int g,
                                              const bool (&row_ok)[COLS], const int (&row_t)[COLS],
                                              const int (&row_h)[COLS], v4f (&o)[NDT][COLS],
                                              const float (&m_ref)[COLS], const float (&m_true)[COLS],
                                              const float (&l_part)[COLS]) {
  constexpr int DV = NDT * 16;
  const int64_t T = a.total_q;
#pragma unroll
  for (int c = 0; c < COLS; ++c) {
    const float l_tot = group4_sum(l_part[c]);
    if (!row_ok[c]) continue;
    const int64_t rowidx = (int64_t)row_t[c] * a.hq + row_h[c];
    if (gr.splits > 1) {
      float *po = gr.part_o + ((int64_t)split * T * a.hq + rowidx) * DV;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<v4f *>(po + dt * 16 + 4 * g) = o[dt][c];
      if (g == 0) {
        float *pm = gr.part_ml + ((int64_t)split * T * a.hq + rowidx) * 4;
        *reinterpret_cast<v4f *>(pm) = (v4f){m_ref[c], l_tot, m_true[c], 0.f};
      }
      continue;
    }
    const bool has_sink = a.sink != nullptr;
    const float zs = has_sink ? a.sink_scale_log2 * a.sink[row_h[c]] : -INFINITY;
    const float M = fmaxf(m_ref[c], zs);
    float Lt = 0.f, fo = 0.f;
    if (M != -INFINITY) {
      const float wk = m_ref[c] == -INFINITY ? 0.f : exp2f(m_ref[c] - M);
      Lt = l_tot * wk + (has_sink ? exp2f(zs - M) : 0.f);
      fo = Lt > 0.f ? wk * a.v_scale / Lt : 0.f;
    }
    uint16_t *orow = a.out + rowidx * DV;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const v4f x = o[dt][c] * fo;
      uint2 pk = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
      *reinterpret_cast<uint2 *>(orow + dt * 16 + 4 * g) = pk;
    }
    if (g == 0) {
      a.lse[rowidx] = Lt > 0.f ? (M + log2f(Lt)) * kLn2 : -INFINITY;
      a.max_logits[rowidx] = m_true[c] * kLn2;
    }
  }
}

// Block-mode kernels with pipelined K/V tiles (attention_block.hip): prefill
// (256-row tiles, double-buffered) and decode (small single-buffered tiles).
constexpr size_t kMaxLds = 160 * 1024;   // LDS per workgroup on gfx950
size_t block_prefill_lds(const Grid &gr);
int block_prefill_rows();
size_t vt_page_bytes();   // one pre-converted V^T tile
int launch_block_prefill(const AttnArgs &a, const Grid &gr, int64_t nblocks, hipStream_t stream);
size_t block_decode_lds(const Grid &gr);
int block_decode_rows();
int launch_block_decode(const AttnArgs &a, const Grid &gr, int64_t nblocks, hipStream_t stream);
// Block-mode decode with every wave streaming its own blocks
// (attention_decode.hip): one 16-row tile (tokens x q heads of one kv head).
size_t block_stream_decode_lds(const Grid &gr);
int launch_block_stream_decode(const AttnArgs &a, const Grid &gr, int64_t nblocks, hipStream_t stream);
// Token-mode MLA kernel with pipelined K/V tiles (attention_token.hip): 128 q
// heads of one token per workgroup.  token_mla_fits: the caches are small
// enough for its 32-bit byte offsets.
size_t token_mla_lds(int topk, int splits);
int token_mla_rows();
bool token_mla_fits(const AttnArgs &a);
int launch_token_mla(const AttnArgs &a, const Grid &gr, int64_t nblocks, hipStream_t stream);
// Token-mode MLA kernel for the latent layout, V = the leading 512 bytes of
// each K row (attention_latent.hip): only K is staged, and PV runs on e4m3
// MFMA with P as a hi + lo pair of e4m3 codes.
size_t token_latent_lds(int topk, int splits);
bool token_latent_fits(const AttnArgs &a, int splits);
int launch_token_latent(const AttnArgs &a, const Grid &gr, int64_t nblocks, hipStream_t stream);

}  // namespace fp8ts
