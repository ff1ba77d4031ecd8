// Sparse attention forward over selected KV tokens (token mode) or blocks
// (block mode), e4m3 Q/K/V, bf16 output, fp32 max_logits / lse.
//
// Semantics: sglang PR 25751 digest (code excerpt of
// sparse_mla_q8kv8_prefill_fwd: out [s_q, h_q, d_v] bf16, max_logits and lse
// [s_q, h_q] fp32, optional attn_sink and topk_length, d_v = 512 for MLA) and
// sglang PR 30971 digest (summary and implementation step 3: q_scale folded
// into sm_scale so it scales the QK dot and the sink logit, k_scale never
// touches the sink, v_scale on the output, None = unit).
//
// Design (gfx950, wave64):
//  * A workgroup owns ROWS = WAVES * COLS * 16 query rows.  Block mode: rows
//    are (token, head) pairs of one KV head (all heads sharing that KV head,
//    for a tile of consecutive tokens), so one staged K/V block serves every
//    row; token mode: rows are the heads of one query token, which share its
//    index list.
//  * Keys are staged in LDS per tile (block mode: one 128-token page of one KV
//    head, 16 KB contiguous; token mode: 64 gathered KV rows).  V is widened
//    to bf16 and transposed on the way into LDS so that the PV operand is
//    key-contiguous.
//  * S^T = K Q^T on 16x16x128 e4m3 MFMA (plus 16x16x32 e4m3 for the 64-wide
//    tail of d_qk = 576): each lane then holds 4 keys of one query row, which
//    is exactly the B-operand layout of the PV product, so P never leaves
//    registers.  PV runs on 16x16x32 bf16 MFMA with P in bf16: rounding P to
//    e4m3 (the pages' design) costs ~3% of max|out|, above the 2e-2 budget.
//  * Online softmax in the log2 domain with lazy rescaling: the reference
//    maximum only moves when a new tile maximum exceeds it by 2^8, so most
//    tiles skip the accumulator rescale.  The row sum L is accumulated from
//    the fp32 probabilities.
//  * Block mode: every row's block list becomes an LDS bitmap; the workgroup
//    walks the union of its rows' lists in ascending order and masks rows
//    that did not select the current block.  Keys j > p are masked (causal).
//  * Decode and small token-mode workloads split the key list across
//    workgroups; partial (O, m, l) go to the workspace and a combine kernel
//    merges them by log-sum-exp.
#include "attn_common.h"

namespace fp8ts {
namespace {

// block-mode prefill whose block bitmaps leave no room for the pipelined
// kernel's two K/V buffers: 8 waves x 32 rows per 256-row workgroup
constexpr int kPrefillWaves = 8;

// Dynamic LDS layout sizes.
template <int DQK, int DV, int KT>
struct Lds {
  static constexpr int KP = DQK + 16;          // K row pitch (bytes)
  static constexpr int VP = 2 * KT + 8;        // V^T row pitch (bytes), see vt_offset
  static_assert(KT / 4 >= 8, "the V^T swizzle needs at least 8 key units per row");
  static constexpr int K_BYTES = KT * KP;
  static constexpr int V_BYTES = DV * VP;
  static constexpr int IDX_OFF = K_BYTES + V_BYTES;
  static constexpr int BASE = IDX_OFF + KT * 4;
};

template <int DQK, int DV, int WAVES, int COLS, int KT, bool BLOCK>
__global__ __launch_bounds__(WAVES * 64) void attn_kernel(AttnArgs a, Grid gr) {
  static_assert(DQK % 128 == 0 || DQK % 128 == 64, "d_qk must be a multiple of 64");
  static_assert(DV % 16 == 0 && KT % 64 == 0, "tile shape");
  constexpr int NT = WAVES * 64;
  constexpr int NKC = DQK / 128;               // full 128-wide K slices
  constexpr bool TAIL = (DQK % 128) == 64;
  constexpr int NDT = DV / 16;
  using L = Lds<DQK, DV, KT>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t *kt_s = smem;
  uint8_t *vt_s = smem + L::K_BYTES;
  int32_t *idx_s = reinterpret_cast<int32_t *>(smem + L::IDX_OFF);

  const int tid = thread_index();
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int col = lane & 15;
  const int64_t T = a.total_q;

  // ---------------------------------------------------------------- work item
  int bid = block_index();
  const int split = bid % gr.splits;
  bid /= gr.splits;

  // per-row metadata for the lane's column in each of its column tiles
  int row_t[COLS], row_h[COLS], row_p[COLS], row_li[COLS];
  bool row_ok[COLS];

  // block mode
  int b = 0, kvh = 0, cu0 = 0, q_len = 0, seq_len = 0, t0 = 0;
  uint32_t *bits = nullptr;      // [NL][W] list bitmaps, then [W] union
  int32_t *ulist = nullptr;      // ascending union of block ids
  int32_t *ucount = nullptr;
  // token mode
  int tok = 0, list_len = 0;

  int range_lo = 0, range_hi = 0;  // positions (union list / index list) of this split

  if constexpr (BLOCK) {
    BlockRows<COLS> br;
    if (!block_rows<COLS>(a, gr, bid, wave, col, br)) return;
    b = br.b;
    kvh = br.kvh;
    cu0 = br.cu0;
    q_len = br.q_len;
    seq_len = br.seq_len;
    t0 = br.t0;
#pragma unroll
    for (int c = 0; c < COLS; ++c) {
      row_ok[c] = br.row_ok[c];
      row_t[c] = br.row_t[c];
      row_h[c] = br.row_h[c];
      row_p[c] = br.row_p[c];
      row_li[c] = br.row_li[c];
    }
    bits = reinterpret_cast<uint32_t *>(smem + L::BASE);
    ucount = reinterpret_cast<int32_t *>(bits + (gr.NL + 1) * gr.W);
    ulist = ucount + 4;
    const int U = block_union<NT>(a, gr, kvh, cu0, q_len, seq_len, t0, bits, ucount, ulist);
    const int chunk = (U + gr.splits - 1) / gr.splits;
    range_lo = min(U, split * chunk);
    range_hi = min(U, range_lo + chunk);
  } else {
    const int hg = bid % gr.n_tiles;
    tok = bid / gr.n_tiles;
#pragma unroll
    for (int c = 0; c < COLS; ++c) {
      const int r = (wave * COLS + c) * 16 + col;
      const int h = hg * (WAVES * COLS * 16) + r;
      row_ok[c] = h < a.hq;
      row_t[c] = tok;
      row_h[c] = h;
      row_p[c] = 0;
      row_li[c] = 0;
    }
    list_len = a.topk;
    if (a.topk_length) list_len = max(0, min(a.topk, a.topk_length[tok]));
    const int chunk = ((list_len + gr.splits - 1) / gr.splits + KT - 1) / KT * KT;
    range_lo = min(list_len, split * chunk);
    range_hi = min(list_len, range_lo + chunk);
  }

  // ---------------------------------------------------------------- Q operands
  v8i qb[COLS][NKC > 0 ? NKC : 1];
  long qt[COLS][2];
#pragma unroll
  for (int c = 0; c < COLS; ++c) {
    const int64_t qr = row_ok[c] ? (int64_t)row_t[c] * a.hq + row_h[c] : 0;
    const uint8_t *qrow = a.q + qr * DQK;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      qb[c][kc] = row_ok[c] ? gload32(qrow + 128 * kc + 32 * g) : (v8i){0, 0, 0, 0, 0, 0, 0, 0};
    }
    if constexpr (TAIL) {
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        qt[c][mm] = row_ok[c] ? *reinterpret_cast<const long *>(qrow + NKC * 128 + 32 * mm + 8 * g) : 0;
      }
    }
  }

  // ---------------------------------------------------------------- state
  v4f o[NDT][COLS];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int c = 0; c < COLS; ++c) o[dt][c] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_used[COLS], m_true[COLS], lsum[COLS];
#pragma unroll
  for (int c = 0; c < COLS; ++c) {
    m_used[c] = -INFINITY;
    m_true[c] = -INFINITY;
    lsum[c] = 0.f;
  }
  const float ck = a.key_scale_log2;

  // ---------------------------------------------------------------- key tiles
  const int n_iter = BLOCK ? (range_hi - range_lo) : (range_hi - range_lo + KT - 1) / KT;

  // Block mode stages tile it+1 from HBM into registers while tile it is being
  // computed (one page of one KV head: K and V are 16 KB contiguous each).
  constexpr int K_CHUNKS = KT * (DQK / 16);            // 16-byte chunks of K
  constexpr int K_PER = BLOCK ? (K_CHUNKS + NT - 1) / NT : 1;
  constexpr int V_UNITS = (KT / 4) * (DV / 16);        // 4-key x 16-dim units of V
  constexpr int V_PER = BLOCK ? (V_UNITS + NT - 1) / NT : 1;
  v4i kreg[K_PER];
  v4i vreg[V_PER][4];
  int cur_page = -1, next_page = -1;

  auto page_of = [&](int it) -> int {
    const int blk = ulist[range_lo + it];
    const int page = a.block_table[(int64_t)b * a.max_blocks + blk];
    return (page >= 0 && page < a.num_kv) ? page : -1;
  };
  auto issue_block_loads = [&](int page) {
    if (page < 0) return;
    const uint8_t *kp = a.k + ((int64_t)page * a.hkv + kvh) * kPage * DQK;
    const uint8_t *vp = a.v + ((int64_t)page * a.hkv + kvh) * kPage * DV;
#pragma unroll
    for (int j = 0; j < K_PER; ++j) {
      const int ch = tid + j * NT;
      if (ch < K_CHUNKS) kreg[j] = *reinterpret_cast<const v4i *>(kp + 16 * ch);
    }
#pragma unroll
    for (int j = 0; j < V_PER; ++j) {
      const int u = tid + j * NT;
      if (u < V_UNITS) {
        const int kg = u / (DV / 16);
        const int dg = u - kg * (DV / 16);
        const uint8_t *r = vp + (4 * kg) * DV + 16 * dg;
#pragma unroll
        for (int q = 0; q < 4; ++q) vreg[j][q] = *reinterpret_cast<const v4i *>(r + q * DV);
      }
    }
  };

  for (int pass = 0; pass < 2; ++pass) {
  bool overflow = false;
  if constexpr (BLOCK) {
    if (n_iter > 0) {
      next_page = page_of(0);
      issue_block_loads(next_page);
    }
  }

  for (int it = 0; it < n_iter; ++it) {
    int key_base = 0;        // absolute key position of tile row 0 (block mode)
    int n_valid_keys = KT;
    __syncthreads();         // previous tile fully consumed
    if constexpr (BLOCK) {
      cur_page = next_page;
      key_base = ulist[range_lo + it] * kPage;
      if (cur_page >= 0) {
#pragma unroll
        for (int j = 0; j < K_PER; ++j) {
          const int ch = tid + j * NT;
          if (ch < K_CHUNKS) {
            const int key = ch / (DQK / 16);
            const int part = ch - key * (DQK / 16);
            *reinterpret_cast<v4i *>(kt_s + key * L::KP + 16 * part) = kreg[j];
          }
        }
#pragma unroll
        for (int j = 0; j < V_PER; ++j) {
          const int u = tid + j * NT;
          if (u < V_UNITS) {
            const int kg = u / (DV / 16);
            const int dg = u - kg * (DV / 16);
            stage_v_regs(vt_s, L::VP, kg, 16 * dg, vreg[j]);
          }
        }
      }
      __syncthreads();
      if (it + 1 < n_iter) {
        next_page = page_of(it + 1);
        issue_block_loads(next_page);   // in flight during this tile's compute
      }
      if (cur_page < 0) continue;       // uniform: the block has no keys
    } else {
      const int pos0 = range_lo + it * KT;
      for (int j = tid; j < KT; j += NT) {
        int id = -1;
        if (pos0 + j < range_hi) {
          id = a.indices[(int64_t)tok * a.topk + pos0 + j];
          if (id < 0 || id >= a.num_kv) id = -1;
        }
        idx_s[j] = id;
      }
      n_valid_keys = wg_count<WAVES>(tid < KT && idx_s[tid < KT ? tid : 0] >= 0);
      for (int ch = tid; ch < KT * (DQK / 16); ch += NT) {
        const int key = ch / (DQK / 16);
        const int part = ch - key * (DQK / 16);
        const int id = idx_s[key];
        v4i val = {0, 0, 0, 0};
        if (id >= 0) val = *reinterpret_cast<const v4i *>(a.k + (int64_t)id * a.k_row_stride + 16 * part);
        *reinterpret_cast<v4i *>(kt_s + key * L::KP + 16 * part) = val;
      }
      for (int u = tid; u < (KT / 4) * (DV / 16); u += NT) {
        const int kg = u / (DV / 16);
        const int dg = u - kg * (DV / 16);
        v4i rows[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int id = idx_s[4 * kg + q];
          // absent keys read row 0 (any finite bytes); their P is exactly 0
          rows[q] = *reinterpret_cast<const v4i *>(a.v + (int64_t)(id >= 0 ? id : 0) * a.v_row_stride + 16 * dg);
        }
        stage_v_regs(vt_s, L::VP, kg, 16 * dg, rows);
      }
      __syncthreads();
    }

    // rows taking part in this tile, and their last visible key position
    bool rsel[COLS];
    int rp[COLS];
#pragma unroll
    for (int c = 0; c < COLS; ++c) {
      if constexpr (BLOCK) {
        const int blk = key_base / kPage;
        rsel[c] = row_ok[c] && ((bits[row_li[c] * gr.W + (blk >> 5)] >> (blk & 31)) & 1u);
        rp[c] = row_p[c];
      } else {
        rsel[c] = row_ok[c];
        rp[c] = 0x7fffffff;
      }
    }
    bool any_sel = false;
#pragma unroll
    for (int c = 0; c < COLS; ++c) any_sel |= rsel[c];
    if (!__any(any_sel)) continue;      // uniform per wave; no barrier until the next tile

#pragma unroll 1
    for (int koff = 0; koff < KT; koff += 64) {
      // ---- S^T = K Q^T for 64 keys
      v4f s[4][COLS];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int c = 0; c < COLS; ++c) s[kt][c] = (v4f){0.f, 0.f, 0.f, 0.f};
        const uint8_t *krow = kt_s + (koff + kt * 16 + col) * L::KP;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          const v8i ka = lds_read32(krow + 128 * kc + 32 * g);
#pragma unroll
          for (int c = 0; c < COLS; ++c) s[kt][c] = mfma_16x16x128_e4m3(ka, qb[c][kc], s[kt][c]);
        }
        if constexpr (TAIL) {
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            const long ka = *reinterpret_cast<const long *>(krow + NKC * 128 + 32 * mm + 8 * g);
#pragma unroll
            for (int c = 0; c < COLS; ++c) s[kt][c] = mfma_16x16x32_e4m3(ka, qt[c][mm], s[kt][c]);
          }
        }
      }
      // ---- masks, only where some row of the wave needs one
      if constexpr (BLOCK) {
        const int kpos0 = key_base + koff;
        bool part = false;
#pragma unroll
        for (int c = 0; c < COLS; ++c) part |= rsel[c] && rp[c] < kpos0 + 63;
        if (__any(part)) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int pos = kpos0 + kt * 16 + 4 * g + i;
#pragma unroll
              for (int c = 0; c < COLS; ++c)
                if (pos > rp[c]) s[kt][c][i] = -INFINITY;
            }
        }
      } else {
        if (n_valid_keys < KT) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (idx_s[koff + kt * 16 + 4 * g + i] < 0) {
#pragma unroll
                for (int c = 0; c < COLS; ++c) s[kt][c][i] = -INFINITY;
              }
            }
        }
      }
      // ---- online softmax (log2 domain, fixed per-row reference maximum)
#pragma unroll
      for (int c = 0; c < COLS; ++c) {
        float smax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          smax = fmaxf(fmaxf(smax, fmaxf(s[kt][c][0], s[kt][c][1])), fmaxf(s[kt][c][2], s[kt][c][3]));
        smax = group4_max(smax);
        const float mt = rsel[c] ? smax * ck : -INFINITY;
        m_true[c] = fmaxf(m_true[c], mt);
        m_used[c] = m_used[c] == -INFINITY ? mt : m_used[c];   // O and L are still 0 here
        overflow |= mt > m_used[c] + kHeadroom;
      }
      v8bf pb[COLS][2];
#pragma unroll
      for (int c = 0; c < COLS; ++c) {
        // rows not in this tile subtract +inf: every probability is exactly 0
        const float msub = !rsel[c] ? INFINITY : (m_used[c] == -INFINITY ? 0.f : m_used[c]);
        float p[4][4];
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[kt][i] = __builtin_amdgcn_exp2f(fmaf(s[kt][c][i], ck, -msub));
            ls += p[kt][i];
          }
        lsum[c] += ls;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          v8bf v;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[i] = (__bf16)p[2 * m][i];
            v[4 + i] = (__bf16)p[2 * m + 1][i];
          }
          pb[c][m] = v;
        }
      }
      // ---- O^T += V^T P^T (bf16 MFMA, 32 keys per step)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int u = koff / 4 + 8 * m + g;      // key units {u, u + 4} of this lane group
          const v4bf lo = *reinterpret_cast<const v4bf *>(vt_s + vt_offset(L::VP, dt * 16 + col, u));
          const v4bf hi = *reinterpret_cast<const v4bf *>(vt_s + vt_offset(L::VP, dt * 16 + col, u + 4));
          const v8bf va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int c = 0; c < COLS; ++c) o[dt][c] = mfma_16x16x32_bf16(va, pb[c][m], o[dt][c]);
        }
      }
    }
  }
  // rare second pass: restart from the exact row maxima seen in the first one
  if (pass == 1 || !wg_or<WAVES>(overflow)) break;
#pragma unroll
  for (int c = 0; c < COLS; ++c) {
    m_used[c] = m_true[c];
    lsum[c] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt][c] = (v4f){0.f, 0.f, 0.f, 0.f};
  }
  }  // pass

  // ---------------------------------------------------------------- epilogue
  attn_epilogue<COLS, NDT>(a, gr, split, g, row_ok, row_t, row_h, o, m_used, m_true, lsum);
}

// Merge split partials: out = v_scale * sum_s O_s 2^(m_s - M) / L.
template <int DV>
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a, Grid gr) {
  // one workgroup per (token, head) row; thread i owns DV / 128 consecutive dims
  constexpr int VPT = DV / 128;
  static_assert(VPT == 1 || VPT == 4, "combine: 128 or 512 output dims");
  const int64_t rowidx = block_index();            // t * hq + h
  const int h = (int)(rowidx % a.hq);
  const int64_t TH = (int64_t)a.total_q * a.hq;
  const bool has_sink = a.sink != nullptr;
  const float zs = has_sink ? a.sink_scale_log2 * a.sink[h] : -INFINITY;
  float M = zs, mtrue = -INFINITY;
  for (int s = 0; s < gr.splits; ++s) {
    const v4f pm = *reinterpret_cast<const v4f *>(gr.part_ml + (s * TH + rowidx) * 4);
    M = fmaxf(M, pm[0]);
    mtrue = fmaxf(mtrue, pm[2]);
  }
  // every split's weight exp2(m_s - M) once, then the dims with 16-byte loads
  float Lt = 0.f;
  float acc[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) acc[j] = 0.f;
  const int d0 = thread_index() * VPT;
  if (M != -INFINITY) {
    for (int s = 0; s < gr.splits; ++s) {
      const v4f pm = *reinterpret_cast<const v4f *>(gr.part_ml + (s * TH + rowidx) * 4);
      if (pm[0] == -INFINITY) continue;
      const float w = exp2f(pm[0] - M);
      Lt += pm[1] * w;
      const float *po = gr.part_o + (s * TH + rowidx) * DV + d0;
      if constexpr (VPT == 4) {
        const v4f x = *reinterpret_cast<const v4f *>(po);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += x[j] * w;
      } else {
        acc[0] += po[0] * w;
      }
    }
    if (has_sink) Lt += exp2f(zs - M);
  }
  const float scale = Lt > 0.f ? a.v_scale / Lt : 0.f;
  uint16_t *orow = a.out + rowidx * DV + d0;
  if constexpr (VPT == 4) {
    *reinterpret_cast<uint2 *>(orow) =
        make_uint2(pack_bf16x2(acc[0] * scale, acc[1] * scale), pack_bf16x2(acc[2] * scale, acc[3] * scale));
  } else {
    orow[0] = __builtin_bit_cast(uint16_t, (__bf16)(acc[0] * scale));
  }
  if (thread_index() == 0) {
    a.lse[rowidx] = Lt > 0.f ? (M + log2f(Lt)) * kLn2 : -INFINITY;
    a.max_logits[rowidx] = mtrue * kLn2;
  }
}

// ---------------------------------------------------------------- host side
constexpr int kDecodeChunk = 32;   // union blocks per tile-decode workgroup
constexpr int kStreamChunk = 64;   // most union blocks per streamed-decode workgroup
constexpr int kStreamMin = 8;      // fewest union blocks per streamed-decode workgroup
constexpr int kCUs = 256;          // compute units of an MI355X

struct Plan {
  int kind;   // 0 block prefill (single-buffered), 2 token 128 heads, 3 token 16 heads,
              // 4 block prefill, pipelined, 5 block decode, tile kernel,
              // 6 token 128 heads, pipelined, 7 block decode, streamed per wave
  Grid gr;
  int64_t nblocks;
  size_t lds;
  size_t ws;
  size_t vt_bytes;   // block prefill: pre-converted V^T tiles in the workspace (0: converted in the kernel)
};

template <int DQK, int DV, int KT>
constexpr size_t lds_base() { return Lds<DQK, DV, KT>::BASE; }

Plan make_plan(int mode, int batch, int total_q, int max_q_len, int hq, int hkv, int hidx,
               int dv, int topk, int max_blocks) {
  Plan pl{};
  Grid &gr = pl.gr;
  gr.splits = 1;
  if (mode == FP8TS_BLOCK_MODE) {
    gr.G = hq / hkv;
    gr.gqi = hq / hidx;
    gr.W = (max_blocks + 31) / 32;
    // few query rows per sequence (decode): tiles of at most 64 rows whose
    // block union is split across workgroups to fill the GPU
    const bool decode = (int64_t)max_q_len * gr.G <= 64;
    const int rows = decode ? block_decode_rows() : block_prefill_rows();
    gr.TT = rows / gr.G;
    if (gr.TT < 1) gr.TT = 1;
    gr.n_tiles = (max_q_len + gr.TT - 1) / gr.TT;
    // index heads touched by the q heads of one kv head
    gr.n_il = gr.G >= gr.gqi ? gr.G / gr.gqi : 1;
    gr.NL = gr.TT * gr.n_il;
    if (decode) {
      // decode tiles (at most 64 rows): the tile kernel streams ~kDecodeChunk
      // blocks of the union per workgroup (small single-buffered tiles,
      // several workgroups per CU); its LDS fits any table of up to 4096
      // blocks
      pl.kind = 5;
      int ubound = gr.n_il * (gr.TT < max_q_len ? gr.TT : max_q_len) * topk;
      if (ubound > max_blocks) ubound = max_blocks;
      gr.splits = (ubound + kDecodeChunk - 1) / kDecodeChunk;
      if (gr.splits < 1) gr.splits = 1;
      pl.nblocks = (int64_t)gr.splits * batch * hkv * gr.n_tiles;
      pl.lds = block_decode_lds(gr);
      // decode tiles of at most 16 rows: the streamed decode kernel, every
      // wave walking its own share of ~kStreamChunk blocks of the union
      if (gr.G <= 16 && 16 % gr.G == 0 && (int64_t)max_q_len * gr.G <= 16) {
        Grid sg = gr;
        sg.TT = 16 / sg.G;
        sg.n_tiles = (max_q_len + sg.TT - 1) / sg.TT;
        sg.NL = sg.TT * sg.n_il;
        int sbound = sg.n_il * (sg.TT < max_q_len ? sg.TT : max_q_len) * topk;
        if (sbound > max_blocks) sbound = max_blocks;
        // one workgroup per CU (each holds 128 KB of LDS), but no fewer
        // than kStreamMin and no more than kStreamChunk blocks per workgroup
        const int64_t tiles = (int64_t)batch * hkv * sg.n_tiles;
        const int64_t want = (kCUs + tiles - 1) / tiles;
        const int64_t most = (sbound + kStreamMin - 1) / kStreamMin;
        int64_t sp = want < most ? want : most;
        const int64_t least = (sbound + kStreamChunk - 1) / kStreamChunk;
        if (sp < least) sp = least;
        sg.splits = sp < 1 ? 1 : (int)sp;
        if (block_stream_decode_lds(sg) <= kMaxLds) {
          gr = sg;
          pl.kind = 7;
          pl.nblocks = (int64_t)gr.splits * batch * hkv * gr.n_tiles;
          pl.lds = block_stream_decode_lds(gr);
        }
      }
    } else {
      pl.kind = 0;
      pl.nblocks = (int64_t)batch * hkv * gr.n_tiles;
      pl.lds = lds_base<128, 128, 128>() + 4 * ((size_t)(gr.NL + 1) * gr.W + 4 + (size_t)gr.W * 32);
    }
    // prefill tiles go to the pipelined kernel when its LDS fits; otherwise
    // (block tables of about 4000 blocks) to the single-buffered one, whose
    // tiles are the same 256 rows
    if (pl.kind == 0 && block_prefill_lds(gr) <= kMaxLds) {
      pl.kind = 4;
      pl.lds = block_prefill_lds(gr);
      // sequences spanning several tiles visit each page many times over:
      // convert every V page to its V^T tile once, up front
      const size_t vt = (size_t)batch * max_blocks * hkv * vt_page_bytes();
      if (gr.n_tiles >= 4 && vt <= ((size_t)1 << 30)) pl.vt_bytes = vt;
    }
  } else {
    if (hq % token_mla_rows() == 0) {
      // 128 heads per workgroup; few tokens split their lists so that the
      // grid still covers the GPU (at least 256 keys per split)
      gr.n_tiles = hq / token_mla_rows();
      const int64_t wgs = (int64_t)total_q * gr.n_tiles;
      gr.splits = 1;
      if (wgs < 256) {
        const int want = (int)((256 + wgs - 1) / wgs);
        const int most = topk / 256 > 1 ? topk / 256 : 1;
        gr.splits = want < most ? want : most;
      }
      pl.kind = 6;
      pl.lds = token_mla_lds(topk, gr.splits);
      if (pl.lds > kMaxLds) {
        pl.kind = 2;
        pl.lds = lds_base<576, 512, 64>();
      }
    } else if (hq % 128 == 0) {
      pl.kind = 2;
      gr.n_tiles = hq / 128;
      gr.splits = 1;
      pl.lds = lds_base<576, 512, 64>();
    } else {
      pl.kind = 3;
      gr.n_tiles = (hq + 15) / 16;
      // split the list so that tiny workloads still fill the GPU
      const int per = (topk + 63) / 64;
      gr.splits = per > 8 ? 8 : per;
      if ((int64_t)total_q * gr.n_tiles >= 2048) gr.splits = 1;
      pl.lds = lds_base<576, 512, 64>();
    }
    pl.nblocks = (int64_t)gr.splits * total_q * gr.n_tiles;
  }
  if (gr.splits > 1) {
    pl.ws = (size_t)gr.splits * total_q * hq * dv * 4 + (size_t)gr.splits * total_q * hq * 16 + 256;
  }
  pl.ws += pl.vt_bytes;   // V^T tiles after the partials (256-byte aligned)
  return pl;
}

template <typename K>
int launch_k(K kern, const Plan &pl, int threads, const AttnArgs &a, hipStream_t stream) {
  if (pl.lds > kMaxLds)
    return fail(FP8TS_EUNSUPPORTED, "sparse_attn_fwd: block lists need %zu bytes of LDS (limit %zu); "
                "use fewer blocks per sequence or more q heads per kv head", pl.lds, kMaxLds);
  if (pl.lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)pl.lds);
    if (e != hipSuccess) return fail(FP8TS_EHIP, "sparse_attn_fwd: LDS attribute: %s", hipGetErrorString(e));
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)pl.nblocks), dim3(threads), pl.lds, stream, a, pl.gr);
  return check_launch("sparse_attn_fwd");
}

}  // namespace

size_t attn_workspace_bytes(int32_t mode, int32_t batch, int32_t total_q, int32_t max_q_len,
                            int32_t hq, int32_t hkv, int32_t hidx, int32_t dv, int32_t topk,
                            int32_t max_blocks) {
  return make_plan(mode, batch, total_q, max_q_len, hq, hkv, hidx, dv, topk, max_blocks).ws;
}

int launch_attention(const AttnArgs &a, hipStream_t stream) {
  if (a.total_q == 0) return FP8TS_OK;
  Plan pl = make_plan(a.mode, a.batch, a.total_q, a.max_q_len, a.hq, a.hkv, a.hidx, a.dv, a.topk,
                      a.max_blocks);
  if (pl.gr.splits > 1) {
    uint8_t *ws = static_cast<uint8_t *>(a.workspace);
    pl.gr.part_o = reinterpret_cast<float *>(ws);
    pl.gr.part_ml = reinterpret_cast<float *>(ws + (size_t)pl.gr.splits * a.total_q * a.hq * a.dv * 4);
  }
  if (pl.vt_bytes) pl.gr.vt_pages = static_cast<uint8_t *>(a.workspace) + (pl.ws - pl.vt_bytes);
  if (pl.nblocks == 0) return FP8TS_OK;
  int st = FP8TS_OK;
  switch (pl.kind) {
    case 0: st = launch_k(attn_kernel<128, 128, kPrefillWaves, 16 / kPrefillWaves, 128, true>, pl,
                          kPrefillWaves * 64, a, stream); break;
    case 4: st = launch_block_prefill(a, pl.gr, pl.nblocks, stream); break;
    case 5:
      if (pl.lds > kMaxLds)
        return fail(FP8TS_EUNSUPPORTED, "sparse_attn_fwd: decode block lists need %zu bytes of LDS", pl.lds);
      st = launch_block_decode(a, pl.gr, pl.nblocks, stream);
      break;
    case 7: st = launch_block_stream_decode(a, pl.gr, pl.nblocks, stream); break;
    case 6:
      if (token_latent_fits(a, pl.gr.splits)) {
        st = launch_token_latent(a, pl.gr, pl.nblocks, stream);
        break;
      }
      if (token_mla_fits(a)) {
        st = launch_token_mla(a, pl.gr, pl.nblocks, stream);
        break;
      }
      pl.lds = lds_base<576, 512, 64>();   // caches past 2 GB: the unpipelined kernel
      [[fallthrough]];
    case 2: st = launch_k(attn_kernel<576, 512, 8, 1, 64, false>, pl, 512, a, stream); break;
    default: st = launch_k(attn_kernel<576, 512, 1, 1, 64, false>, pl, 64, a, stream); break;
  }
  if (st || pl.gr.splits == 1) return st;
  if (a.dv == 512) {
    hipLaunchKernelGGL(attn_combine_kernel<512>, dim3((unsigned)((int64_t)a.total_q * a.hq)), dim3(128), 0,
                       stream, a, pl.gr);
  } else {
    hipLaunchKernelGGL(attn_combine_kernel<128>, dim3((unsigned)((int64_t)a.total_q * a.hq)), dim3(128), 0,
                       stream, a, pl.gr);
  }
  return check_launch("sparse_attn_fwd (combine)");
}

}  // namespace fp8ts
