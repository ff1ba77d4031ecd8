// Block-sparse decode attention (d = 128, 128-token pages) for few query rows
// per kv head: the kernel behind sparse_attn_fwd in block mode when a
// sequence's query rows (tokens x q heads of one kv head) fit one 16-row tile.
//
// Semantics as the block prefill kernel (sglang PR 25751 digest: out bf16,
// max_logits and lse fp32, optional attn_sink; vLLM PR 45892 digest: each
// query attends to the 128-token blocks its index head selected, causally;
// sglang PR 30971 digest, implementation step 3: q_scale folded into
// sm_scale, k_scale on the QK dot, v_scale on the output).
//
// Decode is bound by HBM: one pass over the K and V pages of the union of the
// tile's block lists.  Each of the four waves streams its own share of the
// workgroup's blocks (block i of the share goes to wave i mod 4) with its own
// online softmax, so no wave waits for another until the end:
//  * both pages of a block come in by buffer-to-LDS DMA, each instruction
//    reading 1 KB of contiguous HBM (page rows whole, in order), into the
//    wave's own 32 KB of LDS; the wave waits for its own loads only;
//  * the loads of the wave's next block are issued as soon as the current
//    one no longer needs the slot: the next K page once the QK operands have
//    been read, the next V page once the PV operands have been read, so each
//    wave keeps about one block in flight while it computes;
//  * K is stored with its 16-byte chunks permuted within each row (chunk c of
//    row r at position c ^ f(r)), which keeps the DMA reads contiguous and
//    makes the MFMA operand reads (16 rows, one chunk each) free of LDS bank
//    conflicts;
//  * S^T = K Q^T + C on 16x16x128 e4m3 MFMA (C = minus the row's reference
//    maximum);
//  * V^T operands come from the row-major V page through the gfx950
//    transposing LDS read (ds_read_b64_tr_b8: in a 16-lane group, byte j of
//    lane i is byte i mod 8 of the row addressed by lane 2j + i/8), with the
//    8 rows ordered as the keys of the P operand, and are widened to bf16 in
//    registers for the 16x16x32 bf16 PV MFMA;
//  * at the end the four waves' (O, reference maximum, row sum) are merged by
//    log-sum-exp through LDS and written as final outputs or split partials.
#include "attn_common.h"

namespace fp8ts {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kNdt = kD / 16;                 // 16-dim output tiles
constexpr int kPageBytes = kPage * kD;        // one e4m3 page (K or V) of one kv head
// per wave: the K page (chunk-permuted rows) then the V page (row-major); the
// workgroup's 128 KB of slots leave one workgroup per CU, with four waves
// each keeping a block in flight
constexpr int kWaveLds = 2 * kPageBytes;

// position of 16-byte chunk c of K row r within the row: c ^ f(r) with
// f(r) = (r + r / 8) mod 8 on the row's place in its 16-row group.  f takes
// 8 distinct values over rows 0..7, over rows 8..15, over the even and over
// the odd rows of a group, so the operand reads (16 rows, one chunk column)
// spread over all banks whether the LDS serves 8 or 16 lanes per cycle.
__device__ __forceinline__ int k_swz(int r) { return ((r & 7) + ((r >> 3) & 1)) & 7; }

typedef __attribute__((address_space(3))) void lds_void;

// 8 e4m3 bytes (keys of one dim) -> the 8 bf16 of a 16x16x32 A operand
__device__ __forceinline__ v8bf widen8(v2i b) {
  const uint32_t lo = (uint32_t)b[0], hi = (uint32_t)b[1];
  const v4i w = {(int)bf16x2_from_e4m3(lo, false), (int)bf16x2_from_e4m3(lo, true),
                 (int)bf16x2_from_e4m3(hi, false), (int)bf16x2_from_e4m3(hi, true)};
  return __builtin_bit_cast(v8bf, w);
}

// Eight transposing reads (ds_read_b64_tr_b8) at p + 16 dt, dt = 0..7, and a
// wait for them inside the same statement.  Written as one asm statement
// because the compiler, not seeing which LDS bytes the intrinsic reads, would
// wait for every buffer-to-LDS load in flight before it, including those of
// the next block that the kernel keeps in flight on purpose.  The outputs are
// early-clobber: no output may share a register with the address.
__device__ __forceinline__ void tr_read8x8(const uint8_t *p, v2i (&r)[kNdt]) {
  static_assert(kNdt == 8, "eight dim tiles");
  const uint32_t addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
  asm volatile(
      "ds_read_b64_tr_b8 %0, %8\n\t"
      "ds_read_b64_tr_b8 %1, %8 offset:16\n\t"
      "ds_read_b64_tr_b8 %2, %8 offset:32\n\t"
      "ds_read_b64_tr_b8 %3, %8 offset:48\n\t"
      "ds_read_b64_tr_b8 %4, %8 offset:64\n\t"
      "ds_read_b64_tr_b8 %5, %8 offset:80\n\t"
      "ds_read_b64_tr_b8 %6, %8 offset:96\n\t"
      "ds_read_b64_tr_b8 %7, %8 offset:112\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(addr)
      : "memory");
}

__global__ __launch_bounds__(kWaves * 64) void attn_decode_kernel(AttnArgs a, Grid gr) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int col = lane & 15;

  int bid = blockIdx.x;
  const int split = bid % gr.splits;
  bid /= gr.splits;
  // one 16-row tile shared by all waves: rows 0..15 = tokens x q heads
  BlockRows<1> br;
  if (!block_rows<1>(a, gr, bid, 0, col, br)) return;

  uint32_t *bits = reinterpret_cast<uint32_t *>(smem + kWaves * kWaveLds);
  int32_t *ucount = reinterpret_cast<int32_t *>(bits + (gr.NL + 1) * gr.W);
  int32_t *ulist = ucount + 4;
  const int U = block_union<kWaves * 64>(a, gr, br.kvh, br.cu0, br.q_len, br.seq_len, br.t0, bits, ucount, ulist);
  const int chunk = (U + gr.splits - 1) / gr.splits;
  const int lo = min(U, split * chunk);
  const int hi = min(U, lo + chunk);

  const int64_t qr = br.row_ok[0] ? (int64_t)br.row_t[0] * a.hq + br.row_h[0] : 0;
  const v8i qb = br.row_ok[0] ? gload32(a.q + qr * kD + 32 * g) : (v8i){0, 0, 0, 0, 0, 0, 0, 0};

  uint8_t *kl = smem + wave * kWaveLds;     // this wave's K slot
  uint8_t *vl = kl + kPageBytes;            // and V slot
  // physical page of every union block this workgroup visits (-1: none)
  int32_t *plist = ulist + gr.W * 32;
  for (int i = tid; i < hi - lo; i += kWaves * 64) {
    const int page = a.block_table[(int64_t)br.b * a.max_blocks + ulist[lo + i]];
    plist[i] = (page >= 0 && page < a.num_kv) ? page : -1;
  }
  __syncthreads();
  // the Q operands have landed before any page load is issued, so that the
  // waits on the page loads below count those loads alone
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

  const int kvh_s = __builtin_amdgcn_readfirstlane(br.kvh);
  const float ck = a.key_scale_log2;
  // transposing V reads: lane (g, i) addresses row i / 2, half i % 2 of its
  // 16-byte column group; which key each row is follows the key order of the
  // P operand built from the S^T accumulators (below)
  const int tr_row = col >> 1, tr_half = col & 1;
  // K DMA: instruction j, lane l fetches row 8 j + l / 8, chunk (l % 8) ^ f
  // (1 KB of contiguous HBM per instruction) into position l of the j-th KB
  const int kdma_row = lane >> 3;
  // K operand (kt, half hh) of lane (g, col): row 16 kt + col, chunk 2 g + hh
  const int kop0 = 16 * (col * 8 + ((2 * g) ^ k_swz(col)));
  const int kop1 = 16 * (col * 8 + ((2 * g + 1) ^ k_swz(col)));

  // the wave's next block from index i of its share with a page and a row
  // that selected it (hi: none)
  auto next_block = [&](int i) {
    for (; i < hi; i += kWaves) {
      if (plist[i - lo] < 0) continue;
      const int blk = ulist[i];
      const bool sel = br.row_ok[0] && ((bits[br.row_li[0] * gr.W + (blk >> 5)] >> (blk & 31)) & 1u);
      if (__any(sel)) break;
    }
    return __builtin_amdgcn_readfirstlane(i < hi ? i : hi);
  };
  auto page_off = [&](int i) {
    return ((int64_t)__builtin_amdgcn_readfirstlane(plist[i - lo]) * a.hkv + kvh_s) * kPageBytes;
  };
  auto issue_k = [&](int i) {
    const __amdgpu_buffer_rsrc_t rk = make_tile_rsrc(a.k + page_off(i));
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 8 * j + kdma_row;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(kl + 1024 * j), 16,
                                               r * kD + 16 * ((lane & 7) ^ k_swz(r)), 0, 0, 0);
    }
  };
  auto issue_v = [&](int i) {
    const __amdgpu_buffer_rsrc_t rv = make_tile_rsrc(a.v + page_off(i));
#pragma unroll
    for (int j = 0; j < 16; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(vl + 1024 * j), 16, 1024 * j + 16 * lane, 0, 0, 0);
  };

  v4f o[kNdt];
#pragma unroll
  for (int dt = 0; dt < kNdt; ++dt) o[dt] = (v4f){0.f, 0.f, 0.f, 0.f};
  float negm = 0.f, mraw = -INFINITY, lsum = 0.f;
  bool started = false;
  for (int pass = 0; pass < 2; ++pass) {
    bool overflow = false;
    int cur = next_block(lo + wave);
    if (cur < hi) {
      issue_k(cur);
      issue_v(cur);
    }
    while (cur < hi) {
      const int blk = __builtin_amdgcn_readfirstlane(ulist[cur]);
      const bool sel = br.row_ok[0] && ((bits[br.row_li[0] * gr.W + (blk >> 5)] >> (blk & 31)) & 1u);
      const int nxt = next_block(cur + kWaves);
      // in flight: K(cur), V(cur), in that order; K(cur) has landed once at
      // most the 16 V loads remain
      __builtin_amdgcn_s_waitcnt(0x4F70);   // vmcnt(16)

      // ---- S^T = K Q^T + C over the block's 128 keys
      const float cv = sel ? negm : -INFINITY;
      const v4f cinit = {cv, cv, cv, cv};
      v4f s[8];
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const v4i k0 = *reinterpret_cast<const v4i *>(kl + 2048 * kt + kop0);
        const v4i k1 = *reinterpret_cast<const v4i *>(kl + 2048 * kt + kop1);
        const v8i ka = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
        s[kt] = mfma_16x16x128_e4m3(ka, qb, cinit);
      }
      // the K slot is free once its operand reads are done: load the next K
      if (nxt < hi) {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        issue_k(nxt);
      }
      // causal mask where some row of the tile cannot see the whole block
      const int key0 = blk * kPage;
      if (__any(sel && br.row_p[0] < key0 + kPage - 1)) {
#pragma unroll
        for (int kt = 0; kt < 8; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (key0 + 16 * kt + 4 * g + e > br.row_p[0]) s[kt][e] = -INFINITY;
      }
      // ---- row maximum, reference on the row's first selected block
      float m = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) m = fmaxf(fmaxf(m, fmaxf(s[kt][0], s[kt][1])), fmaxf(s[kt][2], s[kt][3]));
      float mx = group4_max_swap(m);
      if (sel) mraw = fmaxf(mraw, mx - negm);
      const bool st = sel && !started;
      if (__any(st)) {
        const float delta = st ? mx : 0.f;
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) s[kt] -= delta;
        mx -= delta;
        negm -= delta;
        started = started || st;
      }
      overflow |= mx * ck > kHeadroom;
      // ---- probabilities, row sums, bf16 P operands: chunk q holds keys
      // 32 q + 4 g + e (e < 4) and 32 q + 16 + 4 g + (e - 4)
      v8bf pb[4];
      float ls = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v8bf v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(s[2 * q][e] * ck);
          const float p1 = __builtin_amdgcn_exp2f(s[2 * q + 1][e] * ck);
          ls += p0 + p1;
          v[e] = (__bf16)p0;
          v[4 + e] = (__bf16)p1;
        }
        pb[q] = v;
      }
      lsum += ls;
      // in flight: V(cur), then K(nxt) when there is a next block
      if (nxt < hi) __builtin_amdgcn_s_waitcnt(0x4F70);   // vmcnt(16)
      else __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0)
      // ---- V^T operands: row tr_row of group g in chunk q is key
      // 32 q + 4 g + r (r < 4) or 32 q + 16 + 4 g + (r - 4)
      v2i vraw[4][kNdt];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int key = 32 * q + (tr_row < 4 ? 4 * g + tr_row : 16 + 4 * g + tr_row - 4);
        tr_read8x8(vl + key * kD + 8 * tr_half, vraw[q]);
      }
      // the V slot is free (the reads have completed): load the next V
      if (nxt < hi) issue_v(nxt);
      // ---- O^T += V^T P^T
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int dt = 0; dt < kNdt; ++dt) o[dt] = mfma_16x16x32_bf16(widen8(vraw[q][dt]), pb[q], o[dt]);
      cur = nxt;
    }
    // rare second pass of this wave: restart from the exact row maxima it saw
    if (pass == 1 || !__any(overflow)) break;
    started = mraw != -INFINITY;
    negm = started ? -mraw : 0.f;
    lsum = 0.f;
#pragma unroll
    for (int dt = 0; dt < kNdt; ++dt) o[dt] = (v4f){0.f, 0.f, 0.f, 0.f};
  }

  // ---- merge the four waves by log-sum-exp (through each wave's own LDS)
  const float m_ref = started ? -negm * ck : -INFINITY;
  const float m_true = mraw * ck;
  float *xs = reinterpret_cast<float *>(kl);
  if (wave > 0) {
#pragma unroll
    for (int dt = 0; dt < kNdt; ++dt) *reinterpret_cast<v4f *>(xs + 4 * (dt * 64 + lane)) = o[dt];
    xs[4 * kNdt * 64 + lane] = m_ref;
    xs[4 * kNdt * 64 + 64 + lane] = m_true;
    xs[4 * kNdt * 64 + 128 + lane] = lsum;
  }
  __syncthreads();
  if (wave != 0) return;
  float M = m_ref, mt = m_true;
  for (int w = 1; w < kWaves; ++w) {
    const float *xw = reinterpret_cast<const float *>(smem + w * kWaveLds);
    M = fmaxf(M, xw[4 * kNdt * 64 + lane]);
    mt = fmaxf(mt, xw[4 * kNdt * 64 + 64 + lane]);
  }
  const float f0 = m_ref == -INFINITY ? 0.f : exp2f(m_ref - M);
  float l_part = lsum * f0;
#pragma unroll
  for (int dt = 0; dt < kNdt; ++dt) o[dt] *= f0;
  for (int w = 1; w < kWaves; ++w) {
    const float *xw = reinterpret_cast<const float *>(smem + w * kWaveLds);
    const float mw = xw[4 * kNdt * 64 + lane];
    const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
    l_part += xw[4 * kNdt * 64 + 128 + lane] * f;
#pragma unroll
    for (int dt = 0; dt < kNdt; ++dt) o[dt] += *reinterpret_cast<const v4f *>(xw + 4 * (dt * 64 + lane)) * f;
  }
  v4f oc[kNdt][1];
#pragma unroll
  for (int dt = 0; dt < kNdt; ++dt) oc[dt][0] = o[dt];
  const float mrefs[1] = {M}, mtrues[1] = {mt}, lps[1] = {l_part};
  attn_epilogue<1, kNdt>(a, gr, split, g, br.row_ok, br.row_t, br.row_h, oc, mrefs, mtrues, lps);
}

}  // namespace

size_t block_stream_decode_lds(const Grid &gr) {
  return (size_t)kWaves * kWaveLds + 4 * ((size_t)(gr.NL + 1) * gr.W + 4 + 2 * (size_t)gr.W * 32);
}

int launch_block_stream_decode(const AttnArgs &a, const Grid &gr, int64_t nblocks, hipStream_t stream) {
  const size_t lds = block_stream_decode_lds(gr);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(attn_decode_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return fail(FP8TS_EHIP, "sparse_attn_fwd: LDS attribute: %s", hipGetErrorString(e));
  hipLaunchKernelGGL(attn_decode_kernel, dim3((unsigned)nblocks), dim3(kWaves * 64), lds, stream, a, gr);
  return check_launch("sparse_attn_fwd (block decode, streamed)");
}

}  // namespace fp8ts
