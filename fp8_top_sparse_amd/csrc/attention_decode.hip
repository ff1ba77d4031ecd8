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
//  * a block's K page is loaded straight into MFMA operand registers and its
//    V page copied linearly (1 KB contiguous per wave load) into the wave's
//    own 16 KB of LDS by buffer-to-LDS DMA; the wave waits for its own loads
//    only, and two workgroups (eight waves) share a CU;
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
// K goes straight into MFMA operand registers; only V passes through LDS
// (the transposing reads need it there), so a workgroup needs 64 KB and two
// share a CU: eight waves, each with a K and a V page in flight (K in LDS
// too, one workgroup per CU, measured 110 µs against 98.5 on the 64 x 32k
// decode workload)
constexpr int kWaveLds = kPageBytes;

typedef __attribute__((address_space(3))) void lds_void;
typedef int v2i_ __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i_ lds_v2i;

// 8 e4m3 bytes (keys of one dim) -> the 8 bf16 of a 16x16x32 A operand
__device__ __forceinline__ v8bf widen8(v2i_ b) {
  const uint32_t lo = (uint32_t)b[0], hi = (uint32_t)b[1];
  const v4i w = {(int)bf16x2_from_e4m3(lo, false), (int)bf16x2_from_e4m3(lo, true),
                 (int)bf16x2_from_e4m3(hi, false), (int)bf16x2_from_e4m3(hi, true)};
  return __builtin_bit_cast(v8bf, w);
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

  uint8_t *vl = smem + wave * kWaveLds;
  const int kvh_s = __builtin_amdgcn_readfirstlane(br.kvh);
  const float ck = a.key_scale_log2;
  // transposing V reads: lane (g, i) addresses row i / 2, half i % 2 of its
  // 16-byte column group; which key each row is follows the key order of the
  // P operand built from the S^T accumulators (below)
  const int tr_row = col >> 1, tr_half = col & 1;

  v4f o[kNdt];
#pragma unroll
  for (int dt = 0; dt < kNdt; ++dt) o[dt] = (v4f){0.f, 0.f, 0.f, 0.f};
  float negm = 0.f, mraw = -INFINITY, lsum = 0.f;
  bool started = false;
  for (int pass = 0; pass < 2; ++pass) {
    bool overflow = false;
    for (int i = lo + wave; i < hi; i += kWaves) {
      const int blk = __builtin_amdgcn_readfirstlane(ulist[i]);
      const int page = __builtin_amdgcn_readfirstlane(a.block_table[(int64_t)br.b * a.max_blocks + blk]);
      if (page < 0 || page >= a.num_kv) continue;
      const bool sel = br.row_ok[0] && ((bits[br.row_li[0] * gr.W + (blk >> 5)] >> (blk & 31)) & 1u);
      if (!__any(sel)) continue;
      // K and V pages into this wave's LDS, 1 KB per instruction
      const int64_t off = ((int64_t)page * a.hkv + kvh_s) * kPageBytes;
      const __amdgpu_buffer_rsrc_t rk = make_tile_rsrc(a.k + off);
      const __amdgpu_buffer_rsrc_t rv = make_tile_rsrc(a.v + off);
      v8i ka[8];
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const int ko = (16 * kt + col) * kD + 32 * g;
        const v4i k0 = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rk, ko, 0, 0));
        const v4i k1 = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rk, ko + 16, 0, 0));
        ka[kt] = (v8i){k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
      }
#pragma unroll
      for (int j = 0; j < 16; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(vl + 1024 * j), 16, 1024 * j + 16 * lane, 0, 0, 0);
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): K in registers, V in LDS

      // ---- S^T = K Q^T + C over the block's 128 keys
      const float cv = sel ? negm : -INFINITY;
      const v4f cinit = {cv, cv, cv, cv};
      v4f s[8];
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        s[kt] = mfma_16x16x128_e4m3(ka[kt], qb, cinit);
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
      // ---- O^T += V^T P^T: row tr_row of group g in chunk q is key
      // 32 q + 4 g + r (r < 4) or 32 q + 16 + 4 g + (r - 4)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int key = 32 * q + (tr_row < 4 ? 4 * g + tr_row : 16 + 4 * g + tr_row - 4);
#pragma unroll
        for (int dt = 0; dt < kNdt; ++dt) {
          const v2i_ raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (lds_v2i *)(vl + key * kD + 16 * dt + 8 * tr_half));
          o[dt] = mfma_16x16x32_bf16(widen8(raw), pb[q], o[dt]);
        }
      }
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
  float *xs = reinterpret_cast<float *>(vl);
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
  return (size_t)kWaves * kWaveLds + 4 * ((size_t)(gr.NL + 1) * gr.W + 4 + (size_t)gr.W * 32);
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
