// HCA prefill attention for bf16, head_dim 512, on CDNA4 matrix cores.
//
// Operation (ERNIE 5.5 Flash Base pages: mirrorspeed page, "Hybrid sparse
// attention" section; ai-club.cn page, hybrid attention section): query t
// attends densely over the compressed entries j < n_c(t) = floor(lo(t)/block)
// and the raw window [lo(t), t], lo(t) = max(0, t - W + 1), with 512-wide
// heads.
//
// Design (one workgroup = 8 waves = 128 consecutive queries of one head,
// two waves per SIMD):
//   * Each wave owns 16 queries and keeps them in registers as the B operand
//     of S^T = K Q^T (v_mfma_f32_16x16x32_bf16, 16 k-steps over d = 512).
//   * Keys stream in tiles of 32: first the compressed entries, then the raw
//     window band.  K rows go global -> LDS with global_load_lds_dwordx4
//     (one 1-KB row per wave instruction).  V rows are loaded into registers
//     (4 keys x 8 dims per lane), transposed with byte permutes and stored as
//     V^T, the A operand of O^T = V^T P^T (v_mfma_f32_16x16x32_bf16).  Both
//     are double-buffered one tile ahead; one barrier per tile.
//   * LDS layouts are chunk-major so that the 16 lanes of every 16-byte read
//     phase touch one contiguous 256-byte span (the measured full-rate case
//     on gfx950; spans shifted between lane groups run at half rate): K is
//     [chunk][key][16 B] and V^T is [chunk][dim + dim/16][16 B] (the padding
//     row every 16 dims also makes the 8-byte transposed writes
//     conflict-free).  Every MFMA operand read is one lane offset plus a
//     compile-time immediate.  A K DMA instruction fills one chunk pair for
//     all 32 keys of the tile.
//   * Computing S^T rather than S puts one query per lane column, so the
//     online-softmax state and all O^T accumulator rows of a lane belong to
//     the same query: no cross-lane row shuffles.  The S^T accumulators of
//     the two 16-key halves are the P^T operand with the keys of each 32-key
//     step in the order {4g..4g+3, 16+4g..16+4g+3} for lane group g, and V^T
//     is stored in that order.
//   * Online softmax in fp32 (log2 domain) with a lazy rescale: the reference
//     maximum only moves when a tile exceeds it by more than 2^8, so O is
//     rescaled rarely and exactly (the final normalisation uses the same
//     reference).
//   * Workgroup ids are remapped so each XCD receives a contiguous range of
//     (head, query tile) work: same-head tiles share that XCD's L2 for the
//     compressed cache.  Within a head, the longest query tiles go first.
//   * Each LDS stage is its own object and the loop handles two tiles per
//     trip with fixed stages, so the compiler can tell the in-flight DMA of
//     the next tile from the stage being read and keeps it in flight during
//     the step.  The explicit vmcnt wait before the per-tile barrier orders
//     DMA and reads.
#include "device_common.h"
#include "launchers.h"

namespace hca {
namespace {

constexpr int D = 512;
constexpr int BM = 128;  // queries per workgroup
constexpr int WQ = 16;   // queries per wave
constexpr int NWAVE = 8;
constexpr int BN = 32;   // keys per tile
constexpr int KSTAGE = (D / 8) * BN * 8;      // K stage: 64 chunks x 32 keys x 8 elements
constexpr int VCH = (D + D / 16) * 8;         // V^T chunk plane: padded dims x 8 elements
constexpr int VSTAGE = 4 * VCH;               // V^T stage: 4 chunks (32 keys)
constexpr float kLazy = 8.f;

struct PrefillParams {
  AttnArgs a;
  int n_qt;   // query tiles per (batch, head)
  int total;  // batch * h_q * n_qt
  float c;    // scale * log2(e)
};

// V^T: chunk g of dim d holds keys {4g..4g+3, 16+4g..16+4g+3} of the tile and
// sits at element g*VCH + (d + d/16)*8.

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void prefill512_kernel(PrefillParams p) {
  // one LDS object per stage: the compiler tracks DMA/read aliasing per object
  __shared__ __attribute__((aligned(16))) uint16_t Ks0[KSTAGE];  // [chunk][key][8]
  __shared__ __attribute__((aligned(16))) uint16_t Ks1[KSTAGE];
  __shared__ __attribute__((aligned(16))) uint16_t Vt0[VSTAGE];  // [chunk][padded dim][8]
  __shared__ __attribute__((aligned(16))) uint16_t Vt1[VSTAGE];

  const AttnArgs& a = p.a;
  const int L = xcd_remap(blockIdx.x, p.total);
  if (L < 0) return;
  const int qt = p.n_qt - 1 - (L % p.n_qt);
  const int bh = L / p.n_qt;
  const int h = bh % a.h_q;
  const int b = bh / a.h_q;
  const int g = h / (a.h_q / a.h_kv);

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar: everything derived from it stays in SGPRs
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int W = a.window, blk = a.block;

  // Positions fit in 32 bits (checked by the host before launch).
  const int qp0 = (int)a.q_pos0, kvp0 = (int)a.kv_pos0;
  const int i0 = qt * BM;
  const int i_last = min(i0 + BM, a.seqlen_q) - 1;
  const int t_first = qp0 + i0, t_last = qp0 + i_last;
  const int lo_first = max(0, t_first - W + 1);
  const int nc_max = max(0, t_last - W + 1) / blk;
  const int n_ct = (nc_max + BN - 1) / BN;
  const int n_wt = (t_last - lo_first + BN) / BN;
  const int ntiles = n_ct + n_wt;

  // this lane's query (rows past the end read the last row and are never stored)
  const int iq = i0 + WQ * w + col;
  const bool qvalid = iq < a.seqlen_q;
  const int tq = qp0 + iq;
  const int lo_q = max(0, tq - W + 1);
  const int nc_q = lo_q / blk;
  // this wave's query range: tiles nobody in the wave sees are skipped, tiles
  // every query of the wave sees entirely need no mask
  const int iw0 = i0 + WQ * w;
  const int iw1 = min(iw0 + WQ - 1, i_last);
  const bool wave_has_q = iw0 <= i_last;
  const bool wave_full = iw0 + WQ - 1 <= i_last;
  const int tw0 = qp0 + iw0, tw1 = qp0 + iw1;
  const int lo_w0 = max(0, tw0 - W + 1), lo_w1 = max(0, tw1 - W + 1);
  const int nc_w0 = lo_w0 / blk, nc_w1 = lo_w1 / blk;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds query `col`, dims 32ks + 8grp .. +8
  bf16x8 qf[16];
  {
    const uint16_t* qp = (const uint16_t*)a.q + b * a.sq.b + (int64_t)min(iq, a.seqlen_q - 1) * a.sq.s +
                         (int64_t)h * a.sq.h + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, ld16(qp + 32 * ks));
    // settle the Q loads here so the tile pipeline's load counting starts clean
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

  const uint16_t* kcb = (const uint16_t*)a.kc + b * a.skc.b + (int64_t)g * a.skc.h;
  const uint16_t* kb = (const uint16_t*)a.k + b * a.sk.b + (int64_t)g * a.sk.h;
  const uint16_t* vcb = (const uint16_t*)a.vc + b * a.svc.b + (int64_t)g * a.svc.h;
  const uint16_t* vb = (const uint16_t*)a.v + b * a.sv.b + (int64_t)g * a.sv.h;

  // ---- K tile: one DMA instruction fills chunk pair cp (chunks 2cp, 2cp+1) of all
  // 32 keys: lane l fetches chunk 2cp + (l >> 5) of key l & 31.  Wave w owns chunk
  // pairs w, w+8, w+16, w+24.  Keys past the valid range re-read a valid row
  // (their logits are masked).
  const int kkey = lane & 31, khalf = lane >> 5;
  auto issue_k = [&](int tt, uint16_t* kdst, const uint16_t* kcp, const uint16_t* kp) __attribute__((always_inline)) {
    const uint16_t* base;
    int64_t stride;
    int row0, row_max;
    if (tt < n_ct) {
      base = kcp; stride = a.skc.s; row0 = tt * BN; row_max = nc_max - 1;
    } else {
      base = kp; stride = a.sk.s; row0 = lo_first + (tt - n_ct) * BN - kvp0; row_max = t_last - kvp0;
    }
    const uint16_t* rowp = base + (int64_t)min(row0 + kkey, row_max) * stride + 8 * khalf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cp = w + 8 * i;
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(rowp + 16 * cp),
                                       (__attribute__((address_space(3))) void*)(kdst + cp * (2 * BN * 8)), 16, 0, 0);
    }
  };

  // ---- V tile: wave w = 4*dh + vg, lane = 2*dgrp + hi holds keys 16hi + 4vg + i
  // (i < 4) at dims 256dh + 8dgrp .. +8.  Rows past the valid range re-read the
  // last valid row, a row some query of this workgroup attends to; their
  // probabilities are exactly 0, so they add nothing.
  const int vg = w & 3, dh = w >> 2;
  const int hi = lane & 1, dgrp = lane >> 1;
  const int vdim0 = 256 * dh + 8 * dgrp;
  u32x4 vr[4];
  auto load_v = [&](int tt) __attribute__((always_inline)) {
    const uint16_t* base;
    int64_t stride;
    int row0, row_max;
    if (tt < n_ct) {
      base = vcb; stride = a.svc.s; row0 = tt * BN; row_max = nc_max - 1;
    } else {
      base = vb; stride = a.sv.s; row0 = lo_first + (tt - n_ct) * BN - kvp0; row_max = t_last - kvp0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + 16 * hi + 4 * vg + i;
      vr[i] = ld16(base + (int64_t)min(row, row_max) * stride + vdim0);
    }
  };
  // V^T write offset (elements) of dim vdim0: chunk vg, half hi (vdim0 % 16 + e < 16,
  // so the padding term is the same for all eight dims of the lane)
  const int vw = vg * VCH + (vdim0 + vdim0 / 16) * 8 + 4 * hi;
  auto store_v = [&](uint16_t* vdst) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      u32x2 x;
      x[0] = __builtin_amdgcn_perm(vr[1][e >> 1], vr[0][e >> 1], sel);
      x[1] = __builtin_amdgcn_perm(vr[3][e >> 1], vr[2][e >> 1], sel);
      *reinterpret_cast<u32x2*>(vdst + vw + 8 * e) = x;
    }
  };

  f32x4 o[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_used = -INFINITY, l_run = 0.f;
  const float c = p.c;

  // per-lane LDS read offsets (elements).  K: chunk 4ks + grp of key 16kt + col.
  // V^T: chunk grp of dim 16dt + col (padded index 17dt + col).
  const int k_off = grp * (BN * 8) + col * 8;
  const int v_off = grp * VCH + col * 8;

  const int last = max(ntiles - 1, 0);
  auto compute = [&](int tt, const uint16_t* __restrict__ kst, const uint16_t* __restrict__ vst,
                     uint16_t* __restrict__ knext, const uint16_t* __restrict__ kcp,
                     const uint16_t* __restrict__ kp) __attribute__((always_inline)) {
    // next tile's K DMA (stage pointers are per-object, see the file comment)
    issue_k(min(tt + 1, last), knext, kcp, kp);
    if (tt >= ntiles) return;  // the odd trip past the last tile only keeps the pipeline uniform
    const bool comp = tt < n_ct;
    const int j0 = tt * BN;
    const int p0 = lo_first + (tt - n_ct) * BN;
    // does any query of this wave see a key of this tile? (wave-uniform)
    const bool active = wave_has_q && (comp ? (j0 < nc_w1) : (p0 <= tw1 && p0 + BN - 1 >= lo_w0));
    if (!active) return;
    const bool full = wave_full && (comp ? (j0 + BN - 1 < nc_w0) : (p0 >= lo_w1 && p0 + BN - 1 <= tw0));
    // S^T = K Q^T : two 16-key halves x 16 queries (two independent chains)
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 ka = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(kst + k_off + 4 * BN * 8 * ks + 16 * 8 * kt));
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[ks], s[kt], 0, 0, 0);
      }
    }
    // online softmax (log2 domain); lane holds keys 16kt + 4grp + r of query `col`
    float sv[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[4 * kt + r] = s[kt][r] * c;
    if (!full) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = 16 * (e >> 2) + 4 * grp + (e & 3);
        const bool valid = comp ? (qvalid && j0 + kk < nc_q) : (qvalid && p0 + kk >= lo_q && p0 + kk <= tq);
        sv[e] = valid ? sv[e] : -INFINITY;
      }
    }
    float mt = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool need = mt > m_used + kLazy;
    if (__any(need)) {
      const float new_m = need ? mt : m_used;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_used - new_m) : 1.f;
      m_used = new_m;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) o[dt] *= alpha;
    }
    // masked logits are -inf and m_used is finite once any key was seen: exp2 gives 0
    const float msafe = m_used == -INFINITY ? 0.f : m_used;
    float ps[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ps[e] = __builtin_amdgcn_exp2f(sv[e] - msafe);
    l_run += ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
    u32x4 pk;
#pragma unroll
    for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(ps[2 * e], ps[2 * e + 1]);
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pk);
    // O^T += V^T P^T : 32 dim tiles, one 32-key step each
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const bf16x8 va = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vst + v_off + 17 * 8 * dt));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf, o[dt], 0, 0, 0);
    }
  };

  // Pipeline: tile tt's K DMA and V loads are issued one iteration ahead.
  // Loads are unconditional (past the end they re-read the last tile) so the
  // load counting stays exact.
  // Two tiles per trip with fixed stages (even tiles in stage 0, odd in stage 1).
  // The trip for tile tt stores its V^T, waits for its K DMA and V loads, then
  // issues the next tile's loads and computes.  Loads are unconditional (past
  // the end they re-read the last tile) so the load counting stays exact.
  if (ntiles > 0) {
    issue_k(0, Ks0, kcb, kb);
    load_v(0);
    for (int tt = 0; tt < ntiles; tt += 2) {
      store_v(Vt0);
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      load_v(min(tt + 1, last));
      compute(tt, Ks0, Vt0, Ks1, kcb, kb);
      store_v(Vt1);
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      load_v(min(tt + 2, last));
      compute(tt + 1, Ks1, Vt1, Ks0, kcb, kb);
    }
  }

  // ---- epilogue: normalise, store bf16 O and the LSE
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!qvalid) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* op = (uint16_t*)a.o + b * a.so.b + (int64_t)iq * a.so.s + (int64_t)h * a.so.h + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) {
    u32x2 pk;
    pk[0] = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
    pk[1] = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
    *reinterpret_cast<u32x2*>(op + 16 * dt) = pk;
  }
  if (a.lse && grp == 0) a.lse[((int64_t)b * a.h_q + h) * a.seqlen_q + iq] = m_used * kLn2 + __logf(l_tot);
}

}  // namespace

hipError_t launch_attn_prefill512(const AttnArgs& a, hipStream_t st) {
  PrefillParams p;
  p.a = a;
  p.n_qt = (a.seqlen_q + BM - 1) / BM;
  p.total = a.batch * a.h_q * p.n_qt;
  p.c = a.scale * kLog2e;
  const int grid = ((p.total + 7) / 8) * 8;
  hipLaunchKernelGGL(prefill512_kernel, dim3(grid), dim3(NWAVE * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace hca
