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
//   * Keys stream in tiles of 16: first the compressed entries, then the raw
//     window band.  Each tile (16 K rows + 16 V rows of 1 KB) is loaded into
//     registers one tile ahead with coalesced 16-byte loads (one row per wave
//     instruction) and stored to one of two LDS stages: K row-major with its
//     16-byte chunks XOR-swizzled by key, V transposed in registers (4 keys x
//     8 dims per thread) into V^T so that V^T is the A operand of
//     O^T = V^T P^T (v_mfma_f32_16x16x16_bf16).  One barrier per tile.
//   * Computing S^T rather than S puts one query per lane column, so the
//     online-softmax state and all O^T accumulator rows of a lane belong to
//     the same query: no cross-lane row shuffles, and the S^T accumulator
//     layout is exactly the P^T operand layout of the PV product.
//   * Online softmax in fp32 (log2 domain) with a lazy rescale: the reference
//     maximum only moves when a tile exceeds it by more than 2^8, so O is
//     rescaled rarely and exactly (the final normalisation uses the same
//     reference).
//   * Workgroup ids are remapped so each XCD receives a contiguous range of
//     (head, query tile) work: same-head tiles share that XCD's L2 for the
//     compressed cache.  Within a head, the longest query tiles go first.
#include "device_common.h"
#include "launchers.h"

namespace hca {
namespace {

constexpr int D = 512;
constexpr int BM = 128;  // queries per workgroup
constexpr int WQ = 16;   // queries per wave
constexpr int NWAVE = 8;
constexpr int BN = 16;   // keys per tile
constexpr float kLazy = 8.f;

struct PrefillParams {
  AttnArgs a;
  int n_qt;   // query tiles per (batch, head)
  int total;  // batch * h_q * n_qt
  float c;    // scale * log2(e)
};

// V^T row = 16 keys = 4 chunks of 8 B (chunk g = keys 4g..4g+3), chunk index XOR-swizzled.
__device__ __forceinline__ int vt_swz(int dim) { return (dim >> 2) & 3; }

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void prefill512_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2 * BN * D];  // 2 stages x [key][dim], chunk c at c ^ (key & 7)
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2 * D * BN];  // 2 stages x [dim][key], chunk swizzle

  const AttnArgs& a = p.a;
  const int L = xcd_remap(blockIdx.x, p.total);
  if (L < 0) return;
  const int qt = p.n_qt - 1 - (L % p.n_qt);
  const int bh = L / p.n_qt;
  const int h = bh % a.h_q;
  const int b = bh / a.h_q;
  const int g = h / (a.h_q / a.h_kv);

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar: everything derived from it (row choice, tile
  // classification) stays in SGPRs and scalar branches
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

  // Tile loads: wave w < 4 loads K rows 4w..4w+3, wave w >= 4 loads V rows
  // 4(w-4)..+3; lane = 16-byte chunk of the row.  The row choice is
  // wave-uniform, so the address is a scalar base plus the lane offset.  Rows
  // past the valid range re-read a valid row: K logits there are masked, V
  // rows are zeroed.
  const bool is_v = w >= 4;
  const int r0 = 4 * (w & 3);
  const uint16_t* cbase = is_v ? (const uint16_t*)a.vc + b * a.svc.b + (int64_t)g * a.svc.h
                               : (const uint16_t*)a.kc + b * a.skc.b + (int64_t)g * a.skc.h;
  const int64_t cstride = is_v ? a.svc.s : a.skc.s;
  const uint16_t* rbase = is_v ? (const uint16_t*)a.v + b * a.sv.b + (int64_t)g * a.sv.h
                               : (const uint16_t*)a.k + b * a.sk.b + (int64_t)g * a.sk.h;
  const int64_t rstride = is_v ? a.sv.s : a.sk.s;
  auto load_tile = [&](int tt, u32x4 (&R)[4]) __attribute__((always_inline)) {
    const uint16_t* base;
    int64_t stride;
    int row0, row_max;
    if (tt < n_ct) {
      base = cbase;
      stride = cstride;
      row0 = tt * BN + r0;
      row_max = nc_max - 1;
    } else {
      base = rbase;
      stride = rstride;
      row0 = lo_first + (tt - n_ct) * BN + r0 - kvp0;
      row_max = t_last - kvp0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + i;
      const uint32_t keep = (row <= row_max || !is_v) ? ~0u : 0u;
      R[i] = ld16(base + (int64_t)min(row, row_max) * stride + 8 * lane) & keep;
    }
  };
  // V^T store offsets of this lane: dim = 8*lane + e; the chunk swizzle depends on e only through e >> 2
  const int vt_off0 = (8 * lane) * BN + (((w & 3) ^ vt_swz(8 * lane)) << 2);
  const int vt_off1 = (8 * lane + 4) * BN + (((w & 3) ^ vt_swz(8 * lane + 4)) << 2);
  auto store_tile = [&](const u32x4 (&R)[4], int st) __attribute__((always_inline)) {
    if (!is_v) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = r0 + i;
        *reinterpret_cast<u32x4*>(Ks + st * (BN * D) + key * D + ((lane ^ (key & 7)) << 3)) = R[i];
      }
    } else {
      // 4 keys x 8 dims -> 8 dims x 4 keys
      uint16_t* vbase = Vt + st * (D * BN);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        u32x2 x;
        x[0] = __builtin_amdgcn_perm(R[1][e >> 1], R[0][e >> 1], sel);
        x[1] = __builtin_amdgcn_perm(R[3][e >> 1], R[2][e >> 1], sel);
        *reinterpret_cast<u32x2*>(vbase + ((e < 4) ? vt_off0 : vt_off1) + (e & 3) * BN) = x;
      }
    }
  };

  f32x4 o[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_used = -INFINITY, l_run = 0.f;
  const float c = p.c;
  // per-lane LDS offsets of the S^T A-operand reads: chunk (4ks + grp) ^ (col & 7)
  // of row col equals 4(ks ^ h) + (grp ^ (col & 3)) with h = (col >> 2) & 1
  const int k_even = col * D + ((grp ^ (col & 3)) << 3) + 32 * ((col >> 2) & 1);
  const int k_odd = col * D + ((grp ^ (col & 3)) << 3) - 32 * ((col >> 2) & 1);
  const int v_rd = col * BN + ((grp ^ vt_swz(col)) << 2);

  auto compute = [&](int tt, int st) __attribute__((always_inline)) {
    const bool comp = tt < n_ct;
    const int j0 = tt * BN;
    const int p0 = lo_first + (tt - n_ct) * BN;
    // does any query of this wave see a key of this tile? (wave-uniform)
    const bool active = wave_has_q && (comp ? (j0 < nc_w1) : (p0 <= tw1 && p0 + BN - 1 >= lo_w0));
    if (!active) return;
    const bool full = wave_full && (comp ? (j0 + BN - 1 < nc_w0) : (p0 >= lo_w1 && p0 + BN - 1 <= tw0));
    const uint16_t* kst = Ks + st * (BN * D);
    const uint16_t* vst = Vt + st * (D * BN);
    // S^T = K Q^T : 16 keys x 16 queries, two independent accumulation chains
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int ks = 0; ks < 16; ks += 2) {
      const bf16x8 ka0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kst + k_even + 32 * ks));
      const bf16x8 ka1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kst + k_odd + 32 * (ks + 1)));
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1, qf[ks + 1], s1, 0, 0, 0);
    }
    // online softmax (log2 domain); lane holds keys 4grp + r of query `col`
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = (s0[r] + s1[r]) * c;
    if (!full) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = 4 * grp + r;
        const bool valid = comp ? (qvalid && j0 + kk < nc_q) : (qvalid && p0 + kk >= lo_q && p0 + kk <= tq);
        sv[r] = valid ? sv[r] : -INFINITY;
      }
    }
    float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
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
    float ps[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ps[r] = __builtin_amdgcn_exp2f(sv[r] - msafe);
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    u32x2 pk;
    pk[0] = pack_bf16x2(ps[0], ps[1]);
    pk[1] = pack_bf16x2(ps[2], ps[3]);
    const bf16x4 pf = __builtin_bit_cast(bf16x4, pk);
    // O^T += V^T P^T : 32 dim tiles, one 16-key step each
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const bf16x4 va = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(vst + v_rd + 16 * BN * dt));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pf, o[dt], 0, 0, 0);
    }
  };

  // One tile in flight in registers, two LDS stages, one barrier per tile.
  // Loads are unconditional (past the end they re-read the last tile) so the
  // compiler's load counting stays exact.
  u32x4 R[4];
  const int last = max(ntiles - 1, 0);
  if (ntiles > 0) load_tile(0, R);
  for (int tt = 0; tt < ntiles; ++tt) {
    store_tile(R, tt & 1);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    load_tile(min(tt + 1, last), R);
    compute(tt, tt & 1);
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
