// Backward of HCA attention for bf16, head_dim 512, on CDNA4 matrix cores.
//
// The forward (ERNIE 5.5 Flash Base pages: mirrorspeed page, "Hybrid sparse
// attention" section; ai-club.cn page, hybrid attention section) is dense
// attention of query t over the compressed entries j < n_c(t) and the raw
// window [lo(t), t].  Its gradients, with p recomputed from the forward's
// log-sum-exp and D = <dO, O>:
//   dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
//
// Two kernels, each on v_mfma_f32_32x32x16_bf16 with the operand layouts of
// the forward prefill kernel:
//   * dq kernel (query-tile major, 64 queries per workgroup): key tiles of 32
//     (compressed entries, then the window band) stream through LDS;
//     S^T = K Q^T and dP^T = V dO^T, then dQ^T += K^T dS^T.  D is computed
//     here from O and dO and stored for the second kernel.
//   * dkv kernel (key-tile major, 64 keys per workgroup): the keys' K^T and
//     V^T stay in registers, query tiles of 32 (Q, dO, lse, D) stream
//     through LDS; S = Q K^T and dP = dO V^T, then dK^T += Q^T dS and
//     dV^T += dO^T P.  A raw key row is seen by the queries of at most
//     W + 63 positions; a compressed entry by every later query, so the
//     query range of a compressed tile is cut into chunks whose fp32
//     partials a small kernel sums in a fixed order (no atomics anywhere).
//
// Register budget: a wave cannot hold both the Q-side and the dO-side
// B operand (128 VGPRs each) next to a 512-wide fp32 accumulator, so every
// 32-row group is served by a pair of waves.  In the dq kernel the even wave
// holds Q^T, the odd wave dO^T; they swap dP^T and dS^T through LDS and each
// accumulates half of the dQ^T dims (128 AGPRs).  In the dkv kernel the even
// wave holds K^T and accumulates dK^T, the odd wave holds V^T and accumulates
// dV^T (256 AGPRs each); they swap P and dP through LDS.
//
// LDS tiles read both row-wise (A operand of the first product) and
// transposed (A operand of the second, ds_read_b64_tr_b16) use a 1072-byte
// row stride: 16 consecutive rows of a 16-byte column fall in distinct bank
// groups, and the four rows x 32 bytes of a transposed read by 16 lanes do
// too.  Tiles read only row-wise use 1040 bytes.
#include "device_common.h"
#include "launchers.h"
#include "mfma_asm.h"

namespace hca {
namespace {

constexpr int D = 512;
constexpr int BT = 32;            // rows per streamed tile
constexpr int ROW2 = 2 * D + 48;  // 1072: tiles read row-wise and transposed
constexpr int ROW1 = 2 * D + 16;  // 1040: tiles read row-wise only
constexpr int TILE2 = BT * ROW2;  // 34304
constexpr int TILE1 = BT * ROW1;  // 33280
constexpr int DQ_XB = 2 * 4096;       // per wave pair: two fp32 32x32 blocks (P, dP)
constexpr int KV_XB = 4096 + 2048;    // per wave pair: fp32 32x32 (dP) + bf16 32x32 (P)

__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void barrier_dma() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); }

// Accumulator row r (0..15) of a lane in half hf: row 8(r/4) + 4hf + r%4.
__device__ __forceinline__ int acc_row(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

// Row offset (bytes) of the lane's 8-byte piece of a transposed A-operand read
// (dims 32dt + 16((lane>>4)&1) + 4(lane&3) .. +4 of rows 16ks + 4hf + (lane&15)/4
// and 8 rows further): add 64 dt + 16 ks ROW.
__device__ __forceinline__ uint32_t tr_off(int lane, int row_bytes) {
  return (4 * (lane >> 5) + ((lane & 15) >> 2)) * row_bytes + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
}

// Pack 16 fp32 accumulator values into the two bf16 B-operand steps.
__device__ __forceinline__ void pack_b(const float* v, bf16x8* out) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    u32x4 pk;
#pragma unroll
    for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(v[8 * ks + 2 * e], v[8 * ks + 2 * e + 1]);
    out[ks] = __builtin_bit_cast(bf16x8, pk);
  }
}

// First product of a tile: acc = A B over d = 512 (32 k-steps), A rows read
// from LDS at `ab` (lane offset included, +32 bytes per step), B from
// registers.  Reads run four steps ahead.  hook(ks) runs before step ks (the
// callers issue the next tile's DMA there, so its issue overlaps the MFMAs).
template <typename Hook>
__device__ __forceinline__ void product_d(f32x16& acc, const unsigned char* ab, const bf16x8* bf, Hook hook) {
  auto ld = [&](int ks) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ab + 32 * ks));
  };
  bf16x8 q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = ld(i);
#pragma unroll
  for (int ks = 0; ks < 32; ++ks) {
    const bf16x8 x = q[ks & 3];
    if (ks + 4 < 32) q[ks & 3] = ld(ks + 4);
    hook(ks);
    if (ks == 0) mfma_s_first(acc, x, bf[ks]);
    else if (ks == 31) mfma_s_last(acc, x, bf[ks]);
    else mfma_s(acc, x, bf[ks]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ------------------------------------------------------------------ dq kernel

constexpr int DQ_BM = 64;
constexpr int DQ_STAGE = TILE2 + TILE1;  // K (row + transposed reads), V (row reads)
constexpr int DQ_SMEM = 2 * DQ_STAGE + 2 * DQ_XB + 2 * 32 * 4;

struct DqParams {
  BwdArgs a;
  int n_qt;   // query tiles of 64 per (batch, head)
  int total;  // batch * h_q * n_qt
  float c;    // scale * log2(e)
};

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd512_dq_kernel(DqParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[DQ_SMEM];
  const BwdArgs& a = p.a;
  const int L = xcd_remap(blockIdx.x, p.total);
  if (L < 0) return;
  const int qt = p.n_qt - 1 - (L % p.n_qt);
  const int bh = L / p.n_qt;
  const int h = bh % a.h_q, b = bh / a.h_q;
  const int g = h / (a.h_q / a.h_kv);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = w >> 1, role = w & 1;
  const int col = lane & 31, hf = lane >> 5;
  const int W = a.window, blk = a.block;
  const int qp0 = (int)a.q_pos0, kvp0 = (int)a.kv_pos0;

  const int i0 = qt * DQ_BM;
  const int i_last = min(i0 + DQ_BM, a.seqlen_q) - 1;
  const int t_first = qp0 + i0, t_last = qp0 + i_last;
  const int lo_first = max(0, t_first - W + 1);
  const int nc_max = max(0, t_last - W + 1) / blk;
  const int n_ct = (nc_max + BT - 1) / BT;
  const int n_wt = (t_last - lo_first + BT) / BT;
  const int ntiles = n_ct + n_wt;

  // this lane's query (rows past the end read the last row and are never stored)
  const int iq = i0 + 32 * pair + col;
  const bool qvalid = iq < a.seqlen_q;
  const int iqc = min(iq, a.seqlen_q - 1);
  const int tq = qp0 + iq;
  const int lo_q = max(0, tq - W + 1);
  const int nc_q = lo_q / blk;
  // the pair's query range (wave-uniform)
  const int iw0 = i0 + 32 * pair;
  const bool pair_has_q = iw0 <= i_last;
  const int iw1 = min(iw0 + 31, i_last);
  const int tw0 = qp0 + iw0, tw1 = qp0 + iw1;
  const int lo_w0 = max(0, tw0 - W + 1), lo_w1 = max(0, tw1 - W + 1);
  const int nc_w1 = lo_w1 / blk;

  // ---- B operand of the first product: Q^T (even wave) or dO^T (odd wave);
  // lane holds query `col`, dims 16ks + 8hf .. +8
  bf16x8 xf[32];
  {
    const uint16_t* src =
        role == 0 ? (const uint16_t*)a.q + b * a.sq.b + (int64_t)iqc * a.sq.s + (int64_t)h * a.sq.h
                  : (const uint16_t*)a.dout + b * a.sdo.b + (int64_t)iqc * a.sdo.s + (int64_t)h * a.sdo.h;
    src += 8 * hf;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) xf[ks] = __builtin_bit_cast(bf16x8, ld16(src + 16 * ks));
  }
  float* xd = (float*)(smem + 2 * DQ_STAGE + 2 * DQ_XB) + 32 * pair;  // D of the pair's queries
  float lse2 = 0.f;
  if (role == 1) {
    // D = <dO, O> for this lane's query (dims split over the two half-waves)
    const uint16_t* op = (const uint16_t*)a.o + b * a.so.b + (int64_t)iqc * a.so.s + (int64_t)h * a.so.h + 8 * hf;
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) {
      const bf16x8 ov = __builtin_bit_cast(bf16x8, ld16(op + 16 * ks));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)ov[e], (float)xf[ks][e], acc);
    }
    acc += __shfl_xor(acc, 32);
    if (hf == 0) {
      xd[col] = acc;
      if (qvalid) a.delta[((int64_t)b * a.h_q + h) * a.seqlen_q + iq] = acc;
    }
  } else {
    lse2 = a.lse[((int64_t)b * a.h_q + h) * a.seqlen_q + iqc] * kLog2e;
  }
  // settle the operand loads before the DMA pipeline (its waits are explicit)
#pragma unroll
  for (int ks = 0; ks < 32; ++ks) asm volatile("" ::"v"(xf[ks]));
  barrier_lds();
  const float dl = xd[col];

  const uint16_t* kcb = (const uint16_t*)a.kc + b * a.skc.b + (int64_t)g * a.skc.h;
  const uint16_t* kb = (const uint16_t*)a.k + b * a.sk.b + (int64_t)g * a.sk.h;
  const uint16_t* vcb = (const uint16_t*)a.vc + b * a.svc.b + (int64_t)g * a.svc.h;
  const uint16_t* vb = (const uint16_t*)a.v + b * a.sv.b + (int64_t)g * a.sv.h;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)smem;

  // DMA of tile tt into stage st: wave w copies K and V rows 8w .. 8w+7, one
  // row per call of dma_row(i), i < 16 (K rows first).
  const uint16_t* d_kbase = kcb;
  const uint16_t* d_vbase = vcb;
  int64_t d_ks = 0, d_vs = 0;
  int d_row0 = 0, d_rmax = 0;
  uint32_t d_kl = 0;
  auto dma_setup = [&](int tt, int st) __attribute__((always_inline)) {
    if (tt < n_ct) {
      d_kbase = kcb; d_vbase = vcb; d_ks = a.skc.s; d_vs = a.svc.s; d_row0 = tt * BT; d_rmax = nc_max - 1;
    } else {
      d_kbase = kb; d_vbase = vb; d_ks = a.sk.s; d_vs = a.sv.s;
      d_row0 = lo_first + (tt - n_ct) * BT - kvp0; d_rmax = t_last - kvp0;
    }
    d_kl = lds0 + st * DQ_STAGE;
  };
  auto dma_row = [&](int i) __attribute__((always_inline)) {
    const int r = 8 * w + (i & 7);
    const int64_t row = min(d_row0 + r, d_rmax);
    if (i < 8) dma16(d_kbase + row * d_ks + 8 * lane, d_kl + r * ROW2);
    else dma16(d_vbase + row * d_vs + 8 * lane, d_kl + TILE2 + r * ROW1);
  };
  auto issue = [&](int tt, int st) __attribute__((always_inline)) {
    dma_setup(tt, st);
#pragma unroll
    for (int i = 0; i < 16; ++i) dma_row(i);
  };

  unsigned char* xb = smem + 2 * DQ_STAGE + pair * DQ_XB;
  const uint32_t a_off = role == 0 ? col * ROW2 + 16 * hf : TILE2 + col * ROW1 + 16 * hf;
  const uint32_t kt_off = tr_off(lane, ROW2);
  const float c = p.c;

  f32x16 dq[8];  // dQ^T dims 256 role + 32 i .. (AGPRs)
  const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
  for (int i = 0; i < 8; ++i) zero_o(dq[i], zero8);

  // compute(tt): tile tt; the next tile's DMA rows are issued inside the
  // first product (or up front when this pair has nothing to do)
  auto compute = [&](int tt, int st, bool next) __attribute__((always_inline)) {
    const bool comp = tt < n_ct;
    const int j0 = tt * BT;
    const int p0 = lo_first + (tt - n_ct) * BT;
    const bool active = pair_has_q && (comp ? (j0 < nc_w1) : (p0 <= tw1 && p0 + BT - 1 >= lo_w0));
    const unsigned char* sb = smem + st * DQ_STAGE;
    f32x16 s;
    bf16x8 dsf[2];
    if (next) dma_setup(tt + 1, st ^ 1);
    if (!active && next) {
#pragma unroll
      for (int i = 0; i < 16; ++i) dma_row(i);
    }
    if (active) {
      product_d(s, sb + a_off, xf, [&](int ks) __attribute__((always_inline)) {
        if (next && (ks & 1)) dma_row(ks >> 1);
      });  // S^T (even) or dP^T (odd): keys x queries
      // even wave: P = exp2(S c - lse2) over the visible keys [klo, klo + kn)
      // of this lane's query (masked logits become -inf, so P = 0); then each
      // wave hands its 32x32 fp32 block to the other
      if (role == 0) {
        const int klo = comp ? 0 : lo_q - p0;
        const int kn = !qvalid ? 0 : comp ? max(nc_q - j0, 0) : tq - lo_q + 1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = s[r] * c - lse2;
          s[r] = __builtin_amdgcn_exp2f((unsigned)(acc_row(r, hf) - klo) < (unsigned)kn ? x : -INFINITY);
        }
      }
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(xb + 4096 * role + 1024 * q4 + 16 * lane) =
            f32x4{s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]};
    }
    barrier_lds();
    if (active) {
      // dS = P (dP - D), formed identically by both waves of the pair
      float ds[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 o4 = *reinterpret_cast<const f32x4*>(xb + 4096 * (1 - role) + 1024 * q4 + 16 * lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q4 + e;
          const float pr = role == 0 ? s[r] : o4[e];
          const float dp = role == 0 ? o4[e] : s[r];
          ds[r] = pr * (dp - dl);
        }
      }
      pack_b(ds, dsf);
      // dQ^T (dims of this wave's half) += K^T dS^T: 8 dim tiles x 2 key steps
      auto ldk = [&](int i) __attribute__((always_inline)) {  // MFMA i: dim tile 8 role + i%8, key step i/8
        return ld_tr_a(sb + kt_off + 64 * (8 * role + (i & 7)) + 16 * (i >> 3) * ROW2, ROW2);
      };
      bf16x8 kq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kq[i] = ldk(i);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bf16x8 ka = kq[i & 3];
        if (i + 4 < 16) kq[i & 3] = ldk(i + 4);
        if (i == 0) mfma_o_first(dq[i & 7], ka, dsf[i >> 3]);
        else mfma_o(dq[i & 7], ka, dsf[i >> 3]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  issue(0, 0);
  for (int tt = 0; tt < ntiles; ++tt) {
    barrier_dma();
    compute(tt, tt & 1, tt + 1 < ntiles);
  }

  // dq rows leave whole: the tile's 64 x 512 fp32 values are staged in the
  // idle LDS ([query][2 KB], 16-byte chunk c of row r in slot c ^ (r % 32)),
  // then each wave stores 16 rows with two 1-KB instructions each.
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
  barrier_lds();  // every wave is done with the last tile's stage
  {
    const float sc = a.scale;
    const int r = 32 * pair + col;  // this lane's query row in the tile
    float* rowp = reinterpret_cast<float*>(smem + r * 2048);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int cch = 8 * (8 * role + i) + 2 * q4 + hf;  // dims 32 (8 role + i) + 8 q4 + 4 hf .. +3
        *reinterpret_cast<f32x4*>(rowp + 4 * (cch ^ (r & 31))) =
            f32x4{dq[i][4 * q4] * sc, dq[i][4 * q4 + 1] * sc, dq[i][4 * q4 + 2] * sc, dq[i][4 * q4 + 3] * sc};
      }
  }
  barrier_lds();
#pragma unroll 4
  for (int j = 0; j < DQ_BM / 4; ++j) {
    const int r = (DQ_BM / 4) * w + j;
    if (i0 + r >= a.seqlen_q) break;
    const float* rowp = reinterpret_cast<const float*>(smem + r * 2048);
    float* dst = a.dq + b * a.sdq.b + (int64_t)(i0 + r) * a.sdq.s + (int64_t)h * a.sdq.h;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int cch = 64 * half + lane;
      *reinterpret_cast<f32x4*>(dst + 4 * cch) = *reinterpret_cast<const f32x4*>(rowp + 4 * (cch ^ (r & 31)));
    }
  }
}

// ------------------------------------------------------------------ dkv kernel

constexpr int KV_BN = 64;                  // keys per workgroup
constexpr int KV_STAGE = 2 * TILE2 + 256;  // Q tile, dO tile, lse[32], D[32]
constexpr int KV_SMEM = 2 * KV_STAGE + 2 * KV_XB;

struct DkvParams {
  BwdArgs a;
  int n_rt;     // raw key tiles of 64 per (batch, KV head)
  int n_ci;     // compressed chunk items per (batch, KV head)
  int lc;       // query tiles (of 32) per chunk; chunk m covers query tiles [lc m, lc (m + 1))
  int mode;     // items launched: 0 all, 1 compressed chunks only, 2 raw tiles only
  int total;    // batch * h_kv * (items per (batch, KV head) of this mode)
  float c;      // scale * log2(e)
  float* part;  // compressed partials [batch*h_kv*n_ci][64][512] for dK, then the same for dV
  // when set (mode 2, after the reduce): raw row r of a whole block also gets
  // the compressor's share w[g, r % block] * dkc[r / block] (resp. dvc)
  const float* fw_k;
  const float* fw_v;
};

// First query tile (of 32) that sees compressed tile ct (entries 64ct ..), or
// -1 when no query does.  Non-decreasing in ct.
__device__ __host__ __forceinline__ int comp_first_qt(int64_t block, int64_t window, int64_t q_pos0, int seqlen_q,
                                                      int ct) {
  const int64_t t_star = block * (64 * ct + 1) + window - 1;  // first position that sees entry 64ct
  const int64_t i_first = t_star - q_pos0 > 0 ? t_star - q_pos0 : 0;
  return i_first > seqlen_q - 1 ? -1 : (int)(i_first / BT);
}

// Compressed work items of one (batch, KV head), chunk-major: for m = m0 ..
// m_last, every compressed tile ct that some query of chunk m sees (a prefix
// 0 .. A(m) - 1 of the tiles, since first_qt grows with ct).  Items of the
// same m read the same query tiles, so running them side by side shares L2.
struct CompPlan {
  int n_ct;    // compressed tiles seen by any query
  int m_last;  // last chunk
  int lc;
};
__device__ __host__ __forceinline__ int comp_tiles_active(const CompPlan& cp, int m, int64_t block, int64_t window,
                                                          int64_t q_pos0, int seqlen_q) {
  int n = 0;
  while (n < cp.n_ct && comp_first_qt(block, window, q_pos0, seqlen_q, n) / cp.lc <= m) ++n;
  return n;
}

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd512_dkv_kernel(DkvParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[KV_SMEM];
  const BwdArgs& a = p.a;
  // items of one (batch, KV head) are contiguous and each XCD takes a
  // contiguous range of items; within a (batch, KV head): compressed chunks
  // (chunk-major), then raw tiles in key order
  const int item = xcd_remap(blockIdx.x, p.total);
  if (item < 0) return;
  const int group = a.h_q / a.h_kv;
  const int W = a.window, blk = a.block;
  const int qp0 = (int)a.q_pos0, kvp0 = (int)a.kv_pos0;
  const int per_bg = p.mode == 0 ? p.n_ci + p.n_rt : p.mode == 1 ? p.n_ci : p.n_rt;
  const int bg = item / per_bg;
  const int local = item % per_bg + (p.mode == 2 ? p.n_ci : 0);
  const int qt_end = (a.seqlen_q - 1) / BT;

  bool comp;
  int row0, qt_lo, qt_hi, pidx = 0;
  if (local < p.n_ci) {
    comp = true;
    pidx = bg * p.n_ci + local;
    CompPlan cp;
    cp.lc = p.lc;
    cp.n_ct = 0;
    while (64 * cp.n_ct < a.n_blocks && comp_first_qt(blk, W, a.q_pos0, a.seqlen_q, cp.n_ct) >= 0) ++cp.n_ct;
    int m = comp_first_qt(blk, W, a.q_pos0, a.seqlen_q, 0) / p.lc;
    int c = local, n;
    while (c >= (n = comp_tiles_active(cp, m, blk, W, a.q_pos0, a.seqlen_q))) {
      c -= n;
      ++m;
    }
    const int ct = c;
    row0 = 64 * ct;  // entries
    qt_lo = max(comp_first_qt(blk, W, a.q_pos0, a.seqlen_q, ct), p.lc * m);
    qt_hi = min(p.lc * (m + 1) - 1, qt_end);
  } else {
    comp = false;
    const int r = local - p.n_ci;
    row0 = KV_BN * r;  // raw rows
    const int px0 = kvp0 + row0, px1 = kvp0 + min(row0 + KV_BN, a.seqlen_kv) - 1;
    const int i_lo = max(0, px0 - qp0), i_hi = min(a.seqlen_q - 1, px1 + W - 1 - qp0);
    qt_lo = i_lo / BT;
    qt_hi = i_lo <= i_hi ? i_hi / BT : qt_lo - 1;
  }
  const int g = bg % a.h_kv, b = bg / a.h_kv;
  const int nq = qt_hi - qt_lo + 1;
  const int ntiles = nq > 0 ? nq * group : 0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = w >> 1, role = w & 1;
  const int col = lane & 31, hf = lane >> 5;

  // this lane's key: raw row or compressed entry row0 + 32 pair + col
  const int n_rows = comp ? a.n_blocks : a.seqlen_kv;
  const int kr = row0 + 32 * pair + col;
  const bool kvalid = kr < n_rows;
  const int krc = min(kr, n_rows - 1);
  const int pk = kvp0 + kr;  // raw key position
  // query positions that see this lane's key: [vt_lo, vt_lo + vt_n).  A raw
  // key at position pk is in the windows of pk .. pk + W - 1; compressed entry
  // kr in the set of every position from blk (kr + 1) + W - 1 on.
  int vt_lo, vt_n;
  {
    const int64_t q_end = (int64_t)qp0 + a.seqlen_q;  // exclusive
    const int64_t lo = comp ? (int64_t)blk * (kr + 1) + W - 1 : (int64_t)pk;
    const int64_t hi = comp ? q_end : (pk + (int64_t)W < q_end ? pk + (int64_t)W : q_end);
    vt_lo = (int)(lo < q_end ? lo : q_end);
    vt_n = kvalid && hi > lo ? (int)(hi - lo) : 0;
  }
  // the pair's keys (wave-uniform): [e0, e1] rows
  const int e0 = row0 + 32 * pair, e1 = min(e0 + 31, n_rows - 1);
  const bool pair_has_k = e0 <= e1;

  // ---- B operand of the first product: K^T (even wave) or V^T (odd wave)
  bf16x8 xf[32];
  {
    const uint16_t* src;
    if (comp)
      src = role == 0 ? (const uint16_t*)a.kc + b * a.skc.b + (int64_t)krc * a.skc.s + (int64_t)g * a.skc.h
                      : (const uint16_t*)a.vc + b * a.svc.b + (int64_t)krc * a.svc.s + (int64_t)g * a.svc.h;
    else
      src = role == 0 ? (const uint16_t*)a.k + b * a.sk.b + (int64_t)krc * a.sk.s + (int64_t)g * a.sk.h
                      : (const uint16_t*)a.v + b * a.sv.b + (int64_t)krc * a.sv.s + (int64_t)g * a.sv.h;
    src += 8 * hf;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) xf[ks] = __builtin_bit_cast(bf16x8, ld16(src + 16 * ks));
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) asm volatile("" ::"v"(xf[ks]));
  }

  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)smem;
  // DMA of tile tt (head g*group + tt / nq, query tile qt_lo + tt % nq) into
  // stage st: wave w copies Q and dO rows 8w .. 8w+7, one row per call of
  // dma_row(i), i < 16; wave 0 also the tile's lse and D (dma_stats).
  const uint16_t* d_qb = nullptr;
  const uint16_t* d_ob = nullptr;
  int d_qi0 = 0;
  int64_t d_sbase = 0;
  uint32_t d_ql = 0;
  auto dma_setup = [&](int tt, int st) __attribute__((always_inline)) {
    const int h = g * group + tt / nq;
    d_qi0 = BT * (qt_lo + tt % nq);
    d_qb = (const uint16_t*)a.q + b * a.sq.b + (int64_t)h * a.sq.h;
    d_ob = (const uint16_t*)a.dout + b * a.sdo.b + (int64_t)h * a.sdo.h;
    d_sbase = ((int64_t)b * a.h_q + h) * a.seqlen_q;
    d_ql = lds0 + st * KV_STAGE;
  };
  auto dma_row = [&](int i) __attribute__((always_inline)) {
    const int r = 8 * w + (i & 7);
    const int64_t row = min(d_qi0 + r, a.seqlen_q - 1);
    if (i < 8) dma16(d_qb + row * a.sq.s + 8 * lane, d_ql + r * ROW2);
    else dma16(d_ob + row * a.sdo.s + 8 * lane, d_ql + TILE2 + r * ROW2);
  };
  auto dma_stats = [&]() __attribute__((always_inline)) {
    if (w == 0) {
      const int qi = min(d_qi0 + (lane & 31), a.seqlen_q - 1);
      dma4(lane < 32 ? (const void*)(a.lse + d_sbase + qi) : (const void*)(a.delta + d_sbase + qi), d_ql + 2 * TILE2);
    }
  };
  auto issue = [&](int tt, int st) __attribute__((always_inline)) {
    dma_setup(tt, st);
#pragma unroll
    for (int i = 0; i < 16; ++i) dma_row(i);
    dma_stats();
  };

  unsigned char* xb = smem + 2 * KV_STAGE + pair * KV_XB;
  const uint32_t a_off = (role == 0 ? 0 : TILE2) + col * ROW2 + 16 * hf;
  const uint32_t t_off = (role == 0 ? 0 : TILE2) + tr_off(lane, ROW2);
  const float c = p.c;

  f32x16 acc[16];  // dK^T (even wave) or dV^T (odd wave): dims 32 i .. x the pair's keys (AGPRs)
  const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
  for (int i = 0; i < 16; ++i) zero_o(acc[i], zero8);

  auto compute = [&](int tt, int st, bool next) __attribute__((always_inline)) {
    const int qi0 = BT * (qt_lo + tt % nq);
    const int ta = qp0 + qi0, tb = qp0 + min(qi0 + BT, a.seqlen_q) - 1;  // the tile's query positions
    bool active;
    if (comp) {
      active = pair_has_k && (max(0, tb - W + 1) / blk > e0);
    } else {
      active = pair_has_k && tb >= kvp0 + e0 && ta <= kvp0 + e1 + W - 1;
    }
    const unsigned char* sb = smem + st * KV_STAGE;
    const float* s_lse = (const float*)(sb + 2 * TILE2);
    f32x16 s;
    float pr[16];
    if (next) {
      dma_setup(tt + 1, st ^ 1);
      dma_stats();
    }
    if (!active && next) {
#pragma unroll
      for (int i = 0; i < 16; ++i) dma_row(i);
    }
    if (active) {
      product_d(s, sb + a_off, xf, [&](int ks) __attribute__((always_inline)) {
        if (next && (ks & 1)) dma_row(ks >> 1);
      });  // S = Q K^T (even) or dP = dO V^T (odd): queries x keys
      if (role == 0) {
        // masked logits become -inf, so P = 0
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qq = acc_row(r, hf);
          const float x = s[r] * c - s_lse[qq] * kLog2e;
          pr[r] = __builtin_amdgcn_exp2f((unsigned)(ta + qq - vt_lo) < vt_n ? x : -INFINITY);
        }
        bf16x8 pf[2];
        pack_b(pr, pf);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) *reinterpret_cast<bf16x8*>(xb + 4096 + 1024 * ks + 16 * lane) = pf[ks];
      } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(xb + 1024 * q4 + 16 * lane) = f32x4{s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]};
      }
    }
    barrier_lds();
    if (active) {
      bf16x8 bf[2];
      if (role == 0) {
        float ds[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 dp = *reinterpret_cast<const f32x4*>(xb + 1024 * q4 + 16 * lane);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * q4 + e;
            ds[r] = pr[r] * (dp[e] - s_lse[32 + acc_row(r, hf)]);
          }
        }
        pack_b(ds, bf);
      } else {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) bf[ks] = *reinterpret_cast<const bf16x8*>(xb + 4096 + 1024 * ks + 16 * lane);
      }
      // dK^T += Q^T dS (even) / dV^T += dO^T P (odd): 16 dim tiles x 2 query steps
      auto ldt = [&](int i) __attribute__((always_inline)) {  // MFMA i: dim tile i%16, query step i/16
        return ld_tr_a(sb + t_off + 64 * (i & 15) + 16 * (i >> 4) * ROW2, ROW2);
      };
      bf16x8 tq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) tq[i] = ldt(i);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const bf16x8 ta_ = tq[i & 3];
        if (i + 4 < 32) tq[i & 3] = ldt(i + 4);
        if (i == 0) mfma_o_first(acc[i & 15], ta_, bf[i >> 4]);
        else mfma_o(acc[i & 15], ta_, bf[i >> 4]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  if (ntiles > 0) {
    issue(0, 0);
    for (int tt = 0; tt < ntiles; ++tt) {
      barrier_dma();
      compute(tt, tt & 1, tt + 1 < ntiles);
    }
  }

  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
  float* dst;
  if (comp) {
    dst = p.part + (size_t)role * a.batch * a.h_kv * p.n_ci * KV_BN * D + ((size_t)pidx * KV_BN + 32 * pair + col) * D;
  } else {
    if (!kvalid) return;
    dst = role == 0 ? a.dk + b * a.sdk.b + (int64_t)kr * a.sdk.s + (int64_t)g * a.sdk.h
                    : a.dv + b * a.sdv.b + (int64_t)kr * a.sdv.s + (int64_t)g * a.sdv.h;
  }
  dst += 4 * hf;
  const float sc = role == 0 ? a.scale : 1.f;
  if (!comp && p.fw_k && kr < a.n_blocks * blk) {
    // fused compressor backward: + w[g, r % block] * d(compressed row r / block)
    const float wgt = (role == 0 ? p.fw_k : p.fw_v)[g * blk + kr % blk];
    const float* cr = role == 0 ? a.dkc + b * a.sdkc.b + (int64_t)(kr / blk) * a.sdkc.s + (int64_t)g * a.sdkc.h
                                : a.dvc + b * a.sdvc.b + (int64_t)(kr / blk) * a.sdvc.s + (int64_t)g * a.sdvc.h;
    cr += 4 * hf;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 cv = *reinterpret_cast<const f32x4*>(cr + 32 * i + 8 * q4);
        *reinterpret_cast<f32x4*>(dst + 32 * i + 8 * q4) =
            f32x4{fmaf(acc[i][4 * q4], sc, wgt * cv[0]), fmaf(acc[i][4 * q4 + 1], sc, wgt * cv[1]),
                  fmaf(acc[i][4 * q4 + 2], sc, wgt * cv[2]), fmaf(acc[i][4 * q4 + 3], sc, wgt * cv[3])};
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<f32x4*>(dst + 32 * i + 8 * q4) =
          f32x4{acc[i][4 * q4] * sc, acc[i][4 * q4 + 1] * sc, acc[i][4 * q4 + 2] * sc, acc[i][4 * q4 + 3] * sc};
}

// Compressed plan of one (batch, KV head) from the host or the device.
__device__ __host__ __forceinline__ CompPlan comp_plan(int64_t block, int64_t window, int64_t q_pos0, int seqlen_q,
                                                       int n_blocks, int lc) {
  CompPlan cp;
  cp.lc = lc;
  cp.n_ct = 0;
  while (64 * cp.n_ct < n_blocks && comp_first_qt(block, window, q_pos0, seqlen_q, cp.n_ct) >= 0) ++cp.n_ct;
  cp.m_last = ((seqlen_q - 1) / BT) / lc;
  return cp;
}

// dkc/dvc[b, j, g, :] = sum over the chunks m (in order) of the partials of
// j's tile.  One workgroup of 128 threads (4 dims each) per (entry, head, batch).
__global__ __launch_bounds__(128) void bwd512_reduce_kernel(DkvParams p) {
  const BwdArgs& a = p.a;
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int ct = j / KV_BN;
  const CompPlan cp = comp_plan(a.block, a.window, a.q_pos0, a.seqlen_q, a.n_blocks, p.lc);
  const int e = 4 * threadIdx.x;
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  if (ct < cp.n_ct) {
    const size_t vofs = (size_t)a.batch * a.h_kv * p.n_ci * KV_BN * D;
    const size_t base = (size_t)(b * a.h_kv + g) * p.n_ci;
    int prefix = 0;
    for (int m = comp_first_qt(a.block, a.window, a.q_pos0, a.seqlen_q, 0) / p.lc; m <= cp.m_last; ++m) {
      const int n = comp_tiles_active(cp, m, a.block, a.window, a.q_pos0, a.seqlen_q);
      if (ct < n) {
        const float* pk = p.part + ((base + prefix + ct) * KV_BN + (j % KV_BN)) * D + e;
        sk += *reinterpret_cast<const f32x4*>(pk);
        sv += *reinterpret_cast<const f32x4*>(pk + vofs);
      }
      prefix += n;
    }
  }
  *reinterpret_cast<f32x4*>(a.dkc + b * a.sdkc.b + (int64_t)j * a.sdkc.s + (int64_t)g * a.sdkc.h + e) = sk;
  *reinterpret_cast<f32x4*>(a.dvc + b * a.sdvc.b + (int64_t)j * a.sdvc.s + (int64_t)g * a.sdvc.h + e) = sv;
}

// Query tiles of 32 per chunk: at least 32, and at most 32 chunks.
int chunk_len(int seqlen_q) {
  const int n_qt = (seqlen_q + BT - 1) / BT;
  return max(32, (n_qt + 31) / 32);
}

// Compressed chunk items per (batch, KV head).
int n_chunk_items(int seqlen_q, int64_t q_pos0, int n_blocks, int block, int window) {
  const int lc = chunk_len(seqlen_q);
  const CompPlan cp = comp_plan(block, window, q_pos0, seqlen_q, n_blocks, lc);
  int n = 0;
  for (int ct = 0; ct < cp.n_ct; ++ct) n += cp.m_last - comp_first_qt(block, window, q_pos0, seqlen_q, ct) / lc + 1;
  return n;
}

}  // namespace

size_t hca_bwd512_workspace_bytes(int batch, int seqlen_q, int64_t q_pos0, int n_blocks, int h_q, int h_kv,
                                  int block, int window) {
  const size_t delta = ((size_t)batch * h_q * seqlen_q * sizeof(float) + 255) / 256 * 256;
  const size_t n_ci = (size_t)n_chunk_items(seqlen_q, q_pos0, n_blocks, block, window);
  return delta + 2 * (size_t)batch * h_kv * n_ci * KV_BN * D * sizeof(float);
}

hipError_t launch_hca_attn_bwd512(BwdArgs a, void* ws, hipStream_t st, const float* fw_k, const float* fw_v) {
  a.delta = (float*)ws;
  DqParams dp;
  dp.a = a;
  dp.n_qt = (a.seqlen_q + DQ_BM - 1) / DQ_BM;
  dp.total = a.batch * a.h_q * dp.n_qt;
  dp.c = a.scale * kLog2e;
  hipLaunchKernelGGL(bwd512_dq_kernel, dim3(((dp.total + 7) / 8) * 8), dim3(256), 0, st, dp);

  DkvParams kp;
  kp.a = a;
  kp.n_rt = (a.seqlen_kv + KV_BN - 1) / KV_BN;
  kp.lc = chunk_len(a.seqlen_q);
  kp.n_ci = n_chunk_items(a.seqlen_q, a.q_pos0, a.n_blocks, a.block, a.window);
  kp.c = dp.c;
  kp.part = (float*)((char*)ws + ((size_t)a.batch * a.h_q * a.seqlen_q * sizeof(float) + 255) / 256 * 256);
  kp.fw_k = nullptr;
  kp.fw_v = nullptr;
  const int bgs = a.batch * a.h_kv;
  if (!fw_k) {
    kp.mode = 0;
    kp.total = bgs * (kp.n_ci + kp.n_rt);
    hipLaunchKernelGGL(bwd512_dkv_kernel, dim3(((kp.total + 7) / 8) * 8), dim3(256), 0, st, kp);
    if (a.n_blocks > 0)
      hipLaunchKernelGGL(bwd512_reduce_kernel, dim3(a.n_blocks, a.h_kv, a.batch), dim3(128), 0, st, kp);
    return hipGetLastError();
  }
  // fused compressor backward: compressed entries first, their sums, then the
  // raw rows (which add the compressor's share of their block)
  if (kp.n_ci > 0) {
    kp.mode = 1;
    kp.total = bgs * kp.n_ci;
    hipLaunchKernelGGL(bwd512_dkv_kernel, dim3(((kp.total + 7) / 8) * 8), dim3(256), 0, st, kp);
  }
  if (a.n_blocks > 0)
    hipLaunchKernelGGL(bwd512_reduce_kernel, dim3(a.n_blocks, a.h_kv, a.batch), dim3(128), 0, st, kp);
  kp.mode = 2;
  kp.total = bgs * kp.n_rt;
  kp.fw_k = fw_k;
  kp.fw_v = fw_v;
  hipLaunchKernelGGL(bwd512_dkv_kernel, dim3(((kp.total + 7) / 8) * 8), dim3(256), 0, st, kp);
  return hipGetLastError();
}

}  // namespace hca
