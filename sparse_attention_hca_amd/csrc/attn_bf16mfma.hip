// HCA attention in bf16 on the matrix cores for head sizes 64, 128 and 256
// (ERNIE 5.5 Flash Base pages: mirrorspeed page, "Hybrid sparse attention"
// section -- each query attends with one softmax over the compressed entries
// of the blocks that end before its window and over its window of the W most
// recent raw positions).  The 512-wide heads of the HCA layers have their own
// kernels; this one serves the narrower heads with no limit on the number of
// keys a query sees.
//
// One workgroup (4 waves) per 64 consecutive queries of one head; wave w owns
// queries 16w .. 16w+15 (the MFMA columns).  The workgroup walks the keys any
// of its queries sees -- compressed entries [0, n_c(last query)) then raw
// positions [lo(first query), last query] -- in tiles of 16 rows staged in
// LDS (rows padded by 16 bytes, so the 16-byte K operand reads of 16
// consecutive rows fall on distinct banks).  Per tile:
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (Q^T fragments in registers,
//     D/32 steps): a lane holds keys 4g .. 4g+3 (g = lane / 16) of its query;
//   * per-pair visibility mask and an online softmax per query (fp32, log2
//     domain, exact running maximum);
//   * O^T += V^T P^T with v_mfma_f32_16x16x16_bf16: the B operand (keys 4g ..
//     4g+3 of the lane's query) is the lane's own four probabilities rounded
//     to bf16, so P needs no exchange; the A operand gathers the same four
//     keys of one dim from the staged V rows.
// The row sum adds the fp32 probabilities; the output is rounded to bf16 once.
#include "device_common.h"
#include "launchers.h"

namespace hca {
namespace {

constexpr int QW = 16;  // queries per wave
constexpr int QB = 64;  // queries per workgroup
constexpr int TK = 16;  // keys per tile

typedef unsigned short us4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(256) void attn_bf16mfma_kernel(AttnArgs a) {
  constexpr int LDB = 2 * D + 16;  // LDS bytes per staged row
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) unsigned char ks[TK * LDB];
  __shared__ __attribute__((aligned(16))) unsigned char vs[TK * LDB];

  const int h = blockIdx.y, b = blockIdx.z;
  const int g_kv = h / (a.h_q / a.h_kv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, grp = lane >> 4;
  const int i0 = blockIdx.x * QB;
  const int i_last = min(i0 + QB, a.seqlen_q) - 1;
  const int i = min(i0 + QW * w + c, i_last);  // this lane's query (clamped past the end)
  const bool live = i0 + QW * w + c <= i_last;
  const int64_t t = a.q_pos0 + i;
  const int64_t lo = t - a.window + 1 > 0 ? t - a.window + 1 : 0;
  const int n_c = (int)(lo / a.block);
  // the workgroup's key ranges
  const int64_t t_first = a.q_pos0 + i0, t_max = a.q_pos0 + i_last;
  const int64_t LO = t_first - a.window + 1 > 0 ? t_first - a.window + 1 : 0;
  const int64_t lo_max = t_max - a.window + 1 > 0 ? t_max - a.window + 1 : 0;
  const int NC = (int)(lo_max / a.block);
  const int n_ct = (NC + TK - 1) / TK;
  const int n_rt = (int)((t_max - LO + 1 + TK - 1) / TK);

  // Q^T fragments (B operand of step s): query i, dims 32s + 8grp .. +7
  bf16x8 qf[D / 32];
  {
    const uint16_t* qp = (const uint16_t*)a.q + b * a.sq.b + (int64_t)i * a.sq.s + (int64_t)h * a.sq.h + 8 * grp;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qf[s] = __builtin_bit_cast(bf16x8, ld16(qp + 32 * s));
  }
  const uint16_t* kcb = (const uint16_t*)a.kc + b * a.skc.b + (int64_t)g_kv * a.skc.h;
  const uint16_t* vcb = (const uint16_t*)a.vc + b * a.svc.b + (int64_t)g_kv * a.svc.h;
  const uint16_t* kb = (const uint16_t*)a.k + b * a.sk.b + (int64_t)g_kv * a.sk.h;
  const uint16_t* vb = (const uint16_t*)a.v + b * a.sv.b + (int64_t)g_kv * a.sv.h;
  const float cl2 = a.scale * kLog2e;

  f32x4 oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int tt = 0; tt < n_ct + n_rt; ++tt) {
    const bool comp = tt < n_ct;
    const int64_t base = comp ? (int64_t)tt * TK : LO + (int64_t)(tt - n_ct) * TK;  // entry / position of row 0
    // stage the tile's K and V rows (rows past the range re-read the last one
    // and are masked below)
    __syncthreads();
    for (int e = tid; e < TK * CPR; e += 256) {
      const int r = e / CPR, c8 = e % CPR;
      const uint16_t *kp, *vp;
      if (comp) {
        const int64_t j = min<int64_t>(base + r, NC - 1);
        kp = kcb + j * a.skc.s;
        vp = vcb + j * a.svc.s;
      } else {
        const int64_t u = min<int64_t>(base + r, t_max) - a.kv_pos0;
        kp = kb + u * a.sk.s;
        vp = vb + u * a.sv.s;
      }
      *reinterpret_cast<u32x4*>(ks + r * LDB + 16 * c8) = ld16(kp + 8 * c8);
      *reinterpret_cast<u32x4*>(vs + r * LDB + 16 * c8) = ld16(vp + 8 * c8);
    }
    __syncthreads();

    // S^T = K Q^T: rows = the tile's keys (A operand: key c, dims 32s + 8grp ..)
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ks + c * LDB + 2 * (32 * s + 8 * grp)));
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[s], sacc, 0, 0, 0);
    }
    // this lane holds keys 4grp + r of query c
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t key = base + 4 * grp + r;
      const bool vis = comp ? key < n_c : (key >= lo && key <= t);
      sv[r] = vis ? sacc[r] * cl2 : -INFINITY;
    }
    float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    float p[4];
    if (m_new == -INFINITY) {  // nothing visible yet for this query
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = 0.f;
    } else {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[db][r] *= alpha;
      l_run *= alpha;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = __builtin_amdgcn_exp2f(sv[r] - m_new);  // 0 for masked keys
        l_run += p[r];
      }
      m_run = m_new;
    }
    // O^T += V^T P^T over the tile's 16 keys: B = this lane's p (keys 4grp ..
    // 4grp+3 of query c), A = dim 16db + c of the same four keys
    u32x2 pk;
    pk[0] = pack_bf16x2(p[0], p[1]);
    pk[1] = pack_bf16x2(p[2], p[3]);
    const bf16x4 pb = __builtin_bit_cast(bf16x4, pk);
    const uint16_t* vrow = reinterpret_cast<const uint16_t*>(vs + 4 * grp * LDB) + c;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const us4 vv = us4{vrow[16 * db], vrow[LDB / 2 + 16 * db], vrow[LDB + 16 * db], vrow[3 * (LDB / 2) + 16 * db]};
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, vv), pb, oacc[db], 0, 0, 0);
    }
  }

  // epilogue: row sums over the lane group, normalise, store O (4 consecutive
  // dims per lane, bf16) and lse
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!live) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* op = (uint16_t*)a.o + b * a.so.b + (int64_t)i * a.so.s + (int64_t)h * a.so.h + 4 * grp;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    u32x2 ov;
    ov[0] = pack_bf16x2(oacc[db][0] * inv, oacc[db][1] * inv);
    ov[1] = pack_bf16x2(oacc[db][2] * inv, oacc[db][3] * inv);
    *reinterpret_cast<u32x2*>(op + 16 * db) = ov;
  }
  if (a.lse && grp == 0)
    a.lse[((int64_t)b * a.h_q + h) * a.seqlen_q + i] = l_tot > 0.f ? m_run * kLn2 + __logf(l_tot) : -INFINITY;
}

}  // namespace

bool attn_bf16mfma_supports(int dt, int head_dim) {
  return dt == 1 && (head_dim == 64 || head_dim == 128 || head_dim == 256);
}

hipError_t launch_attn_bf16mfma(const AttnArgs& a, hipStream_t st) {
  const dim3 grid((a.seqlen_q + QB - 1) / QB, a.h_q, a.batch), block(256);
  switch (a.head_dim) {
    case 64: hipLaunchKernelGGL(attn_bf16mfma_kernel<64>, grid, block, 0, st, a); break;
    case 128: hipLaunchKernelGGL(attn_bf16mfma_kernel<128>, grid, block, 0, st, a); break;
    case 256: hipLaunchKernelGGL(attn_bf16mfma_kernel<256>, grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hca
