// HCA attention in fp32 on the matrix cores (v_mfma_f32_16x16x4_f32), for
// head sizes 32, 64 and 128 (ERNIE 5.5 Flash Base pages: mirrorspeed page,
// "Hybrid sparse attention" section -- each query attends with one softmax
// over the compressed entries of the blocks that end before its window and
// over its window of the W most recent raw positions).
//
// One workgroup (4 waves) per 64 consecutive queries of one head; wave w owns
// queries 16w .. 16w+15 (the MFMA columns).  The workgroup walks the keys any
// of its queries sees -- compressed entries [0, n_c(last query)) then raw
// positions [lo(first query), last query] -- in tiles of 16 rows staged in
// LDS (rows padded to D + 4 floats, which keeps both operand reads on
// distinct banks).  Per tile a wave forms S^T = K Q^T (Q^T fragments held in
// registers, D/4 steps), masks each (query, key) pair by its visibility, and
// runs an online softmax per query (fp32, log2 domain); O^T += V^T P^T then
// takes P^T straight from the S^T accumulators by contracting the tile's keys
// in the order {4g + s} (step s, lane group g), so no exchange is needed.
#include "device_common.h"
#include "launchers.h"

namespace hca {
namespace {

constexpr int QW = 16;   // queries per wave
constexpr int QB = 64;   // queries per workgroup
constexpr int TKF = 16;  // keys per tile

template <int D>
__global__ __launch_bounds__(256) void attn_f32mfma_kernel(AttnArgs a) {
  constexpr int LD = D + 4;  // LDS row stride in floats
  __shared__ __attribute__((aligned(16))) float ks[TKF * LD];
  __shared__ __attribute__((aligned(16))) float vs[TKF * LD];

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
  const int n_ct = (NC + TKF - 1) / TKF;
  const int n_rt = (int)((t_max - LO + 1 + TKF - 1) / TKF);

  // Q^T fragments: query i, dims 4s + grp
  float qf[D / 4];
  {
    const float* qp = (const float*)a.q + b * a.sq.b + (int64_t)i * a.sq.s + (int64_t)h * a.sq.h + grp;
#pragma unroll
    for (int s = 0; s < D / 4; ++s) qf[s] = qp[4 * s];
  }
  const float* kcb = (const float*)a.kc + b * a.skc.b + (int64_t)g_kv * a.skc.h;
  const float* vcb = (const float*)a.vc + b * a.svc.b + (int64_t)g_kv * a.svc.h;
  const float* kb = (const float*)a.k + b * a.sk.b + (int64_t)g_kv * a.sk.h;
  const float* vb = (const float*)a.v + b * a.sv.b + (int64_t)g_kv * a.sv.h;
  const float cl2 = a.scale * kLog2e;

  f32x4 oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int tt = 0; tt < n_ct + n_rt; ++tt) {
    const bool comp = tt < n_ct;
    const int64_t base = comp ? (int64_t)tt * TKF : LO + (int64_t)(tt - n_ct) * TKF;  // entry / position of row 0
    // stage the tile's K and V rows (rows past the range are clamped and masked below)
    __syncthreads();
    for (int e = tid; e < TKF * D / 4; e += 256) {
      const int r = e / (D / 4), c4 = e % (D / 4);
      const float *kp, *vp;
      if (comp) {
        const int64_t j = min<int64_t>(base + r, NC - 1);
        kp = kcb + j * a.skc.s;
        vp = vcb + j * a.svc.s;
      } else {
        const int64_t u = min<int64_t>(base + r, t_max) - a.kv_pos0;
        kp = kb + u * a.sk.s;
        vp = vb + u * a.sv.s;
      }
      *reinterpret_cast<f32x4*>(ks + r * LD + 4 * c4) = *reinterpret_cast<const f32x4*>(kp + 4 * c4);
      *reinterpret_cast<f32x4*>(vs + r * LD + 4 * c4) = *reinterpret_cast<const f32x4*>(vp + 4 * c4);
    }
    __syncthreads();

    // S^T = K Q^T: rows = the tile's keys (lane row c), columns = this wave's queries
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 4; ++s)
      sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(ks[c * LD + 4 * s + grp], qf[s], sacc, 0, 0, 0);
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
    // O^T += V^T P^T, keys contracted in the order 4g + s (step s): the B
    // operand of step s is this lane's own p[s]
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vs[(4 * grp + s) * LD + 16 * db + c], p[s], oacc[db], 0, 0, 0);
  }

  // epilogue: row sums over the lane group, normalise, store O (4 consecutive dims per lane) and lse
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!live) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  float* op = (float*)a.o + b * a.so.b + (int64_t)i * a.so.s + (int64_t)h * a.so.h + 4 * grp;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    f32x4 x = oacc[db];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] *= inv;
    *reinterpret_cast<f32x4*>(op + 16 * db) = x;
  }
  if (a.lse && grp == 0)
    a.lse[((int64_t)b * a.h_q + h) * a.seqlen_q + i] = l_tot > 0.f ? m_run * kLn2 + __logf(l_tot) : -INFINITY;
}

}  // namespace

bool attn_f32mfma_supports(int dt, int head_dim) {
  return dt == 0 && (head_dim == 32 || head_dim == 64 || head_dim == 128);
}

hipError_t launch_attn_f32mfma(const AttnArgs& a, hipStream_t st) {
  const dim3 grid((a.seqlen_q + QB - 1) / QB, a.h_q, a.batch), block(256);
  switch (a.head_dim) {
    case 32: hipLaunchKernelGGL(attn_f32mfma_kernel<32>, grid, block, 0, st, a); break;
    case 64: hipLaunchKernelGGL(attn_f32mfma_kernel<64>, grid, block, 0, st, a); break;
    case 128: hipLaunchKernelGGL(attn_f32mfma_kernel<128>, grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hca
