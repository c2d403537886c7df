// DSA core attention over the top-k selected positions, bf16, d_qk = d_v = 256
// (ERNIE 5.5 Flash Base pages: mirrorspeed page, "Hybrid sparse attention"
// section -- core attention only on the top-k positions; ai-club.cn page,
// hybrid attention section -- 256-wide heads in the full-context layers).
//
// One workgroup (4 waves) per (query position, group of 64 query heads that
// share one KV head).  Every query head of the group attends over the same
// gathered rows, so the group is packed into the MFMA columns: each wave owns
// 16 heads and computes S^T = K Q^T (16 keys x 16 heads,
// v_mfma_f32_16x16x32_bf16) and O^T += V^T P^T (v_mfma_f32_16x16x16_bf16).
// Gathered K/V rows (512 B each) are loaded one 16-key tile ahead into
// registers (half a wave per row, 16-byte lanes), staged in two LDS stages
// (K chunk-swizzled, V transposed in registers to V^T), one barrier per tile.
// Softmax is online in fp32 with a lazy rescale.  Index entries of -1 are
// skipped; a position outside [0, seqlen) poisons the row with NaN.
#include "device_common.h"
#include "launchers.h"

namespace hca {
namespace {

constexpr int D = 256;
constexpr int TK = 16;
constexpr int HPW = 16;  // heads per wave
constexpr int HPB = 64;  // heads per workgroup

struct SparseParams {
  const uint16_t* q; LStrides sq;
  const uint16_t* k; LStrides sk;
  const uint16_t* v; LStrides sv;
  const int32_t* idx;
  uint16_t* o; LStrides so;
  float* lse;
  int seqlen, h_q, h_kv, topk, n_hb;
  float c;
};

__device__ __forceinline__ int vt_swz(int dim) { return (dim >> 2) & 3; }

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void sparse_attn256_kernel(SparseParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2 * TK * D];  // [stage][key][dim], chunk c at c ^ (key & 7)
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2 * D * TK];  // [stage][dim][key], chunk swizzle
  __shared__ int bad_sh;

  const int t = blockIdx.x;
  const int hb = blockIdx.y % p.n_hb;
  const int g = blockIdx.y / p.n_hb;     // KV head
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int group = p.h_q / p.h_kv;
  const int hq = g * group + hb * HPB + w * HPW + col;
  if (tid == 0) bad_sh = 0;

  bf16x8 qf[8];
  {
    const uint16_t* qp = p.q + b * p.sq.b + (int64_t)t * p.sq.s + (int64_t)hq * p.sq.h + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, ld16(qp + 32 * ks));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qf[ks]));
  }
  const int32_t* irow = p.idx + ((int64_t)b * p.seqlen + t) * p.topk;
  const uint16_t* kb = p.k + b * p.sk.b + (int64_t)g * p.sk.h;
  const uint16_t* vb = p.v + b * p.sv.b + (int64_t)g * p.sv.h;

  // loaders: waves 0-1 gather K rows, waves 2-3 gather V rows; thread handles
  // keys 4*kg + i (i < 4) of the tile, kg = 2*(w & 1) + (lane >> 5), dims 8*(lane & 31) .. +8
  const bool is_v = w >= 2;
  const int kg = 2 * (w & 1) + (lane >> 5);
  const int ch = lane & 31;
  const int ntiles = (p.topk + TK - 1) / TK;
  int bad = 0;
  auto load_tile = [&](int tt, u32x4 (&R)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = tt * TK + 4 * kg + i;
      int u = j < p.topk ? irow[j] : -1;
      bad |= (u < -1 || u >= p.seqlen);
      const bool ok = u >= 0 && u < p.seqlen;
      u = ok ? u : 0;
      const uint16_t* src = (is_v ? vb + (int64_t)u * p.sv.s : kb + (int64_t)u * p.sk.s) + 8 * ch;
      R[i] = ld16(src) & ((ok || !is_v) ? ~0u : 0u);
    }
  };
  auto store_tile = [&](const u32x4 (&R)[4], int st) __attribute__((always_inline)) {
    if (!is_v) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 4 * kg + i;
        *reinterpret_cast<u32x4*>(Ks + st * (TK * D) + key * D + ((ch ^ (key & 7)) << 3)) = R[i];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        u32x2 x;
        x[0] = __builtin_amdgcn_perm(R[1][e >> 1], R[0][e >> 1], sel);
        x[1] = __builtin_amdgcn_perm(R[3][e >> 1], R[2][e >> 1], sel);
        const int dim = 8 * ch + e;
        *reinterpret_cast<u32x2*>(Vt + st * (D * TK) + dim * TK + ((kg ^ vt_swz(dim)) << 2)) = x;
      }
    }
  };

  f32x4 o[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_used = -INFINITY, l_run = 0.f;
  const float c = p.c;

  auto compute = [&](int tt, int st) __attribute__((always_inline)) {
    const uint16_t* kst = Ks + st * (TK * D);
    const uint16_t* vst = Vt + st * (D * TK);
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      const int h1 = (col >> 2) & 1;
      const uint16_t* kbase = kst + col * D + ((grp ^ (col & 3)) << 3);
      const uint16_t* keven = kbase + 32 * h1;
      const uint16_t* kodd = kbase - 32 * h1;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const uint16_t* kp = ((ks & 1) ? kodd : keven) + 32 * ks;
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kp)),
                                                    qf[ks], s, 0, 0, 0);
      }
    }
    float sv[4];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = tt * TK + 4 * grp + r;
      const int u = j < p.topk ? irow[j] : -1;
      const bool valid = u >= 0 && u < p.seqlen;
      sv[r] = valid ? s[r] * c : -INFINITY;
      mt = fmaxf(mt, sv[r]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool need = mt > m_used + 8.f;
    if (__any(need)) {
      const float new_m = need ? mt : m_used;
      const float alpha = need ? exp2f(m_used - new_m) : 1.f;
      m_used = new_m;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) o[dt] *= alpha;
    }
    float ps[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ps[r] = sv[r] == -INFINITY ? 0.f : exp2f(sv[r] - m_used);
      l_run += ps[r];
    }
    u32x2 pk;
    pk[0] = pack_bf16x2(ps[0], ps[1]);
    pk[1] = pack_bf16x2(ps[2], ps[3]);
    const bf16x4 pf = __builtin_bit_cast(bf16x4, pk);
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      const int dim = 16 * dt + col;
      const bf16x4 va =
          __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(vst + dim * TK + ((grp ^ vt_swz(dim)) << 2)));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pf, o[dt], 0, 0, 0);
    }
  };

  u32x4 R[4];
  const int last = max(ntiles - 1, 0);
  load_tile(0, R);
  for (int tt = 0; tt < ntiles; ++tt) {
    store_tile(R, tt & 1);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    load_tile(min(tt + 1, last), R);
    compute(tt, tt & 1);
  }
  if (bad) atomicOr(&bad_sh, 1);
  __syncthreads();
  const bool poisoned = bad_sh != 0;

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = poisoned ? __builtin_nanf("") : (l_tot > 0.f ? 1.f / l_tot : 0.f);
  uint16_t* op = p.o + b * p.so.b + (int64_t)t * p.so.s + (int64_t)hq * p.so.h + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) {
    u32x2 pk;
    pk[0] = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
    pk[1] = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
    *reinterpret_cast<u32x2*>(op + 16 * dt) = pk;
  }
  if (p.lse && grp == 0)
    p.lse[((int64_t)b * p.h_q + hq) * p.seqlen + t] =
        poisoned ? __builtin_nanf("") : m_used * kLn2 + __logf(l_tot);
}

}  // namespace

hipError_t launch_dsa_sparse_attn256(const void* q, LStrides sq, const void* k, LStrides sk, const void* v,
                                     LStrides sv, const int32_t* idx, void* o, LStrides so, float* lse, int batch,
                                     int seqlen, int h_q, int h_kv, int topk, float scale, hipStream_t st) {
  SparseParams p;
  p.q = (const uint16_t*)q; p.sq = sq;
  p.k = (const uint16_t*)k; p.sk = sk;
  p.v = (const uint16_t*)v; p.sv = sv;
  p.idx = idx;
  p.o = (uint16_t*)o; p.so = so;
  p.lse = lse;
  p.seqlen = seqlen; p.h_q = h_q; p.h_kv = h_kv; p.topk = topk;
  const int group = h_q / h_kv;
  if (group % HPB != 0) return hipErrorInvalidValue;
  p.n_hb = group / HPB;
  p.c = scale * kLog2e;
  dim3 grid(seqlen, h_kv * p.n_hb, batch);
  hipLaunchKernelGGL(sparse_attn256_kernel, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace hca
