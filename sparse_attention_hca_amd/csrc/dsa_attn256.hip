// DSA core attention over the top-k selected positions, bf16, d_qk = d_v = 256
// (ERNIE 5.5 Flash Base pages: mirrorspeed page, "Hybrid sparse attention"
// section -- core attention only on the top-k positions; ai-club.cn page,
// hybrid attention section -- 256-wide heads in the full-context layers).
//
// One workgroup (4 waves) per (query position, group of 64 query heads that
// share one KV head); every head of the group attends over the same gathered
// rows, so the heads are the MFMA columns: each wave owns 16 heads and
// computes S^T = K Q^T (32 keys x 16 heads, v_mfma_f32_16x16x32_bf16) and
// O^T += V^T P^T (256 dims x 16 heads, v_mfma_f32_16x16x32_bf16, the 32 keys
// of a tile as the contraction).
//
// The step is a gather of 2 x 512 bytes per selected position, so the design
// keeps as many rows in flight as LDS holds:
//   * The query's index row is copied to LDS once (positions past topk read
//     as -1).  Out-of-range positions are detected there; they and the -1
//     entries are fetched as row 0 (valid memory) and masked out.
//   * Tiles of 32 gathered K and V rows move global -> LDS with 16-byte LDS
//     DMA (each instruction fetches two rows, one per half-wave) through a ring
//     of 4 stages: three tiles (96 KB) in flight while one is consumed.  The
//     DMA is written as asm so the compiler does not wait for it before LDS
//     reads; the explicit vmcnt wait and barrier of each tile order them.
//   * Rows are stored with their 16-byte chunks XOR-swizzled (K chunk c of
//     row r in slot c ^ (r mod 16), V chunk c in slot c ^ 2(r mod 8); the DMA
//     lanes fetch the matching chunks), so the 16-byte K operand reads and
//     the gfx950 transposing V reads (ds_read_b64_tr_b16, which hands each
//     lane four consecutive keys of one dim: the V^T operand) hit distinct
//     bank groups.
//   * The S^T accumulators of a lane (one head, keys 4g .. 4g+3 and
//     16+4g .. 16+4g+3) are the P^T operand of the PV product once converted
//     to bf16; the V^T reads fetch keys in that order.
//   * Softmax is online in fp32 with a lazy rescale.
#include "device_common.h"
#include "launchers.h"

namespace hca {
namespace {

constexpr int D = 256;
constexpr int TK = 32;                 // keys per tile
constexpr int HPW = 16;                // heads per wave
constexpr int HPB = 64;                // heads per workgroup
constexpr int ROWB = 2 * D;            // bytes per K or V row
constexpr int KSTB = TK * ROWB;        // K part of a stage
constexpr int STAGEB = 2 * KSTB;       // K rows then V rows
constexpr int NRING = 4;               // ring stages; NRING - 1 tiles in flight
constexpr int MAX_TOPK = 4096;
constexpr int DMA_PER_TILE = 8;        // DMA instructions per wave per tile (4 K + 4 V)

typedef short s16x4 __attribute__((ext_vector_type(4)));

struct SparseParams {
  const uint16_t* q; LStrides sq;
  const uint16_t* k; LStrides sk;
  const uint16_t* v; LStrides sv;
  const int32_t* idx;
  uint16_t* o; LStrides so;
  float* lse;
  int seqlen, n_kv, h_q, h_kv, topk, n_hb;  // seqlen queries; positions < n_kv
  float c;
};

// 16-byte LDS DMA of one wave: lane l copies 16 bytes from g (per lane) to LDS
// byte address lds + 16 l (lds travels in M0).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void sparse_attn256_kernel(SparseParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[NRING * STAGEB];
  __shared__ __attribute__((aligned(16))) int sidx[MAX_TOPK];
  __shared__ int bad_sh;

  const int t = blockIdx.x;
  const int hb = blockIdx.y % p.n_hb;
  const int g = blockIdx.y / p.n_hb;     // KV head
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int group = p.h_q / p.h_kv;
  const int hq = g * group + hb * HPB + w * HPW + col;
  const int ntiles = (p.topk + TK - 1) / TK;

  // ---- index row -> LDS (-1 past topk); out-of-range positions flag the row
  {
    const int32_t* irow = p.idx + ((int64_t)b * p.seqlen + t) * p.topk;
    int bad = 0;
    for (int j = tid; j < ntiles * TK; j += 256) {
      int u = j < p.topk ? irow[j] : -1;
      bad |= (u < -1 || u >= p.n_kv);
      sidx[j] = (u >= 0 && u < p.n_kv) ? u : -1;
    }
    if (tid == 0) bad_sh = 0;
    __syncthreads();
    if (bad) atomicOr(&bad_sh, 1);
  }

  // ---- Q^T fragments (B operand): head `col`, dims 32ks + 8grp .. +8
  bf16x8 qf[8];
  {
    const uint16_t* qp = p.q + b * p.sq.b + (int64_t)t * p.sq.s + (int64_t)hq * p.sq.h + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, ld16(qp + 32 * ks));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qf[ks]));
  }
  __syncthreads();  // sidx and bad_sh complete; Q settled before the DMA ring

  const uint16_t* kb = p.k + b * p.sk.b + (int64_t)g * p.sk.h;
  const uint16_t* vb = p.v + b * p.sv.b + (int64_t)g * p.sv.h;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ring;

  // ---- DMA of tile tt into stage st: wave w fetches rows 8w .. 8w+7 of K and V;
  // instruction i covers rows 8w+2i (lanes 0-31) and 8w+2i+1 (lanes 32-63).
  const int hrow = lane >> 5, hl = lane & 31;
  auto issue = [&](int tt, int st) __attribute__((always_inline)) {
    const uint32_t kl = lds0 + st * STAGEB, vl = kl + KSTB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * w + 2 * i + hrow;
      const int u = max(sidx[tt * TK + r], 0);
      dma16(kb + (int64_t)u * p.sk.s + 8 * (hl ^ (r & 15)), kl + (8 * w + 2 * i) * ROWB);
      dma16(vb + (int64_t)u * p.sv.s + 8 * (hl ^ (2 * (r & 7))), vl + (8 * w + 2 * i) * ROWB);
    }
  };

  // Per-lane LDS read offsets within a stage.
  //   K (A operand, key half kt, step ks): key 16kt + col, chunk 4ks + grp in slot
  //     (4ks + grp) ^ col: k_off[ks % 4] + 256 (ks / 4) + 16 kt ROWB.
  //   V^T (A operand of dim tile dt, read e): row 16e + 4grp + col/4, dims
  //     16dt + 4(col % 4), chunk 2dt + (col % 4)/2 in slot chunk ^ 2(row mod 8):
  //     v_off[dt % 8] + 256 (dt / 8) + 16 e ROWB.
  uint32_t k_off[4], v_off[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) k_off[i] = col * ROWB + 16 * ((4 * i + grp) ^ col);
  {
    const int row = 4 * grp + (col >> 2);
    const int s = row & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      v_off[i] = KSTB + row * ROWB + 32 * (i ^ s) + 16 * ((col & 3) >> 1) + 8 * (col & 1);
  }

  f32x4 o[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_used = -INFINITY, l_run = 0.f;
  const float c = p.c;

  auto compute = [&](int tt, const unsigned char* sb) __attribute__((always_inline)) {
    // S^T = K Q^T for the two 16-key halves
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 ka = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(sb + k_off[ks & 3] + 256 * (ks >> 2) + 16 * kt * ROWB));
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[ks], s[kt], 0, 0, 0);
      }
    // keys of this lane: 16kt + 4grp + r; masked when the entry is -1
    const int4 u0 = *reinterpret_cast<const int4*>(sidx + tt * TK + 4 * grp);
    const int4 u1 = *reinterpret_cast<const int4*>(sidx + tt * TK + 16 + 4 * grp);
    float sv[8];
    sv[0] = u0.x >= 0 ? s[0][0] * c : -INFINITY;
    sv[1] = u0.y >= 0 ? s[0][1] * c : -INFINITY;
    sv[2] = u0.z >= 0 ? s[0][2] * c : -INFINITY;
    sv[3] = u0.w >= 0 ? s[0][3] * c : -INFINITY;
    sv[4] = u1.x >= 0 ? s[1][0] * c : -INFINITY;
    sv[5] = u1.y >= 0 ? s[1][1] * c : -INFINITY;
    sv[6] = u1.z >= 0 ? s[1][2] * c : -INFINITY;
    sv[7] = u1.w >= 0 ? s[1][3] * c : -INFINITY;
    float mt = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool need = mt > m_used + 8.f;
    if (__any(need)) {
      const float new_m = need ? mt : m_used;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_used - new_m) : 1.f;
      m_used = new_m;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) o[dt] *= alpha;
    }
    // masked logits are -inf: exp2 gives 0 (also while m_used is still -inf)
    const float msafe = m_used == -INFINITY ? 0.f : m_used;
    float ps[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) ps[r] = __builtin_amdgcn_exp2f(sv[r] - msafe);
    l_run += ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
    u32x4 pk;
#pragma unroll
    for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(ps[2 * e], ps[2 * e + 1]);
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pk);
    // O^T += V^T P^T : 16 dim tiles, k = the 32 keys of the tile
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      const unsigned char* vp = sb + v_off[dt & 7] + 256 * (dt >> 3);
      const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp));
      const s16x4 hi4 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp + 16 * ROWB));
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf, o[dt], 0, 0, 0);
    }
  };

  // Ring: tiles 0 .. NRING-2 are issued up front; the trip for tile tt waits
  // for its rows (later tiles stay in flight), a barrier makes every wave's
  // rows visible and frees the stage tile tt-1 used, tile tt+NRING-1 is issued
  // into it, then tile tt is computed.
  for (int i = 0; i < NRING - 1; ++i)
    if (i < ntiles) issue(i, i);
  int st = 0;
  for (int tt = 0; tt < ntiles; ++tt) {
    const int after = min(NRING - 2, ntiles - 1 - tt);  // tiles issued after tt
    if (after >= 2) asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
    else if (after == 1) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (tt + NRING - 1 < ntiles) issue(tt + NRING - 1, st == 0 ? NRING - 1 : st - 1);
    compute(tt, ring + st * STAGEB);
    st = st == NRING - 1 ? 0 : st + 1;
  }

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
                                     int seqlen, int n_kv, int h_q, int h_kv, int topk, float scale, hipStream_t st) {
  SparseParams p;
  p.q = (const uint16_t*)q; p.sq = sq;
  p.k = (const uint16_t*)k; p.sk = sk;
  p.v = (const uint16_t*)v; p.sv = sv;
  p.idx = idx;
  p.o = (uint16_t*)o; p.so = so;
  p.lse = lse;
  p.seqlen = seqlen; p.n_kv = n_kv; p.h_q = h_q; p.h_kv = h_kv; p.topk = topk;
  const int group = h_q / h_kv;
  if (group % HPB != 0 || topk > MAX_TOPK) return hipErrorInvalidValue;
  p.n_hb = group / HPB;
  p.c = scale * kLog2e;
  dim3 grid(seqlen, h_kv * p.n_hb, batch);
  hipLaunchKernelGGL(sparse_attn256_kernel, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace hca
