// HCA decode attention for bf16, head_dim 512: one new query per sequence
// over its compressed cache plus the raw window (ERNIE 5.5 Flash Base pages:
// mirrorspeed page, "Hybrid sparse attention" section -- the KV cache is the
// main inference cost and HCA keeps one entry per 128 tokens plus a short
// recent window; the 1M-token inference context is in the page's opening
// summary).
//
// The step is HBM-bound (each cache byte is used once per query-head group),
// so the design keeps as many cache bytes in flight as LDS holds:
//   * The key list of a sequence (compressed entries, then raw window) is cut
//     into `nsplit` contiguous chunks so that the grid is about one workgroup
//     (4 waves) per CU, all with the same amount of work.  Partial results
//     (unnormalised O, running max, sum) go to the workspace and a second
//     kernel merges them.
//   * Tiles of 16 keys of K and V move global -> LDS with 16-byte LDS DMA
//     (global_load_lds) through a ring of 5 stages, four tiles (128 KB) in
//     flight while one is consumed.  Every stage is an LDS object of its own
//     and the loop is unrolled over the ring, so the compiler can tell the
//     DMA in flight from the stage being read and never drains the ring; the
//     explicit vmcnt wait before each barrier orders them.
//   * K and V are stored chunk-major ([16-byte chunk][key]) so that each DMA
//     instruction fills one contiguous KB; K operand reads then cover one
//     256-byte span per 16 lanes.  V is read transposed, 16 bits at a time;
//     odd chunks flip key bit 1 so that those reads hit distinct banks.
//   * All query heads that share the KV head are packed as the 16 columns of
//     one MFMA: S^T = K Q^T (16 keys x 16 heads, v_mfma_f32_16x16x32_bf16).
//     Every wave computes the same S^T (cheap next to the HBM time) and then
//     its own 128-dim slice of O^T = V^T P^T (v_mfma_f32_16x16x16_bf16).
#include "device_common.h"
#include "launchers.h"

namespace hca {
namespace {

constexpr int D = 512;
constexpr int TK = 16;          // keys per tile
constexpr int HG = 16;          // query heads per workgroup
constexpr int STAGE = TK * D;   // elements of one K (or V) stage
constexpr int NRING = 5;        // ring stages; NRING - 1 tiles in flight
constexpr int CPW = 4;          // 1-KB DMA segments per wave and operand (16 KB per tile / 4 waves)

typedef unsigned short us4 __attribute__((ext_vector_type(4)));

// 16-byte LDS DMA of one wave: lane l copies 16 bytes from g (per lane) to LDS
// byte address lds + 16 l (lds travels in M0).  Written as asm so that the
// compiler does not track it as an LDS store: it cannot tell the ring stages
// apart and would wait for every DMA in flight before some LDS reads.  The
// ring's explicit vmcnt waits and barriers order DMA and reads instead.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

struct DecodeParams {
  AttnArgs a;
  int group;        // h_q / h_kv
  int n_hg;         // head groups per KV head
  int nsplit;
  int keys_per_split;
  float c;          // scale * log2(e)
  float* ws_o;      // [batch, h_kv, n_hg, nsplit, HG, D]
  float* ws_ml;     // [batch, h_kv, n_hg, nsplit, HG, 2]
};

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void decode512_kernel(DecodeParams p) {
  // stage i: K tile at S_i[0, STAGE), V tile at S_i[STAGE, 2 STAGE)
  __shared__ __attribute__((aligned(16))) uint16_t S0[2 * STAGE], S1[2 * STAGE], S2[2 * STAGE], S3[2 * STAGE],
      S4[2 * STAGE];

  const AttnArgs& a = p.a;
  const int split = blockIdx.x;
  const int hg = blockIdx.y % p.n_hg;
  const int kvh = blockIdx.y / p.n_hg;
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;

  const int t = (int)a.q_pos0;
  const int lo = max(0, t - a.window + 1);
  const int n_c = lo / a.block;
  const int n_keys = n_c + (t - lo + 1);
  const int x0 = split * p.keys_per_split;
  const int x1 = min(n_keys, x0 + p.keys_per_split);
  const int ntiles = x1 > x0 ? (x1 - x0 + TK - 1) / TK : 0;

  // query head of this lane's column (heads past the group are padding)
  const int hl = hg * HG + col;
  const int hq = kvh * p.group + min(hl, p.group - 1);

  bf16x8 qf[16];
  {
    const uint16_t* qp = (const uint16_t*)a.q + b * a.sq.b + (int64_t)hq * a.sq.h + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, ld16(qp + 32 * ks));
    // consume Q here so that these loads are settled before the DMA ring starts
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

  const uint16_t* kcb = (const uint16_t*)a.kc + b * a.skc.b + (int64_t)kvh * a.skc.h;
  const uint16_t* vcb = (const uint16_t*)a.vc + b * a.svc.b + (int64_t)kvh * a.svc.h;
  const int raw0 = lo - (int)a.kv_pos0;  // raw row of window position lo
  const uint16_t* kb = (const uint16_t*)a.k + b * a.sk.b + (int64_t)kvh * a.sk.h;
  const uint16_t* vb = (const uint16_t*)a.v + b * a.sv.b + (int64_t)kvh * a.sv.h;

  // DMA lane map: within 1-KB segment s (chunks 4s .. 4s+3), lane l fills the
  // 16-byte slot l: chunk 4s + (l >> 4), key (l & 15) for K and, for V, key
  // (l & 15) ^ 2 in odd chunks.  Keys past the chunk re-read its last key (their
  // logits are masked).
  const int kkey = lane & 15;
  const int vkey = (lane & 15) ^ (lane & 16 ? 2 : 0);
  const int lchunk = lane >> 4;
  auto row_of = [&](int x, const uint16_t* cp, int64_t cs, const uint16_t* rp, int64_t rs) {
    x = min(x, x1 - 1);
    return x < n_c ? cp + (int64_t)x * cs : rp + (int64_t)(raw0 + x - n_c) * rs;
  };
  auto issue = [&](int tt, uint16_t* kdst) __attribute__((always_inline)) {
    const uint16_t* krow = row_of(x0 + tt * TK + kkey, kcb, a.skc.s, kb, a.sk.s) + 8 * lchunk;
    const uint16_t* vrow = row_of(x0 + tt * TK + vkey, vcb, a.svc.s, vb, a.sv.s) + 8 * lchunk;
    const uint32_t kl = lds_addr(kdst), vl = kl + 2 * STAGE;
#pragma unroll
    for (int i = 0; i < CPW; ++i) dma16(krow + 32 * (CPW * w + i), kl + 1024 * (CPW * w + i));
#pragma unroll
    for (int i = 0; i < CPW; ++i) dma16(vrow + 32 * (CPW * w + i), vl + 1024 * (CPW * w + i));
  };

  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_used = -INFINITY, l_run = 0.f;
  const float c = p.c;
  // K operand: lane (key col, k-group grp) of step ks reads chunk 4ks + grp
  const int k_off = grp * (TK * 8) + col * 8;
  // V^T operand: lane (dim col, key group grp) of dim tile dt reads dim
  // 128w + 16dt + col (chunk 16w + 2dt + (col >> 3)) of keys 4grp + r
  const int hbit = col >> 3;
  const int v_base = (16 * w + hbit) * (TK * 8) + (col & 7);
  int v_off[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) v_off[r] = v_base + ((4 * grp + r) ^ (2 * hbit)) * 8;

  auto compute = [&](int tt, const uint16_t* kst)
                     __attribute__((always_inline)) {
    const uint16_t* vst = kst + STAGE;
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int ks = 0; ks < 16; ks += 2) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kst + k_off + 512 * ks)), qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kst + k_off + 512 * (ks + 1))), qf[ks + 1],
          s1, 0, 0, 0);
    }
    float sv[4];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int x = x0 + tt * TK + 4 * grp + r;
      sv[r] = x < x1 ? (s0[r] + s1[r]) * c : -INFINITY;
      mt = fmaxf(mt, sv[r]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool need = mt > m_used + 8.f;
    if (__any(need)) {
      const float new_m = need ? mt : m_used;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_used - new_m) : 1.f;
      m_used = new_m;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    }
    const float msafe = m_used == -INFINITY ? 0.f : m_used;
    float ps[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ps[r] = __builtin_amdgcn_exp2f(sv[r] - msafe);
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    u32x2 pk;
    pk[0] = pack_bf16x2(ps[0], ps[1]);
    pk[1] = pack_bf16x2(ps[2], ps[3]);
    const bf16x4 pf = __builtin_bit_cast(bf16x4, pk);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint16_t* vp = vst + 2 * dt * (TK * 8);
      const us4 vv = us4{vp[v_off[0]], vp[v_off[1]], vp[v_off[2]], vp[v_off[3]]};
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, vv), pf, o[dt], 0, 0, 0);
    }
  };

  // One ring trip per tile: wait for this wave's DMA of the tile (the later
  // tiles stay in flight), a bare barrier (a release fence would drain the
  // ring) after which every wave's part has landed and every wave is done with
  // the previous stage, refill that stage, compute.  DMA is issued even past
  // the end (re-reading the last tile) so that exactly NRING - 1 tiles are in
  // flight at every wait.
  const int last = max(ntiles - 1, 0);
  // The whole ring runs inside one function whose stage pointers are restrict
  // parameters: every access then carries alias scopes of one domain, which
  // lets the compiler prove that a stage read does not alias the DMA into the
  // other stages, so it never waits for those.
  [&](uint16_t* __restrict__ s0, uint16_t* __restrict__ s1, uint16_t* __restrict__ s2, uint16_t* __restrict__ s3,
      uint16_t* __restrict__ s4) __attribute__((always_inline)) {
    if (ntiles <= 0) return;
    // One trip per tile: wait for this wave's DMA of the tile (the later tiles
    // stay in flight), a bare barrier (a release fence would drain the ring)
    // after which every wave's part has landed and every wave is done with the
    // previous stage, refill that stage, compute.  DMA is issued even past the
    // end (re-reading the last tile) so that exactly NRING - 1 tiles are in
    // flight at every wait.
    const int last = ntiles - 1;
    auto trip = [&](int tt, const uint16_t* cur, uint16_t* next) __attribute__((always_inline)) {
      asm volatile("s_waitcnt vmcnt(24)\n\ts_barrier" ::: "memory");
      issue(min(tt + NRING - 1, last), next);
      if (tt < ntiles) compute(tt, cur);
    };
    issue(0, s0);
    issue(min(1, last), s1);
    issue(min(2, last), s2);
    issue(min(3, last), s3);
    for (int tt = 0; tt < ntiles; tt += NRING) {
      trip(tt, s0, s4);
      trip(tt + 1, s1, s0);
      trip(tt + 2, s2, s1);
      trip(tt + 3, s3, s2);
      trip(tt + 4, s4, s3);
    }
    // no DMA may still target this workgroup's LDS when it exits
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }(S0, S1, S2, S3, S4);

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const int64_t part = (((int64_t)b * a.h_kv + kvh) * p.n_hg + hg) * p.nsplit + split;
  float* wo = p.ws_o + (part * HG + col) * D + 128 * w + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(wo + 16 * dt) = o[dt];
  if (w == 0 && grp == 0) {
    float* wml = p.ws_ml + (part * HG + col) * 2;
    wml[0] = m_used;
    wml[1] = l_tot;
  }
}

// Merge the split partials of one (sequence, query head).
__global__ __launch_bounds__(256) void decode512_combine(DecodeParams p) {
  const AttnArgs& a = p.a;
  const int hq = blockIdx.x, b = blockIdx.y;
  const int kvh = hq / p.group, hl = hq % p.group;
  const int hg = hl / HG, col = hl % HG;
  const int64_t part0 = (((int64_t)b * a.h_kv + kvh) * p.n_hg + hg) * p.nsplit;
  const float* ml = p.ws_ml + (part0 * HG + col) * 2;  // split s at ml[2 * HG * s]
  const float* po = p.ws_o + part0 * HG * D + (int64_t)col * D + 2 * threadIdx.x;  // split s at po[HG * D * s]
  float M = -INFINITY;
  for (int s = 0; s < p.nsplit; ++s) M = fmaxf(M, ml[2 * HG * s]);
  // splits four at a time: their loads are issued together
  float Lsum = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s0 = 0; s0 < p.nsplit; s0 += 4) {
    float m[4], l[4], x[4], y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = s0 + j < p.nsplit ? s0 + j : s0;
      m[j] = ml[2 * HG * s];
      l[j] = ml[2 * HG * s + 1];
      const float2 v = *reinterpret_cast<const float2*>(po + (int64_t)HG * D * s);
      x[j] = v.x;
      y[j] = v.y;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float wgt = (s0 + j < p.nsplit && m[j] != -INFINITY) ? exp2f(m[j] - M) : 0.f;
      Lsum = fmaf(l[j], wgt, Lsum);
      o0 = fmaf(wgt, x[j], o0);
      o1 = fmaf(wgt, y[j], o1);
    }
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  uint16_t* op = (uint16_t*)a.o + b * a.so.b + (int64_t)hq * a.so.h;
  *reinterpret_cast<uint32_t*>(op + 2 * threadIdx.x) = pack_bf16x2(o0 * inv, o1 * inv);
  if (a.lse && threadIdx.x == 0) a.lse[(int64_t)b * a.h_q + hq] = M * kLn2 + __logf(Lsum);
}

struct SplitPlan {
  int n_hg, nsplit, keys_per_split;
};

SplitPlan plan(int batch, int h_q, int h_kv, int n_keys) {
  SplitPlan s;
  const int group = h_q / h_kv;
  s.n_hg = (group + HG - 1) / HG;
  const long units = (long)batch * h_kv * s.n_hg;
  // about one workgroup per CU (256 on MI355X), at least 4 tiles per chunk
  long ns = (256 + units - 1) / units;
  const long max_ns = (n_keys + 4 * TK - 1) / (4 * TK);
  if (ns > max_ns) ns = max_ns;
  if (ns < 1) ns = 1;
  s.keys_per_split = (int)(((n_keys + ns - 1) / ns + TK - 1) / TK * TK);
  s.nsplit = (n_keys + s.keys_per_split - 1) / s.keys_per_split;
  return s;
}

}  // namespace

size_t decode512_workspace_bytes(int batch, int h_q, int h_kv, int n_keys) {
  const SplitPlan s = plan(batch, h_q, h_kv, n_keys);
  const size_t parts = (size_t)batch * h_kv * s.n_hg * s.nsplit * HG;
  return parts * (D + 2) * sizeof(float);
}

hipError_t launch_attn_decode512(const AttnArgs& a, void* ws, hipStream_t st) {
  const int t = (int)a.q_pos0;
  const int lo = t - a.window + 1 > 0 ? t - a.window + 1 : 0;
  const int n_keys = lo / a.block + (t - lo + 1);
  const SplitPlan s = plan(a.batch, a.h_q, a.h_kv, n_keys);
  DecodeParams p;
  p.a = a;
  p.group = a.h_q / a.h_kv;
  p.n_hg = s.n_hg;
  p.nsplit = s.nsplit;
  p.keys_per_split = s.keys_per_split;
  p.c = a.scale * kLog2e;
  const size_t parts = (size_t)a.batch * a.h_kv * s.n_hg * s.nsplit * HG;
  p.ws_o = (float*)ws;
  p.ws_ml = p.ws_o + parts * D;
  hipLaunchKernelGGL(decode512_kernel, dim3(s.nsplit, a.h_kv * s.n_hg, a.batch), dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode512_combine, dim3(a.h_q, a.batch), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace hca
