// HCA decode attention for bf16, head_dim 512: one new query per sequence
// over its compressed cache plus the raw window (ERNIE 5.5 Flash Base pages:
// mirrorspeed page, "Hybrid sparse attention" section -- the KV cache is the
// main inference cost and HCA keeps one entry per 128 tokens plus a short
// recent window; the 1M-token inference context is in the page's opening
// summary).
//
// The step is HBM-bound (each cache byte is used once per query head group),
// so the design streams the cache at full bandwidth:
//   * The key list of a sequence (compressed entries, then raw window) is cut
//     into `nsplit` contiguous chunks; one workgroup (4 waves) per
//     (sequence, KV head, group of 16 query heads, chunk).  Partial results
//     (unnormalised O, running max, sum) go to the workspace and a second
//     kernel merges them.
//   * Tiles of 16 keys of K and V are loaded into registers two tiles ahead
//     (coalesced 16-byte loads, one 1-KB row per wave instruction) and stored
//     to one of two LDS stages; one barrier per tile.
//   * All query heads that share the KV head are packed as the 16 columns of
//     one MFMA: S^T = K Q^T (16 keys x 16 heads, v_mfma_f32_16x16x32_bf16).
//     Every wave computes the same S^T (cheap next to the HBM time) and then
//     its own 128-dim slice of O^T = V^T P^T (v_mfma_f32_16x16x16_bf16).
#include "device_common.h"
#include "launchers.h"

namespace hca {
namespace {

constexpr int D = 512;
constexpr int TK = 16;      // keys per tile
constexpr int NST = 2;      // LDS stages
constexpr int HG = 16;      // query heads per workgroup
constexpr int TILE_ELEMS = TK * D;

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

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void decode512_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[NST * TILE_ELEMS];  // [stage][key][dim], chunk swizzle
  __shared__ __attribute__((aligned(16))) uint16_t Vs[NST * TILE_ELEMS];  // [stage][key][dim], natural

  const AttnArgs& a = p.a;
  const int split = blockIdx.x;
  const int hg = blockIdx.y % p.n_hg;
  const int kvh = blockIdx.y / p.n_hg;
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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
  const bool hvalid = hl < p.group;
  const int hq = kvh * p.group + min(hl, p.group - 1);

  bf16x8 qf[16];
  {
    const uint16_t* qp = (const uint16_t*)a.q + b * a.sq.b + (int64_t)hq * a.sq.h + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, ld16(qp + 32 * ks));
    // Consume Q here so the compiler settles these loads before the DMA ring
    // (otherwise it re-waits for them, and with them every DMA, inside the loop).
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

  const uint16_t* kcb = (const uint16_t*)a.kc + b * a.skc.b + (int64_t)kvh * a.skc.h;
  const uint16_t* vcb = (const uint16_t*)a.vc + b * a.svc.b + (int64_t)kvh * a.svc.h;
  const int raw0 = lo - (int)a.kv_pos0;  // raw row of window position lo
  const uint16_t* kb = (const uint16_t*)a.k + b * a.sk.b + (int64_t)kvh * a.sk.h;
  const uint16_t* vb = (const uint16_t*)a.v + b * a.sv.b + (int64_t)kvh * a.sv.h;

  // Tile loads: 16 K rows + 16 V rows of 1 KB; in round r thread tid loads row
  // 4r + w (rows 0-15 are K, 16-31 are V), 16-byte chunk `lane`.  Rows past the
  // chunk re-read a valid row; their logits are masked.
  auto load_tile = [&](int tt, u32x4 (&R)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = 4 * r + w;
      const int key = row & (TK - 1);
      const bool is_v = row >= TK;
      const int x = min(x0 + tt * TK + key, x1 - 1);
      const uint16_t* src;
      if (x < n_c) src = (is_v ? vcb : kcb) + (int64_t)x * (is_v ? a.svc.s : a.skc.s);
      else src = (is_v ? vb : kb) + (int64_t)(raw0 + x - n_c) * (is_v ? a.sv.s : a.sk.s);
      R[r] = ld16(src + 8 * lane);
    }
  };
  auto store_tile = [&](const u32x4 (&R)[8], int st) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = 4 * r + w;
      const int key = row & (TK - 1);
      if (row < TK)
        *reinterpret_cast<u32x4*>(Ks + st * TILE_ELEMS + key * D + ((lane ^ (key & 7)) << 3)) = R[r];
      else
        *reinterpret_cast<u32x4*>(Vs + st * TILE_ELEMS + key * D + (lane << 3)) = R[r];
    }
  };

  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_used = -INFINITY, l_run = 0.f;
  const float c = p.c;

  auto compute = [&](int tt, int st) __attribute__((always_inline)) {
    const uint16_t* kst = Ks + st * TILE_ELEMS;
    const uint16_t* vst = Vs + st * TILE_ELEMS;
    // S^T = K Q^T (16 keys x 16 heads)
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const bf16x8 ka = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(kst + col * D + (((4 * ks + grp) ^ (col & 7)) << 3)));
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[ks], s, 0, 0, 0);
    }
    float sv[4];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int x = x0 + tt * TK + 4 * grp + r;
      sv[r] = x < x1 ? s[r] * c : -INFINITY;
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
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
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
    // O^T[this wave's 128 dims] += V^T P^T (k = 16 keys)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int dim = 128 * w + 16 * dt + col;
      u32x2 vv;
      vv[0] = vst[(4 * grp + 0) * D + dim] | ((uint32_t)vst[(4 * grp + 1) * D + dim] << 16);
      vv[1] = vst[(4 * grp + 2) * D + dim] | ((uint32_t)vst[(4 * grp + 3) * D + dim] << 16);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, vv), pf, o[dt], 0, 0, 0);
    }
  };

  // Two tiles in flight in registers (R0/R1), two LDS stages; one barrier per tile.
  // Loads are unconditional (tiles past the end re-read the last one) so that
  // the compiler's load counting stays exact and only waits for the oldest tile.
  u32x4 R0[8], R1[8];
  const int last = max(ntiles - 1, 0);
  if (ntiles > 0) {
    load_tile(0, R0);
    load_tile(min(1, last), R1);
  }
  for (int tt = 0; tt < ntiles; tt += 2) {
    store_tile(R0, 0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    load_tile(min(tt + 2, last), R0);
    compute(tt, 0);
    store_tile(R1, 1);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    load_tile(min(tt + 3, last), R1);
    if (tt + 1 < ntiles) compute(tt + 1, 1);
  }

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
  (void)hvalid;
}

// Merge the split partials of one (sequence, query head).
__global__ __launch_bounds__(256) void decode512_combine(DecodeParams p) {
  const AttnArgs& a = p.a;
  const int hq = blockIdx.x, b = blockIdx.y;
  const int kvh = hq / p.group, hl = hq % p.group;
  const int hg = hl / HG, col = hl % HG;
  const int64_t part0 = (((int64_t)b * a.h_kv + kvh) * p.n_hg + hg) * p.nsplit;
  float M = -INFINITY;
  for (int s = 0; s < p.nsplit; ++s) M = fmaxf(M, p.ws_ml[((part0 + s) * HG + col) * 2]);
  float Lsum = 0.f;
  for (int s = 0; s < p.nsplit; ++s) {
    const float* ml = p.ws_ml + ((part0 + s) * HG + col) * 2;
    Lsum += ml[1] * (ml[0] == -INFINITY ? 0.f : exp2f(ml[0] - M));
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  uint16_t* op = (uint16_t*)a.o + b * a.so.b + (int64_t)hq * a.so.h;
  for (int e = threadIdx.x * 2; e < D; e += 512) {
    float o0 = 0.f, o1 = 0.f;
    for (int s = 0; s < p.nsplit; ++s) {
      const float m = p.ws_ml[((part0 + s) * HG + col) * 2];
      const float wgt = m == -INFINITY ? 0.f : exp2f(m - M);
      const float* src = p.ws_o + ((part0 + s) * HG + col) * D + e;
      o0 = fmaf(wgt, src[0], o0);
      o1 = fmaf(wgt, src[1], o1);
    }
    *reinterpret_cast<uint32_t*>(op + e) = pack_bf16x2(o0 * inv, o1 * inv);
  }
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
  // aim for >= 1024 workgroups, but keep >= 64 keys per chunk
  long ns = (1024 + units - 1) / units;
  const long max_ns = (n_keys + 63) / 64;
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
