// Attention-output epilogues (ERNIE 5.5 Flash Base pages: mirrorspeed page,
// section "More structural improvements, data, and infrastructure"; besthub
// page, section "Core Architectural Innovations"): the output gate computed
// from the layer's low-rank query latent, and Virtual Head Attention's
// low-rank cross-head mixing with an identity skip.
//   y[b,t,h,e] = sigmoid(<c[b,t,:], W_g[h*d_v + e, :]>) * (o[b,t,h,e] + sum_h' (U V)[h,h'] o[b,t,h',e])
//
// Two steps:
//   * the gate projection G = C W_g^T, a plain GEMM, written as the bf16
//     pre-activation into y: by hipBLASLt when each token's heads are
//     contiguous in y (it runs this shape at ~1.3 PFLOP/s), else by
//     gate_proj_kernel, a bf16 MFMA GEMM (v_mfma_f32_32x32x16_bf16, fp32
//     accumulation; ~0.8 PFLOP/s).  Workgroup tile 256 tokens x 256
//     outputs, 8 waves of 64 x 128 (two per SIMD), K streamed in chunks of 32 through a
//     3-stage LDS ring (two chunks in flight) by 16-byte LDS DMA.  The
//     product is formed transposed (W rows as the A operand) so a lane ends
//     with 4 consecutive outputs of one token: 8-byte stores.  W_g is [out, in], so both
//     operands are read K-contiguous.  LDS rows are 64 bytes with the four
//     16-byte chunks of row r stored XOR-swizzled by (r / 4) % 4, which keeps
//     the 16-byte operand reads of 16 consecutive rows on distinct bank groups
//     while each DMA instruction still fills one contiguous kilobyte.
//   * vha_gate_kernel: one workgroup per token, one dim pair per thread; each
//     thread holds the pair for every head, forms p = V o (rank r, padded to
//     4, 8 or 16), then y = sigmoid(y) * (o + U p) in place.  HBM-bound: o
//     and y read once, y written once.
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "device_common.h"
#include "launchers.h"
#include "mfma_asm.h"

namespace hca {
namespace {

constexpr int GM = 256, GN = 256, GK = 32;  // workgroup tile and K chunk
constexpr int G_WAVES = 8;                  // 4 (tokens) x 2 (outputs) waves of 64 x 128
constexpr int A_ST = GM * 64, B_ST = GN * 64, G_STAGE = A_ST + B_ST;
constexpr int G_NST = 3;  // DMA ring stages; chunk kc + 2 is issued while chunk kc is consumed

struct GateParams {
  const uint16_t* c;  // [M = B*S tokens, d_c], token m at c + m*scs
  int64_t scs;
  const uint16_t* w;  // [N, d_c] contiguous, N = h * d_v
  uint16_t* y;        // gate output, token m, head h, dim e at y + m*sys + h*syh + e
  int64_t sys, syh;
  int M, d_c, d_v;
  int m_tiles;
};

// LDS offset of 16-byte chunk `ch` (0..3) of row r in a swizzled 64-byte-row tile.
__device__ __forceinline__ uint32_t swz(int r, int ch) { return (uint32_t)(r * 64 + 16 * (ch ^ ((r >> 2) & 3))); }

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gate_proj_kernel(GateParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[G_NST * G_STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;  // wm 0..3
  const int col = lane & 31, hf = lane >> 5;
  const int mt = blockIdx.x % p.m_tiles, nt = blockIdx.x / p.m_tiles;
  const int M = p.M;
  const int m0 = mt * GM, n0 = nt * GN;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)smem;

  // DMA of K chunk kc into stage st: 16 instructions of A rows and 16 of B
  // rows (16 rows of 64 bytes each); wave w issues instructions w, w+8, ...
  auto row_ptr_a = [&](int r) __attribute__((always_inline)) { return p.c + (int64_t)min(m0 + r, M - 1) * p.scs; };
  auto issue = [&](int kc, int st) __attribute__((always_inline)) {
    const int k0 = kc * GK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ins = w + G_WAVES * i;  // 0..31: A rows for ins < 16, then B rows
      const bool is_a = ins < 16;
      const int r = 16 * (ins & 15) + (lane >> 2);
      const int s = lane & 3;
      const int ch = s ^ ((r >> 2) & 3);  // the global chunk this LDS slot holds
      const uint16_t* src = is_a ? row_ptr_a(r) + k0 + 8 * ch : p.w + (int64_t)(n0 + r) * p.d_c + k0 + 8 * ch;
      dma16(src, lds0 + st * G_STAGE + (is_a ? 0 : A_ST) + 1024 * (ins & 15));
    }
  };

  // acc[j][i] = G^T tile: W rows 128 wn + 32 j .. (A operand) x C rows
  // 64 wm + 32 i .. (B operand); a lane then holds 4 consecutive outputs of
  // one token per accumulator group.
  f32x16 acc[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

  const int nk = p.d_c / GK;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  for (int kc = 0; kc < nk; ++kc) {
    // chunk kc landed: at most the newer chunk's 4 DMAs per wave are still in flight
    if (kc + 1 < nk) asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (kc + 2 < nk) issue(kc + 2, (kc + 2) % G_NST);
    const unsigned char* sa = smem + (kc % G_NST) * G_STAGE;
    const unsigned char* sb = sa + A_ST;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = 2 * ks + hf;
      bf16x8 af[2], bfr[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 64 * wm + 32 * i + col;
        af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sa + swz(r, ch)));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 128 * wn + 32 * j + col;
        bfr[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sb + swz(r, ch)));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[j][i], 0, 0, 0);
    }
  }

  // epilogue: the pre-activation in bf16 (the mixing kernel applies the
  // sigmoid); the lane's token is m, its outputs n .. n+3
  // (one head, since d_v is a multiple of 8) go out as one 8-byte store
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + 64 * wm + 32 * i + col;
    if (m >= M) continue;
    uint16_t* yr = p.y + (int64_t)m * p.sys;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + 128 * wn + 32 * j + 8 * q + 4 * hf;
        u32x2 pk;
        pk[0] = pack_bf16x2(acc[j][i][4 * q], acc[j][i][4 * q + 1]);
        pk[1] = pack_bf16x2(acc[j][i][4 * q + 2], acc[j][i][4 * q + 3]);
        *reinterpret_cast<u32x2*>(yr + (int64_t)(n / p.d_v) * p.syh + n % p.d_v) = pk;
      }
  }
}

struct VhaParams {
  const uint16_t* o;
  LStrides so;
  uint16_t* y;  // holds the gate on entry, the output on exit
  LStrides sy;
  const float* u;  // [H, r]
  const float* v;  // [r, H]
  int batch, seqlen, d_v, r;
};

// R: the rank rounded up to 4, 8 or 16 (U, V zero-padded in LDS).
template <int H, int R>
__global__ __launch_bounds__(256) void vha_gate_kernel(VhaParams p) {
  __shared__ float su[H * R], sv[R * H];
  const int tok = blockIdx.x;
  const int b = tok / p.seqlen, t = tok % p.seqlen;
  for (int i = threadIdx.x; i < H * R; i += 256) {
    const int h = i / R, j = i % R;  // su[h][j], sv[j][h]
    su[i] = j < p.r ? p.u[h * p.r + j] : 0.f;
    sv[j * H + h] = j < p.r ? p.v[j * H + h] : 0.f;
  }
  __syncthreads();
  const uint16_t* ob = p.o + b * p.so.b + (int64_t)t * p.so.s;
  uint16_t* yb = p.y + b * p.sy.b + (int64_t)t * p.sy.s;
  const int e = 2 * threadIdx.x;  // d_v <= 512: one dim pair per thread
  if (e < p.d_v) {
    float o0[H], o1[H];
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const uint32_t x = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(ob + (int64_t)h * p.so.h + e));
      o0[h] = __uint_as_float(x << 16);
      o1[h] = __uint_as_float(x & 0xffff0000u);
    }
    float p0[R], p1[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int h = 0; h < H; ++h) {
        a0 = fmaf(sv[j * H + h], o0[h], a0);
        a1 = fmaf(sv[j * H + h], o1[h], a1);
      }
      p0[j] = a0;
      p1[j] = a1;
    }
#pragma unroll
    for (int h = 0; h < H; ++h) {
      float z0 = o0[h], z1 = o1[h];
#pragma unroll
      for (int j = 0; j < R; ++j) {
        z0 = fmaf(su[h * R + j], p0[j], z0);
        z1 = fmaf(su[h * R + j], p1[j], z1);
      }
      uint32_t* yp = reinterpret_cast<uint32_t*>(yb + (int64_t)h * p.sy.h + e);
      const uint32_t gx = __builtin_nontemporal_load(yp);  // gate pre-activation
      const float g0 = 1.f / (1.f + __expf(-__uint_as_float(gx << 16)));
      const float g1 = 1.f / (1.f + __expf(-__uint_as_float(gx & 0xffff0000u)));
      __builtin_nontemporal_store(pack_bf16x2(g0 * z0, g1 * z1), yp);
    }
  }
}

template <int H>
hipError_t launch_vha(const VhaParams& vp, dim3 grid, hipStream_t st) {
  if (vp.r <= 4) hipLaunchKernelGGL((vha_gate_kernel<H, 4>), grid, dim3(256), 0, st, vp);
  else if (vp.r <= 8) hipLaunchKernelGGL((vha_gate_kernel<H, 8>), grid, dim3(256), 0, st, vp);
  else hipLaunchKernelGGL((vha_gate_kernel<H, 16>), grid, dim3(256), 0, st, vp);
  return hipGetLastError();
}

}  // namespace

// G^T (out x tokens, column-major: y's token rows) = W_g (d_c x out,
// column-major: W_g's [out, in] rows, transposed) ^T . C^T (d_c x tokens,
// column-major: c's token rows), fp32 accumulation, bf16 result, no
// workspace.  One hipBLASLt handle per device and one heuristic pick per
// shape, created on first use.  Returns false when hipBLASLt cannot run the
// product (the caller then uses gate_proj_kernel).
bool gate_gemm_blaslt(const void* c, int64_t ldc_tok, const void* w_g, void* y, int64_t ldy_tok, int tokens, int out,
                      int d_c, hipStream_t st) {
  static std::mutex mu;
  static std::map<int, hipblasLtHandle_t> handles;
  static std::map<std::tuple<int, int, int, int, int64_t, int64_t>, hipblasLtMatmulAlgo_t> algos;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lock(mu);
  hipblasLtHandle_t hdl;
  auto hit = handles.find(dev);
  if (hit == handles.end()) {
    if (hipblasLtCreate(&hdl) != HIPBLAS_STATUS_SUCCESS) return false;
    handles[dev] = hdl;
  } else {
    hdl = hit->second;
  }
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  bool ok = hipblasLtMatmulDescCreate(&op, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  ok = ok && hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, d_c, out, d_c) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, d_c, tokens, ldc_tok) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&ld, HIP_R_16BF, out, tokens, ldy_tok) == HIPBLAS_STATUS_SUCCESS;
  if (ok) {
    const auto key = std::make_tuple(dev, tokens, out, d_c, ldc_tok, ldy_tok);
    auto ait = algos.find(key);
    if (ait == algos.end()) {
      hipblasLtMatmulPreference_t pref = nullptr;
      uint64_t ws = 0;
      hipblasLtMatmulHeuristicResult_t res[1];
      int n = 0;
      ok = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
           hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws, sizeof(ws)) ==
               HIPBLAS_STATUS_SUCCESS &&
           hipblasLtMatmulAlgoGetHeuristic(hdl, op, la, lb, ld, ld, pref, 1, res, &n) == HIPBLAS_STATUS_SUCCESS &&
           n > 0 && res[0].workspaceSize == 0;
      if (pref) hipblasLtMatmulPreferenceDestroy(pref);
      if (ok) ait = algos.emplace(key, res[0].algo).first;
    }
    if (ok) {
      const float alpha = 1.f, beta = 0.f;
      ok = hipblasLtMatmul(hdl, op, &alpha, w_g, la, c, lb, &beta, y, ld, y, ld, &ait->second, nullptr, 0, st) ==
           HIPBLAS_STATUS_SUCCESS;
    }
  }
  if (ld) hipblasLtMatrixLayoutDestroy(ld);
  if (lb) hipblasLtMatrixLayoutDestroy(lb);
  if (la) hipblasLtMatrixLayoutDestroy(la);
  if (op) hipblasLtMatmulDescDestroy(op);
  return ok;
}

hipError_t launch_attn_output_epilogue(const void* o, LStrides so, const void* c, int64_t scs, const void* w_g,
                                       const float* u, const float* v, void* y, LStrides sy, int batch, int seqlen,
                                       int h, int d_v, int d_c, int r, hipStream_t st) {
  const bool lib = sy.h == d_v &&
                   gate_gemm_blaslt(c, scs, w_g, y, sy.s, batch * seqlen, h * d_v, d_c, st);
  if (!lib) {
    GateParams gp;
    gp.c = (const uint16_t*)c;
    gp.scs = scs;
    gp.w = (const uint16_t*)w_g;
    gp.y = (uint16_t*)y;
    gp.sys = sy.s;
    gp.syh = sy.h;
    gp.M = batch * seqlen;
    gp.d_c = d_c;
    gp.d_v = d_v;
    gp.m_tiles = (gp.M + GM - 1) / GM;
    const int n_tiles = h * d_v / GN;
    hipLaunchKernelGGL(gate_proj_kernel, dim3(gp.m_tiles * n_tiles), dim3(64 * G_WAVES), 0, st, gp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  VhaParams vp;
  vp.o = (const uint16_t*)o;
  vp.so = so;
  vp.y = (uint16_t*)y;
  vp.sy = sy;
  vp.u = u;
  vp.v = v;
  vp.batch = batch;
  vp.seqlen = seqlen;
  vp.d_v = d_v;
  vp.r = r;
  const dim3 grid(batch * seqlen);
  switch (h) {
    case 8: return launch_vha<8>(vp, grid, st);
    case 16: return launch_vha<16>(vp, grid, st);
    case 32: return launch_vha<32>(vp, grid, st);
    case 64: return launch_vha<64>(vp, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hca
