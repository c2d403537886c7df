// DSA lightweight indexer and causal top-k (ERNIE 5.5 Flash Base pages:
// mirrorspeed page, "Hybrid sparse attention" section -- an indexer scores the
// historical positions of each query and core attention runs only on the
// top-k; ai-club.cn page, hybrid attention section, says the same).
//
//   s(t, u) = sum_h w[t,h] * max(0, <qI[t,h,:], kI[u,:]>),  u <= t, fp32
//
// Two kernels per chunk of query rows (the host walks the chunks so the score
// workspace stays bounded):
//   1. index_scores: fp32 matrix cores (v_mfma_f32_32x32x2_f32).  One wave
//      computes a 32-key x 32-query tile of S^T per index head and folds it
//      as w * relu(.) into the score tile; operands come straight from global
//      memory (every lane reads contiguous 16-byte runs), no LDS.
//   2. topk_select: one workgroup per query row.  Scores map to
//      order-preserving uint32 keys (-0 counts as +0); three LDS histogram
//      passes (11 + 11 + 10 bits) find the exact k-th largest key T; a final
//      ordered pass emits every key > T and the lowest-position keys == T.
#include "device_common.h"
#include "launchers.h"

namespace hca {
namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int DI_MAX = 128;
constexpr int QT = 32;   // queries per wave tile
constexpr int KT = 32;   // keys per wave tile
constexpr int WAVES = 4; // a workgroup covers 32 queries x 128 keys

struct ScoreParams {
  const float* qI;  // [S, h_i, d_i] of this batch
  const float* kI;  // [S, d_i]
  const float* w;   // [S, h_i]
  float* sc;        // [rows, ld] scores of rows r0 .. r0+rows-1
  int64_t ld;
  int seqlen, h_i, d_i, r0, rows;
};

// S^T tile = kI (32 keys x d) . qI_h^T (d x 32 queries).  The contraction index
// d = 32*(lane/32)... is mapped so that each lane reads a contiguous run: in
// k-step ks lane half hf holds d = hf * (d_i/2) + ks.
template <int DI>
__global__ __launch_bounds__(256) void index_scores_kernel(ScoreParams p) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int qt0 = blockIdx.y * QT;                  // first query (chunk-relative)
  const int t0 = p.r0 + qt0;                        // absolute position
  const int k0 = blockIdx.x * (KT * WAVES) + w * KT;
  const int t_last = min(t0 + QT, p.r0 + p.rows) - 1;
  if (k0 > t_last) return;                          // keys all in the future of every query
  const int col = lane & 31, hf = lane >> 5;
  constexpr int HALF = DI / 2;

  // A operand: this lane's key row, d in [hf*HALF, hf*HALF + HALF)
  const int key = min(k0 + col, p.seqlen - 1);
  float ka[HALF];
  {
    const float* src = p.kI + (int64_t)key * DI + hf * HALF;
#pragma unroll
    for (int i = 0; i < HALF; i += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + i);
      ka[i] = v[0]; ka[i + 1] = v[1]; ka[i + 2] = v[2]; ka[i + 3] = v[3];
    }
  }
  const int tq = min(t0 + col, p.seqlen - 1);      // this lane's query (B operand column)
  f32x16_t score;
#pragma unroll
  for (int r = 0; r < 16; ++r) score[r] = 0.f;
  for (int h = 0; h < p.h_i; ++h) {
    const float* qsrc = p.qI + ((int64_t)tq * p.h_i + h) * DI + hf * HALF;
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < HALF; i += 4) {
      const f32x4 qv = *reinterpret_cast<const f32x4*>(qsrc + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[i + e], qv[e], acc, 0, 0, 0);
    }
    const float wh = p.w[(int64_t)tq * p.h_i + h];
#pragma unroll
    for (int r = 0; r < 16; ++r) score[r] = fmaf(wh, fmaxf(acc[r], 0.f), score[r]);
  }
  // lane holds query col, keys 8*(r/4) + 4*hf + (r%4): four runs of 4 consecutive keys
  const int qrow = qt0 + col;
  if (qrow >= p.rows) return;
  float* dst = p.sc + (int64_t)qrow * p.ld + k0 + 4 * hf;
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) {
    const int kk = k0 + 8 * rg + 4 * hf;
    if (kk < p.seqlen) {  // ld is a multiple of 4 and >= seqlen rounded up to 4
      f32x4 v = f32x4{score[4 * rg], score[4 * rg + 1], score[4 * rg + 2], score[4 * rg + 3]};
      *reinterpret_cast<f32x4*>(dst + 8 * rg) = v;
    }
  }
}

// Order-preserving map float -> uint32 (larger float -> larger key); -0 -> +0.
__device__ __forceinline__ uint32_t okey(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct SelectParams {
  const float* sc;
  int64_t ld;
  int32_t* idx;     // [S, topk] of this batch
  int r0, topk;
};

constexpr int NB = 2048;

__global__ __launch_bounds__(256) void topk_select_kernel(SelectParams p) {
  __shared__ uint32_t hist[NB];
  __shared__ uint32_t part[256];
  __shared__ uint32_t sel_info[4];
  __shared__ uint32_t wave_cnt[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row = blockIdx.x;
  const int t = p.r0 + row;
  const int n = t + 1;
  const int k = p.topk;
  int32_t* out = p.idx + (int64_t)t * k;
  if (n <= k) {
    for (int j = tid; j < k; j += 256) out[j] = j < n ? j : -1;
    return;
  }
  const float* srow = p.sc + (int64_t)row * p.ld;

  // radix passes: bits [31:21], [20:10], [9:0]
  uint32_t prefix = 0;       // fixed high bits so far
  uint32_t prefix_mask = 0;
  int need = k;              // how many still to take among elements matching the prefix
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass];
    const uint32_t nb = 1u << widths[pass];
    for (int i = tid; i < NB; i += 256) hist[i] = 0;
    __syncthreads();
    for (int u = tid; u < n; u += 256) {
      const uint32_t key = okey(srow[u]);
      if ((key & prefix_mask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    // descending scan: thread i owns bins [nb - 8(i+1), nb - 8i)
    const int per = nb / 256;
    uint32_t csum = 0;
    for (int j = 0; j < per; ++j) csum += hist[nb - 1 - (tid * per + j)];
    part[tid] = csum;
    __syncthreads();
    // inclusive scan over part[] (Hillis-Steele)
    for (int off = 1; off < 256; off <<= 1) {
      const uint32_t v = tid >= off ? part[tid - off] : 0u;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    const uint32_t before = tid ? part[tid - 1] : 0u;
    if (before < (uint32_t)need && part[tid] >= (uint32_t)need) {
      uint32_t acc = before;
      for (int j = 0; j < per; ++j) {
        const uint32_t bin = nb - 1 - (tid * per + j);
        const uint32_t c = hist[bin];
        if (acc + c >= (uint32_t)need) {
          sel_info[0] = bin;
          sel_info[1] = acc;  // elements above this bin (within the prefix)
          break;
        }
        acc += c;
      }
    }
    __syncthreads();
    const uint32_t bin = sel_info[0];
    need -= (int)sel_info[1];
    prefix |= bin << sh;
    prefix_mask |= (nb - 1) << sh;
    __syncthreads();
  }
  // prefix is now the exact threshold key T; take every key > T and the `need`
  // lowest positions with key == T
  const uint32_t T = prefix;
  const int n_above = k - need;
  if (tid == 0) sel_info[2] = 0;
  __syncthreads();
  uint32_t eq_base = 0;
  for (int base = 0; base < n; base += 256) {
    const int u = base + tid;
    uint32_t key = 0;
    bool valid = u < n;
    if (valid) key = okey(srow[u]);
    const bool gt = valid && key > T;
    const bool eq = valid && key == T;
    if (gt) {
      const uint32_t slot = atomicAdd(&sel_info[2], 1u);
      out[slot] = u;
    }
    const uint64_t m = __ballot(eq);
    const uint32_t below = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[w] = __popcll(m);
    __syncthreads();
    uint32_t off = eq_base;
    for (int i = 0; i < w; ++i) off += wave_cnt[i];
    const uint32_t total = wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
    if (eq && off + below < (uint32_t)need) out[n_above + off + below] = u;
    eq_base += total;
    __syncthreads();
  }
}

int chunk_rows(int seqlen) {
  // keep one chunk of scores near 256 MB
  int64_t r = ((int64_t)1 << 26) / (((int64_t)seqlen + 3) & ~3ll);
  if (r < 32) r = 32;
  r = r / 32 * 32;
  if (r > seqlen) r = ((seqlen + 31) / 32) * 32;
  return (int)r;
}

}  // namespace

size_t dsa_topk_workspace_bytes(int batch, int seqlen, int topk) {
  (void)batch;
  (void)topk;
  const int64_t ld = ((int64_t)seqlen + 127) / 128 * 128;
  return (size_t)chunk_rows(seqlen) * ld * sizeof(float);
}

hipError_t launch_dsa_index_topk(const float* qI, const float* kI, const float* w, int32_t* idx, int batch,
                                 int seqlen, int h_i, int d_i, int topk, void* ws, size_t ws_bytes, hipStream_t st) {
  (void)ws_bytes;
  const int64_t ld = ((int64_t)seqlen + 127) / 128 * 128;
  const int R = chunk_rows(seqlen);
  for (int b = 0; b < batch; ++b) {
    for (int r0 = 0; r0 < seqlen; r0 += R) {
      const int rows = min(R, seqlen - r0);
      ScoreParams sp;
      sp.qI = qI + (int64_t)b * seqlen * h_i * d_i;
      sp.kI = kI + (int64_t)b * seqlen * d_i;
      sp.w = w + (int64_t)b * seqlen * h_i;
      sp.sc = (float*)ws;
      sp.ld = ld;
      sp.seqlen = seqlen;
      sp.h_i = h_i;
      sp.d_i = d_i;
      sp.r0 = r0;
      sp.rows = rows;
      const int key_tiles = (r0 + rows + KT * WAVES - 1) / (KT * WAVES);
      dim3 grid(key_tiles, (rows + QT - 1) / QT);
      switch (d_i) {
        case 16: hipLaunchKernelGGL(index_scores_kernel<16>, grid, dim3(256), 0, st, sp); break;
        case 32: hipLaunchKernelGGL(index_scores_kernel<32>, grid, dim3(256), 0, st, sp); break;
        case 48: hipLaunchKernelGGL(index_scores_kernel<48>, grid, dim3(256), 0, st, sp); break;
        case 64: hipLaunchKernelGGL(index_scores_kernel<64>, grid, dim3(256), 0, st, sp); break;
        case 80: hipLaunchKernelGGL(index_scores_kernel<80>, grid, dim3(256), 0, st, sp); break;
        case 96: hipLaunchKernelGGL(index_scores_kernel<96>, grid, dim3(256), 0, st, sp); break;
        case 112: hipLaunchKernelGGL(index_scores_kernel<112>, grid, dim3(256), 0, st, sp); break;
        case 128: hipLaunchKernelGGL(index_scores_kernel<128>, grid, dim3(256), 0, st, sp); break;
        default: return hipErrorInvalidValue;
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      SelectParams pp;
      pp.sc = (const float*)ws;
      pp.ld = ld;
      pp.idx = idx + (int64_t)b * seqlen * topk;
      pp.r0 = r0;
      pp.topk = topk;
      hipLaunchKernelGGL(topk_select_kernel, dim3(rows), dim3(256), 0, st, pp);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace hca
