// HCA block compression: each block of `block` consecutive K (or V) rows of one
// head becomes one cache entry, the per-head weighted sum of those rows
// (ERNIE 5.5 Flash Base pages, mirrorspeed page, section "Hybrid sparse
// attention": 128 tokens per cache entry).
//
// HBM-bound streaming kernels; every input byte is read once, so the loads
// are non-temporal (on the box this moved the 32768-token compression from
// 5.45 to 6.8 TB/s).  General shapes: one workgroup per (block j, head h,
// batch b, K-or-V).  Each thread owns one 16-byte column chunk of the head and walks a
// strided subset of the block's rows with 16-byte loads (a wave reads whole
// contiguous rows), accumulating in fp32; row groups are reduced through LDS.
#include "device_common.h"
#include "launchers.h"

namespace hca {

template <typename T, int D>
__global__ __launch_bounds__(256) void compress_kernel(const T* __restrict__ x0, LStrides sx0, const float* __restrict__ w0,
                                                       T* __restrict__ out0, LStrides so0, const T* __restrict__ x1,
                                                       LStrides sx1, const float* __restrict__ w1, T* __restrict__ out1,
                                                       LStrides so1, int block) {
  constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector
  constexpr int TPR = D / EPV;         // threads covering one row
  constexpr int RG = 256 / TPR;        // rows processed side by side
  static_assert(256 % TPR == 0, "head_dim does not tile a 256-thread workgroup");
  __shared__ float red[RG][D];

  const int j = blockIdx.x, h = blockIdx.y;
  const int b = blockIdx.z >> 1;
  const bool second = blockIdx.z & 1;
  const T* x = second ? x1 : x0;
  const LStrides sx = second ? sx1 : sx0;
  const float* w = (second ? w1 : w0) + (int64_t)h * block;
  T* out = second ? out1 : out0;
  const LStrides so = second ? so1 : so0;

  const int tid = threadIdx.x;
  const int c = tid % TPR, r = tid / TPR;
  const T* base = x + (int64_t)b * sx.b + (int64_t)j * block * sx.s + (int64_t)h * sx.h + c * EPV;

  float acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.f;

  int i = r;
  // 8 rows in flight per thread
  for (; i + 7 * RG < block; i += 8 * RG) {
    u32x4 vals[8];
    float wi[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      vals[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (int64_t)(i + u * RG) * sx.s));
      wi[u] = w[i + u * RG];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = fmaf(wi[u], __uint_as_float(vals[u][e] << 16), acc[2 * e]);
          acc[2 * e + 1] = fmaf(wi[u], __uint_as_float(vals[u][e] & 0xffff0000u), acc[2 * e + 1]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(wi[u], __uint_as_float(vals[u][e]), acc[e]);
      }
    }
  }
  for (; i < block; i += RG) {
    const u32x4 val = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (int64_t)i * sx.s));
    const float wi = w[i];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(wi, __uint_as_float(val[e] << 16), acc[2 * e]);
        acc[2 * e + 1] = fmaf(wi, __uint_as_float(val[e] & 0xffff0000u), acc[2 * e + 1]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(wi, __uint_as_float(val[e]), acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < EPV; ++e) red[r][c * EPV + e] = acc[e];
  __syncthreads();

  T* dst = out + (int64_t)b * so.b + (int64_t)j * so.s + (int64_t)h * so.h;
  for (int e = tid * 2; e < D; e += 512) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      s0 += red[g][e];
      s1 += red[g][e + 1];
    }
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<uint32_t*>(dst + e) = pack_bf16x2(s0, s1);
    } else {
      dst[e] = s0;
      dst[e + 1] = s1;
    }
  }
}

// Row-major variant for heads that fill whole waves: one workgroup per
// (block j, batch b, K-or-V) covers every head, so a block's rows stream as
// contiguous h*d spans when the heads are packed.  Thread tid owns the 16-byte
// column pieces tid + 256k (k < CPT) of the row, each within one head, and
// accumulates them over all rows of the block itself (no reduction); U rows
// of loads are in flight per thread.  Requires (d / EPV) % 64 == 0, so that a
// wave's pieces share one head (its weight is wave-uniform), and
// h * d / EPV == 256 * CPT.
template <typename T, int CPT>
__global__ __launch_bounds__(256) void compress_rows_kernel(const T* __restrict__ x0, LStrides sx0,
                                                            const float* __restrict__ w0, T* __restrict__ out0,
                                                            LStrides so0, const T* __restrict__ x1, LStrides sx1,
                                                            const float* __restrict__ w1, T* __restrict__ out1,
                                                            LStrides so1, int block, int d, int nblocks) {
  constexpr int EPV = 16 / sizeof(T);
  constexpr int U = 4;
  const int b = blockIdx.y >> 1;
  const bool second = blockIdx.y & 1;
  const T* x = second ? x1 : x0;
  const LStrides sx = second ? sx1 : sx0;
  const float* w = second ? w1 : w0;
  T* out = second ? out1 : out0;
  const LStrides so = second ? so1 : so0;
  const int tid = threadIdx.x;
  const int dchunks = d / EPV;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // blocks j = blockIdx.x, + gridDim.x, ...: the grid is sized to one round of
  // resident workgroups, so long sequences stream without a second wave of
  // launches
  for (int j = blockIdx.x; j < nblocks; j += gridDim.x) {
  const T* ptr[CPT];
  const float* wp[CPT];
  int hh[CPT], cc[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int q = tid + 256 * k;
    hh[k] = __builtin_amdgcn_readfirstlane((64 * wv + 256 * k) / dchunks);  // one head per wave
    cc[k] = q - hh[k] * dchunks;
    ptr[k] = x + (int64_t)b * sx.b + (int64_t)j * block * sx.s + (int64_t)hh[k] * sx.h + cc[k] * EPV;
    wp[k] = w + (int64_t)hh[k] * block;
  }
  float acc[CPT][EPV];
#pragma unroll
  for (int k = 0; k < CPT; ++k)
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[k][e] = 0.f;
  auto fma_row = [&](const u32x4& v, float wi, float* a) __attribute__((always_inline)) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[2 * e] = fmaf(wi, __uint_as_float(v[e] << 16), a[2 * e]);
        a[2 * e + 1] = fmaf(wi, __uint_as_float(v[e] & 0xffff0000u), a[2 * e + 1]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = fmaf(wi, __uint_as_float(v[e]), a[e]);
    }
  };
  int i = 0;
  for (; i + U <= block; i += U) {
    u32x4 v[U][CPT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < CPT; ++k)
        v[u][k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr[k] + (int64_t)(i + u) * sx.s));
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < CPT; ++k) fma_row(v[u][k], wp[k][i + u], acc[k]);
  }
  for (; i < block; ++i)
#pragma unroll
    for (int k = 0; k < CPT; ++k) fma_row(ld16(ptr[k] + (int64_t)i * sx.s), wp[k][i], acc[k]);
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    T* dst = out + (int64_t)b * so.b + (int64_t)j * so.s + (int64_t)hh[k] * so.h + cc[k] * EPV;
    if constexpr (sizeof(T) == 2) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(acc[k][2 * e], acc[k][2 * e + 1]);
      st16(dst, pk);
    } else {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = __float_as_uint(acc[k][e]);
      st16(dst, pk);
    }
  }
  }
}

template <typename T, int D>
static void launch_t(const void* x, LStrides sx, const float* w, void* out, LStrides so, const void* x2, LStrides sx2,
                     const float* w2, void* out2, LStrides so2, int batch, int seqlen, int h, int block,
                     hipStream_t st) {
  const int nb = seqlen / block;
  dim3 grid(nb, h, 2 * batch);
  hipLaunchKernelGGL((compress_kernel<T, D>), grid, dim3(256), 0, st, (const T*)x, sx, w, (T*)out, so, (const T*)x2,
                     sx2, w2, (T*)out2, so2, block);
}

hipError_t launch_compress(int dt, const void* x, LStrides sx, const float* w, void* out, LStrides so, const void* x2,
                           LStrides sx2, const float* w2, void* out2, LStrides so2, int batch, int seqlen, int h, int d,
                           int block, hipStream_t st) {
  if (seqlen / block == 0) return hipSuccess;
  {
    // heads that fill whole waves: the row-major kernel
    const int epv = dt == 1 ? 8 : 4;
    const int pieces = h * d / epv;
    if ((d / epv) % 64 == 0 && pieces % 256 == 0) {
      // at most 1024 resident workgroups (4 per CU) over every (block, tensor, batch)
      const int nb = seqlen / block;
      const int per = (1024 + 2 * batch - 1) / (2 * batch);
      const dim3 grid(nb < per ? nb : per, 2 * batch);
#define HCA_COMPRESS_ROWS(T, CPT)                                                                               \
  if (pieces == 256 * CPT) {                                                                                    \
    hipLaunchKernelGGL((compress_rows_kernel<T, CPT>), grid, dim3(256), 0, st, (const T*)x, sx, w, (T*)out, so, \
                       (const T*)x2, sx2, w2, (T*)out2, so2, block, d, nb);                                    \
    return hipGetLastError();                                                                                   \
  }
      if (dt == 1) {
        HCA_COMPRESS_ROWS(uint16_t, 1)
        HCA_COMPRESS_ROWS(uint16_t, 2)
        HCA_COMPRESS_ROWS(uint16_t, 4)
        HCA_COMPRESS_ROWS(uint16_t, 8)
      } else {
        HCA_COMPRESS_ROWS(float, 1)
        HCA_COMPRESS_ROWS(float, 2)
        HCA_COMPRESS_ROWS(float, 4)
        HCA_COMPRESS_ROWS(float, 8)
      }
#undef HCA_COMPRESS_ROWS
    }
  }
#define HCA_COMPRESS_CASE(T, DD)                                                                        \
  if (d == DD) {                                                                                        \
    launch_t<T, DD>(x, sx, w, out, so, x2, sx2, w2, out2, so2, batch, seqlen, h, block, st);            \
    return hipGetLastError();                                                                           \
  }
  if (dt == 1) {
    HCA_COMPRESS_CASE(uint16_t, 64)
    HCA_COMPRESS_CASE(uint16_t, 128)
    HCA_COMPRESS_CASE(uint16_t, 256)
    HCA_COMPRESS_CASE(uint16_t, 512)
  } else {
    HCA_COMPRESS_CASE(float, 64)
    HCA_COMPRESS_CASE(float, 128)
    HCA_COMPRESS_CASE(float, 256)
    HCA_COMPRESS_CASE(float, 512)
  }
#undef HCA_COMPRESS_CASE
  return hipErrorInvalidValue;
}

}  // namespace hca
