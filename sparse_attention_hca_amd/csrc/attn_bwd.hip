// Backward of HCA attention, of the block compressor and of DSA sparse
// attention (ERNIE 5.5 Flash Base pages: mirrorspeed page, "Hybrid sparse
// attention" section, gives the forward; training reaches 128K tokens).  The
// gradients are the chain rule through the forward definitions:
//   p = softmax(scale * K q), o = p V,  D = <dO, o>,
//   ds_x = p_x (<dO, v_x> - D),  dq = scale sum_x ds_x k_x,
//   dk_x += scale ds_x q,  dv_x += p_x dO,
// with p recomputed from the forward's log-sum-exp.  All arithmetic is fp32;
// the gradients are written in fp32.
//
// Work split (no atomics, so every gradient is a fixed-order sum):
//   * delta: D per (query, head);
//   * dq: one workgroup per (query, head): the row's ds in LDS (threads over
//     keys), then dq (threads over dims, coalesced key-row reads);
//   * dk/dv: one workgroup per key row (raw row, compressed entry, or DSA
//     position) and KV head walks the (query, head) pairs that see it, 256 at
//     a time: ds and p per pair (threads over pairs), then the row's dk/dv
//     (threads over dims).  HCA pairs come from closed-form query ranges; DSA
//     pairs from an inverted index built in the workspace.
//   * compressor: dk_raw += w * dkc over the block rows, and
//     dw[h, i] = sum_{b, j} <dkc[b, j, h], k[b, j*block + i, h]>.
#include "device_common.h"
#include "launchers.h"

namespace hca {
namespace {

constexpr int NT = 256;

template <typename T>
__device__ __forceinline__ float ldf(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ldf<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

// Dot product of an LDS row with a global row of d elements (one thread).
template <typename T>
__device__ __forceinline__ float dot_row(const float* s, const T* g, int d) {
  float acc = 0.f;
  for (int e = 0; e < d; ++e) acc = fmaf(s[e], ldf(g, e), acc);
  return acc;
}

// D[b, h, i] = <dO[b, i, h, :], O[b, i, h, :]>: one wave per (query, head).
template <typename T>
__global__ __launch_bounds__(64) void bwd_delta_kernel(BwdArgs a) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const T* o = (const T*)a.o + b * a.so.b + (int64_t)i * a.so.s + (int64_t)h * a.so.h;
  const T* g = (const T*)a.dout + b * a.sdo.b + (int64_t)i * a.sdo.s + (int64_t)h * a.sdo.h;
  float acc = 0.f;
  for (int e = threadIdx.x; e < a.d_v; e += 64) acc = fmaf(ldf(o, e), ldf(g, e), acc);
  acc = wave_sum(acc);
  if (threadIdx.x == 0) a.delta[((int64_t)b * a.h_q + h) * a.seqlen_q + i] = acc;
}

// Keys of query i (HCA: compressed entries then the raw window; DSA: the
// listed positions) -> pointers to the key and value rows.
struct KeyRows {
  const void* k;
  const void* v;
};

template <typename T>
__device__ __forceinline__ KeyRows hca_key(const BwdArgs& a, int b, int g, int n_c, int lo_row, int x) {
  if (x < n_c) {
    return KeyRows{(const T*)a.kc + b * a.skc.b + (int64_t)x * a.skc.s + (int64_t)g * a.skc.h,
                   (const T*)a.vc + b * a.svc.b + (int64_t)x * a.svc.s + (int64_t)g * a.svc.h};
  }
  const int64_t r = lo_row + (x - n_c);
  return KeyRows{(const T*)a.k + b * a.sk.b + r * a.sk.s + (int64_t)g * a.sk.h,
                 (const T*)a.v + b * a.sv.b + r * a.sv.s + (int64_t)g * a.sv.h};
}

// dq of one (query i, head h): keys enumerated by `key(x)` for x < nk (nk <=
// kBwdMaxKeys); returns nothing, writes dq.
template <typename T, typename KeyFn>
__device__ __forceinline__ void dq_row(const BwdArgs& a, int b, int i, int h, int nk, KeyFn key, float* s_ds, float* s_q,
                                       float* s_do) {
  const int tid = threadIdx.x;
  const T* qp = (const T*)a.q + b * a.sq.b + (int64_t)i * a.sq.s + (int64_t)h * a.sq.h;
  const T* gp = (const T*)a.dout + b * a.sdo.b + (int64_t)i * a.sdo.s + (int64_t)h * a.sdo.h;
  for (int e = tid; e < a.d; e += NT) s_q[e] = ldf(qp, e);
  for (int e = tid; e < a.d_v; e += NT) s_do[e] = ldf(gp, e);
  __syncthreads();
  const float lse = a.lse[((int64_t)b * a.h_q + h) * a.seqlen_q + i];
  const float dl = a.delta[((int64_t)b * a.h_q + h) * a.seqlen_q + i];
  for (int x = tid; x < nk; x += NT) {
    const KeyRows r = key(x);
    float ds = 0.f;
    if (r.k) {
      const float s = a.scale * dot_row(s_q, (const T*)r.k, a.d);
      const float p = __expf(s - lse);
      ds = p * (dot_row(s_do, (const T*)r.v, a.d_v) - dl);
    }
    s_ds[x] = ds;
  }
  __syncthreads();
  float* dq = a.dq + b * a.sdq.b + (int64_t)i * a.sdq.s + (int64_t)h * a.sdq.h;
  for (int e = tid; e < a.d; e += NT) {
    float acc = 0.f;
    for (int x = 0; x < nk; ++x) {
      const KeyRows r = key(x);
      if (r.k) acc = fmaf(s_ds[x], ldf((const T*)r.k, e), acc);
    }
    dq[e] = a.scale * acc;
  }
}

template <typename T>
__global__ __launch_bounds__(NT) void hca_bwd_dq_kernel(BwdArgs a) {
  __shared__ float s_ds[kBwdMaxKeys];
  __shared__ float s_q[512], s_do[512];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (a.h_q / a.h_kv);
  const int64_t t = a.q_pos0 + i;
  const int64_t lo = t - a.window + 1 > 0 ? t - a.window + 1 : 0;
  const int n_c = (int)(lo / a.block);
  const int nk = n_c + (int)(t - lo + 1);
  const int lo_row = (int)(lo - a.kv_pos0);
  dq_row<T>(a, b, i, h, nk, [&](int x) { return hca_key<T>(a, b, g, n_c, lo_row, x); }, s_ds, s_q, s_do);
}

template <typename T>
__global__ __launch_bounds__(NT) void dsa_bwd_dq_kernel(BwdArgs a) {
  __shared__ float s_ds[kBwdMaxKeys];
  __shared__ float s_q[512], s_do[512];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (a.h_q / a.h_kv);
  const int32_t* row = a.idx + ((int64_t)b * a.seqlen_q + i) * a.topk;
  dq_row<T>(a, b, i, h, a.topk,
            [&](int x) {
              const int u = row[x];
              if (u < 0 || u >= a.seqlen_kv) return KeyRows{nullptr, nullptr};
              return KeyRows{(const T*)a.k + b * a.sk.b + (int64_t)u * a.sk.s + (int64_t)g * a.sk.h,
                             (const T*)a.v + b * a.sv.b + (int64_t)u * a.sv.s + (int64_t)g * a.sv.h};
            },
            s_ds, s_q, s_do);
}

// dk/dv of one key row (k_row, v_row) over pairs (query i, head h) given by
// pair(p) for p < np; writes the fp32 rows dk, dv.
template <typename T, typename PairFn>
__device__ __forceinline__ void dkv_row(const BwdArgs& a, int b, const T* k_row, const T* v_row, int np, PairFn pair,
                                        float* dk, float* dv) {
  __shared__ float s_k[512], s_v[512];
  __shared__ float s_ds[NT], s_p[NT];
  __shared__ int s_i[NT], s_h[NT];
  const int tid = threadIdx.x;
  for (int e = tid; e < a.d; e += NT) s_k[e] = ldf(k_row, e);
  for (int e = tid; e < a.d_v; e += NT) s_v[e] = ldf(v_row, e);
  float acc_k[2] = {0.f, 0.f}, acc_v[2] = {0.f, 0.f};  // dims tid and tid + 256 (d <= 512)
  for (int p0 = 0; p0 < np; p0 += NT) {
    __syncthreads();  // s_k/s_v written; previous chunk's pairs consumed
    const int p = p0 + tid;
    if (p < np) {
      int i, h;
      pair(p, i, h);
      const T* qp = (const T*)a.q + b * a.sq.b + (int64_t)i * a.sq.s + (int64_t)h * a.sq.h;
      const T* gp = (const T*)a.dout + b * a.sdo.b + (int64_t)i * a.sdo.s + (int64_t)h * a.sdo.h;
      const int64_t ih = ((int64_t)b * a.h_q + h) * a.seqlen_q + i;
      const float s = a.scale * dot_row(s_k, qp, a.d);
      const float pr = __expf(s - a.lse[ih]);
      s_ds[tid] = pr * (dot_row(s_v, gp, a.d_v) - a.delta[ih]);
      s_p[tid] = pr;
      s_i[tid] = i;
      s_h[tid] = h;
    }
    __syncthreads();
    const int n = np - p0 < NT ? np - p0 : NT;
    for (int j = 0; j < n; ++j) {
      const int i = s_i[j], h = s_h[j];
      const T* qp = (const T*)a.q + b * a.sq.b + (int64_t)i * a.sq.s + (int64_t)h * a.sq.h;
      const T* gp = (const T*)a.dout + b * a.sdo.b + (int64_t)i * a.sdo.s + (int64_t)h * a.sdo.h;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int e = tid + NT * r;
        if (e < a.d) acc_k[r] = fmaf(s_ds[j], ldf(qp, e), acc_k[r]);
        if (e < a.d_v) acc_v[r] = fmaf(s_p[j], ldf(gp, e), acc_v[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int e = tid + NT * r;
    if (e < a.d) dk[e] = a.scale * acc_k[r];
    if (e < a.d_v) dv[e] = acc_v[r];
  }
}

// One workgroup per (raw row or compressed entry, KV head, batch).
template <typename T>
__global__ __launch_bounds__(NT) void hca_bwd_dkv_kernel(BwdArgs a) {
  const int item = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int group = a.h_q / a.h_kv;
  const int64_t q_end = a.q_pos0 + a.seqlen_q - 1;
  int64_t t0, t1;  // positions of the queries that see this key
  const T *k_row, *v_row;
  float *dk, *dv;
  if (item < a.seqlen_kv) {
    const int64_t px = a.kv_pos0 + item;  // raw key: in the windows of t in [px, px + W - 1]
    t0 = px > a.q_pos0 ? px : a.q_pos0;
    t1 = px + a.window - 1 < q_end ? px + a.window - 1 : q_end;
    k_row = (const T*)a.k + b * a.sk.b + (int64_t)item * a.sk.s + (int64_t)g * a.sk.h;
    v_row = (const T*)a.v + b * a.sv.b + (int64_t)item * a.sv.s + (int64_t)g * a.sv.h;
    dk = a.dk + b * a.sdk.b + (int64_t)item * a.sdk.s + (int64_t)g * a.sdk.h;
    dv = a.dv + b * a.sdv.b + (int64_t)item * a.sdv.s + (int64_t)g * a.sdv.h;
  } else {
    const int j = item - a.seqlen_kv;  // entry j: seen once lo(t) >= block (j + 1)
    const int64_t first = (int64_t)a.block * (j + 1) + a.window - 1;
    t0 = first > a.q_pos0 ? first : a.q_pos0;
    t1 = q_end;
    k_row = (const T*)a.kc + b * a.skc.b + (int64_t)j * a.skc.s + (int64_t)g * a.skc.h;
    v_row = (const T*)a.vc + b * a.svc.b + (int64_t)j * a.svc.s + (int64_t)g * a.svc.h;
    dk = a.dkc + b * a.sdkc.b + (int64_t)j * a.sdkc.s + (int64_t)g * a.sdkc.h;
    dv = a.dvc + b * a.sdvc.b + (int64_t)j * a.sdvc.s + (int64_t)g * a.sdvc.h;
  }
  const int nq = t1 >= t0 ? (int)(t1 - t0 + 1) : 0;
  const int i0 = (int)(t0 - a.q_pos0);
  dkv_row<T>(a, b, k_row, v_row, nq * group,
             [&](int p, int& i, int& h) {
               i = i0 + p / group;
               h = g * group + p % group;
             },
             dk, dv);
}

// One workgroup per (position u, KV head, batch): the queries that listed u
// (inverted index) times the query heads of the group.
template <typename T>
__global__ __launch_bounds__(NT) void dsa_bwd_dkv_kernel(BwdArgs a) {
  const int u = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int group = a.h_q / a.h_kv;
  const int32_t* off = a.inv_off + (int64_t)b * (a.seqlen_kv + 1);
  const int beg = off[u], nq = off[u + 1] - beg;
  const int32_t* list = a.inv_list + (int64_t)b * a.inv_ld + beg;
  dkv_row<T>(a, b, (const T*)a.k + b * a.sk.b + (int64_t)u * a.sk.s + (int64_t)g * a.sk.h,
             (const T*)a.v + b * a.sv.b + (int64_t)u * a.sv.s + (int64_t)g * a.sv.h, nq * group,
             [&](int p, int& i, int& h) {
               i = list[p / group];
               h = g * group + p % group;
             },
             a.dk + b * a.sdk.b + (int64_t)u * a.sdk.s + (int64_t)g * a.sdk.h,
             a.dv + b * a.sdv.b + (int64_t)u * a.sdv.s + (int64_t)g * a.sdv.h);
}

// ---- inverted index of the DSA selections: for every position u, the
// queries whose list holds it (once per occurrence), in query order.
__global__ __launch_bounds__(NT) void inv_zero_kernel(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) p[i] = 0;
}

__global__ __launch_bounds__(NT) void inv_count_kernel(BwdArgs a, int32_t* cnt) {
  const int64_t n = (int64_t)a.seqlen_q * a.topk;
  const int b = blockIdx.y;
  for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < n; e += (int64_t)gridDim.x * NT) {
    const int u = a.idx[(int64_t)b * n + e];
    if (u >= 0 && u < a.seqlen_kv) atomicAdd(&cnt[(int64_t)b * (a.seqlen_kv + 1) + u], 1);
  }
}

// Exclusive prefix of the counts of one batch, in place (cnt[S] = total).
__global__ __launch_bounds__(NT) void inv_scan_kernel(int32_t* cnt, int S) {
  __shared__ int32_t part[NT];
  int32_t* c = cnt + (int64_t)blockIdx.x * (S + 1);
  const int tid = threadIdx.x;
  const int per = (S + NT - 1) / NT;
  const int lo = tid * per, hi = lo + per < S ? lo + per : S;
  int32_t sum = 0;
  for (int u = lo; u < hi; ++u) sum += c[u];
  part[tid] = sum;
  __syncthreads();
  for (int d = 1; d < NT; d <<= 1) {
    const int32_t x = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  int32_t run = part[tid] - sum;
  for (int u = lo; u < hi; ++u) {
    const int32_t x = c[u];
    c[u] = run;
    run += x;
  }
  if (tid == NT - 1) c[S] = part[NT - 1];
}

// One workgroup per (query, batch): its entries go to their positions' lists
// at slots taken from a per-position cursor.  Queries are visited in order by
// the workgroup of each query, so a list is ordered only up to the cursor
// race; the dk/dv sums do not depend on the order beyond rounding.
__global__ __launch_bounds__(NT) void inv_fill_kernel(BwdArgs a, const int32_t* off, int32_t* cur) {
  const int i = blockIdx.x, b = blockIdx.y;
  const int32_t* row = a.idx + ((int64_t)b * a.seqlen_q + i) * a.topk;
  for (int j = threadIdx.x; j < a.topk; j += NT) {
    const int u = row[j];
    if (u < 0 || u >= a.seqlen_kv) continue;
    const int slot = atomicAdd(&cur[(int64_t)b * a.seqlen_kv + u], 1);
    a.inv_list[(int64_t)b * a.inv_ld + off[(int64_t)b * (a.seqlen_kv + 1) + u] + slot] = i;
  }
}

// ---- compressor backward
// dx[b, j*block + i, h, :] += w[h, i] * dxc[b, j, h, :] for K and V: one
// thread per element of the compressed rows' sources.
struct CompBwdArgs {
  const void* k;
  const void* v;
  LStrides sk, sv;
  const float* dkc;
  const float* dvc;
  LStrides sdkc, sdvc;
  const float* wk;
  const float* wv;
  float* dk;
  float* dv;
  LStrides sdk, sdv;
  float* dwk;
  float* dwv;
  int batch, nb, h, d, block;
};

// One workgroup per (compressed block, head): each thread keeps 4 dims of the
// block's dkc and dvc rows and updates those dims of every other source row
// (two rows in flight per step, 128 threads per row, d <= 512).
__global__ __launch_bounds__(NT) void comp_bwd_dx_kernel(CompBwdArgs c) {
  const int bj = blockIdx.x, h = blockIdx.y;
  const int b = bj / c.nb, j = bj % c.nb;
  const int half = threadIdx.x >> 7, e = 4 * (threadIdx.x & 127);
  if (e >= c.d) return;
  const f32x4 gk = *reinterpret_cast<const f32x4*>(c.dkc + b * c.sdkc.b + (int64_t)j * c.sdkc.s + (int64_t)h * c.sdkc.h + e);
  const f32x4 gv = *reinterpret_cast<const f32x4*>(c.dvc + b * c.sdvc.b + (int64_t)j * c.sdvc.s + (int64_t)h * c.sdvc.h + e);
  float* dk0 = c.dk + b * c.sdk.b + (int64_t)j * c.block * c.sdk.s + (int64_t)h * c.sdk.h + e;
  float* dv0 = c.dv + b * c.sdv.b + (int64_t)j * c.block * c.sdv.s + (int64_t)h * c.sdv.h + e;
  for (int i = half; i < c.block; i += 2) {
    const float wk = c.wk[h * c.block + i], wv = c.wv[h * c.block + i];
    f32x4* pk = reinterpret_cast<f32x4*>(dk0 + (int64_t)i * c.sdk.s);
    f32x4* pv = reinterpret_cast<f32x4*>(dv0 + (int64_t)i * c.sdv.s);
    f32x4 xk = *pk, xv = *pv;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      xk[t] = fmaf(wk, gk[t], xk[t]);
      xv[t] = fmaf(wv, gv[t], xv[t]);
    }
    *pk = xk;
    *pv = xv;
  }
}

template <typename T>
__device__ __forceinline__ f32x4 ld4f(const T* p);
template <>
__device__ __forceinline__ f32x4 ld4f<float>(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
template <>
__device__ __forceinline__ f32x4 ld4f<uint16_t>(const uint16_t* p) {
  const u32x2 u = *reinterpret_cast<const u32x2*>(p);
  return f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u), __uint_as_float(u[1] << 16),
               __uint_as_float(u[1] & 0xffff0000u)};
}
// The same for data read once (non-temporal loads).
template <typename T>
__device__ __forceinline__ f32x4 ld4f_nt(const T* p);
template <>
__device__ __forceinline__ f32x4 ld4f_nt<float>(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
template <>
__device__ __forceinline__ f32x4 ld4f_nt<uint16_t>(const uint16_t* p) {
  const u32x2 u = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u), __uint_as_float(u[1] << 16),
               __uint_as_float(u[1] & 0xffff0000u)};
}

// dw[h, i] = sum_{b, j} <dxc[b, j, h, :], x[b, j*block + i, h, :]>: one
// workgroup per (row-in-block i, head h, K or V); threads hold 4 dims and
// walk the (b, j) rows (128 threads per row, two rows in flight), then one
// block reduction.
template <typename T>
__global__ __launch_bounds__(NT) void comp_bwd_dw_kernel(CompBwdArgs c) {
  __shared__ float part[NT / 64];
  const int i = blockIdx.x, h = blockIdx.y, which = blockIdx.z;
  const T* x = (const T*)(which ? c.v : c.k);
  const LStrides sx = which ? c.sv : c.sk;
  const float* dxc = which ? c.dvc : c.dkc;
  const LStrides sd = which ? c.sdvc : c.sdkc;
  const int half = threadIdx.x >> 7, e = 4 * (threadIdx.x & 127);
  float acc = 0.f;
  if (e < c.d) {
    for (int b = 0; b < c.batch; ++b)
#pragma unroll 8
      for (int j = half; j < c.nb; j += 2) {
        const f32x4 g = *reinterpret_cast<const f32x4*>(dxc + b * sd.b + (int64_t)j * sd.s + (int64_t)h * sd.h + e);
        // each K/V row is read once per call: non-temporal
        const f32x4 xv = ld4f_nt<T>(x + b * sx.b + ((int64_t)j * c.block + i) * sx.s + (int64_t)h * sx.h + e);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc = fmaf(g[t], xv[t], acc);
      }
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int w = 0; w < NT / 64; ++w) s += part[w];
    (which ? c.dwv : c.dwk)[h * c.block + i] = s;
  }
}

template <typename T>
hipError_t run_hca_bwd(const BwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(bwd_delta_kernel<T>, dim3(a.seqlen_q, a.h_q, a.batch), dim3(64), 0, st, a);
  hipLaunchKernelGGL(hca_bwd_dq_kernel<T>, dim3(a.seqlen_q, a.h_q, a.batch), dim3(NT), 0, st, a);
  hipLaunchKernelGGL(hca_bwd_dkv_kernel<T>, dim3(a.seqlen_kv + a.n_blocks, a.h_kv, a.batch), dim3(NT), 0, st, a);
  return hipGetLastError();
}

template <typename T>
hipError_t run_dsa_bwd(const BwdArgs& a, int32_t* cnt, int32_t* cur, hipStream_t st) {
  const int64_t ncnt = (int64_t)a.batch * (a.seqlen_kv + 1), ncur = (int64_t)a.batch * a.seqlen_kv;
  hipLaunchKernelGGL(inv_zero_kernel, dim3(256), dim3(NT), 0, st, cnt, ncnt);
  hipLaunchKernelGGL(inv_zero_kernel, dim3(256), dim3(NT), 0, st, cur, ncur);
  const int64_t per_b = (int64_t)a.seqlen_q * a.topk;
  const int gx = (int)((per_b + NT - 1) / NT < 4096 ? (per_b + NT - 1) / NT : 4096);
  hipLaunchKernelGGL(inv_count_kernel, dim3(gx, a.batch), dim3(NT), 0, st, a, cnt);
  hipLaunchKernelGGL(inv_scan_kernel, dim3(a.batch), dim3(NT), 0, st, cnt, a.seqlen_kv);
  hipLaunchKernelGGL(inv_fill_kernel, dim3(a.seqlen_q, a.batch), dim3(NT), 0, st, a, (const int32_t*)cnt, cur);
  BwdArgs b = a;
  b.inv_off = cnt;
  hipLaunchKernelGGL(bwd_delta_kernel<T>, dim3(a.seqlen_q, a.h_q, a.batch), dim3(64), 0, st, b);
  hipLaunchKernelGGL(dsa_bwd_dq_kernel<T>, dim3(a.seqlen_q, a.h_q, a.batch), dim3(NT), 0, st, b);
  hipLaunchKernelGGL(dsa_bwd_dkv_kernel<T>, dim3(a.seqlen_kv, a.h_kv, a.batch), dim3(NT), 0, st, b);
  return hipGetLastError();
}

}  // namespace

static size_t delta_bytes(int batch, int seqlen_q, int h_q) {
  return ((size_t)batch * h_q * seqlen_q * sizeof(float) + 255) / 256 * 256;
}

bool hca_bwd_uses_mfma(int dt, int head_dim) { return dt == 1 && head_dim == 512; }

size_t hca_bwd_workspace_bytes(int dt, int batch, int seqlen_q, int64_t q_pos0, int n_blocks, int h_q, int h_kv,
                               int head_dim, int block, int window) {
  if (hca_bwd_uses_mfma(dt, head_dim))
    return hca_bwd512_workspace_bytes(batch, seqlen_q, q_pos0, n_blocks, h_q, h_kv, block, window);
  return delta_bytes(batch, seqlen_q, h_q);
}

hipError_t launch_hca_attn_bwd(int dt, BwdArgs a, void* ws, hipStream_t st) {
  if (hca_bwd_uses_mfma(dt, a.d)) return launch_hca_attn_bwd512(a, ws, st);
  a.delta = (float*)ws;
  return dt == 1 ? run_hca_bwd<uint16_t>(a, st) : run_hca_bwd<float>(a, st);
}

size_t dsa_bwd_workspace_bytes(int dt, int batch, int seqlen, int h_q, int h_kv, int d_qk, int d_v, int topk) {
  if (dsa_bwd_uses_mfma(dt, d_qk, d_v, h_q, h_kv)) return dsa_bwd256_workspace_bytes(batch, seqlen, h_q, h_kv, topk);
  size_t bytes = delta_bytes(batch, seqlen, h_q);                                  // delta
  bytes += ((size_t)batch * (seqlen + 1) * sizeof(int32_t) + 255) / 256 * 256;      // counts -> offsets
  bytes += ((size_t)batch * seqlen * sizeof(int32_t) + 255) / 256 * 256;            // cursors
  bytes += (size_t)batch * seqlen * topk * sizeof(int32_t);                          // lists
  return bytes;
}

hipError_t launch_dsa_attn_bwd(int dt, BwdArgs a, void* ws, hipStream_t st) {
  if (dsa_bwd_uses_mfma(dt, a.d, a.d_v, a.h_q, a.h_kv)) return launch_dsa_bwd256(a, ws, st);
  char* p = (char*)ws;
  a.delta = (float*)p;
  p += delta_bytes(a.batch, a.seqlen_q, a.h_q);
  int32_t* cnt = (int32_t*)p;
  p += ((size_t)a.batch * (a.seqlen_kv + 1) * sizeof(int32_t) + 255) / 256 * 256;
  int32_t* cur = (int32_t*)p;
  p += ((size_t)a.batch * a.seqlen_kv * sizeof(int32_t) + 255) / 256 * 256;
  a.inv_list = (int32_t*)p;
  a.inv_ld = (int64_t)a.seqlen_q * a.topk;
  return dt == 1 ? run_dsa_bwd<uint16_t>(a, cnt, cur, st) : run_dsa_bwd<float>(a, cnt, cur, st);
}

hipError_t launch_hca_attn_compress_bwd(int dt, BwdArgs a, const float* wk, const float* wv, float* dwk, float* dwv,
                                        void* ws, hipStream_t st) {
  hipError_t e;
  if (hca_bwd_uses_mfma(dt, a.d))
    e = launch_hca_attn_bwd512(a, ws, st, wk, wv);
  else
    e = launch_hca_attn_bwd(dt, a, ws, st);
  if (e != hipSuccess) return e;
  // the weight gradient, plus (generic path) the raw-row update
  return launch_compress_bwd(dt, a.k, a.sk, a.v, a.sv, a.dkc, a.sdkc, a.dvc, a.sdvc, wk, wv, a.dk, a.sdk, a.dv, a.sdv,
                             dwk, dwv, a.batch, a.n_blocks * a.block, a.h_kv, a.d, a.block, st,
                             !hca_bwd_uses_mfma(dt, a.d));
}

hipError_t launch_compress_bwd(int dt, const void* k, LStrides sk, const void* v, LStrides sv, const float* dkc,
                               LStrides sdkc, const float* dvc, LStrides sdvc, const float* wk, const float* wv,
                               float* dk, LStrides sdk, float* dv, LStrides sdv, float* dwk, float* dwv, int batch,
                               int seqlen, int h, int d, int block, hipStream_t st, bool dx) {
  CompBwdArgs c;
  c.k = k; c.v = v; c.sk = sk; c.sv = sv;
  c.dkc = dkc; c.dvc = dvc; c.sdkc = sdkc; c.sdvc = sdvc;
  c.wk = wk; c.wv = wv;
  c.dk = dk; c.dv = dv; c.sdk = sdk; c.sdv = sdv;
  c.dwk = dwk; c.dwv = dwv;
  c.batch = batch; c.nb = seqlen / block; c.h = h; c.d = d; c.block = block;
  if (c.nb > 0 && dx)
    hipLaunchKernelGGL(comp_bwd_dx_kernel, dim3((unsigned)(batch * c.nb), h), dim3(NT), 0, st, c);
  if (dt == 1)
    hipLaunchKernelGGL(comp_bwd_dw_kernel<uint16_t>, dim3(block, h, 2), dim3(NT), 0, st, c);
  else
    hipLaunchKernelGGL(comp_bwd_dw_kernel<float>, dim3(block, h, 2), dim3(NT), 0, st, c);
  return hipGetLastError();
}

}  // namespace hca
