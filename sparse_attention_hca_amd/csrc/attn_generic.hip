// HCA attention, one workgroup per (query, head): the straightforward form of
// the operation, used for fp32 inputs and for head sizes other than 512.
// Keys of query t: compressed entries [0, n_c) then raw positions [lo, t]
// (ERNIE 5.5 Flash Base pages, mirrorspeed page, "Hybrid sparse attention"
// section; window = W newest positions, blocks that end before the window).
// Logits are kept in LDS (up to kGenericMaxKeys per query), softmax in fp32.
#include "device_common.h"
#include "launchers.h"

namespace hca {

template <typename T>
__device__ __forceinline__ float ldf(const T* p) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
  else return *p;
}

template <typename T>
__global__ __launch_bounds__(256) void attn_generic_kernel(AttnArgs a) {
  extern __shared__ float sm[];
  const int d = a.head_dim;
  float* qs = sm;           // [d]
  float* lg = sm + d;       // [n keys]
  __shared__ float red[8];

  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (a.h_q / a.h_kv);
  const int64_t t = a.q_pos0 + i;
  const int64_t lo = t - a.window + 1 > 0 ? t - a.window + 1 : 0;
  const int n_c = (int)(lo / a.block);
  const int n_w = (int)(t - lo + 1);
  const int n = n_c + n_w;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;

  const T* qp = (const T*)a.q + b * a.sq.b + (int64_t)i * a.sq.s + (int64_t)h * a.sq.h;
  for (int e = tid; e < d; e += 256) qs[e] = ldf(qp + e);
  __syncthreads();

  const T* kcb = (const T*)a.kc + b * a.skc.b + (int64_t)g * a.skc.h;
  const T* vcb = (const T*)a.vc + b * a.svc.b + (int64_t)g * a.svc.h;
  const T* kb = (const T*)a.k + b * a.sk.b + (int64_t)g * a.sk.h + (lo - a.kv_pos0) * a.sk.s;
  const T* vb = (const T*)a.v + b * a.sv.b + (int64_t)g * a.sv.h + (lo - a.kv_pos0) * a.sv.s;

  float mx = -INFINITY;
  for (int x = tid; x < n; x += 256) {
    const T* kp = x < n_c ? kcb + (int64_t)x * a.skc.s : kb + (int64_t)(x - n_c) * a.sk.s;
    float acc = 0.f;
    for (int e = 0; e < d; ++e) acc = fmaf(qs[e], ldf(kp + e), acc);
    acc *= a.scale;
    lg[x] = acc;
    mx = fmaxf(mx, acc);
  }
  mx = wave_max(mx);
  if (lane == 0) red[wid] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();

  float sum = 0.f;
  for (int x = tid; x < n; x += 256) {
    const float p = __expf(lg[x] - mx);
    lg[x] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  if (lane == 0) red[wid] = sum;
  __syncthreads();
  sum = red[0] + red[1] + red[2] + red[3];
  const float inv = 1.f / sum;

  T* op = (T*)a.o + b * a.so.b + (int64_t)i * a.so.s + (int64_t)h * a.so.h;
  for (int e = tid; e < d; e += 256) {
    float acc = 0.f;
    for (int x = 0; x < n_c; ++x) acc = fmaf(lg[x], ldf(vcb + (int64_t)x * a.svc.s + e), acc);
    for (int x = n_c; x < n; ++x) acc = fmaf(lg[x], ldf(vb + (int64_t)(x - n_c) * a.sv.s + e), acc);
    acc *= inv;
    if constexpr (sizeof(T) == 2) *reinterpret_cast<uint16_t*>(op + e) = f32_to_bf16(acc);
    else op[e] = acc;
  }
  if (a.lse && tid == 0) a.lse[((int64_t)b * a.h_q + h) * a.seqlen_q + i] = mx + __logf(sum);
}

hipError_t launch_attn_generic(const AttnArgs& a, hipStream_t st) {
  const int64_t t_last = a.q_pos0 + a.seqlen_q - 1;
  int64_t lo = t_last - a.window + 1;
  if (lo < 0) lo = 0;
  // the key count is largest for the last query
  const int64_t n_max = lo / a.block + (t_last - lo + 1);
  const size_t shmem = (size_t)(a.head_dim + n_max) * sizeof(float);
  dim3 grid(a.seqlen_q, a.h_q, a.batch);
  if (shmem > 65536) {
    hipError_t e = a.dt == 1 ? hipFuncSetAttribute((const void*)attn_generic_kernel<uint16_t>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem)
                             : hipFuncSetAttribute((const void*)attn_generic_kernel<float>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  if (a.dt == 1)
    hipLaunchKernelGGL(attn_generic_kernel<uint16_t>, grid, dim3(256), shmem, st, a);
  else
    hipLaunchKernelGGL(attn_generic_kernel<float>, grid, dim3(256), shmem, st, a);
  return hipGetLastError();
}

}  // namespace hca
