// C-ABI layer of libhca: argument validation, error reporting and kernel
// dispatch.  Every argument is checked before anything is launched, so a call
// that fails has written nothing.  No exception, abort or exit crosses the ABI.
#include <algorithm>
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/hca.h"
#include "launchers.h"

namespace {

thread_local std::string g_last_error;

hca_status_t fail(hca_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

hca_status_t hip_fail(hipError_t e, const char* where) {
  return fail(HCA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

hca::LStrides ls(hca_strides_t s) { return hca::LStrides{s.batch, s.seq, s.head}; }

size_t elem_size(hca_dtype_t dt) { return dt == HCA_DTYPE_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Byte range [lo, hi) covered by a [b, s, h, d] tensor with the given strides.
struct Range {
  uintptr_t lo, hi;
};
// Tensors may span at most 2^56 bytes: beyond any device memory, and small
// enough that every offset a kernel forms fits int64 without overflow.
constexpr __int128 kMaxSpan = (__int128)1 << 56;
__int128 span_bytes(hca_strides_t st, int64_t b, int64_t s, int64_t h, int64_t d, size_t es) {
  if (b <= 0 || s <= 0 || h <= 0 || d <= 0) return 0;
  const __int128 last = (__int128)(b - 1) * st.batch + (__int128)(s - 1) * st.seq + (__int128)(h - 1) * st.head + d;
  return last * (__int128)es;
}
// Only called on tensors that passed check_tensor / check_flat, whose span fits.
Range extent(const void* p, hca_strides_t st, int64_t b, int64_t s, int64_t h, int64_t d, size_t es) {
  return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)span_bytes(st, b, s, h, d, es)};
}
Range flat_extent(const void* p, int64_t n, size_t es) { return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)n * es}; }
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Strides must be non-negative multiples of 16 bytes (the kernels use 16-byte vectors).
// [b, s, h, d] is the tensor's shape; its byte span must stay below 2^56 and
// must not wrap the address space.
hca_status_t check_tensor(const char* name, const void* p, hca_strides_t st, int64_t b, int64_t s, int64_t h,
                          int64_t d, size_t es, bool nullable = false) {
  if (!p) {
    if (nullable) return HCA_OK;
    return fail(HCA_ERR_INVALID, "%s is NULL", name);
  }
  if (!aligned16(p)) return fail(HCA_ERR_INVALID, "%s is not 16-byte aligned", name);
  const int64_t q = (int64_t)(16 / es);
  if (st.batch < 0 || st.seq < 0 || st.head < 0 || st.batch % q || st.seq % q || st.head % q)
    return fail(HCA_ERR_INVALID, "%s strides must be non-negative multiples of 16 bytes", name);
  const __int128 span = span_bytes(st, b, s, h, d, es);
  if (span > kMaxSpan || (__int128)(uintptr_t)p + span > (__int128)UINTPTR_MAX)
    return fail(HCA_ERR_INVALID, "%s spans more than 2^56 bytes (or wraps the address space)", name);
  return HCA_OK;
}

// A contiguous tensor of n elements of es bytes (n computed by the caller in 128 bits).
hca_status_t check_flat(const char* name, const void* p, __int128 n, size_t es, unsigned align) {
  if (!p) return fail(HCA_ERR_INVALID, "%s is NULL", name);
  if ((uintptr_t)p % align) return fail(HCA_ERR_INVALID, "%s is not %u-byte aligned", name, align);
  const __int128 span = n * (__int128)es;
  if (n < 0 || span > kMaxSpan || (__int128)(uintptr_t)p + span > (__int128)UINTPTR_MAX)
    return fail(HCA_ERR_INVALID, "%s spans more than 2^56 bytes (or wraps the address space)", name);
  return HCA_OK;
}

#define HCA_TRY(x)                   \
  do {                               \
    hca_status_t _s = (x);           \
    if (_s != HCA_OK) return _s;     \
  } while (0)

constexpr int64_t kPosLimit = (int64_t)1 << 30;

}  // namespace

// Keys seen by the query at position t: compressed entries, then the raw window.
static int n_keys_of(int64_t t, int window, int block) {
  const int64_t lo = t - window + 1 > 0 ? t - window + 1 : 0;
  return (int)(lo / block + (t - lo + 1));
}

static hca_status_t attn_bwd_impl(const char* fn, hca_dtype_t dt, const void* q, hca_strides_t sq, const void* k, hca_strides_t sk,
                          const void* v, hca_strides_t sv, const void* kc, hca_strides_t skc, const void* vc,
                          hca_strides_t svc, const void* o, hca_strides_t so, const float* lse, const void* dout,
                          hca_strides_t sdo, float* dq, hca_strides_t sdq, float* dk, hca_strides_t sdk, float* dv,
                          hca_strides_t sdv, float* dkc, hca_strides_t sdkc, float* dvc, hca_strides_t sdvc,
                          int batch, int seqlen_q, int64_t q_pos0, int seqlen_kv, int64_t kv_pos0, int n_blocks,
                          int h_q, int h_kv, int head_dim, int block, int window, float scale, void* workspace,
                          size_t workspace_bytes, void* stream, const float* w_k, const float* w_v, float* dw_k,
                          float* dw_v) {
  if (dt != HCA_DTYPE_F32 && dt != HCA_DTYPE_BF16) return fail(HCA_ERR_INVALID, "unknown dtype %d", (int)dt);
  if (batch <= 0 || seqlen_q <= 0 || seqlen_kv <= 0 || h_q <= 0 || h_kv <= 0 || head_dim <= 0 || n_blocks < 0)
    return fail(HCA_ERR_INVALID, "%s: sizes must be positive", fn);
  if (h_q % h_kv) return fail(HCA_ERR_INVALID, "h_q (%d) must be a multiple of h_kv (%d)", h_q, h_kv);
  if (window < 1 || block < 1) return fail(HCA_ERR_INVALID, "window and block must be >= 1");
  if (q_pos0 < 0 || kv_pos0 < 0) return fail(HCA_ERR_INVALID, "positions must be >= 0");
  if (q_pos0 + seqlen_q > kPosLimit || kv_pos0 + seqlen_kv > kPosLimit)
    return fail(HCA_ERR_UNSUPPORTED, "positions beyond 2^30 are not supported");
  if (head_dim > 512 || head_dim % 4) return fail(HCA_ERR_UNSUPPORTED, "%s: head_dim must be <= 512, a multiple of 4", fn);
  if (!(scale == scale)) return fail(HCA_ERR_INVALID, "scale is NaN");
  const size_t es = elem_size(dt);
  HCA_TRY(check_tensor("q", q, sq, batch, seqlen_q, h_q, head_dim, es));
  HCA_TRY(check_tensor("k", k, sk, batch, seqlen_kv, h_kv, head_dim, es));
  HCA_TRY(check_tensor("v", v, sv, batch, seqlen_kv, h_kv, head_dim, es));
  HCA_TRY(check_tensor("kc", kc, skc, batch, n_blocks, h_kv, head_dim, es, n_blocks == 0));
  HCA_TRY(check_tensor("vc", vc, svc, batch, n_blocks, h_kv, head_dim, es, n_blocks == 0));
  HCA_TRY(check_tensor("o", o, so, batch, seqlen_q, h_q, head_dim, es));
  HCA_TRY(check_tensor("dout", dout, sdo, batch, seqlen_q, h_q, head_dim, es));
  HCA_TRY(check_tensor("dq", dq, sdq, batch, seqlen_q, h_q, head_dim, 4));
  HCA_TRY(check_tensor("dk", dk, sdk, batch, seqlen_kv, h_kv, head_dim, 4));
  HCA_TRY(check_tensor("dv", dv, sdv, batch, seqlen_kv, h_kv, head_dim, 4));
  HCA_TRY(check_tensor("dkc", dkc, sdkc, batch, n_blocks, h_kv, head_dim, 4, n_blocks == 0));
  HCA_TRY(check_tensor("dvc", dvc, sdvc, batch, n_blocks, h_kv, head_dim, 4, n_blocks == 0));
  HCA_TRY(check_flat("lse", lse, (__int128)batch * h_q * seqlen_q, 4, 4));
  if (w_k) {
    HCA_TRY(check_flat("w_k", w_k, (__int128)h_kv * block, 4, 4));
    HCA_TRY(check_flat("w_v", w_v, (__int128)h_kv * block, 4, 4));
    HCA_TRY(check_flat("dw_k", dw_k, (__int128)h_kv * block, 4, 4));
    HCA_TRY(check_flat("dw_v", dw_v, (__int128)h_kv * block, 4, 4));
  }
  const int64_t t0 = q_pos0, t1 = q_pos0 + seqlen_q - 1;
  const int64_t lo0 = t0 - window + 1 > 0 ? t0 - window + 1 : 0;
  const int64_t lo1 = t1 - window + 1 > 0 ? t1 - window + 1 : 0;
  if (lo0 < kv_pos0 || t1 >= kv_pos0 + seqlen_kv)
    return fail(HCA_ERR_INVALID, "%s: raw K/V must cover every query's window", fn);
  if (lo1 / block > n_blocks) return fail(HCA_ERR_INVALID, "%s: the last query needs more compressed entries", fn);
  const bool mfma = hca::hca_bwd_uses_mfma(dt == HCA_DTYPE_BF16 ? 1 : 0, head_dim);
  if (!mfma && n_keys_of(t1, window, block) > hca::kBwdMaxKeys)
    return fail(HCA_ERR_UNSUPPORTED, "%s: at most %d keys per query", fn, hca::kBwdMaxKeys);
  {
    const Range outs[5] = {extent(dq, sdq, batch, seqlen_q, h_q, head_dim, 4),
                           extent(dk, sdk, batch, seqlen_kv, h_kv, head_dim, 4),
                           extent(dv, sdv, batch, seqlen_kv, h_kv, head_dim, 4),
                           n_blocks ? extent(dkc, sdkc, batch, n_blocks, h_kv, head_dim, 4) : Range{0, 0},
                           n_blocks ? extent(dvc, sdvc, batch, n_blocks, h_kv, head_dim, 4) : Range{0, 0}};
    const Range ins[7] = {extent(q, sq, batch, seqlen_q, h_q, head_dim, es),
                          extent(k, sk, batch, seqlen_kv, h_kv, head_dim, es),
                          extent(v, sv, batch, seqlen_kv, h_kv, head_dim, es),
                          n_blocks ? extent(kc, skc, batch, n_blocks, h_kv, head_dim, es) : Range{0, 0},
                          n_blocks ? extent(vc, svc, batch, n_blocks, h_kv, head_dim, es) : Range{0, 0},
                          extent(o, so, batch, seqlen_q, h_q, head_dim, es),
                          extent(dout, sdo, batch, seqlen_q, h_q, head_dim, es)};
    const Range rl = flat_extent(lse, (int64_t)batch * h_q * seqlen_q, 4);
    for (int x = 0; x < 5; ++x) {
      for (int y = 0; y < 7; ++y)
        if (overlaps(outs[x], ins[y])) return fail(HCA_ERR_INVALID, "%s: a gradient overlaps an input", fn);
      if (overlaps(outs[x], rl)) return fail(HCA_ERR_INVALID, "%s: a gradient overlaps lse", fn);
      for (int y = x + 1; y < 5; ++y)
        if (overlaps(outs[x], outs[y])) return fail(HCA_ERR_INVALID, "%s: gradients overlap each other", fn);
    }
    if (w_k) {
      // the compressor weights' gradients against each other, the weights and every other gradient
      const int64_t nw = (int64_t)h_kv * block;
      const Range rw[4] = {flat_extent(w_k, nw, 4), flat_extent(w_v, nw, 4), flat_extent(dw_k, nw, 4),
                           flat_extent(dw_v, nw, 4)};
      for (int y = 2; y < 4; ++y) {
        for (int x = 0; x < 5; ++x)
          if (overlaps(outs[x], rw[y])) return fail(HCA_ERR_INVALID, "%s: gradients overlap", fn);
        for (int x = 0; x < 4; ++x)
          if (x != y && overlaps(rw[x], rw[y])) return fail(HCA_ERR_INVALID, "%s: weight gradients overlap", fn);
        for (int x = 0; x < 7; ++x)
          if (overlaps(ins[x], rw[y])) return fail(HCA_ERR_INVALID, "%s: a weight gradient overlaps an input", fn);
        if (overlaps(rl, rw[y])) return fail(HCA_ERR_INVALID, "%s: a weight gradient overlaps lse", fn);
      }
    }
  }
  const size_t need = hca::hca_bwd_workspace_bytes(dt == HCA_DTYPE_BF16 ? 1 : 0, batch, seqlen_q, q_pos0, n_blocks,
                                                   h_q, h_kv, head_dim, block, window);
  if (!workspace || workspace_bytes < need)
    return fail(HCA_ERR_WORKSPACE, "%s needs a %zu-byte workspace (got %zu)", fn, need, workspace_bytes);
  if (!aligned16(workspace)) return fail(HCA_ERR_INVALID, "workspace is not 16-byte aligned");
  hca::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.kc = kc; a.vc = vc; a.o = o; a.dout = dout;
  a.sq = ls(sq); a.sk = ls(sk); a.sv = ls(sv); a.skc = ls(skc); a.svc = ls(svc); a.so = ls(so); a.sdo = ls(sdo);
  a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dkc = dkc; a.dvc = dvc;
  a.sdq = ls(sdq); a.sdk = ls(sdk); a.sdv = ls(sdv); a.sdkc = ls(sdkc); a.sdvc = ls(sdvc);
  a.batch = batch; a.seqlen_q = seqlen_q; a.seqlen_kv = seqlen_kv; a.n_blocks = n_blocks;
  a.h_q = h_q; a.h_kv = h_kv; a.d = head_dim; a.d_v = head_dim; a.block = block; a.window = window;
  a.q_pos0 = q_pos0; a.kv_pos0 = kv_pos0; a.scale = scale;
  hipError_t e = w_k ? hca::launch_hca_attn_compress_bwd(dt == HCA_DTYPE_BF16 ? 1 : 0, a, w_k, w_v, dw_k, dw_v,
                                                        workspace, (hipStream_t)stream)
                     : hca::launch_hca_attn_bwd(dt == HCA_DTYPE_BF16 ? 1 : 0, a, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return HCA_OK;
}

extern "C" {

int hca_abi_version(void) { return 1; }

const char* hca_last_error(void) { return g_last_error.c_str(); }

hca_status_t hca_compress_kv(hca_dtype_t dt, const void* k, hca_strides_t sk, const void* v, hca_strides_t sv,
                             const float* w_k, const float* w_v, void* kc, hca_strides_t skc, void* vc,
                             hca_strides_t svc, int batch, int seqlen, int h_kv, int head_dim, int block,
                             void* stream) {
  if (dt != HCA_DTYPE_F32 && dt != HCA_DTYPE_BF16) return fail(HCA_ERR_INVALID, "unknown dtype %d", (int)dt);
  if (batch <= 0 || seqlen <= 0 || h_kv <= 0 || head_dim <= 0 || block <= 0)
    return fail(HCA_ERR_INVALID, "sizes must be positive (batch %d seqlen %d h_kv %d head_dim %d block %d)", batch,
                seqlen, h_kv, head_dim, block);
  if (head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512)
    return fail(HCA_ERR_UNSUPPORTED, "hca_compress_kv: head_dim %d not in {64,128,256,512}", head_dim);
  if (!w_k || !w_v) return fail(HCA_ERR_INVALID, "compressor weights are NULL");
  const size_t es = elem_size(dt);
  const int nb = seqlen / block;
  HCA_TRY(check_tensor("k", k, sk, batch, seqlen, h_kv, head_dim, es));
  HCA_TRY(check_tensor("v", v, sv, batch, seqlen, h_kv, head_dim, es));
  HCA_TRY(check_tensor("kc", kc, skc, batch, nb, h_kv, head_dim, es, nb == 0));
  HCA_TRY(check_tensor("vc", vc, svc, batch, nb, h_kv, head_dim, es, nb == 0));
  if (nb == 0) return HCA_OK;  // no complete block: nothing to write
  if (nb > 0) {
    const Range rk = extent(k, sk, batch, seqlen, h_kv, head_dim, es), rv = extent(v, sv, batch, seqlen, h_kv, head_dim, es);
    const Range rkc = extent(kc, skc, batch, nb, h_kv, head_dim, es), rvc = extent(vc, svc, batch, nb, h_kv, head_dim, es);
    if (overlaps(rkc, rk) || overlaps(rkc, rv) || overlaps(rvc, rk) || overlaps(rvc, rv) || overlaps(rkc, rvc))
      return fail(HCA_ERR_INVALID, "hca_compress_kv: outputs overlap inputs or each other");
  }
  hipError_t e = hca::launch_compress(dt == HCA_DTYPE_BF16 ? 1 : 0, k, ls(sk), w_k, kc, ls(skc), v, ls(sv), w_v, vc,
                                      ls(svc), batch, seqlen, h_kv, head_dim, block, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hca_compress_kv launch");
  return HCA_OK;
}

hca_status_t hca_append_kv(hca_dtype_t dt, const void* k_new, hca_strides_t skn, const void* v_new,
                           hca_strides_t svn, void* k_ring, hca_strides_t skr, void* v_ring, hca_strides_t svr,
                           int ring, const float* w_k, const float* w_v, void* kc, hca_strides_t skc, void* vc,
                           hca_strides_t svc, int n_blocks, int64_t t, int batch, int h_kv, int head_dim, int block,
                           void* stream) {
  if (dt != HCA_DTYPE_F32 && dt != HCA_DTYPE_BF16) return fail(HCA_ERR_INVALID, "unknown dtype %d", (int)dt);
  if (batch <= 0 || h_kv <= 0 || head_dim <= 0 || block <= 0 || ring <= 0 || n_blocks < 0)
    return fail(HCA_ERR_INVALID, "sizes must be positive (batch %d h_kv %d head_dim %d block %d ring %d n_blocks %d)",
                batch, h_kv, head_dim, block, ring, n_blocks);
  if (head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512)
    return fail(HCA_ERR_UNSUPPORTED, "hca_append_kv: head_dim %d not in {64,128,256,512}", head_dim);
  if (ring < block) return fail(HCA_ERR_INVALID, "hca_append_kv: ring (%d) must hold a whole block (%d)", ring, block);
  if (t < 0) return fail(HCA_ERR_INVALID, "position must be >= 0");
  if (t >= kPosLimit) return fail(HCA_ERR_UNSUPPORTED, "positions beyond 2^30 are not supported");
  const bool closes = (t + 1) % block == 0;
  const int64_t j = (t + 1) / block - 1;
  if (closes && j >= n_blocks)
    return fail(HCA_ERR_INVALID, "hca_append_kv: position %lld closes block %lld but kc/vc hold %d blocks",
                (long long)t, (long long)j, n_blocks);
  if (closes && (!w_k || !w_v)) return fail(HCA_ERR_INVALID, "compressor weights are NULL");
  const size_t es = elem_size(dt);
  HCA_TRY(check_tensor("k_new", k_new, skn, batch, 1, h_kv, head_dim, es));
  HCA_TRY(check_tensor("v_new", v_new, svn, batch, 1, h_kv, head_dim, es));
  HCA_TRY(check_tensor("k_ring", k_ring, skr, batch, 2 * (int64_t)ring, h_kv, head_dim, es));
  HCA_TRY(check_tensor("v_ring", v_ring, svr, batch, 2 * (int64_t)ring, h_kv, head_dim, es));
  HCA_TRY(check_tensor("kc", kc, skc, batch, n_blocks, h_kv, head_dim, es, !closes));
  HCA_TRY(check_tensor("vc", vc, svc, batch, n_blocks, h_kv, head_dim, es, !closes));
  {
    const Range rkn = extent(k_new, skn, batch, 1, h_kv, head_dim, es), rvn = extent(v_new, svn, batch, 1, h_kv, head_dim, es);
    const Range rkr = extent(k_ring, skr, batch, 2 * (int64_t)ring, h_kv, head_dim, es);
    const Range rvr = extent(v_ring, svr, batch, 2 * (int64_t)ring, h_kv, head_dim, es);
    if (overlaps(rkr, rvr) || overlaps(rkr, rkn) || overlaps(rkr, rvn) || overlaps(rvr, rkn) || overlaps(rvr, rvn))
      return fail(HCA_ERR_INVALID, "hca_append_kv: the rings overlap each other or the new rows");
    if (closes) {
      const Range rkc = extent(kc, skc, batch, n_blocks, h_kv, head_dim, es);
      const Range rvc = extent(vc, svc, batch, n_blocks, h_kv, head_dim, es);
      if (overlaps(rkc, rvc) || overlaps(rkc, rkr) || overlaps(rkc, rvr) || overlaps(rvc, rkr) || overlaps(rvc, rvr))
        return fail(HCA_ERR_INVALID, "hca_append_kv: kc/vc overlap each other or the rings");
    }
  }
  hipStream_t st = (hipStream_t)stream;
  const int idt = dt == HCA_DTYPE_BF16 ? 1 : 0;
  hipError_t e = hca::launch_ring_write(idt, k_new, ls(skn), v_new, ls(svn), k_ring, ls(skr), v_ring, ls(svr), ring, t,
                                        batch, h_kv, head_dim, st);
  if (e != hipSuccess) return hip_fail(e, "hca_append_kv ring write");
  if (closes) {
    // rows t+1-block .. t are contiguous in the mirrored ring from row (t+1-block) mod ring
    const int64_t start = (t + 1 - block) % ring;
    const char* kb = (const char*)k_ring + start * skr.seq * (int64_t)es;
    const char* vb = (const char*)v_ring + start * svr.seq * (int64_t)es;
    char* kcj = (char*)kc + j * skc.seq * (int64_t)es;
    char* vcj = (char*)vc + j * svc.seq * (int64_t)es;
    e = hca::launch_compress(idt, kb, ls(skr), w_k, kcj, ls(skc), vb, ls(svr), w_v, vcj, ls(svc), batch, block, h_kv,
                             head_dim, block, st);
    if (e != hipSuccess) return hip_fail(e, "hca_append_kv block compression");
  }
  return HCA_OK;
}


size_t hca_attn_fwd_workspace_size(int batch, int seqlen_q, int h_q, int h_kv, int head_dim, int n_blocks,
                                   int window) {
  if (batch <= 0 || seqlen_q != 1 || h_q <= 0 || h_kv <= 0 || h_q % h_kv || head_dim != 512 || window < 1 ||
      n_blocks < 0)
    return 0;
  return hca::decode512_workspace_bytes(batch, h_q, h_kv, n_blocks + window);
}

hca_status_t hca_attn_fwd(hca_dtype_t dt, const void* q, hca_strides_t sq, const void* k, hca_strides_t sk,
                          const void* v, hca_strides_t sv, const void* kc, hca_strides_t skc, const void* vc,
                          hca_strides_t svc, void* o, hca_strides_t so, float* lse, int batch, int seqlen_q,
                          int64_t q_pos0, int seqlen_kv, int64_t kv_pos0, int n_blocks, int h_q, int h_kv,
                          int head_dim, int block, int window, float scale, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (dt != HCA_DTYPE_F32 && dt != HCA_DTYPE_BF16) return fail(HCA_ERR_INVALID, "unknown dtype %d", (int)dt);
  if (batch <= 0 || seqlen_q <= 0 || seqlen_kv <= 0 || h_q <= 0 || h_kv <= 0 || head_dim <= 0)
    return fail(HCA_ERR_INVALID, "sizes must be positive");
  if (n_blocks < 0) return fail(HCA_ERR_INVALID, "n_blocks must be >= 0");
  if (h_q % h_kv) return fail(HCA_ERR_INVALID, "h_q (%d) must be a multiple of h_kv (%d)", h_q, h_kv);
  if (window < 1) return fail(HCA_ERR_INVALID, "window must be >= 1");
  if (block < 1) return fail(HCA_ERR_INVALID, "block must be >= 1");
  if (q_pos0 < 0 || kv_pos0 < 0) return fail(HCA_ERR_INVALID, "positions must be >= 0");
  if (q_pos0 + seqlen_q > kPosLimit || kv_pos0 + seqlen_kv > kPosLimit)
    return fail(HCA_ERR_UNSUPPORTED, "positions beyond 2^30 are not supported");
  if (!(scale == scale)) return fail(HCA_ERR_INVALID, "scale is NaN");
  const size_t es = elem_size(dt);
  HCA_TRY(check_tensor("q", q, sq, batch, seqlen_q, h_q, head_dim, es));
  HCA_TRY(check_tensor("k", k, sk, batch, seqlen_kv, h_kv, head_dim, es));
  HCA_TRY(check_tensor("v", v, sv, batch, seqlen_kv, h_kv, head_dim, es));
  HCA_TRY(check_tensor("kc", kc, skc, batch, n_blocks, h_kv, head_dim, es, n_blocks == 0));
  HCA_TRY(check_tensor("vc", vc, svc, batch, n_blocks, h_kv, head_dim, es, n_blocks == 0));
  HCA_TRY(check_tensor("o", o, so, batch, seqlen_q, h_q, head_dim, es));
  if (lse) HCA_TRY(check_flat("lse", lse, (__int128)batch * h_q * seqlen_q, 4, 4));
  // every query's window must be inside the raw K/V and its compressed entries inside kc/vc
  const int64_t t0 = q_pos0, t1 = q_pos0 + seqlen_q - 1;
  const int64_t lo0 = t0 - window + 1 > 0 ? t0 - window + 1 : 0;
  const int64_t lo1 = t1 - window + 1 > 0 ? t1 - window + 1 : 0;
  if (lo0 < kv_pos0 || t1 >= kv_pos0 + seqlen_kv)
    return fail(HCA_ERR_INVALID, "raw K/V [%lld, %lld) do not cover the windows [%lld, %lld]", (long long)kv_pos0,
                (long long)(kv_pos0 + seqlen_kv), (long long)lo0, (long long)t1);
  if (lo1 / block > n_blocks)
    return fail(HCA_ERR_INVALID, "queries need %lld compressed entries but n_blocks is %d", (long long)(lo1 / block),
                n_blocks);
  // outputs must not overlap inputs
  {
    const Range ro = extent(o, so, batch, seqlen_q, h_q, head_dim, es);
    const Range ins[3] = {extent(q, sq, batch, seqlen_q, h_q, head_dim, es),
                          extent(k, sk, batch, seqlen_kv, h_kv, head_dim, es),
                          extent(v, sv, batch, seqlen_kv, h_kv, head_dim, es)};
    for (const Range& r : ins)
      if (overlaps(ro, r)) return fail(HCA_ERR_INVALID, "o overlaps an input");
    if (n_blocks > 0 && (overlaps(ro, extent(kc, skc, batch, n_blocks, h_kv, head_dim, es)) ||
                         overlaps(ro, extent(vc, svc, batch, n_blocks, h_kv, head_dim, es))))
      return fail(HCA_ERR_INVALID, "o overlaps an input");
    if (lse) {
      const Range rl = flat_extent(lse, (int64_t)batch * h_q * seqlen_q, 4);
      if (overlaps(rl, ro) || overlaps(rl, ins[0]) || overlaps(rl, ins[1]) || overlaps(rl, ins[2]))
        return fail(HCA_ERR_INVALID, "lse overlaps another tensor");
    }
  }

  hca::AttnArgs a;
  a.dt = dt == HCA_DTYPE_BF16 ? 1 : 0;
  a.q = q; a.sq = ls(sq);
  a.k = k; a.sk = ls(sk);
  a.v = v; a.sv = ls(sv);
  a.kc = kc; a.skc = ls(skc);
  a.vc = vc; a.svc = ls(svc);
  a.o = o; a.so = ls(so);
  a.lse = lse;
  a.batch = batch; a.seqlen_q = seqlen_q; a.q_pos0 = q_pos0; a.seqlen_kv = seqlen_kv; a.kv_pos0 = kv_pos0;
  a.n_blocks = n_blocks; a.h_q = h_q; a.h_kv = h_kv; a.head_dim = head_dim; a.block = block; a.window = window;
  a.scale = scale;
  hipStream_t st = (hipStream_t)stream;

  if (dt == HCA_DTYPE_BF16 && head_dim == 512) {
    if (seqlen_q == 1) {
      const size_t need = hca::decode512_workspace_bytes(batch, h_q, h_kv, n_keys_of(q_pos0, window, block));
      if (!workspace || workspace_bytes < need)
        return fail(HCA_ERR_WORKSPACE, "decode needs a %zu-byte workspace (got %zu)", need, workspace_bytes);
      if (!aligned16(workspace)) return fail(HCA_ERR_INVALID, "workspace is not 16-byte aligned");
      hipError_t e = hca::launch_attn_decode512(a, workspace, st);
      if (e != hipSuccess) return hip_fail(e, "hca_attn_fwd decode launch");
      return HCA_OK;
    }
    hipError_t e = hca::launch_attn_prefill512(a, st);
    if (e != hipSuccess) return hip_fail(e, "hca_attn_fwd prefill launch");
    return HCA_OK;
  }
  if (hca::attn_f32mfma_supports(a.dt, head_dim)) {
    hipError_t e = hca::launch_attn_f32mfma(a, st);
    if (e != hipSuccess) return hip_fail(e, "hca_attn_fwd fp32 launch");
    return HCA_OK;
  }
  if (hca::attn_bf16mfma_supports(a.dt, head_dim)) {
    hipError_t e = hca::launch_attn_bf16mfma(a, st);
    if (e != hipSuccess) return hip_fail(e, "hca_attn_fwd bf16 launch");
    return HCA_OK;
  }
  // one-query-per-workgroup kernel: fp32 and bf16 with the remaining head sizes
  if (head_dim > 512 || (head_dim % (16 / (int)es)) != 0)
    return fail(HCA_ERR_UNSUPPORTED, "hca_attn_fwd: head_dim %d unsupported for this dtype", head_dim);
  if (n_keys_of(t1, window, block) > hca::kGenericMaxKeys)
    return fail(HCA_ERR_UNSUPPORTED, "hca_attn_fwd: more than %d keys per query needs bf16 with head_dim 512",
                hca::kGenericMaxKeys);
  hipError_t e = hca::launch_attn_generic(a, st);
  if (e != hipSuccess) return hip_fail(e, "hca_attn_fwd launch");
  return HCA_OK;
}

// ---------------------------------------------------------------------------
// hca_attn_fwd_noalloc: hca_attn_fwd with the decode kernel's split partials in
// a fixed device array instead of a caller workspace.  The array is a
// file-scope __device__ object, so every GPU the library runs on holds its own
// copy from module load until the process ends; its device address is looked
// up once per device (with that device current) and only that address is ever
// passed to kernels.  No memory is allocated or freed by the call.
constexpr size_t kNoAllocScratchBytes = HCA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of `scratch` on the current device (looked up on first use).
hca_status_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hca_attn_fwd_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(HCA_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  ScratchSlot& s = g_scratch[dev];
  std::call_once(s.once, [&s] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
  if (s.err != hipSuccess) return hip_fail(s.err, "hca_attn_fwd_noalloc: hipGetSymbolAddress(scratch)");
  if (!s.ptr) return fail(HCA_ERR_HIP, "hca_attn_fwd_noalloc: scratch has no device address");
  *out = s.ptr;
  return HCA_OK;
}
}  // namespace

hca_status_t hca_attn_fwd_noalloc(hca_dtype_t dt, const void* q, hca_strides_t sq, const void* k, hca_strides_t sk,
                                  const void* v, hca_strides_t sv, const void* kc, hca_strides_t skc, const void* vc,
                                  hca_strides_t svc, void* o, hca_strides_t so, float* lse, int batch, int seqlen_q,
                                  int64_t q_pos0, int seqlen_kv, int64_t kv_pos0, int n_blocks, int h_q, int h_kv,
                                  int head_dim, int block, int window, float scale, void* stream) {
  // the scratch need is an upper bound from the sizes alone (0 for every path
  // but the bf16 / head_dim 512 decode); it is checked before anything else
  const size_t need = dt == HCA_DTYPE_BF16
                          ? hca_attn_fwd_workspace_size(batch, seqlen_q, h_q, h_kv, head_dim, n_blocks, window)
                          : 0;
  if (need > kNoAllocScratchBytes)
    return fail(HCA_ERR_WORKSPACE,
                "hca_attn_fwd_noalloc: these sizes need %zu bytes of scratch, beyond its fixed %zu bytes; "
                "use hca_attn_fwd with a workspace",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need) HCA_TRY(scratch_ptr(&ws));
  return hca_attn_fwd(dt, q, sq, k, sk, v, sv, kc, skc, vc, svc, o, so, lse, batch, seqlen_q, q_pos0, seqlen_kv,
                      kv_pos0, n_blocks, h_q, h_kv, head_dim, block, window, scale, ws,
                      need ? kNoAllocScratchBytes : 0, stream);
}

size_t dsa_index_topk_workspace_size(int batch, int seqlen, int topk) {
  if (batch <= 0 || seqlen <= 0 || topk <= 0) return 0;
  return hca::dsa_topk_workspace_bytes(batch, seqlen, topk);
}

hca_status_t dsa_index_topk(const float* q_idx, const float* k_idx, const float* w_idx, int32_t* idx, int batch,
                            int seqlen, int h_i, int d_i, int topk, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!q_idx || !k_idx || !w_idx || !idx) return fail(HCA_ERR_INVALID, "dsa_index_topk: NULL tensor");
  if (batch <= 0 || seqlen <= 0 || h_i <= 0 || d_i <= 0 || topk <= 0)
    return fail(HCA_ERR_INVALID, "dsa_index_topk: sizes must be positive");
  if (h_i > 8 || d_i % 16 || d_i > 128 || topk > 4096)
    return fail(HCA_ERR_UNSUPPORTED, "dsa_index_topk: needs h_i <= 8, d_i a multiple of 16 <= 128, topk <= 4096");
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w_idx) || !aligned16(idx))
    return fail(HCA_ERR_INVALID, "dsa_index_topk: tensors must be 16-byte aligned");
  if (h_i % 4) return fail(HCA_ERR_UNSUPPORTED, "dsa_index_topk: h_i must be a multiple of 4");
  if ((int64_t)batch * seqlen > kPosLimit)
    return fail(HCA_ERR_UNSUPPORTED, "dsa_index_topk: more than 2^30 positions over the batch");
  {
    const int64_t n = (int64_t)batch * seqlen;
    const Range ri = flat_extent(idx, n * topk, 4), rq = flat_extent(q_idx, n * h_i * d_i, 4);
    const Range rk = flat_extent(k_idx, n * d_i, 4), rw = flat_extent(w_idx, n * h_i, 4);
    if (overlaps(ri, rq) || overlaps(ri, rk) || overlaps(ri, rw))
      return fail(HCA_ERR_INVALID, "dsa_index_topk: idx overlaps an input");
  }
  const size_t need = hca::dsa_topk_workspace_bytes(batch, seqlen, topk);
  if (need && (!workspace || workspace_bytes < need))
    return fail(HCA_ERR_WORKSPACE, "dsa_index_topk needs a %zu-byte workspace (got %zu)", need, workspace_bytes);
  if (need && !aligned16(workspace)) return fail(HCA_ERR_INVALID, "workspace is not 16-byte aligned");
  hipError_t e = hca::launch_dsa_index_topk(q_idx, k_idx, w_idx, idx, batch, seqlen, h_i, d_i, topk, workspace,
                                            workspace_bytes, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "dsa_index_topk launch");
  return HCA_OK;
}

size_t hca_attn_bwd_workspace_size(hca_dtype_t dt, int batch, int seqlen_q, int64_t q_pos0, int n_blocks, int h_q,
                                   int h_kv, int head_dim, int block, int window) {
  if ((dt != HCA_DTYPE_F32 && dt != HCA_DTYPE_BF16) || batch <= 0 || seqlen_q <= 0 || h_q <= 0 || h_kv <= 0 ||
      head_dim <= 0 || n_blocks < 0 || block < 1 || window < 1 || q_pos0 < 0 || q_pos0 + seqlen_q > kPosLimit)
    return 0;
  return hca::hca_bwd_workspace_bytes(dt == HCA_DTYPE_BF16 ? 1 : 0, batch, seqlen_q, q_pos0, n_blocks, h_q, h_kv,
                                      head_dim, block, window);
}

hca_status_t hca_attn_bwd(hca_dtype_t dt, const void* q, hca_strides_t sq, const void* k, hca_strides_t sk,
                          const void* v, hca_strides_t sv, const void* kc, hca_strides_t skc, const void* vc,
                          hca_strides_t svc, const void* o, hca_strides_t so, const float* lse, const void* dout,
                          hca_strides_t sdo, float* dq, hca_strides_t sdq, float* dk, hca_strides_t sdk, float* dv,
                          hca_strides_t sdv, float* dkc, hca_strides_t sdkc, float* dvc, hca_strides_t sdvc,
                          int batch, int seqlen_q, int64_t q_pos0, int seqlen_kv, int64_t kv_pos0, int n_blocks,
                          int h_q, int h_kv, int head_dim, int block, int window, float scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return attn_bwd_impl("hca_attn_bwd", dt, q, sq, k, sk, v, sv, kc, skc, vc, svc, o, so, lse, dout, sdo, dq, sdq, dk,
                       sdk, dv, sdv, dkc, sdkc, dvc, sdvc, batch, seqlen_q, q_pos0, seqlen_kv, kv_pos0, n_blocks, h_q,
                       h_kv, head_dim, block, window, scale, workspace, workspace_bytes, stream, nullptr, nullptr,
                       nullptr, nullptr);
}

hca_status_t hca_attn_compress_bwd(hca_dtype_t dt, const void* q, hca_strides_t sq, const void* k, hca_strides_t sk,
                                   const void* v, hca_strides_t sv, const void* kc, hca_strides_t skc, const void* vc,
                                   hca_strides_t svc, const void* o, hca_strides_t so, const float* lse,
                                   const void* dout, hca_strides_t sdo, const float* w_k, const float* w_v, float* dq,
                                   hca_strides_t sdq, float* dk, hca_strides_t sdk, float* dv, hca_strides_t sdv,
                                   float* dkc, hca_strides_t sdkc, float* dvc, hca_strides_t sdvc, float* dw_k,
                                   float* dw_v, int batch, int seqlen, int n_blocks, int h_q, int h_kv, int head_dim,
                                   int block, int window, float scale, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (!w_k || !w_v || !dw_k || !dw_v)
    return fail(HCA_ERR_INVALID, "hca_attn_compress_bwd: weights or their gradients are NULL");
  if (((uintptr_t)w_k | (uintptr_t)w_v | (uintptr_t)dw_k | (uintptr_t)dw_v) & 3u)
    return fail(HCA_ERR_INVALID, "hca_attn_compress_bwd: weights must be 4-byte aligned");
  if (block >= 1 && n_blocks >= 0 && (int64_t)n_blocks * block > seqlen)
    return fail(HCA_ERR_INVALID, "hca_attn_compress_bwd: n_blocks * block exceeds seqlen");
  return attn_bwd_impl("hca_attn_compress_bwd", dt, q, sq, k, sk, v, sv, kc, skc, vc, svc, o, so, lse, dout, sdo, dq,
                       sdq, dk, sdk, dv, sdv, dkc, sdkc, dvc, sdvc, batch, seqlen, 0, seqlen, 0, n_blocks, h_q, h_kv,
                       head_dim, block, window, scale, workspace, workspace_bytes, stream, w_k, w_v, dw_k, dw_v);
}

hca_status_t hca_compress_kv_bwd(hca_dtype_t dt, const void* k, hca_strides_t sk, const void* v, hca_strides_t sv,
                                 const float* dkc, hca_strides_t sdkc, const float* dvc, hca_strides_t sdvc,
                                 const float* w_k, const float* w_v, float* dk, hca_strides_t sdk, float* dv,
                                 hca_strides_t sdv, float* dw_k, float* dw_v, int batch, int seqlen, int h_kv,
                                 int head_dim, int block, void* stream) {
  if (dt != HCA_DTYPE_F32 && dt != HCA_DTYPE_BF16) return fail(HCA_ERR_INVALID, "unknown dtype %d", (int)dt);
  if (batch <= 0 || seqlen <= 0 || h_kv <= 0 || head_dim <= 0 || block <= 0)
    return fail(HCA_ERR_INVALID, "hca_compress_kv_bwd: sizes must be positive");
  if (head_dim % 4 || head_dim > 512)
    return fail(HCA_ERR_UNSUPPORTED, "hca_compress_kv_bwd: head_dim must be a multiple of 4, at most 512");
  if (!w_k || !w_v || !dw_k || !dw_v) return fail(HCA_ERR_INVALID, "hca_compress_kv_bwd: weights or their gradients are NULL");
  const size_t es = elem_size(dt);
  const int nb = seqlen / block;
  HCA_TRY(check_tensor("k", k, sk, batch, seqlen, h_kv, head_dim, es));
  HCA_TRY(check_tensor("v", v, sv, batch, seqlen, h_kv, head_dim, es));
  HCA_TRY(check_tensor("dkc", dkc, sdkc, batch, nb, h_kv, head_dim, 4, nb == 0));
  HCA_TRY(check_tensor("dvc", dvc, sdvc, batch, nb, h_kv, head_dim, 4, nb == 0));
  HCA_TRY(check_tensor("dk", dk, sdk, batch, seqlen, h_kv, head_dim, 4));
  HCA_TRY(check_tensor("dv", dv, sdv, batch, seqlen, h_kv, head_dim, 4));
  HCA_TRY(check_flat("dw_k", dw_k, (__int128)h_kv * block, 4, 4));
  HCA_TRY(check_flat("dw_v", dw_v, (__int128)h_kv * block, 4, 4));
  {
    const Range rdk = extent(dk, sdk, batch, seqlen, h_kv, head_dim, 4), rdv = extent(dv, sdv, batch, seqlen, h_kv, head_dim, 4);
    const Range rw = flat_extent(dw_k, (int64_t)h_kv * block, 4), rw2 = flat_extent(dw_v, (int64_t)h_kv * block, 4);
    if (overlaps(rdk, rdv) || overlaps(rw, rw2) || overlaps(rdk, rw) || overlaps(rdk, rw2) || overlaps(rdv, rw) ||
        overlaps(rdv, rw2))
      return fail(HCA_ERR_INVALID, "hca_compress_kv_bwd: gradients overlap each other");
    if (nb > 0) {
      const Range rdkc = extent(dkc, sdkc, batch, nb, h_kv, head_dim, 4), rdvc = extent(dvc, sdvc, batch, nb, h_kv, head_dim, 4);
      if (overlaps(rdk, rdkc) || overlaps(rdk, rdvc) || overlaps(rdv, rdkc) || overlaps(rdv, rdvc))
        return fail(HCA_ERR_INVALID, "hca_compress_kv_bwd: dk/dv overlap dkc/dvc");
    }
  }
  hipError_t e = hca::launch_compress_bwd(dt == HCA_DTYPE_BF16 ? 1 : 0, k, ls(sk), v, ls(sv), dkc, ls(sdkc), dvc,
                                          ls(sdvc), w_k, w_v, dk, ls(sdk), dv, ls(sdv), dw_k, dw_v, batch, seqlen,
                                          h_kv, head_dim, block, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hca_compress_kv_bwd launch");
  return HCA_OK;
}

size_t dsa_sparse_attn_bwd_workspace_size(hca_dtype_t dt, int batch, int seqlen, int h_q, int h_kv, int d_qk, int d_v,
                                          int topk) {
  if ((dt != HCA_DTYPE_F32 && dt != HCA_DTYPE_BF16) || batch <= 0 || seqlen <= 0 || h_q <= 0 || h_kv <= 0 ||
      h_q % h_kv || d_qk <= 0 || d_v <= 0 || topk <= 0)
    return 0;
  return hca::dsa_bwd_workspace_bytes(dt == HCA_DTYPE_BF16 ? 1 : 0, batch, seqlen, h_q, h_kv, d_qk, d_v, topk);
}

hca_status_t dsa_sparse_attn_bwd(hca_dtype_t dt, const void* q, hca_strides_t sq, const void* k, hca_strides_t sk,
                                 const void* v, hca_strides_t sv, const int32_t* idx, const void* o, hca_strides_t so,
                                 const float* lse, const void* dout, hca_strides_t sdo, float* dq, hca_strides_t sdq,
                                 float* dk, hca_strides_t sdk, float* dv, hca_strides_t sdv, int batch, int seqlen,
                                 int h_q, int h_kv, int d_qk, int d_v, int topk, float scale, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (dt != HCA_DTYPE_F32 && dt != HCA_DTYPE_BF16) return fail(HCA_ERR_INVALID, "unknown dtype %d", (int)dt);
  if (batch <= 0 || seqlen <= 0 || h_q <= 0 || h_kv <= 0 || d_qk <= 0 || d_v <= 0 || topk <= 0)
    return fail(HCA_ERR_INVALID, "dsa_sparse_attn_bwd: sizes must be positive");
  if (h_q % h_kv) return fail(HCA_ERR_INVALID, "h_q must be a multiple of h_kv");
  if (d_qk > 512 || d_v > 512 || d_qk % 4 || d_v % 4 || topk > 4096)
    return fail(HCA_ERR_UNSUPPORTED, "dsa_sparse_attn_bwd: needs d_qk, d_v <= 512 (multiples of 4), topk <= 4096");
  HCA_TRY(check_flat("idx", idx, (__int128)batch * seqlen * topk, 4, 16));
  HCA_TRY(check_flat("lse", lse, (__int128)batch * h_q * seqlen, 4, 4));
  if (!(scale == scale)) return fail(HCA_ERR_INVALID, "scale is NaN");
  const size_t es = elem_size(dt);
  HCA_TRY(check_tensor("q", q, sq, batch, seqlen, h_q, d_qk, es));
  HCA_TRY(check_tensor("k", k, sk, batch, seqlen, h_kv, d_qk, es));
  HCA_TRY(check_tensor("v", v, sv, batch, seqlen, h_kv, d_v, es));
  HCA_TRY(check_tensor("o", o, so, batch, seqlen, h_q, d_v, es));
  HCA_TRY(check_tensor("dout", dout, sdo, batch, seqlen, h_q, d_v, es));
  HCA_TRY(check_tensor("dq", dq, sdq, batch, seqlen, h_q, d_qk, 4));
  HCA_TRY(check_tensor("dk", dk, sdk, batch, seqlen, h_kv, d_qk, 4));
  HCA_TRY(check_tensor("dv", dv, sdv, batch, seqlen, h_kv, d_v, 4));
  {
    const Range outs[3] = {extent(dq, sdq, batch, seqlen, h_q, d_qk, 4), extent(dk, sdk, batch, seqlen, h_kv, d_qk, 4),
                           extent(dv, sdv, batch, seqlen, h_kv, d_v, 4)};
    const Range ins[6] = {extent(q, sq, batch, seqlen, h_q, d_qk, es), extent(k, sk, batch, seqlen, h_kv, d_qk, es),
                          extent(v, sv, batch, seqlen, h_kv, d_v, es), extent(o, so, batch, seqlen, h_q, d_v, es),
                          extent(dout, sdo, batch, seqlen, h_q, d_v, es),
                          flat_extent(idx, (int64_t)batch * seqlen * topk, 4)};
    for (int x = 0; x < 3; ++x) {
      for (int y = 0; y < 6; ++y)
        if (overlaps(outs[x], ins[y])) return fail(HCA_ERR_INVALID, "dsa_sparse_attn_bwd: a gradient overlaps an input");
      for (int y = x + 1; y < 3; ++y)
        if (overlaps(outs[x], outs[y])) return fail(HCA_ERR_INVALID, "dsa_sparse_attn_bwd: gradients overlap each other");
    }
  }
  const size_t need =
      hca::dsa_bwd_workspace_bytes(dt == HCA_DTYPE_BF16 ? 1 : 0, batch, seqlen, h_q, h_kv, d_qk, d_v, topk);
  if (!workspace || workspace_bytes < need)
    return fail(HCA_ERR_WORKSPACE, "dsa_sparse_attn_bwd needs a %zu-byte workspace (got %zu)", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(HCA_ERR_INVALID, "workspace is not 16-byte aligned");
  hca::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout;
  a.sq = ls(sq); a.sk = ls(sk); a.sv = ls(sv); a.so = ls(so); a.sdo = ls(sdo);
  a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.sdq = ls(sdq); a.sdk = ls(sdk); a.sdv = ls(sdv);
  a.batch = batch; a.seqlen_q = seqlen; a.seqlen_kv = seqlen; a.h_q = h_q; a.h_kv = h_kv;
  a.d = d_qk; a.d_v = d_v; a.topk = topk; a.scale = scale; a.idx = idx;
  hipError_t e = hca::launch_dsa_attn_bwd(dt == HCA_DTYPE_BF16 ? 1 : 0, a, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "dsa_sparse_attn_bwd launch");
  return HCA_OK;
}

}  // extern "C"

namespace {
// Sparse attention of seqlen_q queries per sequence over n_kv key rows.
// A decode row (one query per sequence) runs as `parts` query rows of the
// sparse-attention kernel, each over a contiguous slice of the index row, so
// that about 256 workgroups (one per CU) share the work instead of one per 64
// heads of a sequence; slices hold at least 64 positions and divide topk.
int decode_parts(int batch, int h_q, int topk) {
  const int64_t wg = std::max<int64_t>(1, (int64_t)batch * (h_q / 64));
  int parts = (int)std::min<int64_t>(64, (256 + wg - 1) / wg);
  parts = std::min(parts, topk / 64);
  while (parts > 1 && topk % parts) --parts;
  return std::max(parts, 1);
}
size_t decode_out_bytes(int batch, int h_q, int parts) {
  return ((size_t)batch * parts * h_q * 256 * 2 + 255) / 256 * 256;
}
size_t decode_ws_bytes(int batch, int h_q, int topk) {
  const int parts = decode_parts(batch, h_q, topk);
  if (parts <= 1) return 0;
  return decode_out_bytes(batch, h_q, parts) + (size_t)batch * h_q * parts * sizeof(float);
}

hca_status_t sparse_attn(const char* name, hca_dtype_t dt, const void* q, hca_strides_t sq, const void* k,
                         hca_strides_t sk, const void* v, hca_strides_t sv, const int32_t* idx, void* o,
                         hca_strides_t so, float* lse, int batch, int seqlen_q, int n_kv, int h_q, int h_kv, int d_qk,
                         int d_v, int topk, float scale, void* stream, void* ws = nullptr, size_t ws_bytes = 0) {
  if (dt != HCA_DTYPE_F32 && dt != HCA_DTYPE_BF16) return fail(HCA_ERR_INVALID, "unknown dtype %d", (int)dt);
  if (batch <= 0 || seqlen_q <= 0 || n_kv <= 0 || h_q <= 0 || h_kv <= 0 || d_qk <= 0 || d_v <= 0 || topk <= 0)
    return fail(HCA_ERR_INVALID, "%s: sizes must be positive", name);
  if (h_q % h_kv) return fail(HCA_ERR_INVALID, "h_q must be a multiple of h_kv");
  HCA_TRY(check_flat("idx", idx, (__int128)batch * seqlen_q * topk, 4, 16));
  const size_t es = elem_size(dt);
  HCA_TRY(check_tensor("q", q, sq, batch, seqlen_q, h_q, d_qk, es));
  HCA_TRY(check_tensor("k", k, sk, batch, n_kv, h_kv, d_qk, es));
  HCA_TRY(check_tensor("v", v, sv, batch, n_kv, h_kv, d_v, es));
  HCA_TRY(check_tensor("o", o, so, batch, seqlen_q, h_q, d_v, es));
  if (lse) HCA_TRY(check_flat("lse", lse, (__int128)batch * h_q * seqlen_q, 4, 4));
  if (dt != HCA_DTYPE_BF16 || d_qk != 256 || d_v != 256 || (h_q / h_kv) % 64 || topk > 4096)
    return fail(HCA_ERR_UNSUPPORTED, "%s: needs bf16, d_qk = d_v = 256, h_q/h_kv a multiple of 64, topk <= 4096",
                name);
  {
    const Range ro = extent(o, so, batch, seqlen_q, h_q, d_v, es);
    if (overlaps(ro, extent(q, sq, batch, seqlen_q, h_q, d_qk, es)) ||
        overlaps(ro, extent(k, sk, batch, n_kv, h_kv, d_qk, es)) ||
        overlaps(ro, extent(v, sv, batch, n_kv, h_kv, d_v, es)) ||
        overlaps(ro, flat_extent(idx, (int64_t)batch * seqlen_q * topk, 4)) ||
        (lse && overlaps(ro, flat_extent(lse, (int64_t)batch * h_q * seqlen_q, 4))))
      return fail(HCA_ERR_INVALID, "o overlaps an input");
  }
  const int parts = ws ? decode_parts(batch, h_q, topk) : 1;
  if (seqlen_q == 1 && parts > 1) {
    const size_t need = decode_ws_bytes(batch, h_q, topk);
    if (ws_bytes < need)
      return fail(HCA_ERR_WORKSPACE, "%s needs a %zu-byte workspace (got %zu)", name, need, ws_bytes);
    if (!aligned16(ws)) return fail(HCA_ERR_INVALID, "workspace is not 16-byte aligned");
    const Range rw = flat_extent(ws, (int64_t)need, 1);
    if (overlaps(rw, extent(o, so, batch, 1, h_q, d_v, es)) ||
        overlaps(rw, extent(q, sq, batch, 1, h_q, d_qk, es)) ||
        overlaps(rw, extent(k, sk, batch, n_kv, h_kv, d_qk, es)) ||
        overlaps(rw, extent(v, sv, batch, n_kv, h_kv, d_v, es)) ||
        overlaps(rw, flat_extent(idx, (int64_t)batch * topk, 4)) ||
        (lse && overlaps(rw, flat_extent(lse, (int64_t)batch * h_q, 4))))
      return fail(HCA_ERR_INVALID, "%s: workspace overlaps a tensor", name);
    // part i of sequence b is query row i over idx[b, i*topk/parts ..): q row
    // stride 0, the index row read as parts rows of topk/parts
    hca::LStrides sqp = ls(sq);
    sqp.s = 0;
    const hca::LStrides sop{(int64_t)parts * h_q * 256, (int64_t)h_q * 256, 256};
    float* lp = (float*)((char*)ws + decode_out_bytes(batch, h_q, parts));
    hipError_t e = hca::launch_dsa_sparse_attn256(q, sqp, k, ls(sk), v, ls(sv), idx, ws, sop, lp, batch, parts, n_kv,
                                                  h_q, h_kv, topk / parts, scale, (hipStream_t)stream);
    if (e == hipSuccess)
      e = hca::launch_dsa_decode_combine256(ws, lp, parts, o, ls(so), lse, batch, h_q, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, name);
    return HCA_OK;
  }
  hipError_t e = hca::launch_dsa_sparse_attn256(q, ls(sq), k, ls(sk), v, ls(sv), idx, o, ls(so), lse, batch, seqlen_q,
                                                n_kv, h_q, h_kv, topk, scale, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, name);
  return HCA_OK;
}
}  // namespace

extern "C" {

hca_status_t dsa_sparse_attn_fwd(hca_dtype_t dt, const void* q, hca_strides_t sq, const void* k, hca_strides_t sk,
                                 const void* v, hca_strides_t sv, const int32_t* idx, void* o, hca_strides_t so,
                                 float* lse, int batch, int seqlen, int h_q, int h_kv, int d_qk, int d_v, int topk,
                                 float scale, void* stream) {
  return sparse_attn("dsa_sparse_attn_fwd", dt, q, sq, k, sk, v, sv, idx, o, so, lse, batch, seqlen, seqlen, h_q,
                     h_kv, d_qk, d_v, topk, scale, stream);
}

size_t dsa_sparse_attn_decode_workspace_size(int batch, int h_q, int topk) {
  if (batch <= 0 || h_q <= 0 || topk <= 0) return 0;
  return decode_ws_bytes(batch, h_q, topk);
}

hca_status_t dsa_sparse_attn_decode(hca_dtype_t dt, const void* q, hca_strides_t sq, const void* k, hca_strides_t sk,
                                    const void* v, hca_strides_t sv, const int32_t* idx, void* o, hca_strides_t so,
                                    float* lse, int batch, int n_keys, int h_q, int h_kv, int d_qk, int d_v, int topk,
                                    float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_attn("dsa_sparse_attn_decode", dt, q, sq, k, sk, v, sv, idx, o, so, lse, batch, 1, n_keys, h_q, h_kv,
                     d_qk, d_v, topk, scale, stream, workspace, workspace_bytes);
}

size_t csa_index_topk_workspace_size(int batch, int seqlen, int n_entries, int topk) {
  if (batch <= 0 || seqlen <= 0 || n_entries <= 0 || topk <= 0) return 0;
  return hca::csa_topk_workspace_bytes(batch, seqlen, n_entries, topk);
}

hca_status_t csa_index_topk(const float* q_idx, const float* k_idx, const float* w_idx, int32_t* idx, int batch,
                            int seqlen, int n_entries, int block, int h_i, int d_i, int topk, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!q_idx || !k_idx || !w_idx || !idx) return fail(HCA_ERR_INVALID, "csa_index_topk: NULL tensor");
  if (batch <= 0 || seqlen <= 0 || n_entries <= 0 || block <= 0 || h_i <= 0 || d_i <= 0 || topk <= 0)
    return fail(HCA_ERR_INVALID, "csa_index_topk: sizes must be positive");
  if (seqlen / block > n_entries)
    return fail(HCA_ERR_INVALID, "csa_index_topk: the last query needs %d entries, %d given", seqlen / block,
                n_entries);
  if ((int64_t)seqlen > kPosLimit)
    return fail(HCA_ERR_UNSUPPORTED, "csa_index_topk: positions beyond 2^30 are not supported");
  if (h_i > 8 || h_i % 4 || d_i % 16 || d_i > 128 || topk > 4096)
    return fail(HCA_ERR_UNSUPPORTED,
                "csa_index_topk: needs h_i 4 or 8, d_i a multiple of 16 <= 128, topk <= 4096");
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w_idx) || !aligned16(idx))
    return fail(HCA_ERR_INVALID, "csa_index_topk: tensors must be 16-byte aligned");
  if ((int64_t)batch * seqlen > kPosLimit || (int64_t)batch * n_entries > kPosLimit)
    return fail(HCA_ERR_UNSUPPORTED, "csa_index_topk: more than 2^30 positions over the batch");
  {
    const int64_t n = (int64_t)batch * seqlen;
    const Range ri = flat_extent(idx, n * topk, 4), rq = flat_extent(q_idx, n * h_i * d_i, 4);
    const Range rk = flat_extent(k_idx, (int64_t)batch * n_entries * d_i, 4), rw = flat_extent(w_idx, n * h_i, 4);
    if (overlaps(ri, rq) || overlaps(ri, rk) || overlaps(ri, rw))
      return fail(HCA_ERR_INVALID, "csa_index_topk: idx overlaps an input");
  }
  const size_t need = hca::csa_topk_workspace_bytes(batch, seqlen, n_entries, topk);
  if (!workspace || workspace_bytes < need)
    return fail(HCA_ERR_WORKSPACE, "csa_index_topk needs a %zu-byte workspace (got %zu)", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(HCA_ERR_INVALID, "workspace is not 16-byte aligned");
  hipError_t e = hca::launch_csa_index_topk(q_idx, k_idx, w_idx, idx, batch, seqlen, n_entries, block, h_i, d_i,
                                            topk, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "csa_index_topk launch");
  return HCA_OK;
}

hca_status_t csa_sparse_attn_fwd(hca_dtype_t dt, const void* q, hca_strides_t sq, const void* kc, hca_strides_t skc,
                                 const void* vc, hca_strides_t svc, const int32_t* idx, void* o, hca_strides_t so,
                                 float* lse, int batch, int seqlen, int n_entries, int h_q, int h_kv, int d_qk,
                                 int d_v, int topk, float scale, void* stream) {
  return sparse_attn("csa_sparse_attn_fwd", dt, q, sq, kc, skc, vc, svc, idx, o, so, lse, batch, seqlen, n_entries,
                     h_q, h_kv, d_qk, d_v, topk, scale, stream);
}

hca_status_t attn_output_epilogue(hca_dtype_t dt, const void* o, hca_strides_t so, const void* c, hca_strides_t sc,
                                  const void* w_g, const float* u, const float* v, void* y, hca_strides_t sy,
                                  int batch, int seqlen, int h, int d_v, int d_c, int r, void* stream) {
  if (dt != HCA_DTYPE_BF16) return fail(HCA_ERR_UNSUPPORTED, "attn_output_epilogue: bf16 only");
  if (batch <= 0 || seqlen <= 0 || h <= 0 || d_v <= 0 || d_c <= 0 || r <= 0)
    return fail(HCA_ERR_INVALID, "attn_output_epilogue: sizes must be positive");
  if (!(h == 8 || h == 16 || h == 32 || h == 64) || r > 16 || d_c % 32 || d_v % (256 / h))
    return fail(HCA_ERR_UNSUPPORTED,
                "attn_output_epilogue: needs h in {8, 16, 32, 64}, r <= 16, d_c a multiple of 32, "
                "d_v a multiple of 256 / h");
  if ((int64_t)batch * seqlen > kPosLimit) return fail(HCA_ERR_UNSUPPORTED, "attn_output_epilogue: too many tokens");
  HCA_TRY(check_flat("w_g", w_g, (__int128)h * d_v * d_c, 2, 16));
  HCA_TRY(check_flat("u", u, (__int128)h * r, 4, 4));
  HCA_TRY(check_flat("v", v, (__int128)h * r, 4, 4));
  HCA_TRY(check_tensor("o", o, so, batch, seqlen, h, d_v, 2));
  HCA_TRY(check_tensor("c", c, sc, batch, seqlen, 1, d_c, 2));
  HCA_TRY(check_tensor("y", y, sy, batch, seqlen, h, d_v, 2));
  {
    const Range ry = extent(y, sy, batch, seqlen, h, d_v, 2);
    if (overlaps(ry, extent(o, so, batch, seqlen, h, d_v, 2)) || overlaps(ry, extent(c, sc, batch, seqlen, 1, d_c, 2)) ||
        overlaps(ry, flat_extent(w_g, (int64_t)h * d_v * d_c, 2)) || overlaps(ry, flat_extent(u, (int64_t)h * r, 4)) ||
        overlaps(ry, flat_extent(v, (int64_t)h * r, 4)))
      return fail(HCA_ERR_INVALID, "attn_output_epilogue: y overlaps an input");
  }
  hipError_t e = hca::launch_attn_output_epilogue(o, ls(so), c, sc.batch, sc.seq, w_g, u, v, y, ls(sy), batch, seqlen,
                                                  h, d_v, d_c, r, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attn_output_epilogue launch");
  return HCA_OK;
}

size_t dsa_index_topk_decode_workspace_size(int batch, int n_keys, int topk) {
  if (batch <= 0 || n_keys <= 0 || topk <= 0) return 0;
  return hca::dsa_topk_decode_workspace_bytes(batch, n_keys, topk);
}

hca_status_t dsa_index_topk_decode(const float* q_idx, const float* k_idx, const float* w_idx, int32_t* idx, int batch,
                                   int n_keys, int h_i, int d_i, int topk, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (!q_idx || !k_idx || !w_idx || !idx) return fail(HCA_ERR_INVALID, "dsa_index_topk_decode: NULL tensor");
  if (batch <= 0 || n_keys <= 0 || h_i <= 0 || d_i <= 0 || topk <= 0)
    return fail(HCA_ERR_INVALID, "dsa_index_topk_decode: sizes must be positive");
  if ((h_i != 4 && h_i != 8) || d_i % 16 || d_i > 128 || topk > 4096)
    return fail(HCA_ERR_UNSUPPORTED, "dsa_index_topk_decode: needs h_i in {4, 8}, d_i a multiple of 16 <= 128, "
                                     "topk <= 4096");
  if (n_keys >= (1 << 30)) return fail(HCA_ERR_UNSUPPORTED, "dsa_index_topk_decode: n_keys must be below 2^30");
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w_idx) || !aligned16(idx))
    return fail(HCA_ERR_INVALID, "dsa_index_topk_decode: tensors must be 16-byte aligned");
  if ((int64_t)batch * n_keys > kPosLimit)
    return fail(HCA_ERR_UNSUPPORTED, "dsa_index_topk_decode: more than 2^30 keys over the batch");
  {
    const Range ri = flat_extent(idx, (int64_t)batch * topk, 4), rq = flat_extent(q_idx, (int64_t)batch * h_i * d_i, 4);
    const Range rk = flat_extent(k_idx, (int64_t)batch * n_keys * d_i, 4), rw = flat_extent(w_idx, (int64_t)batch * h_i, 4);
    if (overlaps(ri, rq) || overlaps(ri, rk) || overlaps(ri, rw))
      return fail(HCA_ERR_INVALID, "dsa_index_topk_decode: idx overlaps an input");
  }
  const size_t need = hca::dsa_topk_decode_workspace_bytes(batch, n_keys, topk);
  if (!workspace || workspace_bytes < need)
    return fail(HCA_ERR_WORKSPACE, "dsa_index_topk_decode needs a %zu-byte workspace (got %zu)", need,
                workspace_bytes);
  if (!aligned16(workspace)) return fail(HCA_ERR_INVALID, "workspace is not 16-byte aligned");
  hipError_t e = hca::launch_dsa_index_topk_decode(q_idx, k_idx, w_idx, idx, batch, n_keys, h_i, d_i, topk, workspace,
                                                   (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "dsa_index_topk_decode launch");
  return HCA_OK;
}

}  // extern "C"
