// Drives every entry point of the C-ABI layer through its argument checks and
// its dispatch, for the host-side AddressSanitizer / UndefinedBehaviorSanitizer
// build: the kernel launchers are recording stubs, so no tensor is ever read or
// written; "device" pointers are 256-byte aligned, non-overlapping slices of a
// host arena sized like the tensors they stand for.  Prints "ALL OK" when every
// status is the expected one and every valid call reached a launcher.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/hca.h"

extern int g_launches;

namespace {
std::vector<unsigned char> g_arena(size_t(96) << 20);
size_t g_used = 0;
int g_fail = 0, g_checks = 0;

// A fresh slice of `bytes` bytes.
void* A(size_t bytes) {
  unsigned char* base = g_arena.data();
  size_t off = (g_used + 255) & ~size_t(255);
  if (off + bytes > g_arena.size()) {
    std::printf("FAIL arena exhausted\n");
    ++g_fail;
    return base;
  }
  g_used = off + bytes;
  return base + off;
}
template <class T>
T* AT(size_t n) { return static_cast<T*>(A(n * sizeof(T))); }

hca_strides_t C(int s, int h, int d) {  // contiguous [b, s, h, d]
  return hca_strides_t{int64_t(s) * h * d, int64_t(h) * d, d};
}

void expect(const char* what, hca_status_t got, hca_status_t want, int launches_before = -1) {
  ++g_checks;
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d (%s)\n", what, (int)got, (int)want, hca_last_error());
    ++g_fail;
    return;
  }
  if (want != HCA_OK && std::strlen(hca_last_error()) == 0) {
    std::printf("FAIL %s: no error message\n", what);
    ++g_fail;
  }
  if (launches_before >= 0) {
    const bool launched = g_launches > launches_before;
    if (launched != (want == HCA_OK)) {
      std::printf("FAIL %s: %s\n", what, launched ? "launched after an error" : "valid call launched nothing");
      ++g_fail;
    }
  }
}
#define EXPECT(what, call, want)            \
  do {                                      \
    const int _n = g_launches;              \
    expect(what, (call), (want), _n);       \
  } while (0)
}  // namespace

int main() {
  const hca_dtype_t BF = HCA_DTYPE_BF16, F32 = HCA_DTYPE_F32;
  if (hca_abi_version() != 1) { std::printf("FAIL version\n"); ++g_fail; }

  // ---- hca_compress_kv: [1, 64, 1, 512] bf16 -> 16 blocks of 4
  {
    const int S = 64, H = 1, D = 512, blk = 4, nb = S / blk;
    void* k = A(size_t(S) * H * D * 2); void* v = A(size_t(S) * H * D * 2);
    float* wk = AT<float>(H * blk); float* wv = AT<float>(H * blk);
    void* kc = A(size_t(nb) * H * D * 2); void* vc = A(size_t(nb) * H * D * 2);
    const hca_strides_t s = C(S, H, D), sc = C(nb, H, D);
    EXPECT("compress ok", hca_compress_kv(BF, k, s, v, s, wk, wv, kc, sc, vc, sc, 1, S, H, D, blk, nullptr), HCA_OK);
    EXPECT("compress f32 ok", hca_compress_kv(F32, k, C(S / 2, H, D), v, C(S / 2, H, D), wk, wv, kc, C(nb / 2, H, D),
                                              vc, C(nb / 2, H, D), 1, S / 2, H, D, blk, nullptr), HCA_OK);
    expect("compress short", hca_compress_kv(BF, k, s, v, s, wk, wv, nullptr, sc, nullptr, sc, 1, 3, H, D, blk, nullptr),
           HCA_OK);  // no complete block: nothing to launch, and no error
    EXPECT("compress null k", hca_compress_kv(BF, nullptr, s, v, s, wk, wv, kc, sc, vc, sc, 1, S, H, D, blk, nullptr),
           HCA_ERR_INVALID);
    EXPECT("compress dtype", hca_compress_kv((hca_dtype_t)7, k, s, v, s, wk, wv, kc, sc, vc, sc, 1, S, H, D, blk, nullptr),
           HCA_ERR_INVALID);
    EXPECT("compress block 0", hca_compress_kv(BF, k, s, v, s, wk, wv, kc, sc, vc, sc, 1, S, H, D, 0, nullptr),
           HCA_ERR_INVALID);
    EXPECT("compress head_dim", hca_compress_kv(BF, k, s, v, s, wk, wv, kc, sc, vc, sc, 1, S, H, 96, blk, nullptr),
           HCA_ERR_UNSUPPORTED);
    EXPECT("compress misaligned", hca_compress_kv(BF, (char*)k + 2, s, v, s, wk, wv, kc, sc, vc, sc, 1, S, H, D, blk,
                                                  nullptr), HCA_ERR_INVALID);
    EXPECT("compress stride", hca_compress_kv(BF, k, hca_strides_t{S * D, D + 1, D}, v, s, wk, wv, kc, sc, vc, sc, 1, S,
                                              H, D, blk, nullptr), HCA_ERR_INVALID);
    EXPECT("compress alias", hca_compress_kv(BF, k, s, v, s, wk, wv, k, sc, vc, sc, 1, S, H, D, blk, nullptr),
           HCA_ERR_INVALID);
    EXPECT("compress null w", hca_compress_kv(BF, k, s, v, s, nullptr, wv, kc, sc, vc, sc, 1, S, H, D, blk, nullptr),
           HCA_ERR_INVALID);
    // the largest sizes: the span arithmetic must not overflow (UBSan checks it) and the call is refused
    const hca_strides_t big{int64_t(1) << 40, int64_t(1) << 20, 512};
    EXPECT("compress huge strides", hca_compress_kv(BF, k, big, v, big, wk, wv, kc, big, vc, big, 2147483647,
                                                    2147483647, 1, D, 2147483647, nullptr), HCA_ERR_INVALID);
    const hca_strides_t wrap{int64_t(1) << 52, 512, 512};
    EXPECT("compress wraps", hca_compress_kv(BF, k, wrap, v, s, wk, wv, kc, sc, vc, sc, 64, S, H, D, blk, nullptr),
           HCA_ERR_INVALID);
  }

  // ---- hca_append_kv: ring of 8 rows mirrored, block 4
  {
    const int B = 2, H = 1, D = 512, blk = 4, ring = 8, nb = 16;
    void* kn = A(size_t(B) * H * D * 2); void* vn = A(size_t(B) * H * D * 2);
    void* kr = A(size_t(B) * 2 * ring * H * D * 2); void* vr = A(size_t(B) * 2 * ring * H * D * 2);
    float* wk = AT<float>(H * blk); float* wv = AT<float>(H * blk);
    void* kc = A(size_t(B) * nb * H * D * 2); void* vc = A(size_t(B) * nb * H * D * 2);
    const hca_strides_t sn = C(1, H, D), sr = C(2 * ring, H, D), sc = C(nb, H, D);
    EXPECT("append no close", hca_append_kv(BF, kn, sn, vn, sn, kr, sr, vr, sr, ring, wk, wv, nullptr, sc, nullptr, sc,
                                            nb, 5, B, H, D, blk, nullptr), HCA_OK);
    EXPECT("append close", hca_append_kv(BF, kn, sn, vn, sn, kr, sr, vr, sr, ring, wk, wv, kc, sc, vc, sc, nb, 63, B, H,
                                         D, blk, nullptr), HCA_OK);
    EXPECT("append past kc", hca_append_kv(BF, kn, sn, vn, sn, kr, sr, vr, sr, ring, wk, wv, kc, sc, vc, sc, nb, 67, B,
                                           H, D, blk, nullptr), HCA_ERR_INVALID);
    EXPECT("append ring < block", hca_append_kv(BF, kn, sn, vn, sn, kr, sr, vr, sr, 2, wk, wv, kc, sc, vc, sc, nb, 3, B,
                                                H, D, blk, nullptr), HCA_ERR_INVALID);
    EXPECT("append negative t", hca_append_kv(BF, kn, sn, vn, sn, kr, sr, vr, sr, ring, wk, wv, kc, sc, vc, sc, nb, -1,
                                              B, H, D, blk, nullptr), HCA_ERR_INVALID);
    EXPECT("append huge t", hca_append_kv(BF, kn, sn, vn, sn, kr, sr, vr, sr, ring, wk, wv, kc, sc, vc, sc, nb,
                                          int64_t(1) << 40, B, H, D, blk, nullptr), HCA_ERR_UNSUPPORTED);
    EXPECT("append rings alias", hca_append_kv(BF, kn, sn, vn, sn, kr, sr, kr, sr, ring, wk, wv, kc, sc, vc, sc, nb, 5,
                                               B, H, D, blk, nullptr), HCA_ERR_INVALID);
    EXPECT("append close no w", hca_append_kv(BF, kn, sn, vn, sn, kr, sr, vr, sr, ring, nullptr, wv, kc, sc, vc, sc, nb,
                                              63, B, H, D, blk, nullptr), HCA_ERR_INVALID);
  }

  // ---- hca_attn_fwd: prefill (bf16 512), generic (fp32), decode with a workspace, and its errors
  {
    const int B = 1, S = 64, Hq = 4, Hkv = 1, D = 512, blk = 4, W = 16, nb = S / blk;
    void* q = A(size_t(B) * S * Hq * D * 4); void* k = A(size_t(B) * S * Hkv * D * 4);
    void* v = A(size_t(B) * S * Hkv * D * 4);
    void* kc = A(size_t(B) * nb * Hkv * D * 4); void* vc = A(size_t(B) * nb * Hkv * D * 4);
    void* o = A(size_t(B) * S * Hq * D * 4); float* lse = AT<float>(size_t(B) * Hq * S);
    const hca_strides_t sq = C(S, Hq, D), skv = C(S, Hkv, D), sc = C(nb, Hkv, D);
    auto fwd = [&](hca_dtype_t dt, int seqlen_q, int64_t q_pos0, int seqlen_kv, int64_t kv_pos0, int n_blocks,
                   int head_dim, int window, float scale, void* ws, size_t wsb, void* out = nullptr,
                   float* l = nullptr) {
      return hca_attn_fwd(dt, q, sq, k, skv, v, skv, kc, sc, vc, sc, out ? out : o, sq, l ? l : lse, B, seqlen_q,
                          q_pos0, seqlen_kv, kv_pos0, n_blocks, Hq, Hkv, head_dim, blk, window, scale, ws, wsb,
                          nullptr);
    };
    EXPECT("fwd prefill", fwd(BF, S, 0, S, 0, nb, D, W, 0.04f, nullptr, 0), HCA_OK);
    EXPECT("fwd generic f32", fwd(F32, S, 0, S, 0, nb, D, W, 0.04f, nullptr, 0), HCA_OK);
    EXPECT("fwd generic bf16 128", fwd(BF, S, 0, S, 0, nb, 128, W, 0.04f, nullptr, 0), HCA_OK);
    EXPECT("fwd no lse", hca_attn_fwd(BF, q, sq, k, skv, v, skv, kc, sc, vc, sc, o, sq, nullptr, B, S, 0, S, 0, nb, Hq,
                                      Hkv, D, blk, W, 0.04f, nullptr, 0, nullptr), HCA_OK);
    // decode: query at position 63 over raw rows 48..63 and 12 compressed entries
    const size_t ws = hca_attn_fwd_workspace_size(B, 1, Hq, Hkv, D, nb, W);
    if (ws == 0) { std::printf("FAIL decode workspace size is 0\n"); ++g_fail; }
    void* wsp = A(ws);
    EXPECT("fwd decode", fwd(BF, 1, 63, W, 48, 12, D, W, 0.04f, wsp, ws), HCA_OK);
    EXPECT("fwd decode no ws", fwd(BF, 1, 63, W, 48, 12, D, W, 0.04f, nullptr, 0), HCA_ERR_WORKSPACE);
    EXPECT("fwd decode short ws", fwd(BF, 1, 63, W, 48, 12, D, W, 0.04f, wsp, 16), HCA_ERR_WORKSPACE);
    EXPECT("fwd decode misaligned ws", fwd(BF, 1, 63, W, 48, 12, D, W, 0.04f, (char*)wsp + 8, ws), HCA_ERR_INVALID);
    EXPECT("fwd window not covered", fwd(BF, 1, 63, W - 1, 49, 12, D, W, 0.04f, wsp, ws), HCA_ERR_INVALID);
    EXPECT("fwd entries missing", fwd(BF, 1, 63, W, 48, 11, D, W, 0.04f, wsp, ws), HCA_ERR_INVALID);
    EXPECT("fwd nan scale", fwd(BF, S, 0, S, 0, nb, D, W, std::nanf(""), nullptr, 0), HCA_ERR_INVALID);
    EXPECT("fwd o aliases q", fwd(BF, S, 0, S, 0, nb, D, W, 0.04f, nullptr, 0, q), HCA_ERR_INVALID);
    EXPECT("fwd lse aliases k", fwd(BF, S, 0, S, 0, nb, D, W, 0.04f, nullptr, 0, nullptr, (float*)k), HCA_ERR_INVALID);
    EXPECT("fwd lse misaligned", fwd(BF, S, 0, S, 0, nb, D, W, 0.04f, nullptr, 0, nullptr, (float*)((char*)lse + 2)),
           HCA_ERR_INVALID);
    EXPECT("fwd head_dim 100", fwd(BF, S, 0, S, 0, nb, 100, W, 0.04f, nullptr, 0), HCA_ERR_UNSUPPORTED);
    EXPECT("fwd huge position", fwd(BF, S, int64_t(1) << 31, S, int64_t(1) << 31, nb, D, W, 0.04f, nullptr, 0),
           HCA_ERR_UNSUPPORTED);
    EXPECT("fwd heads", hca_attn_fwd(BF, q, sq, k, skv, v, skv, kc, sc, vc, sc, o, sq, lse, B, S, 0, S, 0, nb, 3, 2, D,
                                     blk, W, 0.04f, nullptr, 0, nullptr), HCA_ERR_INVALID);
    // the variant without allocation: prefill needs no scratch; oversize decodes are refused before any HIP call
    EXPECT("fwd noalloc prefill", hca_attn_fwd_noalloc(BF, q, sq, k, skv, v, skv, kc, sc, vc, sc, o, sq, lse, B, S, 0, S,
                                                       0, nb, Hq, Hkv, D, blk, W, 0.04f, nullptr), HCA_OK);
    EXPECT("fwd noalloc oversize", hca_attn_fwd_noalloc(BF, q, sq, k, skv, v, skv, kc, sc, vc, sc, o, sq, lse, 100000,
                                                        1, 63, W, 48, 2000000, 64, 1, D, blk, W, 0.04f, nullptr),
           HCA_ERR_WORKSPACE);
  }

  // ---- DSA indexer + top-k (prefill and decode)
  {
    const int B = 1, S = 128, hi = 4, di = 64, K = 16;
    float* qI = AT<float>(size_t(B) * S * hi * di); float* kI = AT<float>(size_t(B) * S * di);
    float* w = AT<float>(size_t(B) * S * hi); int32_t* idx = AT<int32_t>(size_t(B) * S * K);
    const size_t ws = dsa_index_topk_workspace_size(B, S, K);
    void* wsp = A(ws ? ws : 16);
    EXPECT("topk ok", dsa_index_topk(qI, kI, w, idx, B, S, hi, di, K, wsp, ws, nullptr), HCA_OK);
    if (ws) EXPECT("topk no ws", dsa_index_topk(qI, kI, w, idx, B, S, hi, di, K, nullptr, 0, nullptr), HCA_ERR_WORKSPACE);
    EXPECT("topk d_i", dsa_index_topk(qI, kI, w, idx, B, S, hi, 60, K, wsp, ws, nullptr), HCA_ERR_UNSUPPORTED);
    EXPECT("topk h_i", dsa_index_topk(qI, kI, w, idx, B, S, 3, di, K, wsp, ws, nullptr), HCA_ERR_UNSUPPORTED);
    EXPECT("topk k", dsa_index_topk(qI, kI, w, idx, B, S, hi, di, 5000, wsp, ws, nullptr), HCA_ERR_UNSUPPORTED);
    EXPECT("topk null", dsa_index_topk(qI, nullptr, w, idx, B, S, hi, di, K, wsp, ws, nullptr), HCA_ERR_INVALID);
    EXPECT("topk idx aliases", dsa_index_topk(qI, kI, w, (int32_t*)qI, B, S, hi, di, K, wsp, ws, nullptr),
           HCA_ERR_INVALID);
    EXPECT("topk too many positions", dsa_index_topk(qI, kI, w, idx, 1 << 16, 1 << 16, hi, di, K, wsp, ws, nullptr),
           HCA_ERR_UNSUPPORTED);
    EXPECT("topk zero batch", dsa_index_topk(qI, kI, w, idx, 0, S, hi, di, K, wsp, ws, nullptr), HCA_ERR_INVALID);
    const int Bd = 2, N = 300;
    float* qd = AT<float>(size_t(Bd) * hi * di); float* kd = AT<float>(size_t(Bd) * N * di);
    float* wd = AT<float>(size_t(Bd) * hi); int32_t* idd = AT<int32_t>(size_t(Bd) * K);
    const size_t wsd = dsa_index_topk_decode_workspace_size(Bd, N, K);
    void* wsdp = A(wsd ? wsd : 16);
    EXPECT("topk decode", dsa_index_topk_decode(qd, kd, wd, idd, Bd, N, hi, di, K, wsdp, wsd, nullptr), HCA_OK);
    if (wsd)
      EXPECT("topk decode no ws", dsa_index_topk_decode(qd, kd, wd, idd, Bd, N, hi, di, K, nullptr, 0, nullptr),
             HCA_ERR_WORKSPACE);
    EXPECT("topk decode h_i", dsa_index_topk_decode(qd, kd, wd, idd, Bd, N, 5, di, K, wsdp, wsd, nullptr),
           HCA_ERR_UNSUPPORTED);
    EXPECT("topk decode huge", dsa_index_topk_decode(qd, kd, wd, idd, Bd, 1 << 30, hi, di, K, wsdp, wsd, nullptr),
           HCA_ERR_UNSUPPORTED);
  }

  // ---- DSA sparse attention (bf16, 256-wide, 64 query heads on one KV head) + decode + backward
  {
    const int B = 1, S = 32, Hq = 64, Hkv = 1, D = 256, K = 16;
    void* q = A(size_t(B) * S * Hq * D * 2); void* k = A(size_t(B) * S * Hkv * D * 2);
    void* v = A(size_t(B) * S * Hkv * D * 2); int32_t* idx = AT<int32_t>(size_t(B) * S * K);
    void* o = A(size_t(B) * S * Hq * D * 2); float* lse = AT<float>(size_t(B) * Hq * S);
    const hca_strides_t sq = C(S, Hq, D), skv = C(S, Hkv, D);
    EXPECT("sparse ok", dsa_sparse_attn_fwd(BF, q, sq, k, skv, v, skv, idx, o, sq, lse, B, S, Hq, Hkv, D, D, K, 0.0625f,
                                            nullptr), HCA_OK);
    EXPECT("sparse heads", dsa_sparse_attn_fwd(BF, q, sq, k, skv, v, skv, idx, o, sq, lse, B, S, 32, Hkv, D, D, K,
                                               0.0625f, nullptr), HCA_ERR_UNSUPPORTED);
    EXPECT("sparse f32", dsa_sparse_attn_fwd(F32, q, sq, k, skv, v, skv, idx, o, sq, lse, B, S, Hq, Hkv, D, D, K,
                                             0.0625f, nullptr), HCA_ERR_UNSUPPORTED);
    EXPECT("sparse idx null", dsa_sparse_attn_fwd(BF, q, sq, k, skv, v, skv, nullptr, o, sq, lse, B, S, Hq, Hkv, D, D,
                                                  K, 0.0625f, nullptr), HCA_ERR_INVALID);
    EXPECT("sparse o aliases v", dsa_sparse_attn_fwd(BF, q, sq, k, skv, v, skv, idx, v, sq, lse, B, S, Hq, Hkv, D, D, K,
                                                     0.0625f, nullptr), HCA_ERR_INVALID);
    const hca_strides_t sqd = C(1, Hq, D);
    EXPECT("sparse decode", dsa_sparse_attn_decode(BF, q, sqd, k, skv, v, skv, idx, o, sqd, lse, B, S, Hq, Hkv, D, D, K,
                                                   0.0625f, nullptr, 0, nullptr), HCA_OK);
    {
      const size_t wsd = dsa_sparse_attn_decode_workspace_size(B, Hq, 128);
      if (!wsd) EXPECT("sparse decode split size", HCA_ERR_INVALID, HCA_OK);
      // top-128 over 64 heads: two slices of 64 positions (idx holds B * S * K >= 128 entries)
      if (wsd) {
        void* w = A(wsd);
        EXPECT("sparse decode split", dsa_sparse_attn_decode(BF, q, sqd, k, skv, v, skv, idx, o, sqd, lse, B, S, Hq, Hkv,
                                                             D, D, 128, 0.0625f, w, wsd, nullptr), HCA_OK);
        EXPECT("sparse decode split small ws", dsa_sparse_attn_decode(BF, q, sqd, k, skv, v, skv, idx, o, sqd, lse, B, S,
                                                                      Hq, Hkv, D, D, 128, 0.0625f, w, wsd - 1, nullptr),
               HCA_ERR_WORKSPACE);
      }
    }
    void* dout = A(size_t(B) * S * Hq * D * 2);
    float* dq = AT<float>(size_t(B) * S * Hq * D); float* dk = AT<float>(size_t(B) * S * D);
    float* dv = AT<float>(size_t(B) * S * D);
    const size_t ws = dsa_sparse_attn_bwd_workspace_size(BF, B, S, Hq, Hkv, D, D, K);
    void* wsp = A(ws ? ws : 16);
    auto bwd = [&](float* gq, float* gk, void* w, size_t wb) {
      return dsa_sparse_attn_bwd(BF, q, sq, k, skv, v, skv, idx, o, sq, lse, dout, sq, gq, sq, gk, skv, dv, skv, B, S,
                                 Hq, Hkv, D, D, K, 0.0625f, w, wb, nullptr);
    };
    EXPECT("dsa bwd", bwd(dq, dk, wsp, ws), HCA_OK);
    if (ws) EXPECT("dsa bwd no ws", bwd(dq, dk, nullptr, 0), HCA_ERR_WORKSPACE);
    EXPECT("dsa bwd grads alias", bwd(dq, dv, wsp, ws), HCA_ERR_INVALID);
    EXPECT("dsa bwd grad aliases input", bwd((float*)q, dk, wsp, ws), HCA_ERR_INVALID);
  }

  // ---- CSA: indexer over compressed entries + sparse attention over them
  {
    const int B = 1, S = 128, blk = 4, n = S / blk, hi = 4, di = 64, K = 8, Hq = 64, D = 256;
    float* qI = AT<float>(size_t(B) * S * hi * di); float* kIc = AT<float>(size_t(B) * n * di);
    float* w = AT<float>(size_t(B) * S * hi); int32_t* idx = AT<int32_t>(size_t(B) * S * K);
    const size_t ws = csa_index_topk_workspace_size(B, S, n, K);
    void* wsp = A(ws ? ws : 16);
    EXPECT("csa topk", csa_index_topk(qI, kIc, w, idx, B, S, n, blk, hi, di, K, wsp, ws, nullptr), HCA_OK);
    EXPECT("csa too few entries", csa_index_topk(qI, kIc, w, idx, B, S, n - 1, blk, hi, di, K, wsp, ws, nullptr),
           HCA_ERR_INVALID);
    EXPECT("csa misaligned", csa_index_topk(qI + 1, kIc, w, idx, B, S, n, blk, hi, di, K, wsp, ws, nullptr),
           HCA_ERR_INVALID);
    void* q = A(size_t(B) * S * Hq * D * 2); void* kc = A(size_t(B) * n * D * 2); void* vc = A(size_t(B) * n * D * 2);
    void* o = A(size_t(B) * S * Hq * D * 2);
    const hca_strides_t sq = C(S, Hq, D), sc = C(n, 1, D);
    EXPECT("csa attn", csa_sparse_attn_fwd(BF, q, sq, kc, sc, vc, sc, idx, o, sq, nullptr, B, S, n, Hq, 1, D, D, K,
                                           0.0625f, nullptr), HCA_OK);
    EXPECT("csa attn heads", csa_sparse_attn_fwd(BF, q, sq, kc, sc, vc, sc, idx, o, sq, nullptr, B, S, n, Hq, 3, D, D,
                                                 K, 0.0625f, nullptr), HCA_ERR_INVALID);
  }

  // ---- attention-output epilogue: gate GEMM + head mixing
  {
    const int B = 1, S = 64, H = 16, Dv = 512, Dc = 2048, R = 4;
    void* o = A(size_t(B) * S * H * Dv * 2); void* c = A(size_t(B) * S * Dc * 2);
    void* wg = A(size_t(Dc) * H * Dv * 2); float* u = AT<float>(size_t(H) * R); float* vv = AT<float>(size_t(H) * R);
    void* y = A(size_t(B) * S * H * Dv * 2);
    const hca_strides_t so = C(S, H, Dv), sc = C(S, 1, Dc);
    EXPECT("epilogue ok", attn_output_epilogue(BF, o, so, c, sc, wg, u, vv, y, so, B, S, H, Dv, Dc, R, nullptr), HCA_OK);
    EXPECT("epilogue f32", attn_output_epilogue(F32, o, so, c, sc, wg, u, vv, y, so, B, S, H, Dv, Dc, R, nullptr),
           HCA_ERR_UNSUPPORTED);
    EXPECT("epilogue y aliases o", attn_output_epilogue(BF, o, so, c, sc, wg, u, vv, o, so, B, S, H, Dv, Dc, R, nullptr),
           HCA_ERR_INVALID);
    EXPECT("epilogue null u", attn_output_epilogue(BF, o, so, c, sc, wg, nullptr, vv, y, so, B, S, H, Dv, Dc, R,
                                                   nullptr), HCA_ERR_INVALID);
  }

  // ---- HCA backward (attention alone, compression alone, and the fused layer)
  {
    const int B = 1, S = 64, Hq = 4, Hkv = 1, D = 512, blk = 4, W = 16, nb = S / blk;
    void* q = A(size_t(B) * S * Hq * D * 2); void* k = A(size_t(B) * S * Hkv * D * 2);
    void* v = A(size_t(B) * S * Hkv * D * 2);
    void* kc = A(size_t(B) * nb * Hkv * D * 2); void* vc = A(size_t(B) * nb * Hkv * D * 2);
    void* o = A(size_t(B) * S * Hq * D * 2); float* lse = AT<float>(size_t(B) * Hq * S);
    void* dout = A(size_t(B) * S * Hq * D * 2);
    float* dq = AT<float>(size_t(B) * S * Hq * D); float* dk = AT<float>(size_t(B) * S * Hkv * D);
    float* dv = AT<float>(size_t(B) * S * Hkv * D); float* dkc = AT<float>(size_t(B) * nb * Hkv * D);
    float* dvc = AT<float>(size_t(B) * nb * Hkv * D);
    float* wk = AT<float>(Hkv * blk); float* wv = AT<float>(Hkv * blk);
    float* dwk = AT<float>(Hkv * blk); float* dwv = AT<float>(Hkv * blk);
    const hca_strides_t sq = C(S, Hq, D), skv = C(S, Hkv, D), sc = C(nb, Hkv, D);
    const size_t ws = hca_attn_bwd_workspace_size(BF, B, S, 0, nb, Hq, Hkv, D, blk, W);
    void* wsp = A(ws ? ws : 16);
    auto bwd = [&](float* gq, float* gk, int window, void* w, size_t wb) {
      return hca_attn_bwd(BF, q, sq, k, skv, v, skv, kc, sc, vc, sc, o, sq, lse, dout, sq, gq, sq, gk, skv, dv, skv, dkc,
                          sc, dvc, sc, B, S, 0, S, 0, nb, Hq, Hkv, D, blk, window, 0.04f, w, wb, nullptr);
    };
    EXPECT("bwd ok", bwd(dq, dk, W, wsp, ws), HCA_OK);
    if (ws) EXPECT("bwd no ws", bwd(dq, dk, W, nullptr, 0), HCA_ERR_WORKSPACE);
    EXPECT("bwd grads alias", bwd(dq, dq, W, wsp, ws), HCA_ERR_INVALID);
    EXPECT("bwd window 0", bwd(dq, dk, 0, wsp, ws), HCA_ERR_INVALID);
    EXPECT("compress bwd", hca_compress_kv_bwd(BF, k, skv, v, skv, dkc, sc, dvc, sc, wk, wv, dk, skv, dv, skv, dwk, dwv,
                                               B, S, Hkv, D, blk, nullptr), HCA_OK);
    EXPECT("compress bwd alias", hca_compress_kv_bwd(BF, k, skv, v, skv, dkc, sc, dvc, sc, wk, wv, dk, skv, dk, skv, dwk,
                                                     dwv, B, S, Hkv, D, blk, nullptr), HCA_ERR_INVALID);
    EXPECT("layer bwd", hca_attn_compress_bwd(BF, q, sq, k, skv, v, skv, kc, sc, vc, sc, o, sq, lse, dout, sq, wk, wv, dq,
                                              sq, dk, skv, dv, skv, dkc, sc, dvc, sc, dwk, dwv, B, S, nb, Hq, Hkv, D,
                                              blk, W, 0.04f, wsp, ws, nullptr), HCA_OK);
    EXPECT("bwd grad aliases lse", bwd((float*)lse, dk, W, wsp, ws), HCA_ERR_INVALID);
    EXPECT("layer bwd dw aliases q", hca_attn_compress_bwd(BF, q, sq, k, skv, v, skv, kc, sc, vc, sc, o, sq, lse, dout,
                                                           sq, wk, wv, dq, sq, dk, skv, dv, skv, dkc, sc, dvc, sc,
                                                           (float*)q, dwv, B, S, nb, Hq, Hkv, D, blk, W, 0.04f, wsp, ws,
                                                           nullptr), HCA_ERR_INVALID);
    EXPECT("layer bwd dw aliases dq", hca_attn_compress_bwd(BF, q, sq, k, skv, v, skv, kc, sc, vc, sc, o, sq, lse, dout,
                                                            sq, wk, wv, dq, sq, dk, skv, dv, skv, dkc, sc, dvc, sc, dwk,
                                                            dq + 8, B, S, nb, Hq, Hkv, D, blk, W, 0.04f, wsp, ws,
                                                            nullptr), HCA_ERR_INVALID);
    EXPECT("layer bwd null w", hca_attn_compress_bwd(BF, q, sq, k, skv, v, skv, kc, sc, vc, sc, o, sq, lse, dout, sq,
                                                     nullptr, wv, dq, sq, dk, skv, dv, skv, dkc, sc, dvc, sc, dwk, dwv,
                                                     B, S, nb, Hq, Hkv, D, blk, W, 0.04f, wsp, ws, nullptr),
           HCA_ERR_INVALID);
  }

  // error messages are per thread and the last error survives later successful calls
  if (std::strlen(hca_last_error()) == 0) { std::printf("FAIL last error cleared\n"); ++g_fail; }
  if (g_fail) {
    std::printf("FAILURES %d of %d checks\n", g_fail, g_checks);
    return 1;
  }
  std::printf("ALL OK (%d checks, %d launches)\n", g_checks, g_launches);
  return 0;
}
