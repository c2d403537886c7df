// Host-side launcher declarations shared between the C-ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hca {

struct LStrides {
  int64_t b, s, h;
};

struct AttnArgs {
  int dt;  // 0 = f32, 1 = bf16
  const void* q; LStrides sq;
  const void* k; LStrides sk;
  const void* v; LStrides sv;
  const void* kc; LStrides skc;
  const void* vc; LStrides svc;
  void* o; LStrides so;
  float* lse;
  int batch, seqlen_q;
  int64_t q_pos0;
  int seqlen_kv;
  int64_t kv_pos0;
  int n_blocks, h_q, h_kv, head_dim, block, window;
  float scale;
};

hipError_t launch_compress(int dt, const void* x, LStrides sx, const float* w, void* out, LStrides so,
                           const void* x2, LStrides sx2, const float* w2, void* out2, LStrides so2,
                           int batch, int seqlen, int h, int d, int block, hipStream_t st);

// Writes the K/V row of position t into rows t mod ring and t mod ring + ring
// of the raw-row rings.
hipError_t launch_ring_write(int dt, const void* k_new, LStrides skn, const void* v_new, LStrides svn, void* k_ring,
                             LStrides skr, void* v_ring, LStrides svr, int ring, int64_t t, int batch, int h_kv,
                             int head_dim, hipStream_t st);

// One workgroup per (query, head): any dtype, head_dim <= 512, keys per query <= kGenericMaxKeys.
constexpr int kGenericMaxKeys = 16384;
hipError_t launch_attn_generic(const AttnArgs& a, hipStream_t st);
// fp32 with head_dim 32, 64 or 128: the fp32 MFMA kernel (attn_f32mfma.hip).
bool attn_f32mfma_supports(int dt, int head_dim);
hipError_t launch_attn_f32mfma(const AttnArgs& a, hipStream_t st);
// bf16 with head_dim 64, 128 or 256: the bf16 MFMA kernel (attn_bf16mfma.hip).
bool attn_bf16mfma_supports(int dt, int head_dim);
hipError_t launch_attn_bf16mfma(const AttnArgs& a, hipStream_t st);

// bf16, head_dim 512, MFMA prefill.
hipError_t launch_attn_prefill512(const AttnArgs& a, hipStream_t st);

// bf16, head_dim 512, one query per sequence, split over keys.
size_t decode512_workspace_bytes(int batch, int h_q, int h_kv, int n_keys);
hipError_t launch_attn_decode512(const AttnArgs& a, void* ws, hipStream_t st);

// Backward (fp32 gradients).  One struct for the HCA and DSA attention
// backward; the DSA fields (idx, inverted index) are unused by HCA.
struct BwdArgs {
  const void *q, *k, *v, *kc, *vc, *o, *dout;
  LStrides sq, sk, sv, skc, svc, so, sdo;
  const float* lse;  // [batch, h_q, seqlen_q] natural log, from the forward
  float* delta;      // workspace: <dO, O> per (query, head)
  float *dq, *dk, *dv, *dkc, *dvc;
  LStrides sdq, sdk, sdv, sdkc, sdvc;
  int batch, seqlen_q, seqlen_kv, n_blocks, h_q, h_kv, d, d_v, block, window, topk;
  int64_t q_pos0, kv_pos0;
  float scale;
  const int32_t* idx;       // DSA selections [batch, seqlen_q, topk]
  const int32_t* inv_off;   // inverted index: offsets [batch, seqlen_kv + 1]
  int32_t* inv_list;        //                 query lists [batch, inv_ld]
  int64_t inv_ld;
};
constexpr int kBwdMaxKeys = 16384;  // keys per query of the generic dq kernel (LDS row of ds)
// bf16 with head_dim 512 runs the MFMA kernels (no key limit); everything else the generic ones.
bool hca_bwd_uses_mfma(int dt, int head_dim);
size_t hca_bwd_workspace_bytes(int dt, int batch, int seqlen_q, int64_t q_pos0, int n_blocks, int h_q, int h_kv,
                               int head_dim, int block, int window);
hipError_t launch_hca_attn_bwd(int dt, BwdArgs a, void* ws, hipStream_t st);
// Attention backward followed by the compressor backward (raw rows of whole
// blocks get w * dkc added; dw written), for kv_pos0 = 0 and kc = compression
// of the given raw rows.
hipError_t launch_hca_attn_compress_bwd(int dt, BwdArgs a, const float* wk, const float* wv, float* dwk, float* dwv,
                                        void* ws, hipStream_t st);
size_t hca_bwd512_workspace_bytes(int batch, int seqlen_q, int64_t q_pos0, int n_blocks, int h_q, int h_kv,
                                  int block, int window);
// fw_k/fw_v non-null: fused compressor backward into the raw-row gradients.
hipError_t launch_hca_attn_bwd512(BwdArgs a, void* ws, hipStream_t st, const float* fw_k = nullptr,
                                  const float* fw_v = nullptr);
// bf16 with d_qk = d_v = 256 and a multiple of 64 query heads per KV head runs
// the MFMA kernels (dsa_bwd256.hip); everything else the generic ones.
bool dsa_bwd_uses_mfma(int dt, int d_qk, int d_v, int h_q, int h_kv);
// The library's second stream of the current device (default priority,
// non-blocking; created on first use): chunk pipelines run their side work on
// it, ordered against the caller's stream by events.
hipError_t side_stream(hipStream_t* out);
size_t dsa_bwd256_workspace_bytes(int batch, int seqlen, int h_q, int h_kv, int topk);
hipError_t launch_dsa_bwd256(const BwdArgs& a, void* ws, hipStream_t st);
size_t dsa_bwd_workspace_bytes(int dt, int batch, int seqlen, int h_q, int h_kv, int d_qk, int d_v, int topk);
hipError_t launch_dsa_attn_bwd(int dt, BwdArgs a, void* ws, hipStream_t st);
// dk/dv (fp32, accumulated) += the compressor's backward of dkc/dvc; dw_k/dw_v written.
hipError_t launch_compress_bwd(int dt, const void* k, LStrides sk, const void* v, LStrides sv, const float* dkc,
                               LStrides sdkc, const float* dvc, LStrides sdvc, const float* wk, const float* wv,
                               float* dk, LStrides sdk, float* dv, LStrides sdv, float* dwk, float* dwv, int batch,
                               int seqlen, int h, int d, int block, hipStream_t st, bool dx = true);

// DSA
size_t dsa_topk_workspace_bytes(int batch, int seqlen, int topk);
hipError_t launch_dsa_index_topk(const float* qI, const float* kI, const float* w, int32_t* idx, int batch,
                                 int seqlen, int h_i, int d_i, int topk, void* ws, size_t ws_bytes, hipStream_t st);
// Decode: one query per sequence over n_keys keys ([batch, 1, h_i, d_i] queries,
// [batch, n_keys, d_i] keys, [batch, 1, topk] output).
size_t dsa_topk_decode_workspace_bytes(int batch, int n_keys, int topk);
hipError_t launch_dsa_index_topk_decode(const float* qI, const float* kI, const float* w, int32_t* idx, int batch,
                                        int n_keys, int h_i, int d_i, int topk, void* ws, hipStream_t st);
// CSA: seqlen queries over n_keys compressed index keys; key u is visible to
// query t when (u + 1) * block - 1 <= t.
size_t csa_topk_workspace_bytes(int batch, int seqlen, int n_keys, int topk);
hipError_t launch_csa_index_topk(const float* qI, const float* kIc, const float* w, int32_t* idx, int batch,
                                 int seqlen, int n_keys, int block, int h_i, int d_i, int topk, void* ws,
                                 hipStream_t st);
// Sparse attention of seqlen queries per sequence; selected positions must lie in [0, n_kv).
hipError_t launch_dsa_sparse_attn256(const void* q, LStrides sq, const void* k, LStrides sk, const void* v,
                                     LStrides sv, const int32_t* idx, void* o, LStrides so, float* lse, int batch,
                                     int seqlen, int n_kv, int h_q, int h_kv, int topk, float scale, hipStream_t st);
// Merge of a split decode row: op [batch, parts, h_q, 256] bf16 partial outputs,
// lp [batch, h_q, parts] their log-sum-exps; writes o (row 0 of each sequence) and lse.
hipError_t launch_dsa_decode_combine256(const void* op, const float* lp, int parts, void* o, LStrides so, float* lse,
                                        int batch, int h_q, hipStream_t st);

// Attention-output epilogue: y = sigmoid(c W_g^T) * (o + (U V) o across heads),
// one fused kernel.  Token (b, t) of c at c + b*scb + t*scs (d_c contiguous);
// W_g [h*d_v, d_c] contiguous; needs h in {8, 16, 32, 64}, d_v a multiple of
// 256 / h, d_c a multiple of 32, r <= 16.
hipError_t launch_attn_output_epilogue(const void* o, LStrides so, const void* c, int64_t scb, int64_t scs,
                                       const void* w_g, const float* u, const float* v, void* y, LStrides sy,
                                       int batch, int seqlen, int h, int d_v, int d_c, int r, hipStream_t st);

}  // namespace hca
