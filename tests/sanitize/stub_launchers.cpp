// Host-only stand-ins for the kernel launchers of libhca, for the sanitizer
// build of the C-ABI layer (hca_abi.cpp) on a machine without a GPU: every
// launcher records that it was reached and returns hipSuccess; the workspace
// size helpers return fixed sizes.  Only the argument checking, error
// reporting and dispatch of the ABI layer run.
#include <hip/hip_runtime.h>

#include "../../sparse_attention_hca_amd/csrc/launchers.h"

int g_launches = 0;

namespace hca {
static hipError_t hit() { ++g_launches; return hipSuccess; }
hipError_t launch_compress(int, const void*, LStrides, const float*, void*, LStrides, const void*, LStrides,
                           const float*, void*, LStrides, int, int, int, int, int, hipStream_t) { return hit(); }
hipError_t launch_ring_write(int, const void*, LStrides, const void*, LStrides, void*, LStrides, void*, LStrides, int,
                             int64_t, int, int, int, hipStream_t) { return hit(); }
hipError_t launch_attn_generic(const AttnArgs&, hipStream_t) { return hit(); }
bool attn_f32mfma_supports(int dt, int head_dim) { return dt == 0 && (head_dim == 32 || head_dim == 64 || head_dim == 128); }
hipError_t launch_attn_f32mfma(const AttnArgs&, hipStream_t) { return hit(); }
bool attn_bf16mfma_supports(int dt, int head_dim) { return dt == 1 && (head_dim == 64 || head_dim == 128 || head_dim == 256); }
hipError_t launch_attn_bf16mfma(const AttnArgs&, hipStream_t) { return hit(); }
hipError_t launch_attn_prefill512(const AttnArgs&, hipStream_t) { return hit(); }
size_t decode512_workspace_bytes(int batch, int h_q, int, int n_keys) {
  return (size_t)batch * h_q * (size_t)(n_keys / 64 + 1) * 2056;
}
hipError_t launch_attn_decode512(const AttnArgs&, void*, hipStream_t) { return hit(); }
bool hca_bwd_uses_mfma(int dt, int head_dim) { return dt == 1 && head_dim == 512; }
size_t hca_bwd_workspace_bytes(int, int batch, int seqlen_q, int64_t, int, int h_q, int, int, int, int) {
  return (size_t)batch * seqlen_q * h_q * 4 + 256;
}
hipError_t launch_hca_attn_bwd(int, BwdArgs, void*, hipStream_t) { return hit(); }
hipError_t launch_hca_attn_compress_bwd(int, BwdArgs, const float*, const float*, float*, float*, void*, hipStream_t) {
  return hit();
}
size_t hca_bwd512_workspace_bytes(int batch, int seqlen_q, int64_t, int, int h_q, int, int, int) {
  return (size_t)batch * seqlen_q * h_q * 4 + 256;
}
hipError_t launch_hca_attn_bwd512(BwdArgs, void*, hipStream_t, const float*, const float*) { return hit(); }
size_t dsa_bwd_workspace_bytes(int dt, int batch, int seqlen, int h_q, int, int d_qk, int, int topk) {
  return (size_t)batch * seqlen * (h_q * 4 + (size_t)topk * 4 + 8) + (dt == 1 && d_qk == 256 ? (size_t)seqlen * topk * 1024 : 0);
}
hipError_t launch_dsa_attn_bwd(int, BwdArgs, void*, hipStream_t) { return hit(); }
hipError_t launch_compress_bwd(int, const void*, LStrides, const void*, LStrides, const float*, LStrides, const float*,
                               LStrides, const float*, const float*, float*, LStrides, float*, LStrides, float*, float*,
                               int, int, int, int, int, hipStream_t, bool) { return hit(); }
size_t dsa_topk_workspace_bytes(int batch, int seqlen, int) { return (size_t)batch * seqlen * 64 + 1024; }
hipError_t launch_dsa_index_topk(const float*, const float*, const float*, int32_t*, int, int, int, int, int, void*,
                                 size_t, hipStream_t) { return hit(); }
size_t dsa_topk_decode_workspace_bytes(int batch, int n_keys, int) { return (size_t)batch * n_keys * 8 + 1024; }
hipError_t launch_dsa_index_topk_decode(const float*, const float*, const float*, int32_t*, int, int, int, int, int,
                                        void*, hipStream_t) { return hit(); }
size_t csa_topk_workspace_bytes(int batch, int seqlen, int n_keys, int) {
  return (size_t)batch * seqlen * 16 + (size_t)n_keys * 4 + 1024;
}
hipError_t launch_csa_index_topk(const float*, const float*, const float*, int32_t*, int, int, int, int, int, int, int,
                                 void*, hipStream_t) { return hit(); }
hipError_t launch_dsa_sparse_attn256(const void*, LStrides, const void*, LStrides, const void*, LStrides,
                                     const int32_t*, void*, LStrides, float*, int, int, int, int, int, int, float,
                                     hipStream_t) { return hit(); }
hipError_t launch_dsa_decode_combine256(const void*, const float*, int, void*, LStrides, float*, int, int,
                                        hipStream_t) { return hit(); }
hipError_t launch_attn_output_epilogue(const void*, LStrides, const void*, int64_t, int64_t, const void*,
                                       const float*, const float*, void*, LStrides, int, int, int, int, int, int,
                                       hipStream_t) { return hit(); }
}  // namespace hca
