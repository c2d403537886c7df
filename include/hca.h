/*
 * hca.h -- C ABI of libhca.so: hybrid sparse attention (HCA heavily
 * compressed attention + DSA top-k sparse attention) for AMD Instinct MI355X
 * (gfx950): the forward path, decode-time cache upkeep, and the backward of
 * both attentions and of the block compressor.
 *
 * The method is the one described on the ERNIE 5.5 Flash Base pages:
 *   - mirrorspeed page, section "Hybrid sparse attention, 1/7 full context
 *     access": every 128 tokens of K/V become one cache entry; HCA layers
 *     attend over the compressed entries plus a recent short uncompressed
 *     window; the full-context layers use DSA, where a lightweight indexer
 *     scores past positions per query and core attention runs on the top-k.
 *   - ai-club.cn page, section on hybrid attention (MLA + HCA): the attention
 *     over compressed entries plus recent tokens is dense; HCA heads are 512
 *     wide, the token-level layers use 256-wide heads.
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers on the current HIP device, owned by
 *     the caller.  The library never allocates or frees memory and keeps no
 *     pointer after a call returns.  Scratch memory is passed in
 *     as a caller-owned workspace whose size is given by the
 *     *_workspace_size() queries.
 *   - Tensors are batch/sequence/head/dim with the dim axis contiguous
 *     (stride 1).  The other three axes take element strides through
 *     hca_strides_t.  Base pointers must be 16-byte aligned and every stride
 *     a multiple of 16 bytes.
 *   - `stream` is a hipStream_t (NULL = the default stream) of the current
 *     device.  Work is only enqueued; no call synchronizes.  Device faults
 *     surface at the caller's next synchronization.  The chunked calls
 *     (dsa_index_topk, csa_index_topk, dsa_sparse_attn_bwd) may run part of
 *     their work on a library-owned second stream of the current device,
 *     joined back to `stream` by events before they return.
 *   - Errors: every argument is validated before anything is launched, so a
 *     call that returns an error has written nothing.  hca_last_error()
 *     returns a message for the last non-OK status on the calling thread.
 *     No exception, abort or exit crosses this ABI.  Calls are thread-safe.
 */
#ifndef HCA_H_
#define HCA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HCA_OK = 0,
  HCA_ERR_INVALID = 1,     /* null pointer, bad size, misalignment, aliasing, window not covered */
  HCA_ERR_UNSUPPORTED = 2, /* a valid request this build has no kernel for (never a silent fallback) */
  HCA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the size query says */
  HCA_ERR_HIP = 4          /* a HIP runtime or launch error; the HIP text is in hca_last_error() */
} hca_status_t;

/* The two range markers are not dtypes: they give the type every 32-bit value,
 * so an unknown value a caller passes is rejected (HCA_ERR_INVALID) instead of
 * being an out-of-range enum inside the C++ library. */
typedef enum {
  HCA_DTYPE_F32 = 0,
  HCA_DTYPE_BF16 = 1,
  HCA_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
  HCA_DTYPE_RANGE_MAX_ = 0x7fffffff
} hca_dtype_t;

/* Element strides of a [batch, seq, head, dim] tensor whose dim axis is contiguous. */
typedef struct {
  int64_t batch;
  int64_t seq;
  int64_t head;
} hca_strides_t;

/* Version of this ABI (1). */
int hca_abi_version(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* hca_last_error(void);

/*
 * hca_compress_kv -- HCA block compression (mirrorspeed page, "Hybrid sparse
 * attention" section: 128 tokens -> one cache entry).  For every batch b,
 * block j < seqlen / block and KV head h:
 *     kc[b, j, h, :] = sum_{i < block} w_k[h, i] * k[b, j*block + i, h, :]
 *     vc[b, j, h, :] = sum_{i < block} w_v[h, i] * v[b, j*block + i, h, :]
 * accumulated in fp32, stored in `dt`.  A trailing partial block is not
 * compressed.
 *   k, v   : [batch, seqlen, h_kv, head_dim] device, dtype dt (read)
 *   w_k,w_v: [h_kv, block] fp32 device, contiguous (read)
 *   kc, vc : [batch, seqlen/block, h_kv, head_dim] device, dtype dt (written)
 * Supported: head_dim in {64, 128, 256, 512}; any block >= 1.
 */
hca_status_t hca_compress_kv(hca_dtype_t dt,
                             const void* k, hca_strides_t sk,
                             const void* v, hca_strides_t sv,
                             const float* w_k, const float* w_v,
                             void* kc, hca_strides_t skc,
                             void* vc, hca_strides_t svc,
                             int batch, int seqlen, int h_kv, int head_dim, int block,
                             void* stream);

/*
 * hca_append_kv -- decode-time upkeep of the HCA caches (mirrorspeed page,
 * "Hybrid sparse attention" section: every 128 tokens become one cache entry
 * while the most recent tokens stay uncompressed).  Appends the K/V row of
 * position t (the same t for every sequence of the batch) to a mirrored ring
 * of raw rows and, when t closes a block, compresses that block:
 *     k_ring[b, t mod R, h, :] = k_ring[b, t mod R + R, h, :] = k_new[b, 0, h, :]
 *     (v_ring likewise), and if (t + 1) % block == 0, with j = (t + 1) / block - 1:
 *     kc[b, j, h, :] = sum_{i < block} w_k[h, i] * (ring row of position t + 1 - block + i)
 *     vc[b, j, h, :] likewise with w_v
 * in fp32, stored in `dt` -- the same values hca_compress_kv gives for block j
 * of the whole history.  The rows of positions lo .. t (t - lo < R) sit
 * contiguously at ring rows lo mod R .. lo mod R + (t - lo), so a decode
 * query at t reads its window straight from the ring: hca_attn_fwd with
 * k = k_ring + (lo mod R) rows, kv_pos0 = lo, seqlen_kv = t - lo + 1.
 *   k_new, v_new : [batch, 1, h_kv, head_dim] (read)
 *   k_ring, v_ring: [batch, 2 * ring, h_kv, head_dim] (two rows written; when a
 *                   block closes its rows are read back -- positions
 *                   t + 1 - block .. t - 1 must have been appended before)
 *   w_k, w_v     : [h_kv, block] fp32 contiguous (read when a block closes)
 *   kc, vc       : [batch, n_blocks, h_kv, head_dim] (row j written when block j
 *                   closes; may be NULL otherwise)
 * Errors: HCA_ERR_INVALID when ring < block, when t closes a block j >=
 * n_blocks, or when the rings overlap each other, the new rows or kc/vc.
 * Supported: head_dim in {64, 128, 256, 512}.
 */
hca_status_t hca_append_kv(hca_dtype_t dt,
                           const void* k_new, hca_strides_t sk_new,
                           const void* v_new, hca_strides_t sv_new,
                           void* k_ring, hca_strides_t sk_ring,
                           void* v_ring, hca_strides_t sv_ring,
                           int ring,
                           const float* w_k, const float* w_v,
                           void* kc, hca_strides_t skc,
                           void* vc, hca_strides_t svc,
                           int n_blocks, int64_t t,
                           int batch, int h_kv, int head_dim, int block,
                           void* stream);

/*
 * Workspace bytes hca_attn_fwd needs for these sizes (0 when none is needed).
 * n_blocks and window are the values that will be passed to hca_attn_fwd.
 */
size_t hca_attn_fwd_workspace_size(int batch, int seqlen_q, int h_q, int h_kv, int head_dim,
                                   int n_blocks, int window);

/*
 * hca_attn_fwd -- HCA attention (mirrorspeed page, "Hybrid sparse attention"
 * section; ai-club.cn page, hybrid attention section: dense attention over
 * the compressed sequence plus the most recent uncompressed tokens).
 *
 * Query i sits at absolute position t = q_pos0 + i.  It sees
 *   - the raw window [lo, t] with lo = max(0, t - window + 1), i.e. the
 *     `window` most recent positions including itself, and
 *   - the compressed entries j < n_c = floor(lo / block): exactly the blocks
 *     that end before the window (no block overlaps the window).
 * For query head h and KV head g = h / (h_q / h_kv):
 *   o[b,i,h,:] = sum_x softmax_x(scale * <q[b,i,h], key_x>) * value_x
 * over keys kc[b, 0..n_c-1, g] and k[b, lo-kv_pos0 .. t-kv_pos0, g] (values
 * from vc and v likewise).  Softmax in fp32; output in dt.
 *   q   : [batch, seqlen_q, h_q, head_dim]            (read)
 *   k, v: [batch, seqlen_kv, h_kv, head_dim]          raw K/V at positions kv_pos0 + s (read)
 *   kc, vc: [batch, n_blocks, h_kv, head_dim]         compressed entries (read)
 *   o   : [batch, seqlen_q, h_q, head_dim]            (written)
 *   lse : [batch, h_q, seqlen_q] fp32 contiguous, natural-log logsumexp of the
 *         scaled logits; may be NULL.
 * Prefill: q_pos0 = kv_pos0 = 0 and seqlen_kv = seqlen_q.  Decode: seqlen_q = 1.
 * Errors: HCA_ERR_INVALID when some query's window is not inside
 * [kv_pos0, kv_pos0 + seqlen_kv) or needs more than n_blocks entries, or when
 * h_q % h_kv != 0, window < 1 or block < 1.
 * Kernels: bf16 with head_dim 512 runs the MFMA prefill kernel (seqlen_q > 1)
 * or the split-key decode kernel (seqlen_q == 1, which uses the workspace);
 * fp32 with head_dim 32, 64 or 128 and bf16 with head_dim 64, 128 or 256 run
 * MFMA kernels of 64 queries per workgroup (any number of keys); fp32 with
 * another head_dim (multiple of 4) and bf16 with another head_dim (multiple
 * of 8), both <= 512, run a one-query-per-workgroup kernel limited to 16384
 * keys per query (HCA_ERR_UNSUPPORTED beyond).
 */
hca_status_t hca_attn_fwd(hca_dtype_t dt,
                          const void* q, hca_strides_t sq,
                          const void* k, hca_strides_t sk,
                          const void* v, hca_strides_t sv,
                          const void* kc, hca_strides_t skc,
                          const void* vc, hca_strides_t svc,
                          void* o, hca_strides_t so,
                          float* lse,
                          int batch, int seqlen_q, int64_t q_pos0,
                          int seqlen_kv, int64_t kv_pos0, int n_blocks,
                          int h_q, int h_kv, int head_dim, int block, int window, float scale,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * hca_attn_fwd_noalloc -- hca_attn_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, semantics, validation and kernels as
 * hca_attn_fwd, without the workspace: the decode path's split partials go to
 * a fixed device array inside the library (HCA_NOALLOC_SCRATCH_BYTES, 16 MiB;
 * one copy per GPU, held from library load until the process exits).  The call allocates and frees nothing; the caller still passes q,
 * k, v, kc, vc, o and lse.  Every fully written partial is consumed by the
 * same call, so nothing needs clearing between calls.
 * Calls that overlap on one GPU (two streams, or two threads) race on that
 * array and must be serialized by the caller.
 * Errors: as hca_attn_fwd; HCA_ERR_WORKSPACE (checked first) when
 * hca_attn_fwd_workspace_size(batch, seqlen_q, h_q, h_kv, head_dim, n_blocks,
 * window) exceeds the array (the c4 decode shape -- 64 sequences, 16 heads on
 * one KV head, 8192 + 128 keys -- needs 8.4 MB).
 */
#define HCA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

hca_status_t hca_attn_fwd_noalloc(hca_dtype_t dt,
                                  const void* q, hca_strides_t sq,
                                  const void* k, hca_strides_t sk,
                                  const void* v, hca_strides_t sv,
                                  const void* kc, hca_strides_t skc,
                                  const void* vc, hca_strides_t svc,
                                  void* o, hca_strides_t so,
                                  float* lse,
                                  int batch, int seqlen_q, int64_t q_pos0,
                                  int seqlen_kv, int64_t kv_pos0, int n_blocks,
                                  int h_q, int h_kv, int head_dim, int block, int window, float scale,
                                  void* stream);

/* Workspace bytes dsa_index_topk needs: score rows for one chunk of queries,
 * two chunks' worth when the call has more than one chunk. */
size_t dsa_index_topk_workspace_size(int batch, int seqlen, int topk);

/*
 * dsa_index_topk -- DSA lightweight indexer and causal top-k (mirrorspeed
 * page, "Hybrid sparse attention" section: the indexer scores historical
 * positions for each query; attention runs on the top-k).
 *   s(t, u) = sum_{h < h_i} w_idx[b,t,h] * max(0, <q_idx[b,t,h,:], k_idx[b,u,:]>),  u <= t
 * computed in fp32.  Row t of idx receives the min(t+1, topk) positions with
 * the largest s (ties: the smaller position wins; -0 counts as +0) in
 * unspecified order, then -1 padding.
 *   q_idx: [batch, seqlen, h_i, d_i] fp32 contiguous (read)
 *   k_idx: [batch, seqlen, d_i]      fp32 contiguous (read)
 *   w_idx: [batch, seqlen, h_i]      fp32 contiguous (read)
 *   idx  : [batch, seqlen, topk]     int32 contiguous (written)
 * Supported: h_i <= 8, d_i a multiple of 16 and <= 128, topk <= 4096.
 * Streams: the scores run on `stream` in chunks of query rows.  When there
 * is more than one chunk, each chunk's selection runs on a library-owned
 * second stream of the current device (default priority, created on first
 * use), ordered by events.  `stream` waits for the last selection before any
 * work queued after the call, so the call behaves as if it ran entirely on
 * `stream`.  Calls from several host threads take the second stream in turn.
 */
hca_status_t dsa_index_topk(const float* q_idx, const float* k_idx, const float* w_idx,
                            int32_t* idx,
                            int batch, int seqlen, int h_i, int d_i, int topk,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/* Workspace bytes dsa_index_topk_decode needs (one score row per sequence plus
 * the two-stage selection's candidates). */
size_t dsa_index_topk_decode_workspace_size(int batch, int n_keys, int topk);

/*
 * dsa_index_topk_decode -- the DSA indexer and top-k for one new query per
 * sequence (mirrorspeed page, "Hybrid sparse attention" section: the indexer
 * scores the historical positions of each query, so the per-query attention
 * cost stops growing with the context).  The query of sequence b sits at
 * position n_keys - 1 and sees keys 0 .. n_keys - 1:
 *   s(u) = sum_{h < h_i} w_idx[b,0,h] * max(0, <q_idx[b,0,h,:], k_idx[b,u,:]>)
 * in fp32; idx[b,0,:] receives the min(n_keys, topk) positions with the largest
 * s (ties: the smaller position wins; -0 counts as +0) in unspecified order,
 * then -1 padding -- the same set dsa_index_topk gives for row n_keys - 1.
 * Rows longer than 65536 keys are selected in two exact stages (each 65536-key
 * segment, then the segments' winners).
 *   q_idx: [batch, 1, h_i, d_i] fp32 contiguous (read)
 *   k_idx: [batch, n_keys, d_i] fp32 contiguous (read)
 *   w_idx: [batch, 1, h_i]      fp32 contiguous (read)
 *   idx  : [batch, 1, topk]     int32 contiguous (written)
 * Supported: h_i in {4, 8}, d_i a multiple of 16 and <= 128, topk <= 4096,
 * n_keys < 2^30.
 */
hca_status_t dsa_index_topk_decode(const float* q_idx, const float* k_idx, const float* w_idx,
                                   int32_t* idx,
                                   int batch, int n_keys, int h_i, int d_i, int topk,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * dsa_sparse_attn_fwd -- DSA core attention over the selected positions
 * (mirrorspeed page, "Hybrid sparse attention" section; 256-wide heads per
 * the ai-club.cn page).  For query t and head h, with g = h / (h_q / h_kv):
 *   o[b,t,h,:] = sum_{u in idx[b,t,:], u >= 0} softmax_u(scale * <q[b,t,h], k[b,u,g]>) * v[b,u,g,:]
 * Entries equal to -1 are skipped; any order is accepted; every listed
 * position must lie in [0, seqlen) (checked on the device: a row holding an
 * out-of-range position is written as NaN).  A row with no valid entry
 * yields zeros and lse = -inf.
 *   q: [batch, seqlen, h_q, d_qk]; k: [batch, seqlen, h_kv, d_qk];
 *   v: [batch, seqlen, h_kv, d_v]; o: [batch, seqlen, h_q, d_v];
 *   idx: [batch, seqlen, topk] int32 contiguous; lse: [batch, h_q, seqlen] fp32 or NULL.
 * Supported: bf16, d_qk = d_v = 256, (h_q / h_kv) a multiple of 64, topk <= 4096.
 */
hca_status_t dsa_sparse_attn_fwd(hca_dtype_t dt,
                                 const void* q, hca_strides_t sq,
                                 const void* k, hca_strides_t sk,
                                 const void* v, hca_strides_t sv,
                                 const int32_t* idx,
                                 void* o, hca_strides_t so,
                                 float* lse,
                                 int batch, int seqlen, int h_q, int h_kv, int d_qk, int d_v,
                                 int topk, float scale,
                                 void* stream);

/*
 * dsa_sparse_attn_decode -- DSA core attention for one query per sequence
 * over a key history of n_keys rows (mirrorspeed page, "Hybrid sparse
 * attention" section).  For head h, g = h / (h_q / h_kv):
 *   o[b,0,h,:] = sum_{u in idx[b,0,:], u >= 0} softmax_u(scale * <q[b,0,h], k[b,u,g]>) * v[b,u,g,:]
 * with the same conventions as dsa_sparse_attn_fwd (every listed position in
 * [0, n_keys), else the row is written as NaN).
 *   q: [batch, 1, h_q, d_qk]; k: [batch, n_keys, h_kv, d_qk]; v: [batch, n_keys, h_kv, d_v];
 *   idx: [batch, 1, topk] int32 contiguous; o: [batch, 1, h_q, d_v]; lse: [batch, h_q] fp32 or NULL.
 * Supported: as dsa_sparse_attn_fwd.
 * workspace: NULL runs one workgroup per sequence and 64 query heads.  Else
 * it must hold dsa_sparse_attn_decode_workspace_size(batch, h_q, topk) bytes
 * (16-byte aligned, caller-owned, overlapping no tensor; contents need no
 * initialisation and are overwritten): the index row is then split into
 * contiguous slices that run as separate workgroups (about one per CU), and a
 * second kernel merges the slices' bf16 outputs by their log-sum-exps.  A size
 * of 0 means the shape gains nothing from the split (workspace ignored).
 * HCA_ERR_WORKSPACE when a non-NULL workspace is too small.
 */
size_t dsa_sparse_attn_decode_workspace_size(int batch, int h_q, int topk);
hca_status_t dsa_sparse_attn_decode(hca_dtype_t dt,
                                    const void* q, hca_strides_t sq,
                                    const void* k, hca_strides_t sk,
                                    const void* v, hca_strides_t sv,
                                    const int32_t* idx,
                                    void* o, hca_strides_t so,
                                    float* lse,
                                    int batch, int n_keys, int h_q, int h_kv, int d_qk, int d_v,
                                    int topk, float scale,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream);

/* ---------------------------------------------------------------------------
 * CSA (compressed sparse attention): the history compressed 4x, then a top-k
 * selection over the compressed entries (mirrorspeed page, "Hybrid sparse
 * attention" section: the common CSA + HCA design; besthub page, "Core
 * Architectural Innovations -- 1. Hybrid Sparse Attention").  The compressed
 * K, V and index keys come from hca_compress_kv with block = 4 (the index
 * keys as one fp32 head).  Entry j covers positions block*j .. block*j +
 * block - 1 and belongs to the history of position t once its block is
 * complete: block*j + block - 1 <= t.
 * ------------------------------------------------------------------------- */

/* Workspace bytes csa_index_topk needs: score rows for one chunk of queries,
 * two chunks' worth when the call has more than one chunk. */
size_t csa_index_topk_workspace_size(int batch, int seqlen, int n_entries, int topk);

/*
 * csa_index_topk -- the DSA indexer over the compressed entries visible to each
 * position, then the top-k of them (same ranking as dsa_index_topk: larger
 * fp32 score first, the smaller entry index on a tie):
 *   s(t, j) = sum_h w[b,t,h] * max(0, <q_idx[b,t,h,:], k_idx[b,j,:]>),  j < (t + 1) / block
 *   q_idx: [batch, seqlen, h_i, d_i] fp32 contiguous; w_idx: [batch, seqlen, h_i] fp32 contiguous
 *   k_idx: [batch, n_entries, d_i] fp32 contiguous (the compressed index keys)
 *   idx  : [batch, seqlen, topk] int32 contiguous (written): the selected entry
 *          indices in unspecified order, then -1 (a position before the first
 *          complete block lists none).
 * Errors: HCA_ERR_INVALID when n_entries < seqlen / block (the last position
 * needs more entries), for NULL or misaligned tensors, or when idx overlaps an
 * input; HCA_ERR_WORKSPACE for a missing or short workspace.
 * Supported: h_i in {4, 8}, d_i a multiple of 16 <= 128, topk <= 4096.
 * Streams: as dsa_index_topk (selections of all but a single chunk run on the
 * library's second stream; `stream` waits for them).
 */
hca_status_t csa_index_topk(const float* q_idx, const float* k_idx, const float* w_idx,
                            int32_t* idx,
                            int batch, int seqlen, int n_entries, int block,
                            int h_i, int d_i, int topk,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * csa_sparse_attn_fwd -- attention of each position over the compressed
 * entries listed in its row of idx (from csa_index_topk):
 *   o[b,t,h,:] = sum_{j in idx[b,t,:], j >= 0} softmax_j(scale * <q[b,t,h], kc[b,j,g]>) * vc[b,j,g,:]
 * with g = h / (h_q / h_kv); conventions as dsa_sparse_attn_fwd (every listed
 * entry in [0, n_entries), else the row is NaN; a row listing none gives o = 0,
 * lse = -inf).
 *   q: [batch, seqlen, h_q, d_qk]; kc: [batch, n_entries, h_kv, d_qk]; vc: [batch, n_entries, h_kv, d_v];
 *   idx: [batch, seqlen, topk] int32; o: [batch, seqlen, h_q, d_v]; lse: [batch, h_q, seqlen] fp32 or NULL.
 * Supported: as dsa_sparse_attn_fwd (bf16, d_qk = d_v = 256, h_q / h_kv a multiple of 64).
 */
hca_status_t csa_sparse_attn_fwd(hca_dtype_t dt,
                                 const void* q, hca_strides_t sq,
                                 const void* kc, hca_strides_t skc,
                                 const void* vc, hca_strides_t svc,
                                 const int32_t* idx,
                                 void* o, hca_strides_t so,
                                 float* lse,
                                 int batch, int seqlen, int n_entries, int h_q, int h_kv, int d_qk, int d_v,
                                 int topk, float scale,
                                 void* stream);

/*
 * attn_output_epilogue -- the two attention-output epilogues of the pages
 * (mirrorspeed page, section "More structural improvements, data, and
 * infrastructure"; besthub page, section "Core Architectural Innovations"):
 * the output gate computed from the layer's low-rank query latent c (a
 * quarter of the hidden size) and Virtual Head Attention's low-rank mixing
 * of the heads with an identity skip; heads are mixed first, then gated:
 *   y[b,t,h,e] = sigmoid(<c[b,t,:], w_g[h*d_v + e, :]>) * (o[b,t,h,e] + sum_h' (u v)[h,h'] o[b,t,h',e])
 *   o  : [batch, seqlen, h, d_v] bf16, the attention output (read)
 *   c  : [batch, seqlen, 1, d_c] bf16, the query latent (read)
 *   w_g: [h * d_v, d_c] bf16 contiguous (the [out, in] layout of a linear layer)
 *   u  : [h, r] fp32 contiguous; v: [r, h] fp32 contiguous
 *   y  : [batch, seqlen, h, d_v] bf16 (written; must not overlap an input)
 * One kernel: the gate projection runs on the matrix cores (bf16 operands,
 * fp32 accumulation) and its epilogue applies the sigmoid, the head mixing
 * and the product in fp32 before the single bf16 rounding of y; the gate
 * pre-activations never reach memory.
 * Supported: bf16, h in {8, 16, 32, 64}, r <= 16, d_c a multiple of 32,
 * d_v a multiple of 256 / h.
 */
hca_status_t attn_output_epilogue(hca_dtype_t dt,
                                  const void* o, hca_strides_t so,
                                  const void* c, hca_strides_t sc,
                                  const void* w_g,
                                  const float* u, const float* v,
                                  void* y, hca_strides_t sy,
                                  int batch, int seqlen, int h, int d_v, int d_c, int r,
                                  void* stream);

/* ---------------------------------------------------------------------------
 * Backward.  The pages describe the forward only (mirrorspeed page, "Hybrid
 * sparse attention" section; training reaches 128K-token contexts).  The
 * gradients below are the chain rule through the forward definitions above:
 * with p the softmax weights recomputed from the forward's lse and
 * D = <dO, O> per (query, head),
 *   ds_x = p_x (<dO, value_x> - D),  dq = scale * sum_x ds_x key_x,
 *   dkey_x += scale * ds_x q,        dvalue_x += p_x dO.
 * All gradients are fp32 (their strides follow the same 16-byte rule, i.e.
 * multiples of 4 elements) and are overwritten, except where a call says it
 * accumulates.  Sums run in a fixed order without atomics, except the DSA
 * key/value gradients (see dsa_sparse_attn_bwd).
 * ------------------------------------------------------------------------- */

/*
 * Workspace bytes hca_attn_bwd needs for these arguments (the values that will
 * be passed to it; 0 for invalid sizes): D per query and head and, on the
 * bf16 / head_dim 512 path, fp32 partial gradients of the compressed entries
 * (one 64-entry x 512 block per chunk of at most max(32, seqlen_q / 1024)
 * query tiles of 32 that see the block).
 */
size_t hca_attn_bwd_workspace_size(hca_dtype_t dt, int batch, int seqlen_q, int64_t q_pos0, int n_blocks, int h_q,
                                   int h_kv, int head_dim, int block, int window);

/*
 * hca_attn_bwd -- gradients of hca_attn_fwd's output o with respect to q, the
 * raw K/V and the compressed entries, given dout = dL/do and the forward's o
 * and lse (same keys per query as hca_attn_fwd: compressed entries j < n_c
 * plus the raw window [lo, t]).
 *   q, k, v, kc, vc, o, dout: as in hca_attn_fwd, dtype dt (read)
 *   lse : [batch, h_q, seqlen_q] fp32 contiguous from hca_attn_fwd (read)
 *   dq  : [batch, seqlen_q, h_q, head_dim] fp32 (written)
 *   dk, dv  : [batch, seqlen_kv, h_kv, head_dim] fp32 (written; rows no query
 *             sees get zeros)
 *   dkc, dvc: [batch, n_blocks, h_kv, head_dim] fp32 (written; may be NULL
 *             when n_blocks == 0)
 * To reach the raw K/V through the compressor, follow with
 * hca_compress_kv_bwd, which adds its share into dk/dv.
 * Errors: as hca_attn_fwd; HCA_ERR_INVALID when a gradient overlaps an input
 * or another gradient; HCA_ERR_WORKSPACE for a missing or short workspace.
 * Kernels: bf16 with head_dim 512 runs two MFMA kernels (query-tile major
 * for dq and D, key-tile major for dk/dv/dkc/dvc) and a fixed-order sum of the
 * compressed-entry partials; other shapes run one-row-per-workgroup kernels.
 * Supported: fp32 and bf16, head_dim <= 512 (multiple of 4); outside the MFMA
 * path at most 16384 keys per query.
 */
hca_status_t hca_attn_bwd(hca_dtype_t dt,
                          const void* q, hca_strides_t sq,
                          const void* k, hca_strides_t sk,
                          const void* v, hca_strides_t sv,
                          const void* kc, hca_strides_t skc,
                          const void* vc, hca_strides_t svc,
                          const void* o, hca_strides_t so,
                          const float* lse,
                          const void* dout, hca_strides_t sdout,
                          float* dq, hca_strides_t sdq,
                          float* dk, hca_strides_t sdk,
                          float* dv, hca_strides_t sdv,
                          float* dkc, hca_strides_t sdkc,
                          float* dvc, hca_strides_t sdvc,
                          int batch, int seqlen_q, int64_t q_pos0,
                          int seqlen_kv, int64_t kv_pos0, int n_blocks,
                          int h_q, int h_kv, int head_dim, int block, int window, float scale,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * hca_compress_kv_bwd -- backward of hca_compress_kv given dkc, dvc = dL/dkc,
 * dL/dvc (fp32):
 *   dk[b, j*block + i, h, :] += w_k[h, i] * dkc[b, j, h, :]   (v likewise; rows
 *                                                              past the last whole block untouched)
 *   dw_k[h, i] = sum_{b, j} <dkc[b, j, h, :], k[b, j*block + i, h, :]>  (dw_v likewise)
 *   k, v   : [batch, seqlen, h_kv, head_dim] dtype dt (read)
 *   dkc, dvc: [batch, seqlen/block, h_kv, head_dim] fp32 (read)
 *   w_k, w_v: [h_kv, block] fp32 contiguous (read)
 *   dk, dv : [batch, seqlen, h_kv, head_dim] fp32 (ACCUMULATED: pass the raw
 *            gradients from hca_attn_bwd, or zeros)
 *   dw_k, dw_v: [h_kv, block] fp32 contiguous (written)
 * Errors: HCA_ERR_INVALID for null pointers, bad sizes or overlapping gradients.
 * Supported: fp32 and bf16, head_dim a multiple of 4, at most 512.
 */
hca_status_t hca_compress_kv_bwd(hca_dtype_t dt,
                                 const void* k, hca_strides_t sk,
                                 const void* v, hca_strides_t sv,
                                 const float* dkc, hca_strides_t sdkc,
                                 const float* dvc, hca_strides_t sdvc,
                                 const float* w_k, const float* w_v,
                                 float* dk, hca_strides_t sdk,
                                 float* dv, hca_strides_t sdv,
                                 float* dw_k, float* dw_v,
                                 int batch, int seqlen, int h_kv, int head_dim, int block,
                                 void* stream);

/*
 * hca_attn_compress_bwd -- the backward of a whole HCA layer's attention for a
 * sequence processed from position 0: hca_compress_kv (K, V -> kc, vc with
 * w_k, w_v) followed by hca_attn_fwd (queries 0 .. seqlen-1 over kc, vc and the
 * raw window).  Gives the same values as hca_attn_bwd followed by
 * hca_compress_kv_bwd, in one call:
 *   dq, dkc, dvc as hca_attn_bwd;
 *   dk[b, r, g, :] = (window part of hca_attn_bwd) + w_k[g, r % block] * dkc[b, r / block, g, :]
 *                    for rows r < n_blocks * block (window part only beyond), dv likewise;
 *   dw_k[g, i] = sum_{b, j} <dkc[b, j, g, :], k[b, j*block + i, g, :]>, dw_v likewise.
 *   q, o, dout: [batch, seqlen, h_q, head_dim]; k, v: [batch, seqlen, h_kv, head_dim]
 *   kc, vc: [batch, n_blocks, h_kv, head_dim], the compression of k, v (read)
 *   w_k, w_v, dw_k, dw_v: [h_kv, block] fp32 contiguous
 *   dq, dk, dv, dkc, dvc: fp32, overwritten.
 * On the bf16 / head_dim 512 path the compressor's share is added inside the
 * key-tile kernel, saving a read-modify-write pass over dk and dv.
 * Workspace: hca_attn_bwd_workspace_size with q_pos0 = 0 and seqlen_q = seqlen.
 * Errors: as hca_attn_bwd, and HCA_ERR_INVALID when a weight pointer is NULL,
 * n_blocks * block > seqlen, or the weight gradients overlap other outputs.
 */
hca_status_t hca_attn_compress_bwd(hca_dtype_t dt,
                                   const void* q, hca_strides_t sq,
                                   const void* k, hca_strides_t sk,
                                   const void* v, hca_strides_t sv,
                                   const void* kc, hca_strides_t skc,
                                   const void* vc, hca_strides_t svc,
                                   const void* o, hca_strides_t so,
                                   const float* lse,
                                   const void* dout, hca_strides_t sdout,
                                   const float* w_k, const float* w_v,
                                   float* dq, hca_strides_t sdq,
                                   float* dk, hca_strides_t sdk,
                                   float* dv, hca_strides_t sdv,
                                   float* dkc, hca_strides_t sdkc,
                                   float* dvc, hca_strides_t sdvc,
                                   float* dw_k, float* dw_v,
                                   int batch, int seqlen, int n_blocks,
                                   int h_q, int h_kv, int head_dim, int block, int window, float scale,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Workspace bytes dsa_sparse_attn_bwd needs for these arguments (0 for
 * invalid sizes): an inverted index of idx, and on the bf16 / 256-wide path
 * the position-ordered contribution rows of one chunk of queries (at most
 * 8 GiB plus the index; proportionally less for short sequences), twice when
 * the call has more than one chunk (the chunks are pipelined). */
size_t dsa_sparse_attn_bwd_workspace_size(hca_dtype_t dt, int batch, int seqlen, int h_q, int h_kv, int d_qk,
                                          int d_v, int topk);

/*
 * dsa_sparse_attn_bwd -- gradients of dsa_sparse_attn_fwd's output with
 * respect to q, k and v, given dout, the forward's o and lse, and the same
 * idx.  Every occurrence of a position in a query's list counts (a position
 * listed twice receives both contributions); entries outside [0, seqlen),
 * -1 included, are skipped.
 *   q, k, v, o, dout, idx: as in dsa_sparse_attn_fwd, dtype dt (read)
 *   lse : [batch, h_q, seqlen] fp32 contiguous from the forward (read)
 *   dq  : [batch, seqlen, h_q, d_qk] fp32 (written)
 *   dk  : [batch, seqlen, h_kv, d_qk] fp32, dv: [batch, seqlen, h_kv, d_v] fp32
 *         (written; positions no query lists get zeros)
 * dk and dv sum over the queries that list a position in an order set by
 * atomic slot claims, so they are reproducible up to fp32 rounding only.
 * Kernels: bf16 with d_qk = d_v = 256 and h_q / h_kv a multiple of 64 (the
 * DSA workload) runs the MFMA path -- one workgroup per (query, 64 heads)
 * over the gathered rows, dq accumulated in fp32, each (query, position)
 * pair's dk and dv contributions written as bf16 rows ordered by position and
 * summed in fp32 per position, queries taken in chunks (launches several
 * kernels per chunk; with more than one chunk, each chunk's index building
 * and reduction run on the library's second stream of the current device
 * beside the next chunk's MFMA kernel, ordered by events, and `stream` waits
 * for the last of them); everything else the generic fp32 kernels.
 * Errors: HCA_ERR_INVALID for bad pointers, sizes or overlaps;
 * HCA_ERR_WORKSPACE for a missing or short workspace.
 * Supported: fp32 and bf16, d_qk and d_v <= 512 (multiples of 4), any
 * h_q / h_kv, topk <= 4096.
 */
hca_status_t dsa_sparse_attn_bwd(hca_dtype_t dt,
                                 const void* q, hca_strides_t sq,
                                 const void* k, hca_strides_t sk,
                                 const void* v, hca_strides_t sv,
                                 const int32_t* idx,
                                 const void* o, hca_strides_t so,
                                 const float* lse,
                                 const void* dout, hca_strides_t sdout,
                                 float* dq, hca_strides_t sdq,
                                 float* dk, hca_strides_t sdk,
                                 float* dv, hca_strides_t sdv,
                                 int batch, int seqlen, int h_q, int h_kv, int d_qk, int d_v,
                                 int topk, float scale,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HCA_H_ */
