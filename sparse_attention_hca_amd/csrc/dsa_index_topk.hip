// DSA lightweight indexer and causal top-k (ERNIE 5.5 Flash Base pages:
// mirrorspeed page, "Hybrid sparse attention" section -- an indexer scores the
// historical positions of each query and core attention runs only on the
// top-k; ai-club.cn page, hybrid attention section, says the same).
//
//   s(t, u) = sum_h w[t,h] * max(0, <qI[t,h,:], kI[u,:]>),  u <= t, fp32
//
// Two kernels per chunk of query rows (the host walks the chunks so the score
// workspace stays bounded; with more than one chunk each chunk's selection
// runs on the library's second stream beside the next chunk's scores, the
// scores alternating between two buffers):
//   1. index_scores: fp32 matrix cores (v_mfma_f32_32x32x2_f32).  One wave
//      computes a 32-key x 32-query tile of S^T per index head and folds it
//      as w * relu(.) into the score tile; operands come straight from global
//      memory (every lane reads contiguous 16-byte runs), no LDS.
//   2. topk_select: one workgroup per query row.  Scores map to
//      order-preserving uint32 keys (-0 counts as +0).  Rows of 4096 keys or
//      more first bracket the k-th largest key with two order statistics of a
//      1024-key sample (256 spread groups of 4 adjacent keys); one pass over
//      the row emits the keys above the bracket and gathers those inside it
//      into LDS, where radix passes find the exact k-th largest key T.
//      Otherwise (short rows, or a bracket that missed) an 11-bit LDS
//      histogram locates the bin of T, one ordered pass emits everything above
//      that bin and gathers the bin, and 11- and 10-bit passes find T; rows
//      whose boundary bin is too large use four radix passes over the row.  A
//      bracket that holds the k-th key but too many candidates (a mass of
//      equal scores) first tries one histogram pass over the bracket: when the
//      k-th key's bin holds a single value, one ordered pass finishes.  In
//      every path keys > T and the lowest positions with key == T are emitted.
#include <mutex>

#include "device_common.h"
#include "launchers.h"

namespace hca {
namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int DI_MAX = 128;
// max(x, 0) as one integer max on the bits: a set sign bit (negative, -0)
// reads as a negative int and gives +0, a clear one keeps x (a float max would
// add a NaN-quieting instruction per value).
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

constexpr int QT = 32;   // queries per wave tile
constexpr int KT = 32;   // keys per wave tile
constexpr int WAVES = 4; // a workgroup covers 32 queries x 128 keys

struct ScoreParams {
  const float* qI;  // [S, h_i, d_i] of this batch
  const float* kI;  // [n_keys, d_i]
  const float* w;   // [S, h_i]
  float* sc;        // [rows, ld] scores of rows r0 .. r0+rows-1
  int64_t ld;
  int seqlen, h_i, d_i, r0, rows;
  // key u stands for positions block*u .. block*u + block - 1 and is visible
  // to query t when its last position is <= t (block 1: u <= t)
  int n_keys, block;
};

// Last key visible to query t (-1 when none).
__device__ __forceinline__ int last_key(const ScoreParams& p, int t) { return (t + 1) / p.block - 1; }

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
  if (k0 > last_key(p, t_last)) return;             // keys all in the future of every query
  const int col = lane & 31, hf = lane >> 5;
  constexpr int HALF = DI / 2;

  // A operand: this lane's key row, d in [hf*HALF, hf*HALF + HALF)
  const int key = min(k0 + col, p.n_keys - 1);
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
    for (int r = 0; r < 16; ++r) score[r] = fmaf(wh, relu(acc[r]), score[r]);
  }
  // lane holds query col, keys 8*(r/4) + 4*hf + (r%4): four runs of 4 consecutive keys
  const int qrow = qt0 + col;
  if (qrow >= p.rows) return;
  float* dst = p.sc + (int64_t)qrow * p.ld + k0 + 4 * hf;
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) {
    const int kk = k0 + 8 * rg + 4 * hf;
    if (kk < p.n_keys) {  // ld is a multiple of 4 and >= n_keys rounded up to 4
      f32x4 v = f32x4{score[4 * rg], score[4 * rg + 1], score[4 * rg + 2], score[4 * rg + 3]};
      *reinterpret_cast<f32x4*>(dst + 8 * rg) = v;
    }
  }
}

// Q-stationary variant for h_i * d_i / 2 <= 128: a wave keeps the B operands
// of its 32 queries (all index heads, 128 floats per lane at most) in
// registers and walks KG key tiles of 32, prefetching the next key tile's A
// operand while the current one runs.  Each query block's Q is then read once
// per KG key tiles instead of once per tile.  Two heads' MFMA chains are
// interleaved so consecutive MFMAs are independent.
constexpr int KG = 8;  // key tiles per wave

template <int DI, int HI>
__global__ __launch_bounds__(256) void index_scores_qs_kernel(ScoreParams p) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int qt0 = blockIdx.y * QT;                  // first query (chunk-relative)
  const int t0 = p.r0 + qt0;                        // absolute position
  const int t_last = min(t0 + QT, p.r0 + p.rows) - 1;
  const int kbase = (blockIdx.x * WAVES + w) * (KG * KT);
  const int k_last = last_key(p, t_last);
  if (kbase > k_last) return;                       // keys all in the future of every query
  const int col = lane & 31, hf = lane >> 5;
  constexpr int HALF = DI / 2;

  // B operands: this lane's query, d in [hf*HALF, hf*HALF + HALF), every head
  const int tq = min(t0 + col, p.seqlen - 1);
  float qb[HI][HALF];
  float wq[HI];
#pragma unroll
  for (int h = 0; h < HI; ++h) {
    const float* qsrc = p.qI + ((int64_t)tq * HI + h) * DI + hf * HALF;
#pragma unroll
    for (int i = 0; i < HALF; i += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(qsrc + i);
      qb[h][i] = v[0]; qb[h][i + 1] = v[1]; qb[h][i + 2] = v[2]; qb[h][i + 3] = v[3];
    }
    wq[h] = p.w[(int64_t)tq * HI + h];
  }
  // A operand of key tile kt: this lane's key row
  auto load_k = [&](int kt, float (&ka)[HALF]) __attribute__((always_inline)) {
    const int key = min(kbase + kt * KT + col, p.n_keys - 1);
    const float* src = p.kI + (int64_t)key * DI + hf * HALF;
#pragma unroll
    for (int i = 0; i < HALF; i += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + i);
      ka[i] = v[0]; ka[i + 1] = v[1]; ka[i + 2] = v[2]; ka[i + 3] = v[3];
    }
  };
  const int n_kt = min(KG, (k_last - kbase) / KT + 1);
  const int qrow = qt0 + col;
  // One key tile: two heads' MFMA chains at a time (independent, so
  // consecutive MFMAs do not wait on each other), each pair folded as
  // w * relu(.) into the score tile.
  auto tile = [&](int kt, const float (&ka)[HALF]) __attribute__((always_inline)) {
    f32x16_t score;
#pragma unroll
    for (int r = 0; r < 16; ++r) score[r] = 0.f;
#pragma unroll
    for (int h = 0; h < HI; h += 2) {
      f32x16_t a0, a1;
#pragma unroll
      for (int r = 0; r < 16; ++r) a0[r] = a1[r] = 0.f;
#pragma unroll
      for (int i = 0; i < HALF; ++i) {
        a0 = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[i], qb[h][i], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[i], qb[h + 1][i], a1, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        score[r] = fmaf(wq[h], relu(a0[r]), score[r]);
        score[r] = fmaf(wq[h + 1], relu(a1[r]), score[r]);
      }
    }
    // lane holds query col, keys 8*(r/4) + 4*hf + (r%4) of the tile
    const int k0 = kbase + kt * KT;
    if (qrow < p.rows) {
      float* dst = p.sc + (int64_t)qrow * p.ld + k0 + 4 * hf;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int kk = k0 + 8 * rg + 4 * hf;
        if (kk < p.n_keys) {  // ld is a multiple of 4 and >= n_keys rounded up to 4
          f32x4 v = f32x4{score[4 * rg], score[4 * rg + 1], score[4 * rg + 2], score[4 * rg + 3]};
          *reinterpret_cast<f32x4*>(dst + 8 * rg) = v;
        }
      }
    }
  };
  // two key-row register sets taken in turn (no copies); the next tile's rows
  // are loaded while the current tile runs
  float ka[HALF], kb[HALF];
  load_k(0, ka);
  // settle the prologue loads here: otherwise the loop's waits, placed for its
  // first iteration, would also hold every later iteration until the next
  // tile's prefetch has landed
#pragma unroll
  for (int h = 0; h < HI; ++h)
#pragma unroll
    for (int i = 0; i < HALF; ++i) asm volatile("" ::"v"(qb[h][i]));
#pragma unroll
  for (int i = 0; i < HALF; ++i) asm volatile("" ::"v"(ka[i]));
  for (int kt = 0; kt < n_kt; kt += 2) {
    load_k(min(kt + 1, n_kt - 1), kb);
    tile(kt, ka);
    if (kt + 1 >= n_kt) break;
    load_k(min(kt + 2, n_kt - 1), ka);
    tile(kt + 1, kb);
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
  int32_t* idx;     // [S, topk] of this batch (prefill rows) or [rows, topk] (decode rows)
  int r0, topk;
  // Decode rows (nseg > 0): row r holds keys seg * seg_len .. of sequence
  // r / nseg (seg = r % nseg; n_total keys in all), scores at sc + (r / nseg) * ld
  // + seg * seg_len.  Element u stands for position seg * seg_len + u, or for
  // pos[(r / nseg) * ld + seg * seg_len + u] when pos is given (then ascending
  // in u).  Prefill rows (nseg == 0): row r is query t = r0 + r over positions
  // 0 .. t.
  int nseg, seg_len, n_total;
  const int32_t* pos;
  // prefill rows: the candidates of query t are keys 0 .. (t + 1) / block - 1
  // (block <= 1: 0 .. t)
  int block;
};

constexpr int NB = 2048;   // bins of the general radix passes (11 + 11 + 10 bits)
constexpr int HB = 2048;   // bins of the first pass of the fast path (top 11 bits)
// candidates resolved in LDS; with HB this keeps the selection under 40 KB of
// LDS, so four workgroups share a CU
constexpr int CAP = 3840;
// The first stage of a decode selection runs few, long rows (65536 keys, k =
// 2048: the bracket admits ~3300 candidates with a spread of ~450, so about
// one row in ten would exceed CAP and take the multi-pass paths, and the
// slowest row sets the launch's time).  It uses this capacity instead (69 KB
// of LDS, two workgroups per CU).
constexpr int CAP_WIDE = 7680;

// Descending prefix over nb bins held in hist[] (256 threads, nb a multiple
// of 256): returns in sel[0] the bin holding the need-th largest element and in
// sel[1] the number of elements in higher bins.  Wave scans by lane shuffles,
// one LDS exchange of the wave totals (part[] holds 4 entries).
__device__ __forceinline__ void find_bin(const uint32_t* hist, int nb, uint32_t need, uint32_t* part,
                                         uint32_t* sel) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = nb / 256;
  uint32_t csum = 0;
  for (int j = 0; j < per; ++j) csum += hist[nb - 1 - (tid * per + j)];
  uint32_t x = csum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) part[w] = x;
  __syncthreads();
  uint32_t wbase = 0;
  for (int i = 0; i < w; ++i) wbase += part[i];
  const uint32_t incl = x + wbase, before = incl - csum;
  if (before < need && incl >= need) {
    uint32_t acc = before;
    for (int j = 0; j < per; ++j) {
      const uint32_t bin = nb - 1 - (tid * per + j);
      const uint32_t c = hist[bin];
      if (acc + c >= need) {
        sel[0] = bin;
        sel[1] = acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

// Ordered compaction helper: every thread of the workgroup has one flag; the
// flagged threads get consecutive ranks in thread order (wave ballots plus a
// cross-wave prefix in LDS).  Returns this thread's rank and the total.
__device__ __forceinline__ uint32_t ordered_rank(bool flag, uint32_t* wave_cnt, uint32_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint64_t m = __ballot(flag);
  const uint32_t below = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wave_cnt[w] = __popcll(m);
  __syncthreads();
  uint32_t off = 0;
  for (int i = 0; i < w; ++i) off += wave_cnt[i];
  total = wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
  __syncthreads();
  return off + below;
}

// Wave-aggregated LDS slot allocation: the flagged lanes of a wave get
// consecutive slots from *ctr (one atomic per wave).  Returns the lane's slot.
__device__ __forceinline__ uint32_t wave_alloc(bool flag, uint32_t* ctr) {
  const int lane = threadIdx.x & 63;
  const uint64_t m = __ballot(flag);
  uint32_t base = 0;
  const int leader = __ffsll((unsigned long long)m) - 1;
  if (m && lane == leader) base = atomicAdd(ctr, (uint32_t)__popcll(m));
  base = __builtin_amdgcn_readlane(base, leader < 0 ? 0 : leader);
  return base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
}

// Workgroup barrier that orders LDS accesses only: global loads in flight
// (the next step of a row scan) are not waited for.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Workgroup-wide exclusive prefixes, in thread order, of two per-thread
// counts in [0, 31] packed as a | b << 16 (ballots of the count bits; one LDS
// exchange).  Returns the packed prefix; total receives the packed sums.
__device__ __forceinline__ uint32_t wg_prefix2(uint32_t cnt, uint32_t* wave_cnt, uint32_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t pre = 0, wtot = 0;
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int bit = 0; bit < 5; ++bit) {
      const int sh = 16 * f + bit;
      const uint64_t m = __ballot((cnt >> sh) & 1u);
      pre += (uint32_t)__popcll(m & lt) << sh;
      wtot += (uint32_t)__popcll(m) << sh;
    }
  if (lane == 0) wave_cnt[w] = wtot;
  lds_barrier();
  uint32_t off = 0;
  for (int i = 0; i < w; ++i) off += wave_cnt[i];
  total = wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
  lds_barrier();
  return off + pre;
}

// The float F with okey(x) >= K  <=>  x >= F for every non-NaN x (IEEE
// compares; fp32 denormals are preserved in these kernels): the key's inverse
// image, -inf below the key of -inf and NaN (never true) above that of +inf.
__device__ __forceinline__ float key_ge_float(uint32_t K) {
  if (K <= 0x007fffffu) return -INFINITY;
  if (K > 0xff800000u) return __uint_as_float(0x7fc00000u);
  return __uint_as_float((K & 0x80000000u) ? (K & 0x7fffffffu) : ~K);
}

constexpr int NS = 1024;  // samples of a row used to bracket the k-th largest key

// One workgroup per query row: the k largest scores (ties to the lower
// position) of positions 0 .. t.
//   Fast path: an 11-bit histogram finds the bin B holding the k-th largest
//   key; one ordered pass emits every position above B and collects the
//   positions in B (in position order) into LDS; 11- and 10-bit passes over that
//   short list find the exact threshold key T; positions above T are emitted
//   and the lowest positions equal to T complete the set.  Two reads of the
//   row in all.
//   General path (bin B holds more than CAP positions, e.g. massive ties): three
//   radix passes over the row find T, then one ordered pass emits the set.
//   Long rows first try a sampling path: two order statistics of 1024 sampled
//   keys (256 spread groups of 4) bracket the k-th largest key; one pass emits
//   the keys above the bracket and collects the keys inside it (at most CAP),
//   where T and the tie-break are resolved in LDS.  When the bracket misses, the paths above run.
// POS: positions come from p.pos (the candidate rows of the decode merge)
// rather than being the element index; without it the row scans hold no
// load besides the row's own, so the next step's loads stay in flight while
// a step's elements are emitted.
// CAPN: the candidate capacity in LDS (CAP by default; see CAP_WIDE).
template <bool POS, int CAPN = CAP>
__global__ __launch_bounds__(256) void topk_select_kernel(SelectParams p) {
  static_assert(CAPN % 256 == 0 && CAPN >= 2048, "the candidate arrays double as 2048-bin tables");
  __shared__ uint32_t hist[HB];
  __shared__ uint32_t ckey[CAPN];
  __shared__ int cpos[CAPN];
  __shared__ uint32_t part[4];
  __shared__ uint32_t sel_info[4];
  __shared__ uint32_t wave_cnt[4];
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int k = p.topk;
  int n, off = 0;
  const float* srow;
  int32_t* out;
  const int32_t* prow = nullptr;
  if (p.nseg > 0) {
    const int b = row / p.nseg;
    off = (row % p.nseg) * p.seg_len;
    n = min(p.seg_len, p.n_total - off);
    srow = p.sc + (int64_t)b * p.ld + off;
    out = p.idx + (int64_t)row * k;
    if (POS) prow = p.pos + (int64_t)b * p.ld + off;
  } else {
    const int t = p.r0 + row;
    n = p.block > 1 ? (t + 1) / p.block : t + 1;
    srow = p.sc + (int64_t)row * p.ld;
    out = p.idx + (int64_t)t * k;
  }
  // position of element u (monotonic in u)
  auto P = [&](int u) __attribute__((always_inline)) { return POS ? prow[u] : u + off; };
  if (n <= k) {
    for (int j = tid; j < k; j += 256) out[j] = j < n ? P(j) : -1;
    return;
  }

  // ---- sampling path: bracket the k-th largest key with two order
  // statistics of a sample of 256 spread groups of 4 adjacent keys, then one
  // pass over the row emits the keys above the bracket and collects the keys
  // inside it; the exact threshold is resolved in LDS.
  if (n >= 4 * NS) {
    uint32_t* skey = hist;  // the sample lives in the histogram space
    {
      // 256 aligned groups of 4 adjacent keys (one 16-byte load per thread,
      // 256 cache lines of the row)
      const int u = (int)(((int64_t)tid * (n - 4) / 255) & ~3ll);
      const f32x4 x = *reinterpret_cast<const f32x4*>(srow + u);
#pragma unroll
      for (int j = 0; j < 4; ++j) skey[4 * tid + j] = okey(x[j]) >> 16;
    }
    if (tid == 0) sel_info[2] = sel_info[3] = 0;
    __syncthreads();
    // Bracket the k-th largest key between two order statistics of the
    // 1024-key sample (ranks r -+ delta, 3 standard deviations of the sample
    // rank of the row's k-th key plus 4), on the top 16 key bits: a coarser bracket
    // stays correct, it only admits a few more candidates.  A bracket that
    // misses the k-th key (a few rows in a thousand) or admits more than the
    // LDS list holds sends the row to the multi-pass paths; at 3.5 deviations
    // plus 6, one 65536-key row in twelve overflowed the 3840-entry list.  One wave per
    // statistic bisects over the whole sample (16 keys per lane, counts by
    // ballot): the largest T with #(sample >= T) >= rank + 1 is the sample key
    // of that rank (0 = largest).
    const int r = (int)((int64_t)k * NS / n);
    const int delta = (int)(3.0f * sqrtf((float)r * (1.f - (float)r / NS))) + 4;
    uint32_t hi = 0xffffffffu, lo = 0u;  // keys > hi are in, keys < lo are out
    {
      // wave 0 finds the upper statistic, wave 1 the lower one
      const int lane = tid & 63, wv = tid >> 6;
      if (wv < 2) {
        uint32_t sv[NS / 64];
#pragma unroll
        for (int j = 0; j < NS / 64; ++j) sv[j] = skey[lane + 64 * j];
        const int rank = wv == 0 ? r - delta : r + delta;
        uint32_t res = 0xffffffffu;
        if (rank >= 0 && rank < NS) {
          uint32_t t = 0;
          for (int bit = 15; bit >= 0; --bit) {
            const uint32_t cand = t | (1u << bit);
            uint32_t cnt = 0;
#pragma unroll
            for (int j = 0; j < NS / 64; ++j) cnt += (uint32_t)__popcll(__ballot(sv[j] >= cand));
            if (cnt >= (uint32_t)rank + 1) t = cand;
          }
          res = t;
        }
        if (lane == 0) wave_cnt[wv] = res;
      }
      lds_barrier();
      if (wave_cnt[0] != 0xffffffffu) hi = (wave_cnt[0] << 16) | 0xffffu;
      if (wave_cnt[1] != 0xffffffffu) lo = wave_cnt[1] << 16;
      lds_barrier();
    }
    {
      // Steps of 4096 elements: thread tid classifies elements
      // base + 1024e + 4tid + j (bit 4e + j of its masks) with two float
      // compares; a workgroup prefix of the mask counts gives every flagged
      // element its slot.  The loads of step s+1 are issued before step s is
      // classified.
      const float f_above = hi == 0xffffffffu ? __uint_as_float(0x7fc00000u) : key_ge_float(hi + 1u);
      const float f_in = key_ge_float(lo);
      uint32_t run_a = 0, run_i = 0;  // slots used so far (workgroup-uniform)
      auto classify = [&](const f32x4 v0, const f32x4 v1, const f32x4 v2, const f32x4 v3, int base)
                          __attribute__((always_inline)) {
        const f32x4 v[4] = {v0, v1, v2, v3};
        uint32_t fa = 0, fi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x = v[e][j];
            const bool above = x >= f_above;
            const bool in_or_above = x >= f_in;
            fa |= (uint32_t)above << (4 * e + j);
            fi |= (uint32_t)(in_or_above && !above) << (4 * e + j);
          }
        uint32_t tot;
        const uint32_t pre = wg_prefix2((uint32_t)__popc(fa) | ((uint32_t)__popc(fi) << 16), wave_cnt, tot);
        uint32_t oa = run_a + (pre & 0xffffu), oi = run_i + (pre >> 16);
        const int ub = base + 4 * tid;
        // emit: one iteration per flagged element of this thread
        for (uint32_t m = fa; m; m &= m - 1u) {
          const int bit = __builtin_ctz(m);
          if (oa < (uint32_t)k) out[oa] = P(ub + 1024 * (bit >> 2) + (bit & 3));
          ++oa;
        }
        for (uint32_t m = fi; m; m &= m - 1u) {
          const int bit = __builtin_ctz(m);
          // select the element by the bits of its index (no dynamic register indexing)
          const f32x4 h = (bit & 8) ? ((bit & 4) ? v3 : v2) : ((bit & 4) ? v1 : v0);
          const float x = (bit & 2) ? ((bit & 1) ? h[3] : h[2]) : ((bit & 1) ? h[1] : h[0]);
          if (oi < (uint32_t)CAPN) {
            ckey[oi] = okey(x);
            cpos[oi] = P(ub + 1024 * (bit >> 2) + (bit & 3));
          }
          ++oi;
        }
        run_a += tot & 0xffffu;
        run_i += tot >> 16;
      };
      // full steps: unguarded loads, those of step s+1 issued before step s
      // is classified, in two register sets taken in turn (no copies).  The
      // next step's loads are issued on every path (the last step re-reads
      // the final full step), so the wait before a classification counts
      // exactly the four loads issued after its own.
      const int n_full = n & ~4095;
      auto load_full = [&](int base, f32x4 (&v)[4]) __attribute__((always_inline)) {
        base = base < n_full - 4096 ? base : n_full - 4096;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = *reinterpret_cast<const f32x4*>(srow + base + 1024 * e + 4 * tid);
      };
      if (n_full > 0) {
        f32x4 va[4], vb[4];
        load_full(0, va);
        for (int base = 0; base < n_full; base += 8192) {
          load_full(base + 4096, vb);
          classify(va[0], va[1], va[2], va[3], base);
          if (base + 4096 >= n_full) break;
          load_full(base + 8192, va);
          classify(vb[0], vb[1], vb[2], vb[3], base + 4096);
        }
      }
      if (n_full < n) {
        // the partial step: keys past the row read as NaN, neither above nor inside
        f32x4 v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int u = n_full + 1024 * e + 4 * tid + j;
            v[e][j] = u < n ? srow[u] : __uint_as_float(0x7fc00000u);
          }
        classify(v[0], v[1], v[2], v[3], n_full);
      }
      if (tid == 0) {
        sel_info[2] = run_a;
        sel_info[3] = run_i;
      }
    }
    __syncthreads();
    const uint32_t c_hi = sel_info[2], nc = sel_info[3];
    if (c_hi < (uint32_t)k && nc <= (uint32_t)CAPN && c_hi + nc >= (uint32_t)k) {
      // exact threshold among the candidates: need-th largest key
      uint32_t need = (uint32_t)k - c_hi;
      uint32_t prefix = 0, pmask = 0;
      // every candidate lies in [lo, hi]: bits they all share need no pass
      int pass0 = 0;
      if ((lo >> 21) == (hi >> 21)) {
        prefix = hi & 0xffe00000u;
        pmask = 0xffe00000u;
        pass0 = 1;
      }
      for (int pass = pass0; pass < 3; ++pass) {
        const int sh = pass == 0 ? 21 : pass == 1 ? 10 : 0;
        const uint32_t nb = pass == 2 ? 1024u : 2048u;  // bits 31..21, 20..10, 9..0
        __syncthreads();
        for (int i = tid; i < (int)nb; i += 256) hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < (int)nc; i += 256)
          if ((ckey[i] & pmask) == prefix) atomicAdd(&hist[(ckey[i] >> sh) & (nb - 1)], 1u);
        __syncthreads();
        find_bin(hist, (int)nb, need, part, sel_info);
        need -= sel_info[1];
        prefix |= sel_info[0] << sh;
        pmask |= (nb - 1) << sh;
      }
      const uint32_t T = prefix;
      const uint32_t n_gt = (uint32_t)k - need;  // keys > T in the whole row
      // candidates above T go out directly; the slots of the candidates equal
      // to T are listed in hist (free now), then their positions gathered
      // into ckey[0, neq)
      __syncthreads();
      if (tid == 0) sel_info[2] = c_hi, sel_info[3] = 0;
      __syncthreads();
      for (int base = 0; base < (int)nc; base += 256) {
        const int i = base + tid;
        const bool valid = i < (int)nc;
        const uint32_t key = valid ? ckey[i] : 0u;
        const bool gt = valid && key > T;
        const uint32_t sa = wave_alloc(gt, &sel_info[2]);
        if (gt) out[sa] = cpos[i];
        const bool eq = valid && key == T;
        const uint32_t se = wave_alloc(eq, &sel_info[3]);
        if (eq && se < (uint32_t)NB) hist[se] = (uint32_t)i;
      }
      __syncthreads();
      if (sel_info[3] <= (uint32_t)NB) {
        const uint32_t ne = sel_info[3];
        uint32_t tp[NB / 256];  // ne <= NB here
#pragma unroll
        for (int j = 0; j < NB / 256; ++j) {
          const int i = tid + 256 * j;
          tp[j] = i < (int)ne ? (uint32_t)cpos[hist[i]] : 0u;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NB / 256; ++j)
          if (tid + 256 * j < (int)ne) ckey[tid + 256 * j] = tp[j];
      } else {
        // many ties: compact their positions in place, in steps of 256 (every
        // slot written in a step is below its end, i.e. already read)
        if (tid == 0) sel_info[3] = 0;
        __syncthreads();
        for (int base = 0; base < (int)nc; base += 256) {
          const int i = base + tid;
          const bool valid = i < (int)nc;
          const bool eq = valid && ckey[i] == T;
          const int pos = valid ? cpos[i] : 0;
          const uint32_t se = wave_alloc(eq, &sel_info[3]);
          __syncthreads();
          if (eq) ckey[se] = (uint32_t)pos;
          __syncthreads();
        }
      }
      __syncthreads();
      const uint32_t neq = sel_info[3];
      // the `need` lowest positions among the ties: need-th largest of ~position
      uint32_t pmax = 0xffffffffu;
      if (neq > need) {
        uint32_t nd = need, pre = 0, pm = 0;
        for (int pass = 0; pass < 3; ++pass) {
          const int sh = pass == 0 ? 21 : pass == 1 ? 10 : 0;
          const uint32_t nb = pass == 2 ? 1024u : 2048u;  // bits 31..21, 20..10, 9..0
          __syncthreads();
          for (int i = tid; i < (int)nb; i += 256) hist[i] = 0;
          __syncthreads();
          for (int i = tid; i < (int)neq; i += 256) {
            const uint32_t kp = ~ckey[i];
            if ((kp & pm) == pre) atomicAdd(&hist[(kp >> sh) & (nb - 1)], 1u);
          }
          __syncthreads();
          find_bin(hist, (int)nb, nd, part, sel_info);
          nd -= sel_info[1];
          pre |= sel_info[0] << sh;
          pm |= (nb - 1) << sh;
        }
        pmax = ~pre;  // the need-th lowest tied position
      }
      __syncthreads();
      if (tid == 0) sel_info[2] = n_gt;
      __syncthreads();
      for (int base = 0; base < (int)neq; base += 256) {
        const int i = base + tid;
        const bool take = i < (int)neq && ckey[i] <= pmax;
        const uint32_t sa = wave_alloc(take, &sel_info[2]);
        if (take) out[sa] = (int)ckey[i];
      }
      return;
    }
    if (c_hi < (uint32_t)k && c_hi + nc >= (uint32_t)k) {
      // The bracket holds the k-th key but more than CAP candidates (a mass of
      // equal scores, e.g. ReLU zeros).  One pass histograms the keys inside
      // [lo, hi] into 2048 bins of width 2^bs, with each bin's smallest and
      // largest key (in the free candidate arrays); when the bin holding the
      // k-th key has a single key value T, one ordered pass emits the bracket's
      // keys above T and the lowest positions equal to T.  Otherwise the general
      // path below runs.
      uint32_t* bmin = ckey;
      uint32_t* bmax = reinterpret_cast<uint32_t*>(cpos);
      const uint32_t span = hi - lo;
      int bs = 0;
      while ((span >> bs) >= 2048u) ++bs;
      __syncthreads();
      for (int i = tid; i < 2048; i += 256) {
        hist[i] = 0;
        bmin[i] = 0xffffffffu;
        bmax[i] = 0;
      }
      __syncthreads();
      auto add = [&](float x) __attribute__((always_inline)) {
        const uint32_t key = okey(x);
        if (key >= lo && key <= hi) {
          const uint32_t bin = (key - lo) >> bs;
          atomicAdd(&hist[bin], 1u);
          atomicMin(&bmin[bin], key);
          atomicMax(&bmax[bin], key);
        }
      };
      {
        const int n4 = n & ~3;
        for (int u = 4 * tid; u < n4; u += 1024) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(srow + u);
          add(v[0]);
          add(v[1]);
          add(v[2]);
          add(v[3]);
        }
        for (int u = n4 + tid; u < n; u += 256) add(srow[u]);
      }
      __syncthreads();
      find_bin(hist, 2048, (uint32_t)k - c_hi, part, sel_info);
      const uint32_t bt = sel_info[0], above = sel_info[1];
      const uint32_t T = bmin[bt];
      if (T == bmax[bt]) {
        const uint32_t need = (uint32_t)k - c_hi - above;  // taken from the keys equal to T
        __syncthreads();
        if (tid == 0) sel_info[2] = c_hi;
        __syncthreads();
        uint32_t eq_base = 0;
        for (int base = 0; base < n; base += 256) {
          const int u = base + tid;
          uint32_t key = 0;
          const bool valid = u < n;
          if (valid) key = okey(srow[u]);
          if (valid && key > T && key <= hi) out[atomicAdd(&sel_info[2], 1u)] = P(u);
          uint32_t tot;
          const bool eq = valid && key == T;
          const uint32_t r = ordered_rank(eq, wave_cnt, tot);
          if (eq && eq_base + r < need) out[c_hi + above + eq_base + r] = P(u);
          eq_base += tot;
        }
        return;
      }
    }
    __syncthreads();
  }

  // ---- pass 1: histogram of the top 11 bits
  for (int i = tid; i < HB; i += 256) hist[i] = 0;
  if (tid == 0) sel_info[2] = 0;
  __syncthreads();
  {
    const int n4 = n & ~3;
    for (int u = 4 * tid; u < n4; u += 1024) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(srow + u);
      atomicAdd(&hist[okey(v[0]) >> 21], 1u);
      atomicAdd(&hist[okey(v[1]) >> 21], 1u);
      atomicAdd(&hist[okey(v[2]) >> 21], 1u);
      atomicAdd(&hist[okey(v[3]) >> 21], 1u);
    }
    for (int u = n4 + tid; u < n; u += 256) atomicAdd(&hist[okey(srow[u]) >> 21], 1u);
  }
  __syncthreads();
  find_bin(hist, HB, (uint32_t)k, part, sel_info);
  const uint32_t B = sel_info[0];
  const uint32_t above_b = sel_info[1];
  const uint32_t in_b = hist[B];

  if (in_b <= (uint32_t)CAPN) {
    // ---- pass 2: emit bins above B, collect bin B in position order
    uint32_t nc = 0;
    for (int base = 0; base < n; base += 256) {
      const int u = base + tid;
      uint32_t key = 0;
      const bool valid = u < n;
      if (valid) key = okey(srow[u]);
      const uint32_t bin = key >> 21;
      if (valid && bin > B) out[atomicAdd(&sel_info[2], 1u)] = P(u);
      uint32_t tot;
      const bool inb = valid && bin == B;
      const uint32_t r = ordered_rank(inb, wave_cnt, tot);
      if (inb) {
        ckey[nc + r] = key;
        cpos[nc + r] = P(u);
      }
      nc += tot;
    }
    __syncthreads();
    // ---- resolve the threshold among the nc = in_b candidates (bits 20..10, 9..0)
    uint32_t need = (uint32_t)k - above_b;
    uint32_t prefix = B << 21, pmask = 0xffe00000u;
    for (int pass = 0; pass < 2; ++pass) {
      const int sh = pass == 0 ? 10 : 0;
      const uint32_t nb = pass == 0 ? 2048u : 1024u;
      for (int i = tid; i < (int)nb; i += 256) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < (int)nc; i += 256)
        if ((ckey[i] & pmask) == prefix) atomicAdd(&hist[(ckey[i] >> sh) & (nb - 1)], 1u);
      __syncthreads();
      find_bin(hist, (int)nb, need, part, sel_info);
      need -= sel_info[1];
      prefix |= sel_info[0] << sh;
      pmask |= (nb - 1) << sh;
      __syncthreads();
    }
    const uint32_t T = prefix;
    const uint32_t n_gt = (uint32_t)k - need;  // keys > T, all emitted below
    // candidates above T (unordered), then the `need` lowest positions equal to T
    uint32_t eq_base = 0;
    for (int base = 0; base < (int)nc; base += 256) {
      const int i = base + tid;
      const bool valid = i < (int)nc;
      const uint32_t key = valid ? ckey[i] : 0u;
      if (valid && key > T) out[atomicAdd(&sel_info[2], 1u)] = cpos[i];
      uint32_t tot;
      const bool eq = valid && key == T;
      const uint32_t r = ordered_rank(eq, wave_cnt, tot);
      if (eq && eq_base + r < need) out[n_gt + eq_base + r] = cpos[i];
      eq_base += tot;
    }
    return;
  }

  // ---- general path: radix passes over the row (bits [31:21], [20:10], [9:0])
  uint32_t prefix = 0, prefix_mask = 0;
  uint32_t need = (uint32_t)k;
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
    find_bin(hist, (int)nb, need, part, sel_info);
    need -= sel_info[1];
    prefix |= sel_info[0] << sh;
    prefix_mask |= (nb - 1) << sh;
    __syncthreads();
  }
  // prefix is now the exact threshold key T; take every key > T and the `need`
  // lowest positions with key == T
  const uint32_t T = prefix;
  const uint32_t n_above = (uint32_t)k - need;
  if (tid == 0) sel_info[2] = 0;
  __syncthreads();
  uint32_t eq_base = 0;
  for (int base = 0; base < n; base += 256) {
    const int u = base + tid;
    uint32_t key = 0;
    const bool valid = u < n;
    if (valid) key = okey(srow[u]);
    if (valid && key > T) out[atomicAdd(&sel_info[2], 1u)] = P(u);
    uint32_t tot;
    const bool eq = valid && key == T;
    const uint32_t r = ordered_rank(eq, wave_cnt, tot);
    if (eq && eq_base + r < need) out[n_above + eq_base + r] = P(u);
    eq_base += tot;
  }
}

// ---- decode: one query per sequence over n keys.
// Scores stream the key rows (HBM-bound: 4 * d_i bytes per key); the query's
// operands sit in LDS and are read as broadcasts.
template <int DI, int HI>
__global__ __launch_bounds__(256) void decode_scores_kernel(const float* qI, const float* kI, const float* w,
                                                            float* sc, int64_t ld, int n) {
  __shared__ __attribute__((aligned(16))) float qs[HI * DI];
  __shared__ float wsh[HI];
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  for (int i = tid; i < HI * DI; i += 256) qs[i] = qI[(int64_t)b * HI * DI + i];
  if (tid < HI) wsh[tid] = w[(int64_t)b * HI + tid];
  __syncthreads();
  const int u = blockIdx.x * 256 + tid;
  if (u >= n) return;
  const float* kr = kI + ((int64_t)b * n + u) * DI;
  float acc[HI];
#pragma unroll
  for (int h = 0; h < HI; ++h) acc[h] = 0.f;
#pragma unroll
  for (int c = 0; c < DI; c += 4) {
    const f32x4 kv = *reinterpret_cast<const f32x4*>(kr + c);
#pragma unroll
    for (int h = 0; h < HI; ++h) {
      const f32x4 qv = *reinterpret_cast<const f32x4*>(qs + h * DI + c);
      acc[h] = fmaf(kv[0], qv[0], acc[h]);
      acc[h] = fmaf(kv[1], qv[1], acc[h]);
      acc[h] = fmaf(kv[2], qv[2], acc[h]);
      acc[h] = fmaf(kv[3], qv[3], acc[h]);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int h = 0; h < HI; ++h) s = fmaf(wsh[h], relu(acc[h]), s);
  sc[(int64_t)b * ld + u] = s;
}

// The same scores for 64-wide index keys with whole-line loads: each wave
// covers 64 keys in 8 blocks of 8, eight lanes per key; load c of a block
// reads dims 32c .. 32c+31 of its 8 keys (lane l: key l/8, dims 32c + 4(l%8)
// .. +3), so every instruction reads 8 whole 128-byte lines, which no other
// instruction touches: the loads are non-temporal.  The eight partial dot
// products of a key are summed across its lane octet.
template <int HI>
__global__ __launch_bounds__(256) void decode_scores64_kernel(const float* qI, const float* kI, const float* w,
                                                              float* sc, int64_t ld, int n) {
  constexpr int DI = 64;
  __shared__ __attribute__((aligned(16))) float qs[HI * DI];
  __shared__ float wsh[HI];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w4 = tid >> 6;
  for (int i = tid; i < HI * DI; i += 256) qs[i] = qI[(int64_t)b * HI * DI + i];
  if (tid < HI) wsh[tid] = w[(int64_t)b * HI + tid];
  __syncthreads();
  const int key0 = blockIdx.x * 256 + 64 * w4;
  if (key0 >= n) return;
  const int p8 = lane & 7;
  float acc[8][HI];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb)
#pragma unroll
    for (int h = 0; h < HI; ++h) acc[kb][h] = 0.f;
  f32x4 kv[8][2];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    const int u = min(key0 + 8 * kb + (lane >> 3), n - 1);
    const float* kr = kI + ((int64_t)b * n + u) * DI + 4 * p8;
#pragma unroll
    for (int c = 0; c < 2; ++c) kv[kb][c] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(kr + 32 * c));
  }
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int h = 0; h < HI; ++h) {
      const f32x4 qv = *reinterpret_cast<const f32x4*>(qs + h * DI + 32 * c + 4 * p8);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        acc[kb][h] = fmaf(kv[kb][c][0], qv[0], acc[kb][h]);
        acc[kb][h] = fmaf(kv[kb][c][1], qv[1], acc[kb][h]);
        acc[kb][h] = fmaf(kv[kb][c][2], qv[2], acc[kb][h]);
        acc[kb][h] = fmaf(kv[kb][c][3], qv[3], acc[kb][h]);
      }
    }
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    float s = 0.f;
#pragma unroll
    for (int h = 0; h < HI; ++h) {
      float a = acc[kb][h];
      a += __shfl_xor(a, 1);
      a += __shfl_xor(a, 2);
      a += __shfl_xor(a, 4);
      s = fmaf(wsh[h], relu(a), s);
    }
    const int u = key0 + 8 * kb + (lane >> 3);
    if (p8 == 0 && u < n) sc[(int64_t)b * ld + u] = s;
  }
}

constexpr int SEG = 65536;  // keys per first-stage row of a decode selection

// The first stage leaves, per (sequence, segment), the segment's selected
// positions in no particular order.  One workgroup per (sequence, segment)
// marks them in an LDS bitmap and writes them back in ascending order with
// their scores, at offset seg * k of the sequence's candidate row: every
// segment but the last contributes exactly k, so the rows are contiguous.
__global__ __launch_bounds__(256) void decode_compact_kernel(const int32_t* sel, const float* sc, int64_t ld, int nseg,
                                                             int n_total, int k, float* cand_sc, int32_t* cand_pos,
                                                             int64_t ld2) {
  __shared__ uint32_t bits[SEG / 32];
  __shared__ uint32_t part[256];
  const int tid = threadIdx.x;
  const int row = blockIdx.x, b = row / nseg, seg = row % nseg;
  const int off = seg * SEG;
  for (int i = tid; i < SEG / 32; i += 256) bits[i] = 0;
  __syncthreads();
  for (int j = tid; j < k; j += 256) {
    const int pz = sel[(int64_t)row * k + j];
    if (pz >= 0) atomicOr(&bits[(pz - off) >> 5], 1u << ((pz - off) & 31));
  }
  __syncthreads();
  // thread tid owns words 8 tid .. 8 tid + 7
  constexpr int WPT = SEG / 32 / 256;
  uint32_t cnt = 0;
#pragma unroll
  for (int i = 0; i < WPT; ++i) cnt += __popc(bits[WPT * tid + i]);
  part[tid] = cnt;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const uint32_t x = tid >= d ? part[tid - d] : 0u;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  uint32_t o = part[tid] - cnt;
  const int64_t base = (int64_t)b * ld2 + (int64_t)seg * k;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    uint32_t m = bits[WPT * tid + i];
    while (m) {
      const int pz = off + 32 * (WPT * tid + i) + __builtin_ctz(m);
      m &= m - 1u;
      cand_pos[base + o] = pz;
      cand_sc[base + o] = sc[(int64_t)b * ld + pz];
      ++o;
    }
  }
}

// Query rows per chunk of score rows of row_len keys: keep one chunk near 1 GB
// (few, large launches fill the GPU), at most all n_rows rows.
int chunk_rows(int n_rows, int row_len) {
  int64_t r = ((int64_t)1 << 28) / (((int64_t)row_len + 3) & ~3ll);
  if (r < 32) r = 32;
  r = r / 32 * 32;
  if (r > n_rows) r = ((n_rows + 31) / 32) * 32;
  return (int)r;
}

int64_t score_ld(int n_keys) { return ((int64_t)n_keys + 127) / 128 * 128; }

// Number of score chunks of a call: the workspace holds two chunk buffers
// when there is more than one, so that the selection of one chunk runs beside
// the scores of the next.
int64_t n_chunks(int batch, int seqlen, int R) { return (int64_t)batch * ((seqlen + R - 1) / R); }

// Events of the indexer's chunk pipeline, created once per device on first use.
struct IndexEvents {
  bool ready = false;
  hipEvent_t sc[2] = {nullptr, nullptr};   // scores of buffer i written (recorded on the caller's stream)
  hipEvent_t sel[2] = {nullptr, nullptr};  // selection of buffer i done (recorded on the side stream)
};
std::mutex g_index_mu;
IndexEvents g_index_ev[64];

hipError_t index_events(IndexEvents*& out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  IndexEvents& ev = g_index_ev[dev];
  if (!ev.ready) {
    for (int i = 0; i < 2 && e == hipSuccess; ++i) {
      e = hipEventCreateWithFlags(&ev.sc[i], hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&ev.sel[i], hipEventDisableTiming);
    }
    if (e != hipSuccess) return e;
    ev.ready = true;
  }
  out = &ev;
  return hipSuccess;
}

// Scores + selection of seqlen queries over n_keys keys of granularity block
// (DSA: n_keys = seqlen, block = 1), in chunks of query rows.  With more than
// one chunk the scores run on the caller's stream into two alternating
// buffers and each chunk's selection runs on the side stream as soon as its
// scores are written: the selection (memory-latency bound) overlaps the next
// chunk's scores (matrix cores).  A buffer is rewritten only after the
// selection that read it is done, and the caller's stream waits for the last
// selection before anything queued after this call.  Enqueueing holds a lock,
// so concurrent callers share the side stream in turn.
hipError_t launch_index_topk_rows(const float* qI, const float* kI, const float* w, int32_t* idx, int batch,
                                  int seqlen, int n_keys, int block, int h_i, int d_i, int topk, void* ws,
                                  hipStream_t st) {
  const int64_t ld = score_ld(n_keys);
  const int R = chunk_rows(seqlen, n_keys);
  const bool overlap = n_chunks(batch, seqlen, R) > 1;
  std::unique_lock<std::mutex> lock(g_index_mu, std::defer_lock);
  IndexEvents* ev = nullptr;
  hipStream_t side = nullptr;
  if (overlap) {
    lock.lock();
    hipError_t e = index_events(ev);
    if (e == hipSuccess) e = side_stream(&side);
    if (e != hipSuccess) return e;
  }
  int c = 0;  // chunk counter over the call
  for (int b = 0; b < batch; ++b) {
    for (int r0 = 0; r0 < seqlen; r0 += R, ++c) {
      const int rows = min(R, seqlen - r0);
      float* buf = (float*)ws + (overlap ? (size_t)(c & 1) * (size_t)R * (size_t)ld : 0);
      hipStream_t sel_st = st;
      if (overlap) {
        // the selection that last read this buffer is done
        hipError_t e = hipStreamWaitEvent(st, ev->sel[c & 1], 0);
        if (e != hipSuccess) return e;
      }
      ScoreParams sp;
      sp.qI = qI + (int64_t)b * seqlen * h_i * d_i;
      sp.kI = kI + (int64_t)b * n_keys * d_i;
      sp.w = w + (int64_t)b * seqlen * h_i;
      sp.sc = buf;
      sp.ld = ld;
      sp.seqlen = seqlen;
      sp.h_i = h_i;
      sp.d_i = d_i;
      sp.r0 = r0;
      sp.rows = rows;
      sp.n_keys = n_keys;
      sp.block = block;
      // keys visible to the chunk's last query
      const int keys = min(n_keys, (r0 + rows) / block);
      if (keys > 0) {
        const int key_tiles = (keys + KT * WAVES - 1) / (KT * WAVES);
        dim3 grid(key_tiles, (rows + QT - 1) / QT);
        const dim3 grid_qs((keys + KT * WAVES * KG - 1) / (KT * WAVES * KG), (rows + QT - 1) / QT);
        bool qs = true;
        if (h_i == 4 && d_i == 16) hipLaunchKernelGGL((index_scores_qs_kernel<16, 4>), grid_qs, dim3(256), 0, st, sp);
        else if (h_i == 4 && d_i == 32) hipLaunchKernelGGL((index_scores_qs_kernel<32, 4>), grid_qs, dim3(256), 0, st, sp);
        else if (h_i == 4 && d_i == 48) hipLaunchKernelGGL((index_scores_qs_kernel<48, 4>), grid_qs, dim3(256), 0, st, sp);
        else if (h_i == 4 && d_i == 64) hipLaunchKernelGGL((index_scores_qs_kernel<64, 4>), grid_qs, dim3(256), 0, st, sp);
        else if (h_i == 8 && d_i == 16) hipLaunchKernelGGL((index_scores_qs_kernel<16, 8>), grid_qs, dim3(256), 0, st, sp);
        else if (h_i == 8 && d_i == 32) hipLaunchKernelGGL((index_scores_qs_kernel<32, 8>), grid_qs, dim3(256), 0, st, sp);
        else qs = false;
        if (!qs) switch (d_i) {
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
      }
      if (overlap) {
        hipError_t e = hipEventRecord(ev->sc[c & 1], st);
        if (e == hipSuccess) e = hipStreamWaitEvent(side, ev->sc[c & 1], 0);
        if (e != hipSuccess) return e;
        sel_st = side;
      }
      SelectParams pp{};
      pp.sc = buf;
      pp.ld = ld;
      pp.idx = idx + (int64_t)b * seqlen * topk;
      pp.r0 = r0;
      pp.topk = topk;
      pp.block = block;
      hipLaunchKernelGGL(topk_select_kernel<false>, dim3(rows), dim3(256), 0, sel_st, pp);
      hipError_t e = hipGetLastError();
      if (e == hipSuccess && overlap) e = hipEventRecord(ev->sel[c & 1], side);
      if (e != hipSuccess) return e;
    }
  }
  if (overlap) {
    // the caller's stream sees every selection (the side stream runs them in order)
    hipError_t e = hipStreamWaitEvent(st, ev->sel[(c - 1) & 1], 0);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t side_stream(hipStream_t* out) {
  static std::mutex mu;
  static hipStream_t streams[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!streams[dev]) {
    e = hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking);
    if (e != hipSuccess) {
      streams[dev] = nullptr;
      return e;
    }
  }
  *out = streams[dev];
  return hipSuccess;
}

size_t dsa_topk_workspace_bytes(int batch, int seqlen, int topk) {
  (void)topk;
  const int R = chunk_rows(seqlen, seqlen);
  return (n_chunks(batch, seqlen, R) > 1 ? 2 : 1) * (size_t)R * score_ld(seqlen) * sizeof(float);
}

hipError_t launch_dsa_index_topk(const float* qI, const float* kI, const float* w, int32_t* idx, int batch,
                                 int seqlen, int h_i, int d_i, int topk, void* ws, size_t ws_bytes, hipStream_t st) {
  (void)ws_bytes;
  return launch_index_topk_rows(qI, kI, w, idx, batch, seqlen, seqlen, 1, h_i, d_i, topk, ws, st);
}

size_t csa_topk_workspace_bytes(int batch, int seqlen, int n_keys, int topk) {
  (void)topk;
  const int R = chunk_rows(seqlen, n_keys);
  return (n_chunks(batch, seqlen, R) > 1 ? 2 : 1) * (size_t)R * score_ld(n_keys) * sizeof(float);
}

hipError_t launch_csa_index_topk(const float* qI, const float* kIc, const float* w, int32_t* idx, int batch,
                                 int seqlen, int n_keys, int block, int h_i, int d_i, int topk, void* ws,
                                 hipStream_t st) {
  return launch_index_topk_rows(qI, kIc, w, idx, batch, seqlen, n_keys, block, h_i, d_i, topk, ws, st);
}

size_t dsa_topk_decode_workspace_bytes(int batch, int n_keys, int topk) {
  const int64_t ld = ((int64_t)n_keys + 127) / 128 * 128;
  const int64_t nseg = ((int64_t)n_keys + SEG - 1) / SEG;
  const int64_t ld2 = (nseg * topk + 127) / 128 * 128;
  size_t bytes = (size_t)batch * ld * sizeof(float);                                // scores
  if (nseg > 1) {
    bytes += ((size_t)batch * nseg * topk * sizeof(int32_t) + 255) / 256 * 256;     // first-stage selections
    bytes += (size_t)batch * ld2 * (sizeof(float) + sizeof(int32_t));                // ordered candidates
  }
  return bytes;
}

hipError_t launch_dsa_index_topk_decode(const float* qI, const float* kI, const float* w, int32_t* idx, int batch,
                                        int n_keys, int h_i, int d_i, int topk, void* ws, hipStream_t st) {
  const int64_t ld = ((int64_t)n_keys + 127) / 128 * 128;
  const int nseg = (n_keys + SEG - 1) / SEG;
  const int64_t ld2 = ((int64_t)nseg * topk + 127) / 128 * 128;
  float* sc = (float*)ws;
  const dim3 gs((n_keys + 255) / 256, batch);
#define HCA_DEC_SCORES(DI_, HI_) hipLaunchKernelGGL((decode_scores_kernel<DI_, HI_>), gs, dim3(256), 0, st, qI, kI, w, sc, ld, n_keys)
  bool ok = true;
  if (h_i == 4) {
    switch (d_i) {
      case 16: HCA_DEC_SCORES(16, 4); break;
      case 32: HCA_DEC_SCORES(32, 4); break;
      case 48: HCA_DEC_SCORES(48, 4); break;
      case 64: hipLaunchKernelGGL((decode_scores64_kernel<4>), gs, dim3(256), 0, st, qI, kI, w, sc, ld, n_keys); break;
      case 80: HCA_DEC_SCORES(80, 4); break;
      case 96: HCA_DEC_SCORES(96, 4); break;
      case 112: HCA_DEC_SCORES(112, 4); break;
      case 128: HCA_DEC_SCORES(128, 4); break;
      default: ok = false;
    }
  } else if (h_i == 8) {
    switch (d_i) {
      case 16: HCA_DEC_SCORES(16, 8); break;
      case 32: HCA_DEC_SCORES(32, 8); break;
      case 48: HCA_DEC_SCORES(48, 8); break;
      case 64: hipLaunchKernelGGL((decode_scores64_kernel<8>), gs, dim3(256), 0, st, qI, kI, w, sc, ld, n_keys); break;
      case 80: HCA_DEC_SCORES(80, 8); break;
      case 96: HCA_DEC_SCORES(96, 8); break;
      case 112: HCA_DEC_SCORES(112, 8); break;
      case 128: HCA_DEC_SCORES(128, 8); break;
      default: ok = false;
    }
  } else {
    ok = false;
  }
#undef HCA_DEC_SCORES
  if (!ok) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // first stage: exact top-k of every segment of SEG keys (the whole row when
  // it fits one segment, written straight to idx)
  int32_t* sel = nseg > 1 ? (int32_t*)(sc + (size_t)batch * ld) : idx;
  SelectParams s1{};
  s1.sc = sc;
  s1.ld = ld;
  s1.idx = sel;
  s1.topk = topk;
  s1.nseg = nseg;
  s1.seg_len = SEG;
  s1.n_total = n_keys;
  hipLaunchKernelGGL((topk_select_kernel<false, CAP_WIDE>), dim3(batch * nseg), dim3(256), 0, st, s1);
  e = hipGetLastError();
  if (e != hipSuccess || nseg == 1) return e;
  // second stage: the segments' selections, in position order, hold the top-k
  // of the whole row (each of its members is in its segment's top-k)
  // the candidate rows start on a 256-byte boundary (16-byte loads)
  float* cand_sc = (float*)((char*)sel + ((size_t)batch * nseg * topk * sizeof(int32_t) + 255) / 256 * 256);
  int32_t* cand_pos = (int32_t*)(cand_sc + (size_t)batch * ld2);
  hipLaunchKernelGGL(decode_compact_kernel, dim3(batch * nseg), dim3(256), 0, st, sel, sc, ld, nseg, n_keys, topk,
                     cand_sc, cand_pos, ld2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int last = n_keys - (nseg - 1) * SEG;
  const int n2 = (nseg - 1) * topk + (last < topk ? last : topk);
  SelectParams s2{};
  s2.sc = cand_sc;
  s2.ld = ld2;
  s2.idx = idx;
  s2.topk = topk;
  s2.nseg = 1;
  s2.seg_len = n2;
  s2.n_total = n2;
  s2.pos = cand_pos;
  hipLaunchKernelGGL(topk_select_kernel<true>, dim3(batch), dim3(256), 0, st, s2);
  return hipGetLastError();
}

}  // namespace hca
