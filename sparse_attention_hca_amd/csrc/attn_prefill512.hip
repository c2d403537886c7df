// HCA prefill attention for bf16, head_dim 512, on CDNA4 matrix cores.
//
// Operation (ERNIE 5.5 Flash Base pages: mirrorspeed page, "Hybrid sparse
// attention" section; ai-club.cn page, hybrid attention section): query t
// attends densely over the compressed entries j < n_c(t) = floor(lo(t)/block)
// and the raw window [lo(t), t], lo(t) = max(0, t - W + 1), with 512-wide
// heads.
//
// Design (one workgroup = 4 waves = 128 consecutive queries of one head; one
// wave per SIMD with the whole 512-entry register file):
//   * Each wave owns 32 queries.  Q^T stays in registers as the B operand of
//     S^T = K Q^T (v_mfma_f32_32x32x16_bf16, 32 k-steps over d = 512) and the
//     O^T accumulators (512 dims x 32 queries, fp32) take 256 registers.
//     32 queries per wave halve the LDS bytes read per MFMA flop compared
//     with 16, which keeps the operand reads well under LDS bandwidth.
//   * Keys stream in tiles of 32 (compressed entries first, then the raw
//     window band).  Both K and V rows go global -> LDS with 16-byte LDS DMA,
//     one 1-KB row per wave instruction, double-buffered one tile ahead; one
//     barrier per tile.
//   * K rows are stored with a 16-byte pad (row stride 1040 B): the 16-byte
//     A-operand reads of 16 consecutive keys then hit 16 distinct bank
//     groups.  V rows are padded by 64 B (stride 1088 B) and read with the
//     gfx950 transposing LDS load (ds_read_b64_tr_b16), which hands each lane
//     four consecutive keys of one dim: exactly the V^T A operand of
//     O^T = V^T P^T, with no register transpose.  With that stride the four
//     rows x four 16-byte chunks read by 32 lanes fall in 16 distinct bank
//     groups.
//   * The S^T accumulator of a lane (one query, 16 keys) is the P^T operand
//     once converted to bf16; the V^T reads fetch the keys in the matching
//     order, so no data moves between lanes.
//   * Online softmax in fp32 (log2 domain) with a lazy rescale: the reference
//     maximum only moves when a tile exceeds it by more than 2^8, so O is
//     rescaled rarely and exactly (the final normalisation uses the same
//     reference).
//   * Workgroup ids are remapped so each XCD receives a contiguous range of
//     (head, query tile) work: same-head tiles share that XCD's L2 for the
//     compressed cache.  Within a head, the longest query tiles go first.
#include "device_common.h"
#include "launchers.h"
#include "mfma_asm.h"

namespace hca {
namespace {

constexpr int D = 512;
constexpr int BM = 128;             // queries per workgroup
constexpr int WQ = 32;              // queries per wave
constexpr int NWAVE = 4;
constexpr int BN = 32;              // keys per tile
constexpr int KROW = 2 * D + 16;    // LDS bytes per K row
constexpr int VROW = 2 * D + 64;    // LDS bytes per V row
constexpr int KST = BN * KROW;      // K stage bytes
constexpr int VST = BN * VROW;      // V stage bytes
constexpr int STAGE = KST + VST;
constexpr float kGuard = 64.f;  // log2 headroom of the fixed softmax reference

struct PrefillParams {
  AttnArgs a;
  int n_qt;   // query tiles per (batch, head)
  int total;  // batch * h_q * n_qt
  float c;    // scale * log2(e)
};

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void prefill512_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];
  __shared__ int redo_flag;

  const AttnArgs& a = p.a;
  const int L = xcd_remap(blockIdx.x, p.total);
  if (L < 0) return;
  const int qt = p.n_qt - 1 - (L % p.n_qt);
  const int bh = L / p.n_qt;
  const int h = bh % a.h_q;
  const int b = bh / a.h_q;
  const int g = h / (a.h_q / a.h_kv);

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar: everything derived from it stays in SGPRs
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hf = lane >> 5;
  const int W = a.window, blk = a.block;

  // Positions fit in 32 bits (checked by the host before launch).
  const int qp0 = (int)a.q_pos0, kvp0 = (int)a.kv_pos0;
  const int i0 = qt * BM;
  const int i_last = min(i0 + BM, a.seqlen_q) - 1;
  const int t_first = qp0 + i0, t_last = qp0 + i_last;
  const int lo_first = max(0, t_first - W + 1);
  const int nc_max = max(0, t_last - W + 1) / blk;
  const int n_ct = (nc_max + BN - 1) / BN;
  const int n_wt = (t_last - lo_first + BN) / BN;
  const int ntiles = n_ct + n_wt;

  // this lane's query (rows past the end read the last row and are never stored)
  const int iq = i0 + WQ * w + col;
  const bool qvalid = iq < a.seqlen_q;
  const int tq = qp0 + iq;
  const int lo_q = max(0, tq - W + 1);
  const int nc_q = lo_q / blk;
  // this wave's query range: tiles nobody in the wave sees are skipped, tiles
  // every query of the wave sees entirely need no mask
  const int iw0 = i0 + WQ * w;
  const int iw1 = min(iw0 + WQ - 1, i_last);
  const bool wave_has_q = iw0 <= i_last;
  const bool wave_full = iw0 + WQ - 1 <= i_last;
  const int tw0 = qp0 + iw0, tw1 = qp0 + iw1;
  const int lo_w0 = max(0, tw0 - W + 1), lo_w1 = max(0, tw1 - W + 1);
  const int nc_w0 = lo_w0 / blk, nc_w1 = lo_w1 / blk;

  // ---- Q^T fragments (B operand): lane holds query `col`, dims 16ks + 8hf .. +8
  bf16x8 qf[32];
  {
    const uint16_t* qp = (const uint16_t*)a.q + b * a.sq.b + (int64_t)min(iq, a.seqlen_q - 1) * a.sq.s +
                         (int64_t)h * a.sq.h + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, ld16(qp + 16 * ks));
    // settle the Q loads before the DMA pipeline (its waits are explicit)
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

  const uint16_t* kcb = (const uint16_t*)a.kc + b * a.skc.b + (int64_t)g * a.skc.h;
  const uint16_t* kb = (const uint16_t*)a.k + b * a.sk.b + (int64_t)g * a.sk.h;
  const uint16_t* vcb = (const uint16_t*)a.vc + b * a.svc.b + (int64_t)g * a.svc.h;
  const uint16_t* vb = (const uint16_t*)a.v + b * a.sv.b + (int64_t)g * a.sv.h;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)smem;

  // ---- DMA of tile tt into stage st: wave w copies K rows and V rows 8w .. 8w+7.
  // Rows past the valid range re-read the last valid row: their logits are
  // masked and their probabilities are exactly 0.
  auto issue = [&](int tt, int st) __attribute__((always_inline)) {
    const uint16_t *kbase, *vbase;
    int64_t ks_, vs_;
    int row0, row_max;
    if (tt < n_ct) {
      kbase = kcb; vbase = vcb; ks_ = a.skc.s; vs_ = a.svc.s; row0 = tt * BN; row_max = nc_max - 1;
    } else {
      kbase = kb; vbase = vb; ks_ = a.sk.s; vs_ = a.sv.s;
      row0 = lo_first + (tt - n_ct) * BN - kvp0; row_max = t_last - kvp0;
    }
    const uint32_t kl = lds0 + st * STAGE, vl = kl + KST;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * w + i;
      const int64_t row = min(row0 + r, row_max);
      dma16(kbase + row * ks_ + 8 * lane, kl + r * KROW);
      dma16(vbase + row * vs_ + 8 * lane, vl + r * VROW);
    }
  };

  f32x16 o[16];
  // Softmax reference (log2 domain, per query): fixed at the maximum of the
  // first tile the query sees, never moved afterwards, so O^T is never
  // rescaled.  m_true tracks the real running maximum; `risk` records a tile
  // exceeding the reference by more than 2^kGuard (probabilities that large
  // could overflow fp32), in which case the whole loop runs again with the
  // exact maximum as reference.
  float m_ref = -INFINITY, m_true = -INFINITY, l_run = 0.f;
  bool risk = false;
  const float c = p.c;

  // Per-lane LDS read offsets (bytes within a stage).
  //   K (A operand of step ks): key `col`, dims 16ks + 8hf .. +8.
  //   V^T (A operand of dim tile dt, key step ks, read e): dim 32dt + 16((lane>>4)&1) + lane%16,
  //   rows 16ks + 8e + 4hf + (lane%16)/4 (each lane of a 16-lane group fetches 4 dims of one row).
  const uint32_t k_off = col * KROW + 16 * hf;
  const uint32_t v_off = KST + (4 * hf + ((lane & 15) >> 2)) * VROW + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

  auto compute = [&](int tt, int st) __attribute__((always_inline)) {
    const bool comp = tt < n_ct;
    const int j0 = tt * BN;
    const int p0 = lo_first + (tt - n_ct) * BN;
    // does any query of this wave see a key of this tile? (wave-uniform)
    const bool active = wave_has_q && (comp ? (j0 < nc_w1) : (p0 <= tw1 && p0 + BN - 1 >= lo_w0));
    if (!active) return;
    const bool full = wave_full && (comp ? (j0 + BN - 1 < nc_w0) : (p0 >= lo_w1 && p0 + BN - 1 <= tw0));
    const unsigned char* sb = smem + st * STAGE;
    // S^T = K Q^T : 32 keys x 32 queries, 32 k-steps.  Operand reads run four
    // steps ahead; the scheduling barriers keep that order (left alone, the
    // scheduler hoists every read and runs out of registers).
    auto ldk = [&](int ks) __attribute__((always_inline)) {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sb + k_off + 32 * ks));
    };
    f32x16 s;
    bf16x8 kq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kq[i] = ldk(i);
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) {
      const bf16x8 ka = kq[ks & 3];
      if (ks + 4 < 32) kq[ks & 3] = ldk(ks + 4);
      if (ks == 0) mfma_s_first(s, ka, qf[ks]);
      else if (ks == 31) mfma_s_last(s, ka, qf[ks]);
      else mfma_s(s, ka, qf[ks]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // online softmax (log2 domain); lane holds keys 8(r/4) + 4hf + r%4 of query `col`
    float sv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[r] = s[r] * c;
    if (!full) {
      // this query's visible keys, relative to the tile: [klo, klo + kn)
      const int klo = comp ? 0 : lo_q - p0;
      const int kn = !qvalid ? 0 : comp ? max(nc_q - j0, 0) : tq - lo_q + 1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 8 * (r >> 2) + 4 * hf + (r & 3);
        sv[r] = (unsigned)(kk - klo) < (unsigned)kn ? sv[r] : -INFINITY;
      }
    }
    float mt = sv[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sv[r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    m_true = fmaxf(m_true, mt);
    // first tile with a visible key for this query: O^T is still zero, so the
    // reference may be set freely
    if (m_ref == -INFINITY) m_ref = mt;
    risk |= mt > m_ref + kGuard;
    // masked logits are -inf: exp2 gives 0 (also while m_ref is still -inf)
    const float msafe = m_ref == -INFINITY ? 0.f : m_ref;
    float ps[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) ps[r] = __builtin_amdgcn_exp2f(fminf(sv[r] - msafe, kGuard));
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) lsum += ps[r];
    l_run += lsum;
    bf16x8 pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(ps[8 * ks + 2 * e], ps[8 * ks + 2 * e + 1]);
      pf[ks] = __builtin_bit_cast(bf16x8, pk);
    }
    // O^T += V^T P^T : 16 dim tiles x 2 key steps; V^T reads run four MFMAs ahead
    auto ldv = [&](int i) __attribute__((always_inline)) {  // MFMA i: dim tile i%16, key step i/16
      const unsigned char* vp = sb + v_off + 64 * (i & 15) + (16 * (i >> 4)) * VROW;
      const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp));
      const s16x4 hi4 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp + 8 * VROW));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // key step major (i = 16 ks + dt), so consecutive MFMAs use different accumulators
    bf16x8 vq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vq[i] = ldv(i);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const bf16x8 va = vq[i & 3];
      if (i + 4 < 32) vq[i & 3] = ldv(i + 4);
      if (i == 0) mfma_o_first(o[i & 15], va, pf[i >> 4]);
      else mfma_o(o[i & 15], va, pf[i >> 4]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  if (tid == 0) redo_flag = 0;
  // Pipeline: tile tt+1's DMA is issued right after the barrier that opens
  // tile tt, into the stage tile tt-1 used (every wave has left it by then).
  // The second pass (rare, see m_ref) is decided for the whole workgroup, as
  // the loop holds barriers.
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) zero_o(o[dt], zero8);
    l_run = 0.f;
    if (ntiles > 0) {
      issue(0, 0);
      for (int tt = 0; tt < ntiles; ++tt) {
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if (tt + 1 < ntiles) issue(tt + 1, (tt + 1) & 1);
        compute(tt, tt & 1);
      }
    }
    if (pass == 1) break;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (__any(risk) && lane == 0) redo_flag = 1;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (redo_flag == 0) break;
    m_ref = m_true;  // exact maximum: every probability is at most 1
    risk = false;
  }

  // ---- epilogue: normalise, then stage this wave's bf16 O rows in the DMA
  // ring (idle once every wave has passed the barrier below; each wave owns a
  // disjoint 32-row slice) and store whole 1-KB rows with one coalesced
  // 16-byte store per lane: storing straight from the accumulator layout
  // writes each row in 16-byte pieces spread over 64 instructions, which costs
  // about a third more HBM write traffic than the output holds.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // wait states: O^T is read right after the last MFMA wrote it
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
  float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  constexpr int OROW = 2 * D + 16;  // LDS bytes per staged O row
  static_assert(NWAVE * WQ * OROW <= 2 * STAGE, "O staging must fit in the DMA ring");
  unsigned char* ow = smem + w * (WQ * OROW);
#pragma unroll
  for (int dt = 0; dt < 16; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2 pk;
      pk[0] = pack_bf16x2(o[dt][4 * q4] * inv, o[dt][4 * q4 + 1] * inv);
      pk[1] = pack_bf16x2(o[dt][4 * q4 + 2] * inv, o[dt][4 * q4 + 3] * inv);
      *reinterpret_cast<u32x2*>(ow + col * OROW + 2 * (32 * dt + 8 * q4 + 4 * hf)) = pk;
    }
  // rows of this wave that exist (none when the wave's queries are all past the end)
  const int nrow = min(WQ, a.seqlen_q - iw0);
  uint16_t* obase = (uint16_t*)a.o + b * a.so.b + (int64_t)h * a.so.h + 8 * lane;
#pragma unroll 8
  for (int r = 0; r < WQ; ++r) {
    if (r >= nrow) break;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ow + r * OROW + 16 * lane);
    *reinterpret_cast<u32x4*>(obase + (int64_t)(iw0 + r) * a.so.s) = v;
  }
  if (a.lse && hf == 0 && qvalid) a.lse[((int64_t)b * a.h_q + h) * a.seqlen_q + iq] = m_ref * kLn2 + __logf(l_tot);
}

}  // namespace

hipError_t launch_attn_prefill512(const AttnArgs& a, hipStream_t st) {
  PrefillParams p;
  p.a = a;
  p.n_qt = (a.seqlen_q + BM - 1) / BM;
  p.total = a.batch * a.h_q * p.n_qt;
  p.c = a.scale * kLog2e;
  const int grid = ((p.total + 7) / 8) * 8;
  hipLaunchKernelGGL(prefill512_kernel, dim3(grid), dim3(NWAVE * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace hca
