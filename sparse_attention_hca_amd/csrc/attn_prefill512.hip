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
//   * Wave w owns query block w (32 queries) for the logits and the softmax:
//     its Q^T stays in 128 registers as the B operand of S^T = K Q^T
//     (v_mfma_f32_32x32x16_bf16, 32 k-steps over d = 512).
//   * The output is split by head dims instead: wave w accumulates
//     O^T[dims 128w .. 128w+127][all 128 queries] (4 dim tiles x 4 query
//     blocks of 32 x 32 fp32 = the 256 AGPRs).  Each wave publishes its
//     block's P^T (bf16, 2 KB per tile) in LDS and reads all four, so every
//     V^T byte is read from LDS by one wave instead of four: per 32-key tile
//     and wave, 32 K reads, 16 transposing V^T reads and 10 P^T accesses
//     (was 32 + 64).
//   * Keys stream in tiles of 32 (compressed entries first, then the raw
//     window band in aligned 32-position blocks, rotated so that neighbouring
//     query tiles fetch a shared block at the same step) through two K stages
//     and two V stages filled by 16-byte LDS DMA; P^T is double-buffered.
//   * What bounds it: every 32-key tile moves 64 KB of K/V rows through the
//     CU's vector-memory path (about 1 KB per 33 cycles), and a DMA
//     instruction holds up the wave that issues it, so with one wave per SIMD
//     the matrix cores wait while DMA is issued.  A bare loop of this tile's
//     64 MFMAs and 16 DMAs per wave takes about 3700 cycles from L2 against
//     2048 for the MFMAs alone.  The DMA instructions are spread over the S^T
//     steps (one every other step), where they cost least.  The PV product of tile t-1 runs during
//     tile t: its first half interleaved with the S^T steps of tile t, its
//     second half with the softmax of tile t, so the matrix cores have work
//     while the VALU computes probabilities.  At the top of tile t the DMA of
//     K(t+1) and V(t) goes out; one barrier per tile (after the P^T store)
//     makes P^T(t), K(t+1) and V(t) visible and frees the stages read in
//     tile t.
//   * K rows are stored with a 16-byte pad (row stride 1040 B): the 16-byte
//     A-operand reads of 16 consecutive keys hit 16 distinct bank groups.  V
//     rows are padded by 64 B (stride 1088 B) and read with the gfx950
//     transposing LDS load (ds_read_b64_tr_b16), which hands each lane four
//     consecutive keys of one dim: the V^T A operand, in the key order of the
//     S^T accumulator layout (so P^T needs no permutation).
//   * Softmax in fp32 (log2 domain) against a fixed reference per query: the
//     maximum of the first tile it sees.  O^T is never rescaled, so it never
//     leaves the AGPRs.  If a later tile exceeds the reference by more than
//     2^64 the whole workgroup runs the loop again with the exact maximum.
//   * Only tiles that some query of the wave's block does not see entirely
//     are masked; a block that sees nothing of a tile gets zero probabilities.
//   * Workgroup ids are remapped so each XCD receives a contiguous range of
//     (head, query tile) work: same-head tiles share that XCD's L2 for the
//     compressed cache and the overlapping window rows.  Within a head, the
//     longest query tiles go first.
#include "device_common.h"
#include "launchers.h"
#include "mfma_asm.h"

#include <type_traits>

namespace hca {
namespace {

constexpr int D = 512;
constexpr int BM = 128;             // queries per workgroup
constexpr int WQ = 32;              // queries per wave (logits, softmax)
constexpr int NWAVE = 4;
constexpr int BN = 32;              // keys per tile
constexpr int KROW = 2 * D + 16;    // LDS bytes per K row
constexpr int VROW = 2 * D + 64;    // LDS bytes per V row
constexpr int KST = BN * KROW;      // K stage bytes
constexpr int VST = BN * VROW;      // V stage bytes
constexpr int PST = NWAVE * 2 * 64 * 16;  // P^T of one tile: 4 blocks x 2 key steps x 64 lanes x 16 B
constexpr int V0 = 2 * KST;         // first V stage
constexpr int P0 = 2 * KST + 2 * VST;  // first P^T buffer
constexpr int SMEM = P0 + 2 * PST;
constexpr float kGuard = 64.f;  // log2 headroom of the fixed softmax reference

struct PrefillParams {
  AttnArgs a;
  int n_qt;   // query tiles per (batch, head)
  int total;  // batch * h_q * n_qt
  float c;    // scale * log2(e)
};

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void prefill512_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  __shared__ float lsh[BM];
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
  // Window tiles are aligned 32-position blocks of the band [lo_first,
  // t_last], visited in a rotated order: at window step s the block whose
  // absolute index is congruent to s modulo n_wt.  Neighbouring query tiles
  // share most of their band blocks and run side by side on one XCD, so each
  // shared block is fetched by all of them at the same step (one L2 miss)
  // rather than a few steps apart (a miss each).
  const int a0 = lo_first / BN;
  const int n_wt = t_last / BN - a0 + 1;
  const int ntiles = n_ct + n_wt;
  const int j0 = (n_wt - a0 % n_wt) % n_wt;  // band block visited at window step 0
  auto win_p0 = [&](int tt) __attribute__((always_inline)) {
    int j = j0 + (tt - n_ct);
    j -= j >= n_wt ? n_wt : 0;
    return (a0 + j) * BN;
  };

  // this lane's query in the wave's own block (rows past the end read the
  // last row and are never stored)
  const int iq = i0 + WQ * w + col;
  const bool qvalid = iq < a.seqlen_q;
  const int tq = qp0 + iq;
  const int lo_q = max(0, tq - W + 1);
  const int nc_q = lo_q / blk;

  // Whether the wave's own block sees every key of tile tt (no mask needed;
  // wave-uniform).
  auto own_full = [&](int tt) __attribute__((always_inline)) {
    const int iw0 = i0 + WQ * w;
    if (iw0 + WQ - 1 > i_last) return false;
    const int tw0 = qp0 + iw0, tw1 = tw0 + WQ - 1;
    const int lo_w0 = max(0, tw0 - W + 1), lo_w1 = max(0, tw1 - W + 1);
    if (tt < n_ct) return tt * BN + BN - 1 < lo_w0 / blk;
    const int p0 = win_p0(tt);
    return p0 >= lo_w1 && p0 + BN - 1 <= tw0;
  };

  // ---- Q^T fragments (B operand): lane holds query `col`, dims 16ks + 8hf .. +8
  bf16x8 qf[32];
  {
    const uint16_t* qp = (const uint16_t*)a.q + b * a.sq.b + (int64_t)min(iq, a.seqlen_q - 1) * a.sq.s +
                         (int64_t)h * a.sq.h + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, ld16(qp + 16 * ks));
  }

  const uint16_t* kcb = (const uint16_t*)a.kc + b * a.skc.b + (int64_t)g * a.skc.h;
  const uint16_t* kb = (const uint16_t*)a.k + b * a.sk.b + (int64_t)g * a.sk.h;
  const uint16_t* vcb = (const uint16_t*)a.vc + b * a.svc.b + (int64_t)g * a.svc.h;
  const uint16_t* vb = (const uint16_t*)a.v + b * a.sv.b + (int64_t)g * a.sv.h;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)smem;

  // ---- DMA: K (isv = 0) or V (isv = 1) rows of tile tt; wave w copies rows
  // 8w .. 8w+7, one 1-KB row per instruction, from a wave-uniform row address
  // plus the lane's 16-byte offset.  Rows past the valid range re-read the
  // last valid row: their logits are masked and their probabilities are
  // exactly 0.
  struct RowSrc {
    const uint16_t* base;    // row 0 of K, V, kc or vc
    int64_t rs;              // row stride (elements)
    int r0;                  // row of tile row 8w
    int row_min, row_max;    // rows that exist for this tile (others re-read the nearest one)
    uint32_t dst;            // LDS byte address of row 8w
    uint32_t step;           // LDS bytes per row
  };
  auto row_src = [&](int tt, int isv) __attribute__((always_inline)) {
    RowSrc r;
    int row0;
    if (tt < n_ct) {
      r.base = isv ? vcb : kcb; r.rs = isv ? a.svc.s : a.skc.s; row0 = tt * BN; r.row_min = 0; r.row_max = nc_max - 1;
    } else {
      r.base = isv ? vb : kb; r.rs = isv ? a.sv.s : a.sk.s;
      row0 = win_p0(tt) - kvp0; r.row_min = lo_first - kvp0; r.row_max = t_last - kvp0;
    }
    r.r0 = row0 + 8 * w;
    r.dst = isv ? lds0 + V0 + (tt & 1) * VST + 8 * w * VROW : lds0 + (tt & 1) * KST + 8 * w * KROW;
    r.step = isv ? VROW : KROW;
    return r;
  };
  // The source is a per-lane VGPR address: a wave-uniform SGPR base read by
  // the DMA itself would need wait states after any VALU write of that SGPR
  // (a spill reload, for one), which the compiler does not insert around
  // inline asm.
  // lane16 is marked as rewritten at the top of each pass, so the DMA
  // addresses are not hoisted out of the pass loop (they would stay live
  // across the tile loop and spill).
  int lane16 = 16 * lane;
  auto dma_row = [&](const RowSrc& r, int i) __attribute__((always_inline)) {
    const int row = min(max(r.r0 + i, r.row_min), r.row_max);
    const unsigned char* src = reinterpret_cast<const unsigned char*>(r.base + (int64_t)row * r.rs) + lane16;
    dma16_m0(src, r.dst + i * r.step);
  };

  f32x16 o[16];  // o[4 dt + qb]: O^T dims 128w + 32dt .. +32, queries of block qb
  // Softmax reference (log2 domain, per query): fixed at the maximum of the
  // first tile the query sees, never moved afterwards, so O^T is never
  // rescaled.  m_true tracks the real running maximum; `risk` records a tile
  // exceeding the reference by more than 2^kGuard (probabilities that large
  // could overflow fp32), in which case the whole loop runs again with the
  // exact maximum as reference.
  float m_ref = -INFINITY, m_true = -INFINITY, l_run = 0.f;
  bool risk = false;
  const float c = p.c;

  // Per-lane LDS read offsets.
  //   K (A operand of step ks): key `col`, dims 16ks + 8hf .. +8.
  //   V^T (A operand of dim tile dg, key step ks, read e): dim 32dg + 16((lane>>4)&1) + lane%16,
  //   rows 16ks + 8e + 4hf + (lane%16)/4 (each lane of a 16-lane group fetches 4 dims of one row).
  //   P^T (B operand of query block qb, key step ks): the 16 bytes lane `lane` of wave qb stored.
  const uint32_t k_off = col * KROW + 16 * hf;
  const uint32_t v_off = (4 * hf + ((lane & 15) >> 2)) * VROW + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

  auto ldk = [&](const unsigned char* ks_base, int ks) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ks_base + k_off + 32 * ks));
  };
  // V^T operand of this wave's dim tile dt (global dim tile 4w + dt), key step ks
  auto ldv = [&](const unsigned char* vs_base, int dt, int ks) __attribute__((always_inline)) {
    const unsigned char* vp = vs_base + v_off + 64 * (4 * w + dt) + (16 * ks) * VROW;
    const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp));
    const s16x4 hi4 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp + 8 * VROW));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto ldp = [&](const unsigned char* ps_base, int qb, int ks) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ps_base + ((qb * 2 + ks) * 64 + lane) * 16));
  };

  // One tile.  S^T(tt) for the wave's own block and the PV product of tile
  // tt-1 (PREV: tt > 0) run interleaved: PV key step 0 between the S^T steps,
  // key step 1 between the softmax steps.  The DMA of K(tt+1) (of tile
  // ntiles-1 again on the last tile, into the free stage) and V(tt) goes out
  // between the first S^T steps.  A block that sees no key of the tile gets
  // all-masked logits, hence zero probabilities (the products run anyway:
  // one code path keeps O^T in the AGPRs).
  auto tile = [&](auto prev_c, int tt) __attribute__((always_inline)) {
    constexpr bool PREV = decltype(prev_c)::value;
    const unsigned char* ksb = smem + (tt & 1) * KST;                 // K(tt)
    const unsigned char* vsb = smem + V0 + ((tt - 1) & 1) * VST;     // V(tt-1)
    const unsigned char* prb = smem + P0 + ((tt - 1) & 1) * PST;     // P^T(tt-1)
    unsigned char* pwb = smem + P0 + (tt & 1) * PST;                 // P^T(tt)
    const int tk = min(tt + 1, ntiles - 1);
    RowSrc srck = row_src(tk, 0);
    srck.dst = lds0 + ((tt + 1) & 1) * KST + 8 * w * KROW;
    const RowSrc srcv = row_src(tt, 1);

    // ---- phase 1: S^T(tt) steps with K read eight steps ahead (LDS latency
    // under load is 200+ cycles); PV(tt-1) key step 0 from slot 8 on, when its
    // operands (read before slot 0) have arrived; the DMA on even slots; the
    // key-step-1 operands of PV (all of them, phase 2 reads nothing) in the
    // last slots.
    f32x16 s;
    bf16x8 kq[8], vq0[4], vq1[4], pqa[2], pqb[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) kq[i] = ldk(ksb, i);
    if constexpr (PREV) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) vq0[dt] = ldv(vsb, dt, 0);
      pqa[0] = ldp(prb, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) {
      {
        const bf16x8 ka = kq[ks & 7];
        if (ks + 8 < 32) kq[ks & 7] = ldk(ksb, ks + 8);
        if (ks == 0) mfma_s_first(s, ka, qf[ks]);
        else mfma_s(s, ka, qf[ks]);
      }
      if constexpr (PREV) {
        if (ks >= 8 && ks < 24) {
          const int m = ks - 8, qb = m >> 2, dt = m & 3;
          if (dt == 0 && qb < 3) pqa[(qb + 1) & 1] = ldp(prb, qb + 1, 0);
          mfma_o(o[4 * dt + qb], vq0[dt], pqa[qb & 1]);
        } else if (ks >= 24 && ks < 28) {
          vq1[ks - 24] = ldv(vsb, ks - 24, 1);
        } else if (ks >= 28) {
          pqb[ks - 28] = ldp(prb, ks - 28, 1);
        }
      }
      // DMA, one instruction every other slot (the CU's DMA path takes about
      // 33 cycles per 1-KB instruction; issued in a burst they stall the wave
      // longer): K(tt+1) rows on slots 0, 4, .., 28, V(tt) rows on 2, .., 30
      if (!(ks & 1)) {
        if (ks & 2) dma_row(srcv, ks >> 2);
        else dma_row(srck, ks >> 2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- phase 2: softmax of tile tt interleaved with PV(tt-1) key step 1
    // (MFMA j = block j/4, dim tile j%4), about four VALU instructions per
    // MFMA: a wave issuing more than ~6 VALU (or ~2 transcendental)
    // instructions per 32-cycle MFMA delays the next one.
    float sv[16], ps[16];
    const bool full = own_full(tt);
    int klo = 0, kn = 0;
    {
      const bool comp = tt < n_ct;
      const int p0 = comp ? 0 : win_p0(tt);
      klo = comp ? 0 : lo_q - p0;
      kn = !qvalid ? 0 : comp ? max(nc_q - tt * BN, 0) : tq - lo_q + 1;
    }
    auto pv1 = [&](int j) __attribute__((always_inline)) {
      if constexpr (PREV) mfma_o(o[4 * (j & 3) + (j >> 2)], vq1[j & 3], pqb[j >> 2]);
    };
    __builtin_amdgcn_sched_barrier(0);
    pv1(0);
    // wait states: the S^T accumulator is read by VALU after the last step
    asm volatile("s_nop 15\n\ts_nop 15" : "+v"(s));
    __builtin_amdgcn_sched_barrier(0);
    // slots 0..3: scale (and, on partially visible tiles, mask) four logits
    // each; lane holds keys 8(r/4) + 4hf + r%4 of query `col`
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j > 0) pv1(j);
      if (full) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[4 * j + e] = s[4 * j + e] * c;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * j + e;
          const int kk = 8 * (r >> 2) + 4 * hf + (r & 3);
          sv[r] = (unsigned)(kk - klo) < (unsigned)kn ? s[r] * c : -INFINITY;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // slots 4..5: row maximum over this lane's 16 keys, then over the other
    // half of the query's keys (lane ^ 32)
    float mt, mt2;
    {
      pv1(4);
      float m4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) m4[e] = fmaxf(fmaxf(sv[4 * e], sv[4 * e + 1]), fmaxf(sv[4 * e + 2], sv[4 * e + 3]));
      mt2 = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
      __builtin_amdgcn_sched_barrier(0);
      pv1(5);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt2), __float_as_uint(mt2), false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      __builtin_amdgcn_sched_barrier(0);
    }
    // slot 6: the reference; first tile with a visible key for this query:
    // O^T is still zero, so the reference may be set freely.  Later logits
    // above it by more than 2^kGuard set `risk` (the workgroup then runs again
    // with the exact maximum, discarding this pass), so exp2 needs no clamp.
    float msafe;
    {
      pv1(6);
      m_true = fmaxf(m_true, mt);
      if (m_ref == -INFINITY) m_ref = mt;
      risk |= mt > m_ref + kGuard;
      // masked logits are -inf: exp2 gives 0 (also while m_ref is still -inf)
      msafe = m_ref == -INFINITY ? 0.f : m_ref;
      __builtin_amdgcn_sched_barrier(0);
    }
    // slots 7..14: two probabilities each, added to the row sum and packed to
    // bf16; P^T of this block (lane order is the B operand's) goes to LDS for
    // every wave once a key step's eight probabilities are done
    u32x4 pk[2];
    float lsum = 0.f;
#pragma unroll
    for (int j = 7; j < 15; ++j) {
      pv1(j);
      const int r = 2 * (j - 7);
      ps[r] = __builtin_amdgcn_exp2f(sv[r] - msafe);
      ps[r + 1] = __builtin_amdgcn_exp2f(sv[r + 1] - msafe);
      lsum += ps[r] + ps[r + 1];
      pk[r >> 3][(r & 7) >> 1] = pack_bf16x2(ps[r], ps[r + 1]);
      if (j == 10) *reinterpret_cast<u32x4*>(pwb + ((w * 2 + 0) * 64 + lane) * 16) = pk[0];
      __builtin_amdgcn_sched_barrier(0);
    }
    pv1(15);
    *reinterpret_cast<u32x4*>(pwb + ((w * 2 + 1) * 64 + lane) * 16) = pk[1];
    l_run += lsum;
  };

  // PV of the last tile (after the loop): both key steps of every block.
  auto pv_only = [&](int tt) __attribute__((always_inline)) {
    const unsigned char* vsb = smem + V0 + (tt & 1) * VST;
    const unsigned char* prb = smem + P0 + (tt & 1) * PST;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 vq[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) vq[dt] = ldv(vsb, dt, ks);
#pragma unroll
      for (int qb = 0; qb < NWAVE; ++qb) {
        const bf16x8 pq = ldp(prb, qb, ks);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) mfma_o(o[4 * dt + qb], vq[dt], pq);
      }
    }
  };

  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  if (tid == 0) redo_flag = 0;
  // Pipeline: K(0) is issued before the loop; in tile tt the DMA of K(tt+1)
  // and V(tt) goes out (into the stages of K(tt-1) and V(tt-2), both freed by
  // the barrier that ended tile tt-1), and the barrier at the end of tile tt
  // waits for them.  The second pass (rare, see m_ref) is decided for the
  // whole workgroup, as the loop holds barriers.
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int i = 0; i < 16; ++i) zero_o(o[i], zero8);
    l_run = 0.f;
    asm volatile("" : "+v"(lane16));
    if (ntiles > 0) {
      {
        const RowSrc sk0 = row_src(0, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) dma_row(sk0, i);
      }
      // The first K tile's DMA goes out while the Q loads are still in flight.
      // The compiler's waits for Q (its loads were issued before the DMA, and
      // loads complete in order) and the explicit wait below leave both landed.
#pragma unroll
      for (int ks = 0; ks < 32; ++ks) asm volatile("" ::"v"(qf[ks]));
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      tile(F_{}, 0);
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      for (int tt = 1; tt < ntiles; ++tt) {
        tile(T_{}, tt);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
      pv_only(ntiles - 1);
    }
    if (pass == 1) break;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (__any(risk) && lane == 0) redo_flag = 1;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (redo_flag == 0) break;
    m_ref = m_true;  // exact maximum: every probability is at most 1
    risk = false;
  }

  // ---- epilogue: row sums of every query (each lives with the wave that owns
  // the query's block), normalise, stage the bf16 O rows in the DMA ring (idle
  // once every wave has passed the barrier below) and store whole 1-KB rows
  // with one coalesced 16-byte store per lane; wave w stores block w's rows.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // wait states: O^T is read right after the last MFMA wrote it
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (hf == 0) lsh[WQ * w + col] = l_tot;
  if (a.lse && hf == 0 && qvalid) a.lse[((int64_t)b * a.h_q + h) * a.seqlen_q + iq] = m_ref * kLn2 + __logf(l_tot);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  constexpr int OROW = 2 * D + 16;  // LDS bytes per staged O row
  static_assert(BM * OROW <= P0, "O staging must fit in the K/V stages");
#pragma unroll
  for (int qb = 0; qb < NWAVE; ++qb) {
    const float lt = lsh[WQ * qb + col];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    unsigned char* orow = smem + (WQ * qb + col) * OROW + 2 * (128 * w + 4 * hf);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16& acc = o[4 * dt + qb];
        u32x2 pk;
        pk[0] = pack_bf16x2(acc[4 * q4] * inv, acc[4 * q4 + 1] * inv);
        pk[1] = pack_bf16x2(acc[4 * q4 + 2] * inv, acc[4 * q4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + 2 * (32 * dt + 8 * q4)) = pk;
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // rows of block w that exist (none when the block is past the end)
  const int iw0 = i0 + WQ * w;
  const int nrow = min(WQ, a.seqlen_q - iw0);
  const unsigned char* ow = smem + (WQ * w) * OROW;
  uint16_t* obase = (uint16_t*)a.o + b * a.so.b + (int64_t)h * a.so.h + 8 * lane;
#pragma unroll 8
  for (int r = 0; r < WQ; ++r) {
    if (r >= nrow) break;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ow + r * OROW + 16 * lane);
    *reinterpret_cast<u32x4*>(obase + (int64_t)(iw0 + r) * a.so.s) = v;
  }
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
