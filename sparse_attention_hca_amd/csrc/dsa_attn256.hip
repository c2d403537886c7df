// DSA core attention over the top-k selected positions, bf16, d_qk = d_v = 256
// (ERNIE 5.5 Flash Base pages: mirrorspeed page, "Hybrid sparse attention"
// section -- core attention only on the top-k positions; ai-club.cn page,
// hybrid attention section -- 256-wide heads in the full-context layers).
//
// One workgroup (4 waves) per (query position, group of 64 query heads that
// share one KV head); every head of the group attends over the same gathered
// rows, so the heads are the MFMA columns.  Wave w owns heads 16w .. 16w+15
// for S^T = K Q^T (32 keys x 16 heads, v_mfma_f32_16x16x32_bf16) and their
// softmax, publishes its P^T (bf16, 1 KB per tile) in LDS, and then computes
// O^T += V^T P^T for dims 64w .. 64w+63 of all 64 heads (the 32 keys of a
// tile as the contraction), each V^T byte read from LDS by one wave.  The PV
// product of a tile runs interleaved with the next tile's S^T steps.  With
// one wave per SIMD the per-wave chain S -> softmax -> exchange -> PV and the
// per-query start-up are serial, so for rows of up to 2048 entries the ring
// is kept small enough for two workgroups to share a CU.
//
// The step is a gather of 2 x 512 bytes per selected position:
//   * The query's index row is copied to LDS once, with a 32-bit validity mask
//     per 32-entry tile (a wave ballot); -1 entries and out-of-range positions
//     are fetched as row 0 (valid memory) and masked, an out-of-range position
//     also turns the row's output into NaN.  Trailing tiles with no valid entry
//     are not visited, so rows shorter than topk cost what they hold; an
//     interior tile with none takes the masked path (all probabilities 0).
//   * Q and the index row are loaded with every load in flight at once.
//   * Tiles of 32 gathered K and V rows move global -> LDS with 16-byte LDS
//     DMA through a ring of NRING stages (NRING - 1 tiles in flight while one
//     is consumed), the next tile's DMA instructions interleaved with the
//     S^T steps.  DMA instruction i of wave w fetches entries 8w+i (lanes
//     0-31) and 8w+4+i (lanes 32-63) into the adjacent LDS rows 8w+2i and
//     8w+2i+1, so a lane's four row numbers are one 16-byte LDS read; the
//     addresses are a scalar base plus a 32-bit row offset (64-bit addresses
//     when a plane of K or V spans 2 GiB or more).  Keys sit in the tile in
//     this row order: S, the masks and the PV contraction all use it.
//   * Rows are stored with their 16-byte chunks XOR-swizzled (K chunk c of
//     row r in slot c ^ (r mod 16), V chunk c in slot c ^ 2(r mod 8); the DMA
//     lanes fetch the matching chunks), so the 16-byte K operand reads and
//     the gfx950 transposing V reads (ds_read_b64_tr_b16, which hands each
//     lane four consecutive keys of one dim: the V^T operand) hit distinct
//     bank groups.
//   * The S^T accumulators of a lane (one head, rows 4g .. 4g+3 and
//     16+4g .. 16+4g+3) are the P^T operand of the PV product once converted
//     to bf16; the V^T reads fetch rows in that order.
//   * Softmax in fp32 (log2 domain) against a fixed reference per head: the
//     maximum of the first tile holding a valid key.  O^T is never rescaled,
//     so it stays in AGPRs (the products are inline asm with explicit
//     accumulator classes and wait states).  If a later logit exceeds the
//     reference by more than 2^kGuard the whole row runs again with the exact
//     maximum as reference.  The row sum of P comes from one more MFMA with an
//     all-ones A operand, so it is the sum of the same bf16 probabilities
//     that enter O.
#include "device_common.h"
#include "launchers.h"

namespace hca {
namespace {

constexpr int D = 256;
constexpr int TK = 32;                 // keys per tile
constexpr int HPW = 16;                // heads per wave
constexpr int HPB = 64;                // heads per workgroup
constexpr int ROWB = 2 * D;            // bytes per K or V row
constexpr int KSTB = TK * ROWB;        // K part of a stage
constexpr int STAGEB = 2 * KSTB;       // K rows then V rows
constexpr int MAX_TOPK = 4096;
constexpr float kGuard = 64.f;         // log2 headroom of the fixed softmax reference

typedef short s16x4 __attribute__((ext_vector_type(4)));

struct SparseParams {
  const uint16_t* q; LStrides sq;
  const uint16_t* k; LStrides sk;
  const uint16_t* v; LStrides sv;
  const int32_t* idx;
  uint16_t* o; LStrides so;
  float* lse;
  int seqlen, n_kv, h_q, h_kv, topk, n_hb;  // seqlen queries; positions < n_kv
  uint32_t k_row_bytes, v_row_bytes;        // position strides of K and V in bytes
  float c;
};

// 16-byte LDS DMA of one wave (lane l copies 16 bytes to LDS byte address
// lds + 16 l; lds travels in M0): from a per-lane 64-bit address, or from a
// scalar base plus a per-lane 32-bit offset.  Written as asm so the compiler
// does not wait for it before LDS reads; the explicit vmcnt wait and barrier
// of each tile order them.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma16_so(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}

// v_mfma_f32_16x16x32_bf16 as inline asm: S^T accumulates in VGPRs (the
// softmax reads it), O^T and the row sum in AGPRs.  The compiler does not see
// these as MFMAs, so the required wait states are explicit: after the last
// S^T step (VALU reads it), before the first PV step of a tile (P^T was just
// written by VALU) and before the AGPRs are read back.
__device__ __forceinline__ void mfma_s_first(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_o(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_o_first(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 4\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void zero_o(f32x4& acc, const bf16x8& z) {
  asm volatile("s_nop 4\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %1, 0" : "=&a"(acc) : "v"(z));
}

// NRING ring stages (NRING - 1 tiles in flight) and rows of up to MAXK
// entries: <2, 2048> keeps a workgroup under 80 KB of LDS so that two run on
// a CU (two waves per SIMD, whose serial S -> softmax -> PV chains and
// per-query start-up interleave); <4, 4096> is one workgroup per CU (rows
// longer than 2048, and grids too small to fill the chip twice over).
template <bool POS, bool WIDE, int NRING, int MAXK>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(NRING == 2 ? 2 : 1)))
void sparse_attn256_kernel(SparseParams p) {
  constexpr int MAX_TILES = MAXK / TK;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[NRING * STAGEB];
  __shared__ __attribute__((aligned(16))) int sidx[MAXK];
  __shared__ uint32_t tvalid[MAX_TILES];
  __shared__ __attribute__((aligned(16))) unsigned char pbuf[HPB * TK * 2];  // P^T of the 4 head blocks
  __shared__ float lsh[HPB];                                                  // row sums per head
  __shared__ int bad_sh, last_sh, redo_sh;

  const int t = blockIdx.x;
  const int hb = blockIdx.y % p.n_hb;
  const int g = blockIdx.y / p.n_hb;     // KV head
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int group = p.h_q / p.h_kv;
  const int hq = g * group + hb * HPB + w * HPW + col;
  const int ntiles_all = (p.topk + TK - 1) / TK;

  // ---- Q^T fragments (B operand): head `col`, dims 32ks + 8grp .. +8, and
  // the query's index row; every load is in flight at once (one round trip)
  if (tid == 0) { bad_sh = 0; last_sh = -1; redo_sh = 0; }
  bf16x8 qf[8];
  {
    const uint16_t* qp = p.q + b * p.sq.b + (int64_t)t * p.sq.s + (int64_t)hq * p.sq.h + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, ld16(qp + 32 * ks));
  }
  constexpr int NJ = MAXK / 256;
  int uv[NJ];
  {
    const int32_t* irow = p.idx + ((int64_t)b * p.seqlen + t) * p.topk;
#pragma unroll
    for (int k = 0; k < NJ; ++k) {
      const int j = 256 * k + tid;
      uv[k] = j < p.topk ? irow[j] : -1;
    }
  }
  __syncthreads();  // flags initialised
  // index row -> LDS (fetch row, 0 where invalid), per-tile validity masks,
  // the last tile holding a valid entry, out-of-range flag
  {
    int bad = 0, last = -1;
#pragma unroll
    for (int k = 0; k < NJ; ++k) {
      const int j0 = 256 * k;
      if (j0 >= ntiles_all * TK) break;
      const int j = j0 + tid;
      const int u = uv[k];
      bad |= (u < -1 || u >= p.n_kv);
      const bool ok = u >= 0 && u < p.n_kv;
      if (j < ntiles_all * TK) sidx[j] = ok ? u : 0;
      const uint64_t bal = __ballot(ok);
      const int tile = (j0 + 64 * w) / TK;
      if (lane == 0) {
        if (tile < ntiles_all) tvalid[tile] = (uint32_t)bal;
        if (tile + 1 < ntiles_all) tvalid[tile + 1] = (uint32_t)(bal >> 32);
      }
      if ((uint32_t)(bal >> 32) != 0u) last = tile + 1;
      else if ((uint32_t)bal != 0u) last = tile;
    }
    if (bad) atomicOr(&bad_sh, 1);
    if (lane == 0 && last >= 0) atomicMax(&last_sh, last);
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qf[ks]));
  __syncthreads();  // sidx, tvalid, flags complete; Q settled before the DMA ring
  const int ntiles = __builtin_amdgcn_readfirstlane(last_sh + 1);

  const uint16_t* kb = p.k + b * p.sk.b + (int64_t)g * p.sk.h;
  const uint16_t* vb = p.v + b * p.sv.b + (int64_t)g * p.sv.h;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ring;

  // ---- DMA of tile tt into stage st.  Instruction i of wave w: lanes 0-31
  // fetch entry 8w+i into LDS row 8w+2i, lanes 32-63 entry 8w+4+i into row
  // 8w+2i+1; lane hl of a half fetches the chunk that lands in slot hl.
  const int hrow = lane >> 5, hl = lane & 31;
  uint32_t kch[4], vch[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * w + 2 * i + hrow;
    kch[i] = 16 * (hl ^ (r & 15));
    vch[i] = 16 * (hl ^ (2 * (r & 7)));
  }
  auto rows_of = [&](int tt) __attribute__((always_inline)) {
    return *reinterpret_cast<const int4*>(sidx + tt * TK + 8 * w + 4 * hrow);
  };
  // instruction j of a tile: K (j even) or V (j odd) rows of pair j/2
  auto dma_one = [&](const int4& u4, int st, int j) __attribute__((always_inline)) {
    const int i = j >> 1;
    const uint32_t u = (uint32_t)(i == 0 ? u4.x : i == 1 ? u4.y : i == 2 ? u4.z : u4.w);
    const uint32_t lds = lds0 + st * STAGEB + (j & 1) * KSTB + (8 * w + 2 * i) * ROWB;
    if constexpr (WIDE) {
      if (j & 1) dma16(reinterpret_cast<const unsigned char*>(vb) + (uint64_t)u * p.v_row_bytes + vch[i], lds);
      else dma16(reinterpret_cast<const unsigned char*>(kb) + (uint64_t)u * p.k_row_bytes + kch[i], lds);
    } else {
      if (j & 1) dma16_so(vb, __umul24(u, p.v_row_bytes) + vch[i], lds);
      else dma16_so(kb, __umul24(u, p.k_row_bytes) + kch[i], lds);
    }
  };
  auto issue = [&](int tt, int st) __attribute__((always_inline)) {
    const int4 u4 = rows_of(tt);
#pragma unroll
    for (int j = 0; j < 8; ++j) dma_one(u4, st, j);
  };

  // Per-lane LDS read offsets within a stage.
  //   K (A operand, key half kt, step ks): row 16kt + col, chunk 4ks + grp in slot
  //     (4ks + grp) ^ col: k_off[ks % 4] + 256 (ks / 4) + 16 kt ROWB.
  //   V^T (A operand of dim tile dt = 4w + i, read e): row 16e + 4grp + col/4,
  //     dims 16dt + 4(col % 4), chunk 2dt + (col % 4)/2 in slot chunk ^ 2(row mod 8):
  //     v_off[i] + 16 e ROWB.
  uint32_t k_off[4], v_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) k_off[i] = col * ROWB + 16 * ((4 * i + grp) ^ col);
  {
    const int row = 4 * grp + (col >> 2);
    const int s = row & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int dt = 4 * w + i;
      v_off[i] = KSTB + row * ROWB + 32 * ((dt & 7) ^ s) + 256 * (dt >> 3) + 16 * ((col & 3) >> 1) + 8 * (col & 1);
    }
  }
  // Entry number (bit of the tile's validity mask) of the S^T rows this lane
  // holds: row 16kt + 4grp + r sits in LDS row order, see the DMA above.
  int ebit[8];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rho = 16 * kt + 4 * grp + r;
      ebit[4 * kt + r] = 8 * (rho >> 3) + 4 * (rho & 1) + ((rho & 7) >> 1);
    }

  f32x4 o[4][4], lacc;  // o[dim tile 4w + i][head block]
  const float c = p.c;
  const float NEG = POS ? -INFINITY : INFINITY;  // raw score that maps to a -inf logit
  float m_ref = -INFINITY;                       // reference (scaled, log2 domain) of this lane's head
  float m_run = NEG;                             // running max (POS) / min of this lane's raw scores
  bool have_ref = false;                         // same for every lane of the workgroup
  const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  const bf16x8 ones8 = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

  auto ext = [](float a, float x) __attribute__((always_inline)) { return POS ? fmaxf(a, x) : fminf(a, x); };
  // extreme of three raw scores (v_max3 / v_min3; written as asm so that no
  // canonicalising moves are added around the MFMA results)
  auto ext3 = [](float a, float x, float y) __attribute__((always_inline)) {
    float r;
    if constexpr (POS) asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(x), "v"(y));
    else asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(x), "v"(y));
    return r;
  };
  // first tile with a valid key: O^T is still zero, so the reference (the
  // head's maximum logit over this tile) may be set freely
  auto set_ref = [&](const float* sv) __attribute__((always_inline)) {
    float mt = ext(ext3(sv[0], sv[1], sv[2]), ext3(sv[3], sv[4], ext(sv[5], ext(sv[6], sv[7]))));
    mt = ext(mt, __shfl_xor(mt, 16));
    mt = ext(mt, __shfl_xor(mt, 32));
    m_ref = mt * c;
    have_ref = true;
  };

  // One tile.  When `dma` is set, the 8 DMA instructions of tile tt+NRING-1
  // go out between the first S^T steps, so their issue overlaps the products.
  // The PV product of the previous tile (its V^T and P^T operands held in vq
  // and pq since then, when `pend` is set) is interleaved with this tile's S^T
  // steps; on return vq and pq hold this tile's operands.
  auto compute = [&](uint32_t vmask, const unsigned char* sb, bool dma, const int4& u4, int dst, bool pend,
                     bf16x8 (&vq)[4], bf16x8 (&pq)[4]) __attribute__((always_inline)) {
    // S^T = K Q^T for the two 16-key halves; MFMA i is step i/2 of half i%2,
    // its K operand is read four MFMAs ahead (the scheduling barriers keep
    // that order)
    auto ldk = [&](int i) __attribute__((always_inline)) {
      return __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(sb + k_off[(i >> 1) & 3] + 256 * (i >> 3) + 16 * (i & 1) * ROWB));
    };
    auto ldv = [&](int i) __attribute__((always_inline)) {  // dim tile 4w + i
      const unsigned char* vp = sb + v_off[i];
      const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp));
      const s16x4 hi4 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp + 16 * ROWB));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    f32x4 s[2];
    bf16x8 kq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kq[i] = ldk(i);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bf16x8 ka = kq[i & 3];
      if (i + 4 < 16) kq[i & 3] = ldk(i + 4);
      if (i < 2) mfma_s_first(s[i & 1], ka, qf[i >> 1]);
      else mfma_s(s[i & 1], ka, qf[i >> 1]);
      if (pend) mfma_o(o[i >> 2][i & 3], vq[i >> 2], pq[i & 3]);
      if (i < 8 && dma) dma_one(u4, dst, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the V^T operands do not depend on P: their reads overlap the softmax
#pragma unroll
    for (int i = 0; i < 4; ++i) vq[i] = ldv(i);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 3" : "+v"(s[0]), "+v"(s[1]));
    float sv[8] = {s[0][0], s[0][1], s[0][2], s[0][3], s[1][0], s[1][1], s[1][2], s[1][3]};
    float ps[8];
    if (vmask == 0xffffffffu) {
      m_run = ext3(m_run, ext3(sv[0], sv[1], sv[2]), ext3(sv[3], sv[4], ext(sv[5], ext(sv[6], sv[7]))));
      if (!have_ref) set_ref(sv);
#pragma unroll
      for (int r = 0; r < 8; ++r) ps[r] = __builtin_amdgcn_exp2f(fmaf(sv[r], c, -m_ref));
    } else {
      bool ok[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        ok[r] = (vmask >> ebit[r]) & 1u;
        sv[r] = ok[r] ? sv[r] : NEG;
      }
      m_run = ext(m_run, ext(ext3(sv[0], sv[1], sv[2]), ext3(sv[3], sv[4], ext(sv[5], ext(sv[6], sv[7])))));
      if (!have_ref && vmask != 0u) set_ref(sv);
#pragma unroll
      for (int r = 0; r < 8; ++r) ps[r] = ok[r] ? __builtin_amdgcn_exp2f(fmaf(sv[r], c, -m_ref)) : 0.f;
    }
    u32x4 pk;
#pragma unroll
    for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(ps[2 * e], ps[2 * e + 1]);
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pk);
    // P^T of this wave's heads to LDS (lane order is the B operand's), the row
    // sums of its heads, then every wave takes all four head blocks
    *reinterpret_cast<u32x4*>(pbuf + w * (HPW * TK * 2) + 16 * lane) = pk;
    mfma_o_first(lacc, ones8, pf);  // the ones operand may have just been rematerialised by VALU
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int hk = 0; hk < 4; ++hk)
      pq[hk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(pbuf + hk * (HPW * TK * 2) + 16 * lane));
    __builtin_amdgcn_sched_barrier(0);
  };
  // O^T += V^T P^T of one tile: this wave's 4 dim tiles x the 4 head blocks,
  // k = the 32 keys of the tile
  auto pv = [&](const bf16x8 (&vq)[4], const bf16x8 (&pq)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int hk = 0; hk < 4; ++hk) mfma_o(o[i][hk], vq[i], pq[hk]);
  };

  // Ring: tiles 0 .. NRING-2 are issued up front; the trip for tile tt waits
  // for its rows (later tiles stay in flight), a barrier makes every wave's
  // rows visible and frees the stage tile tt-1 used, then tile tt is computed
  // while tile tt+NRING-1 is issued into that stage.  Every tile up to the
  // last valid one is computed (a tile with no valid entry contributes
  // nothing).  The second pass (rare, see m_ref) is
  // decided for the whole workgroup, as the loop holds barriers.
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int hk = 0; hk < 4; ++hk) zero_o(o[i][hk], zero8);
    zero_o(lacc, zero8);
    for (int i = 0; i < NRING - 1; ++i)
      if (i < ntiles) issue(i, i);
    int st = 0;
    bf16x8 vq[4], pq[4];                        // operands of the PV product still to do
    uint32_t vm = ntiles > 0 ? tvalid[0] : 0u;  // validity word of the next tile, read ahead
    for (int tt = 0; tt < ntiles; ++tt) {
      const uint32_t vmask = __builtin_amdgcn_readfirstlane(vm);
      vm = tvalid[min(tt + 1, ntiles - 1)];
      const int4 u4 = rows_of(min(tt + NRING - 1, ntiles - 1));  // rows of the tile issued in this trip
      const int after = min(NRING - 2, ntiles - 1 - tt);  // tiles issued after tt
      if (after >= 2) asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
      else if (after == 1) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      compute(vmask, ring + st * STAGEB, tt + NRING - 1 < ntiles, u4, st == 0 ? NRING - 1 : st - 1, tt > 0, vq, pq);
      st = st == NRING - 1 ? 0 : st + 1;
    }
    if (ntiles > 0) pv(vq, pq);  // the last tile's PV product
    if (pass == 1) break;
    float mh = ext(m_run, __shfl_xor(m_run, 16));
    mh = ext(mh, __shfl_xor(mh, 32));
    const float top = mh * c;  // exact maximum logit of this lane's head
    const bool risk = have_ref && top > m_ref + kGuard;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (__any(risk) && lane == 0) redo_sh = 1;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (redo_sh == 0) break;
    m_ref = top;  // every probability of the second pass is at most 1
  }

  // ---- epilogue (wait states: the AGPRs are read right after the last MFMA).
  // Each head's row sum lives with the wave that owns the head; O^T of every
  // head is spread over the four waves by dims.
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int hk = 0; hk < 4; ++hk) asm volatile("" : "+a"(o[i][hk]));
  asm volatile("" : "+a"(lacc));
  const bool poisoned = bad_sh != 0;
  const float l_own = lacc[0];
  if (grp == 0) lsh[HPW * w + col] = l_own;
  if (p.lse && grp == 0)
    p.lse[((int64_t)b * p.h_q + hq) * p.seqlen + t] =
        poisoned ? __builtin_nanf("") : (have_ref ? m_ref * kLn2 + __logf(l_own) : -INFINITY);
  __syncthreads();
#pragma unroll
  for (int hk = 0; hk < 4; ++hk) {
    const float l_tot = lsh[HPW * hk + col];
    const float inv = poisoned ? __builtin_nanf("") : (l_tot > 0.f ? 1.f / l_tot : 0.f);
    const int hq_k = g * group + hb * HPB + HPW * hk + col;
    uint16_t* op = p.o + b * p.so.b + (int64_t)t * p.so.s + (int64_t)hq_k * p.so.h + 4 * grp;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 pk;
      pk[0] = pack_bf16x2(o[i][hk][0] * inv, o[i][hk][1] * inv);
      pk[1] = pack_bf16x2(o[i][hk][2] * inv, o[i][hk][3] * inv);
      *reinterpret_cast<u32x2*>(op + 16 * (4 * w + i)) = pk;
    }
  }
}

// Merge of a decode row whose selected positions ran as `parts` query rows
// (one per contiguous slice of the index row): each part's normalised output
// is weighted by exp(lse_p - max lse), the log-sum-exp of the parts' softmax
// denominators.  A part with no position (lse -inf) weighs nothing; a row with
// no position at all is written as 0 with lse -inf; a poisoned part (NaN)
// poisons the row, as in the single-pass kernel.  One workgroup per (head,
// sequence), one thread per value dim.
__global__ __launch_bounds__(256) void decode_combine256_kernel(const uint16_t* op, const float* lp, int parts,
                                                                uint16_t* o, LStrides so, float* lse, int h_q) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const float* l = lp + ((int64_t)b * h_q + h) * parts;
  float m = -INFINITY;
  bool nan = false;
#pragma unroll 8
  for (int i = 0; i < parts; ++i) {
    const float x = l[i];
    nan |= x != x;
    m = fmaxf(m, x);
  }
  float acc = 0.f, s = 0.f;
  if (m != -INFINITY) {
    // unrolled so that several slices' loads are in flight at once
#pragma unroll 8
    for (int i = 0; i < parts; ++i) {
      const float wgt = __expf(l[i] - m);  // 0 for a part with no position
      s += wgt;
      acc = fmaf(wgt, bf16_to_f32(op[(((int64_t)b * parts + i) * h_q + h) * 256 + d]), acc);
    }
  }
  float out = s > 0.f ? acc / s : 0.f;
  float ls = s > 0.f ? m + __logf(s) : -INFINITY;
  if (nan) out = ls = __builtin_nanf("");
  o[b * so.b + (int64_t)h * so.h + d] = (uint16_t)(pack_bf16x2(out, 0.f) & 0xffffu);
  if (lse && d == 0) lse[(int64_t)b * h_q + h] = ls;
}

}  // namespace

hipError_t launch_dsa_decode_combine256(const void* op, const float* lp, int parts, void* o, LStrides so, float* lse,
                                        int batch, int h_q, hipStream_t st) {
  hipLaunchKernelGGL(decode_combine256_kernel, dim3(h_q, batch), dim3(256), 0, st, (const uint16_t*)op, lp, parts,
                     (uint16_t*)o, so, lse, h_q);
  return hipGetLastError();
}

hipError_t launch_dsa_sparse_attn256(const void* q, LStrides sq, const void* k, LStrides sk, const void* v,
                                     LStrides sv, const int32_t* idx, void* o, LStrides so, float* lse, int batch,
                                     int seqlen, int n_kv, int h_q, int h_kv, int topk, float scale, hipStream_t st) {
  SparseParams p;
  p.q = (const uint16_t*)q; p.sq = sq;
  p.k = (const uint16_t*)k; p.sk = sk;
  p.v = (const uint16_t*)v; p.sv = sv;
  p.idx = idx;
  p.o = (uint16_t*)o; p.so = so;
  p.lse = lse;
  p.seqlen = seqlen; p.n_kv = n_kv; p.h_q = h_q; p.h_kv = h_kv; p.topk = topk;
  const int group = h_q / h_kv;
  if (group % HPB != 0 || topk > MAX_TOPK || sk.s < 0 || sv.s < 0) return hipErrorInvalidValue;
  p.n_hb = group / HPB;
  p.c = scale * kLog2e;
  // 32-bit row offsets (with __umul24) while every gathered byte of a K or V
  // plane lies below 2^31 from its base
  const uint64_t kr = 2ull * (uint64_t)sk.s, vr = 2ull * (uint64_t)sv.s;
  const uint64_t span = (uint64_t)(n_kv - 1) * (kr > vr ? kr : vr) + ROWB;
  const bool wide = n_kv >= (1 << 24) || kr >= (1ull << 24) || vr >= (1ull << 24) || span >= (1ull << 31);
  p.k_row_bytes = (uint32_t)kr;
  p.v_row_bytes = (uint32_t)vr;
  const bool pos = !(p.c < 0.f);
  dim3 grid(seqlen, h_kv * p.n_hb, batch);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, p); };
  // Two workgroups per CU pay off when there are enough of them to fill the
  // chip; a small grid (decode: one workgroup per sequence) keeps the deeper
  // ring, which hides more gather latency per workgroup.
  const int64_t n_wg = (int64_t)seqlen * h_kv * p.n_hb * batch;
  if (topk <= 2048 && n_wg >= 1024) {
    if (wide) pos ? go(sparse_attn256_kernel<true, true, 2, 2048>) : go(sparse_attn256_kernel<false, true, 2, 2048>);
    else pos ? go(sparse_attn256_kernel<true, false, 2, 2048>) : go(sparse_attn256_kernel<false, false, 2, 2048>);
  } else {
    if (wide) pos ? go(sparse_attn256_kernel<true, true, 4, 4096>) : go(sparse_attn256_kernel<false, true, 4, 4096>);
    else pos ? go(sparse_attn256_kernel<true, false, 4, 4096>) : go(sparse_attn256_kernel<false, false, 4, 4096>);
  }
  return hipGetLastError();
}

}  // namespace hca
