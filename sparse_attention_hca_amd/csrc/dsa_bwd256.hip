// Backward of DSA core attention over the top-k selected positions, bf16,
// d_qk = d_v = 256 (ERNIE 5.5 Flash Base pages: mirrorspeed page, "Hybrid
// sparse attention" section, gives the forward; ai-club.cn page, hybrid
// attention section -- 256-wide heads in the full-context layers; training
// runs at 128K, so the backward runs at the full DSA shape).  The gradients
// are the chain rule through the forward (the generic kernels' comment gives
// the formulas): p = exp(scale q.k - lse), dS = p (dO.v - <dO, o>),
// dq = scale dS K, dk_u = scale sum dS q, dv_u = sum p dO.
//
// One workgroup (4 waves) per (query, group of 64 query heads sharing one KV
// head), the forward's layout: the selected K and V rows are gathered 32 at a
// time into LDS by 16-byte DMA (three stages, two tiles in flight), and for
// each tile
//   * wave w forms S^T = K Q^T and dP^T = V dO^T for heads 16w .. 16w+15
//     (v_mfma_f32_16x16x32_bf16, Q and dO fragments in registers), then P and
//     dS = P (dP - D) in fp32;
//   * scale dS is published in LDS twice (packed per head block, the B
//     operand of dQ; and [key][head], the B operand of dK), P once
//     ([key][head]);
//   * wave w accumulates dQ^T += K^T dS^T for dims 64w .. 64w+63 of all 64
//     heads (K^T by transposing LDS reads, dQ in registers for the whole row);
//   * wave w forms the tile's dK^T = Q^T dS^T and dV^T = dO^T P^T for its 64
//     dims (Q^T and dO^T fragments held in registers, read once per query by
//     transposing LDS reads) and writes them, bf16, as the tile's
//     contributions.
// The key gradients are a sum over every (query, head) that selected the
// position: the contributions go to rows of a workspace ordered by position
// (an inverted index of the selections: count, exclusive scan, slot fill)
// and a reduction kernel sums each position's rows in fp32 into dk, dv.  The
// queries are taken in chunks so that the contribution rows stay within a
// fixed workspace; each chunk's reduction adds into dk, dv.  (fp32 atomics
// instead of the sorted rows: measured ~1.3 TB/s of row updates on MI355X,
// five times slower than writing and re-reading bf16 rows.)
#include <mutex>

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
constexpr int NSTAGE = 3;
constexpr int MAX_TOPK = 4096;
constexpr int CROW = 2 * D;            // contribution row: dk (256 bf16) then dv (256 bf16)
constexpr size_t kContribBudget = (size_t)8 << 30;  // workspace for the contribution rows of one chunk

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

struct DsaBwdParams {
  const uint16_t *q, *k, *v, *o, *dout;
  LStrides sq, sk, sv, so, sdo;
  const float* lse;
  const int32_t* idx;
  float* dq;
  LStrides sdq;
  const int32_t* pslot;   // [chunk queries, topk]: contribution row of each entry, -1 if none
  uint16_t* contrib;      // rows of CROW bf16, G per slot
  uint16_t* dummy;        // one CROW row per workgroup: the stores of entries without a slot
  int b, q0, seqlen, n_kv, h_q, h_kv, topk, n_hb, G;
  float scale, c;         // c = scale * log2(e)
};

__device__ __forceinline__ bf16x8 tr_read(const unsigned char* p, int step) {
  const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p + step));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

// Byte offset of head-byte hb of key row rho in the [key][head] exchange
// buffers (64 bf16 heads = 128 B per row): the 8-byte chunk index is XORed with
// rho % 16, so the dK/dV operand reads of 16 rows (each lane 8 bytes of one
// row) spread over the banks instead of piling onto two.
__device__ __forceinline__ uint32_t xoff(int rho, int hb) {
  return rho * (HPB * 2) + 8 * ((hb >> 3) ^ (rho & 15)) + (hb & 7);
}

// Transposing read offset of the A operand of a 16x16x32 step whose 16 rows
// are consecutive 16-element columns of a row-major LDS tile: lane (col, grp)
// reads, for read e (0, 1), 4 elements of row 16e + 4grp + col/4 at columns
// 16 tile + 4(col % 4); with 16-byte chunk c of row r stored in slot
// c ^ 2(r % 8).  The k order the lanes receive is rows {4grp .. 4grp+3,
// 16+4grp .. 16+4grp+3} (+32 per further step).
__device__ __forceinline__ uint32_t tr_off(int col, int grp, int tile) {
  const int row = 4 * grp + (col >> 2);
  const int c = 2 * tile + ((col & 3) >> 1);  // 16-byte chunk of columns 16 tile + 4(col % 4)
  return row * ROWB + 16 * (c ^ (2 * (row & 7))) + 8 * (col & 1);
}

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void dsa_bwd256_kernel(DsaBwdParams p) {
  constexpr int MAX_TILES = MAX_TOPK / TK;
  // the ring; before the tiles it holds the query's Q and dO rows (64 heads x 512 B each)
  __shared__ __attribute__((aligned(1024))) unsigned char ring[NSTAGE * STAGEB];
  __shared__ __attribute__((aligned(16))) int sidx[MAX_TOPK];
  __shared__ __attribute__((aligned(16))) int sslot[MAX_TOPK];
  __shared__ uint32_t tvalid[MAX_TILES];
  __shared__ __attribute__((aligned(16))) unsigned char xq[HPB * TK * 2];   // scale dS, B operand of dQ
  __shared__ __attribute__((aligned(16))) unsigned char xk[TK * HPB * 2];   // scale dS [key][head]
  __shared__ __attribute__((aligned(16))) unsigned char xp[TK * HPB * 2];   // P [key][head]
  __shared__ int last_sh;

  const int t = p.q0 + blockIdx.x;
  const int hb = blockIdx.y % p.n_hb;
  const int g = blockIdx.y / p.n_hb;  // KV head
  const int b = p.b;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int group = p.h_q / p.h_kv;
  const int h0 = g * group + hb * HPB;       // first head of the workgroup
  const int hq = h0 + w * HPW + col;         // this lane's head for S / dP
  const int ntiles_all = (p.topk + TK - 1) / TK;

  if (tid == 0) last_sh = -1;
  // ---- Q and dO rows of the 64 heads into the ring (row-major, chunk c of
  // row r in slot c ^ 2(r % 8)), the query's index row and slots
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ring;
  {
    // 64 rows x 32 chunks per tensor: 8 instructions per wave per tensor
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 16 * w + 2 * i + (lane >> 5);  // head row
      const int slot = lane & 31;
      const int c = slot ^ (2 * (r & 7));
      const uint16_t* qs = p.q + b * p.sq.b + (int64_t)t * p.sq.s + (int64_t)(h0 + r) * p.sq.h + 8 * c;
      const uint16_t* ds = p.dout + b * p.sdo.b + (int64_t)t * p.sdo.s + (int64_t)(h0 + r) * p.sdo.h + 8 * c;
      dma16(qs, lds0 + (16 * w + 2 * i) * ROWB);
      dma16(ds, lds0 + STAGEB + (16 * w + 2 * i) * ROWB);
    }
  }
  constexpr int NJ = MAX_TOPK / 256;
  {
    const int32_t* irow = p.idx + ((int64_t)b * p.seqlen + t) * p.topk;
    const int32_t* srow = p.pslot + (int64_t)blockIdx.x * p.topk;
    int last = -1;
#pragma unroll
    for (int k = 0; k < NJ; ++k) {
      const int j0 = 256 * k;
      if (j0 >= ntiles_all * TK) break;
      const int j = j0 + tid;
      const int u = j < p.topk ? irow[j] : -1;
      const bool ok = u >= 0 && u < p.n_kv;
      if (j < ntiles_all * TK) {
        sidx[j] = ok ? u : 0;
        sslot[j] = (ok && j < p.topk) ? srow[j] : -1;
      }
      const uint64_t bal = __ballot(ok);
      const int tile = (j0 + 64 * w) / TK;
      if (lane == 0) {
        if (tile < ntiles_all) tvalid[tile] = (uint32_t)bal;
        if (tile + 1 < ntiles_all) tvalid[tile + 1] = (uint32_t)(bal >> 32);
      }
      if ((uint32_t)(bal >> 32) != 0u) last = tile + 1;
      else if ((uint32_t)bal != 0u) last = tile;
    }
    __syncthreads();  // last_sh initialised
    if (lane == 0 && last >= 0) atomicMax(&last_sh, last);
  }
  // D = <dO, O> and the log2-domain lse of this lane's head (lanes of one
  // column share the head: each takes 64 of its dims)
  float dlt, lse2;
  {
    const uint16_t* op = p.o + b * p.so.b + (int64_t)t * p.so.s + (int64_t)hq * p.so.h + 64 * grp;
    const uint16_t* gp = p.dout + b * p.sdo.b + (int64_t)t * p.sdo.s + (int64_t)hq * p.sdo.h + 64 * grp;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 x = ld16(op + 8 * i), y = ld16(gp + 8 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(__uint_as_float(x[e] << 16), __uint_as_float(y[e] << 16), acc);
        acc = fmaf(__uint_as_float(x[e] & 0xffff0000u), __uint_as_float(y[e] & 0xffff0000u), acc);
      }
    }
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    dlt = acc;
    lse2 = p.lse[((int64_t)b * p.h_q + hq) * p.seqlen + t] * kLog2e;
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");  // Q, dO rows landed; sidx, tvalid, last_sh complete
  const int ntiles = __builtin_amdgcn_readfirstlane(last_sh + 1);

  // ---- per-query fragments from the staged rows.
  //   qf, df: Q^T / dO^T as the B operand of S^T / dP^T: head 16w + col, dims
  //   32ks + 8grp .. +8 (16-byte reads).
  //   qa, da: Q^T / dO^T as the A operand of dK^T / dV^T: rows = dims 64w + 16i
  //   + col, k = heads 32ks + {4grp .. +3, 16+4grp .. +3} (transposing reads).
  bf16x8 qf[8], df[8], qa[4][2], da[4][2];
  {
    const int r = 16 * w + col;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int c = 4 * ks + grp;
      const uint32_t off = r * ROWB + 16 * (c ^ (2 * (r & 7)));
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ring + off));
      df[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ring + STAGEB + off));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint32_t off = tr_off(col, grp, 4 * w + i) + 32 * ks * ROWB;
        qa[i][ks] = tr_read(ring + off, 16 * ROWB);
        da[i][ks] = tr_read(ring + STAGEB + off, 16 * ROWB);
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // the ring is free for the tiles

  const uint16_t* kb = p.k + b * p.sk.b + (int64_t)g * p.sk.h;
  const uint16_t* vb = p.v + b * p.sv.b + (int64_t)g * p.sv.h;
  // DMA of tile tt into stage st: instruction i of wave w fetches entry 8w+i
  // (lanes 0-31) into LDS row 8w+2i and entry 8w+4+i (lanes 32-63) into row
  // 8w+2i+1.  K rows: chunk c in slot c ^ 2(r % 8) (transposing reads for
  // dQ); V rows: chunk c in slot c ^ (r % 16) (plain 16-byte reads for dP).
  const int hrow = lane >> 5, hl = lane & 31;
  auto issue = [&](int tt, int st) __attribute__((always_inline)) {
    const int4 u4 = *reinterpret_cast<const int4*>(sidx + tt * TK + 8 * w + 4 * hrow);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * w + 2 * i + hrow;
      const int u = i == 0 ? u4.x : i == 1 ? u4.y : i == 2 ? u4.z : u4.w;
      const uint32_t lk = lds0 + st * STAGEB + (8 * w + 2 * i) * ROWB;
      dma16(kb + (int64_t)u * p.sk.s + 8 * (hl ^ (2 * (r & 7))), lk);
      dma16(vb + (int64_t)u * p.sv.s + 8 * (hl ^ (r & 15)), lk + KSTB);
    }
  };
  // entry number of LDS row rho (the DMA above)
  auto entry_of = [](int rho) { return 8 * (rho >> 3) + 4 * (rho & 1) + ((rho & 7) >> 1); };

  f32x4 dqa[4][4];  // dQ^T: dim tile 4w + i, head block hk
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int hk = 0; hk < 4; ++hk) dqa[i][hk] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float c = p.c, sc = p.scale;

  // Two tiles in flight.  Every wave issues exactly 8 DMA instructions per
  // tile (re-reading the last tile past the end) and 16 contribution stores
  // per tile (entries without a slot store to the workgroup's dummy row), so
  // the wait for tile tt counts what was issued after its DMA: the stores of
  // tiles tt-2 and tt-1 and the DMA of tile tt+1 -- the stores stay in flight.
  const int last = ntiles - 1;
  if (ntiles > 0) {
    issue(0, 0);
    issue(min(1, last), 1);
  }
  for (int tt = 0; tt < ntiles; ++tt) {
    const int st = tt % NSTAGE;
    // tile tt landed; every wave is done with the exchange buffers and with
    // the stage of tile tt - 1, which the DMA of tile tt + 2 refills
    if (tt >= 2) asm volatile("s_waitcnt vmcnt(40)\n\ts_barrier" ::: "memory");
    else if (tt == 1) asm volatile("s_waitcnt vmcnt(24)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    issue(min(tt + 2, last), (tt + 2) % NSTAGE);
    const unsigned char* sk_ = ring + st * STAGEB;
    const unsigned char* sv_ = sk_ + KSTB;
    const uint32_t vmask = tvalid[tt];

    // S^T = K Q^T and dP^T = V dO^T: rows = keys 16kt + col, k = dims
    f32x4 s[2], dp[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = 16 * kt + col;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int cc = 4 * ks + grp;
        const bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sk_ + r * ROWB + 16 * (cc ^ (2 * (r & 7)))));
        const bf16x8 va = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sv_ + r * ROWB + 16 * (cc ^ (r & 15))));
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[ks], s[kt], 0, 0, 0);
        dp[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, df[ks], dp[kt], 0, 0, 0);
      }
    }
    // P and scale dS of this lane's 8 keys (rows 16kt + 4grp + r) of head hq
    float pv[8], dsv[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rho = 16 * kt + 4 * grp + r;
        const bool ok = (vmask >> entry_of(rho)) & 1u;
        const float pr = ok ? __builtin_amdgcn_exp2f(fmaf(s[kt][r], c, -lse2)) : 0.f;
        pv[4 * kt + r] = pr;
        dsv[4 * kt + r] = sc * pr * (dp[kt][r] - dlt);
      }
    // publish: packed per head block (xq), [key][head] (xk, xp)
    {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(dsv[2 * e], dsv[2 * e + 1]);
      *reinterpret_cast<u32x4*>(xq + w * (HPW * TK * 2) + 16 * lane) = pk;
      const int hl_ = w * HPW + col;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rho = 16 * kt + 4 * grp + r;
          const uint32_t ds2 = pack_bf16x2(dsv[4 * kt + r], 0.f), p2 = pack_bf16x2(pv[4 * kt + r], 0.f);
          *reinterpret_cast<uint16_t*>(xk + xoff(rho, 2 * hl_)) = (uint16_t)ds2;
          *reinterpret_cast<uint16_t*>(xp + xoff(rho, 2 * hl_)) = (uint16_t)p2;
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // dQ^T += K^T dS^T: this wave's dim tiles x the 4 head blocks, k = the tile's keys
    {
      bf16x8 bq[4];
#pragma unroll
      for (int hk = 0; hk < 4; ++hk)
        bq[hk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xq + hk * (HPW * TK * 2) + 16 * lane));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 ka = tr_read(sk_ + tr_off(col, grp, 4 * w + i), 16 * ROWB);
#pragma unroll
        for (int hk = 0; hk < 4; ++hk) dqa[i][hk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, bq[hk], dqa[i][hk], 0, 0, 0);
      }
    }
    // dK^T = Q^T dS^T and dV^T = dO^T P^T for this wave's 64 dims and the
    // tile's 32 keys (columns: key half kh, key row 16kh + col), k = 64 heads
    // in the transposing reads' order.  At most 47 memory operations may be
    // in flight before the tile's 16 stores (the counter holds 63).
    asm volatile("s_waitcnt vmcnt(47)" ::: "memory");
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const unsigned char* xs = which ? xp : xk;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int rho = 16 * kh + col;
        bf16x8 bk[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int hb = 2 * (32 * ks + 4 * grp);  // heads 32ks + 4grp .. +3, then 16 further
          const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(xs + xoff(rho, hb));
          const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(xs + xoff(rho, hb + 32));
          bk[ks] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        }
        const int slot = sslot[tt * TK + entry_of(rho)];
        uint16_t* dst = (slot >= 0 ? p.contrib + ((int64_t)slot * p.G + (g * p.n_hb + hb)) * CROW
                                   : p.dummy + ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * CROW) +
                        which * D + 64 * w + 4 * grp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(which ? da[i][ks] : qa[i][ks], bk[ks], acc, 0, 0, 0);
          u32x2 pk;
          pk[0] = pack_bf16x2(acc[0], acc[1]);
          pk[1] = pack_bf16x2(acc[2], acc[3]);
          *reinterpret_cast<u32x2*>(dst + 16 * i) = pk;
        }
      }
    }
  }

  // no DMA may still target this workgroup's LDS when it exits
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- dq (the scale is in dS): lane holds dims 16(4w+i) + 4grp .. +3 of head 16hk + col
#pragma unroll
  for (int hk = 0; hk < 4; ++hk) {
    float* dp_ = p.dq + b * p.sdq.b + (int64_t)t * p.sdq.s + (int64_t)(h0 + HPW * hk + col) * p.sdq.h + 4 * grp;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4*>(dp_ + 16 * (4 * w + i)) = dqa[i][hk];
  }
}

// ---- inverted index of one chunk's selections, and the reduction
__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

// dk, dv rows of batch b to zero (general strides; d floats per row)
__global__ __launch_bounds__(256) void zero_rows_kernel(float* x, LStrides s, int b, int rows, int h, int d) {
  const int64_t n = (int64_t)rows * h * d;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int e = (int)(i % d);
    const int64_t rh = i / d;
    x[b * s.b + (rh / h) * s.s + (rh % h) * s.h + e] = 0.f;
  }
}

__global__ __launch_bounds__(256) void chunk_count_kernel(const int32_t* idx, int b, int seqlen, int n_kv, int topk,
                                                          int q0, int nq, int32_t* cnt) {
  const int64_t n = (int64_t)nq * topk;
  const int32_t* base = idx + ((int64_t)b * seqlen + q0) * topk;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int u = base[e];
    if (u >= 0 && u < n_kv) atomicAdd(&cnt[u], 1);
  }
}

// exclusive prefix of cnt[0 .. n) in place, cnt[n] = total (one workgroup)
__global__ __launch_bounds__(256) void chunk_scan_kernel(int32_t* cnt, int n) {
  __shared__ int32_t part[256];
  const int tid = threadIdx.x;
  const int per = (n + 255) / 256;
  const int lo = tid * per, hi = min(lo + per, n);
  int32_t sum = 0;
  for (int u = lo; u < hi; ++u) sum += cnt[u];
  part[tid] = sum;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const int32_t x = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  int32_t run = part[tid] - sum;
  for (int u = lo; u < hi; ++u) {
    const int32_t x = cnt[u];
    cnt[u] = run;
    run += x;
  }
  if (tid == 255) cnt[n] = part[255];
}

// pslot of every entry of the chunk: off[u] + a per-position cursor (the
// order inside a position's rows is the cursor race's; sums do not depend on
// it beyond rounding)
__global__ __launch_bounds__(256) void chunk_fill_kernel(const int32_t* idx, int b, int seqlen, int n_kv, int topk,
                                                         int q0, int nq, const int32_t* off, int32_t* cur,
                                                         int32_t* pslot) {
  const int64_t n = (int64_t)nq * topk;
  const int32_t* base = idx + ((int64_t)b * seqlen + q0) * topk;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int u = base[e];
    pslot[e] = (u >= 0 && u < n_kv) ? off[u] + atomicAdd(&cur[u], 1) : -1;
  }
}

// dk[u, g] += scale-free sum of its rows (the scale is in dS), dv likewise:
// one wave per (position, KV head); lane l sums 8 values (16 bytes) of the
// 1 KB rows: dk dims 8l (l < 32), dv dims 8(l - 32).
__global__ __launch_bounds__(64) void chunk_reduce_kernel(const uint16_t* contrib, const int32_t* off, int G,
                                                          int n_hb, float* dk, LStrides sdk, float* dv, LStrides sdv,
                                                          int b) {
  const int u = blockIdx.x, g = blockIdx.y, l = threadIdx.x;
  const int beg = off[u], end = off[u + 1];
  if (beg == end) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const u32x4& x) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __uint_as_float(x[e] << 16);
      acc[2 * e + 1] += __uint_as_float(x[e] & 0xffff0000u);
    }
  };
  // the rows of (u, g): n_hb per slot; eight loads in flight at a time
  const int64_t r0 = (int64_t)beg * G + g * n_hb, nr = (int64_t)(end - beg) * n_hb;
  auto row = [&](int64_t i) __attribute__((always_inline)) {
    const int64_t s = i / n_hb, hb = i - s * n_hb;
    return contrib + (r0 + s * G + hb) * CROW + 8 * l;
  };
  int64_t i = 0;
  for (; i + 8 <= nr; i += 8) {
    u32x4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = ld16(row(i + j));
#pragma unroll
    for (int j = 0; j < 8; ++j) add(x[j]);
  }
  for (; i < nr; ++i) add(ld16(row(i)));
  float* dst = l < 32 ? dk + b * sdk.b + (int64_t)u * sdk.s + (int64_t)g * sdk.h + 8 * l
                      : dv + b * sdv.b + (int64_t)u * sdv.s + (int64_t)g * sdv.h + 8 * (l - 32);
  f32x4 a0 = *reinterpret_cast<const f32x4*>(dst), a1 = *reinterpret_cast<const f32x4*>(dst + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a0[e] += acc[e];
    a1[e] += acc[4 + e];
  }
  *reinterpret_cast<f32x4*>(dst) = a0;
  *reinterpret_cast<f32x4*>(dst + 4) = a1;
}

int chunk_queries(int seqlen, int topk, int G) {
  const size_t per_q = (size_t)topk * G * CROW * 2;
  const size_t cq = kContribBudget / per_q;
  return (int)(cq < (size_t)seqlen ? (cq > 0 ? cq : 1) : seqlen);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// One set of chunk buffers: counts -> offsets, cursors, slots, contribution rows.
size_t chunk_set_bytes(int n_kv, int cq, int topk, int G) {
  return align256((size_t)(n_kv + 1) * 4) + align256((size_t)n_kv * 4) + align256((size_t)cq * topk * 4) +
         align256((size_t)cq * topk * G * CROW * 2);
}

// Events of the backward's chunk pipeline, created once per device.
struct BwdEvents {
  bool ready = false;
  hipEvent_t start = nullptr;                // the caller's stream reached the call (dk, dv zeroed)
  hipEvent_t idx[2] = {nullptr, nullptr};    // inverted index of buffer set i built (side stream)
  hipEvent_t main[2] = {nullptr, nullptr};   // contributions of buffer set i written (caller's stream)
  hipEvent_t end = nullptr;                  // last reduction done (side stream)
};
std::mutex g_bwd_mu;
BwdEvents g_bwd_ev[64];

hipError_t bwd_events(BwdEvents*& out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  BwdEvents& ev = g_bwd_ev[dev];
  if (!ev.ready) {
    hipEvent_t* all[6] = {&ev.start, &ev.idx[0], &ev.idx[1], &ev.main[0], &ev.main[1], &ev.end};
    for (int i = 0; i < 6 && e == hipSuccess; ++i) e = hipEventCreateWithFlags(all[i], hipEventDisableTiming);
    if (e != hipSuccess) return e;
    ev.ready = true;
  }
  out = &ev;
  return hipSuccess;
}

}  // namespace

bool dsa_bwd_uses_mfma(int dt, int d_qk, int d_v, int h_q, int h_kv) {
  return dt == 1 && d_qk == D && d_v == D && h_kv > 0 && h_q % h_kv == 0 && (h_q / h_kv) % HPB == 0;
}

size_t dsa_bwd256_workspace_bytes(int batch, int seqlen, int h_q, int h_kv, int topk) {
  const int G = h_kv * (h_q / h_kv / HPB);
  const int cq = chunk_queries(seqlen, topk, G);
  const int64_t chunks = (int64_t)batch * ((seqlen + cq - 1) / cq);
  return (chunks > 1 ? 2 : 1) * chunk_set_bytes(seqlen, cq, topk, G)  // one or two buffer sets
         + (size_t)cq * G * CROW * 2;                                 // one dummy row per workgroup
}

// The call runs in chunks of cq queries; chunk c uses buffer set c % 2.  With
// more than one chunk the inverted index of each chunk (zero, count, scan,
// fill) and its per-position reduction run on the library's side stream, and
// the MFMA kernel on the caller's stream, ordered by events: the MFMA kernel
// of chunk c needs its index; its reduction needs its contributions; the index
// of chunk c + 2 (same buffer set) is built after the reduction of chunk c,
// and the MFMA kernel of chunk c + 2 waits for that index, hence for the
// reduction too.  So the reduction of chunk c - 1 and the index of chunk c + 1
// run beside the MFMA kernel of chunk c.  The reductions add into dk, dv in
// chunk order on the one side stream.
hipError_t launch_dsa_bwd256(const BwdArgs& a, void* ws, hipStream_t st) {
  const int group = a.h_q / a.h_kv;
  const int n_hb = group / HPB, G = a.h_kv * n_hb;
  const int cq = chunk_queries(a.seqlen_q, a.topk, G);
  if (a.topk > MAX_TOPK) return hipErrorInvalidValue;
  const int per_batch = (a.seqlen_q + cq - 1) / cq;
  const int total = a.batch * per_batch;
  const bool overlap = total > 1;

  struct Set {
    int32_t *cnt, *cur, *pslot;
    uint16_t* contrib;
  } set[2];
  char* pw = (char*)ws;
  for (int k = 0; k < (overlap ? 2 : 1); ++k) {
    set[k].cnt = (int32_t*)pw;
    pw += align256((size_t)(a.seqlen_kv + 1) * 4);
    set[k].cur = (int32_t*)pw;
    pw += align256((size_t)a.seqlen_kv * 4);
    set[k].pslot = (int32_t*)pw;
    pw += align256((size_t)cq * a.topk * 4);
    set[k].contrib = (uint16_t*)pw;
    pw += align256((size_t)cq * a.topk * G * CROW * 2);
  }
  uint16_t* dummy = (uint16_t*)pw;

  DsaBwdParams p;
  p.q = (const uint16_t*)a.q; p.k = (const uint16_t*)a.k; p.v = (const uint16_t*)a.v;
  p.o = (const uint16_t*)a.o; p.dout = (const uint16_t*)a.dout;
  p.sq = a.sq; p.sk = a.sk; p.sv = a.sv; p.so = a.so; p.sdo = a.sdo;
  p.lse = a.lse; p.idx = a.idx; p.dq = a.dq; p.sdq = a.sdq;
  p.dummy = dummy;
  p.seqlen = a.seqlen_q; p.n_kv = a.seqlen_kv; p.h_q = a.h_q; p.h_kv = a.h_kv; p.topk = a.topk;
  p.n_hb = n_hb; p.G = G;
  p.scale = a.scale; p.c = a.scale * kLog2e;

  std::unique_lock<std::mutex> lock(g_bwd_mu, std::defer_lock);
  BwdEvents* ev = nullptr;
  hipStream_t side = st;
  if (overlap) {
    lock.lock();
    hipError_t e = bwd_events(ev);
    if (e == hipSuccess) e = side_stream(&side);
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipSuccess;
  // dk, dv of every sequence start at zero; the side stream starts after them
  // (and after everything queued before this call)
  for (int b = 0; b < a.batch; ++b) {
    hipLaunchKernelGGL(zero_rows_kernel, dim3(1024), dim3(256), 0, st, a.dk, a.sdk, b, a.seqlen_kv, a.h_kv, a.d);
    hipLaunchKernelGGL(zero_rows_kernel, dim3(1024), dim3(256), 0, st, a.dv, a.sdv, b, a.seqlen_kv, a.h_kv, a.d_v);
  }
  if (overlap) {
    e = hipEventRecord(ev->start, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(side, ev->start, 0);
    if (e != hipSuccess) return e;
  }
  auto chunk_b = [&](int c) { return c / per_batch; };
  auto chunk_q0 = [&](int c) { return (c % per_batch) * cq; };
  auto chunk_nq = [&](int c) { return cq < a.seqlen_q - chunk_q0(c) ? cq : a.seqlen_q - chunk_q0(c); };
  auto build_index = [&](int c) -> hipError_t {
    const Set& S = set[c & 1];
    const int b = chunk_b(c), q0 = chunk_q0(c), nq = chunk_nq(c);
    const int64_t ne = (int64_t)nq * a.topk;
    const int gx = (int)((ne + 255) / 256 < 4096 ? (ne + 255) / 256 : 4096);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(256), dim3(256), 0, side, S.cnt, (int64_t)a.seqlen_kv + 1);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(256), dim3(256), 0, side, S.cur, (int64_t)a.seqlen_kv);
    hipLaunchKernelGGL(chunk_count_kernel, dim3(gx), dim3(256), 0, side, a.idx, b, a.seqlen_q, a.seqlen_kv, a.topk,
                       q0, nq, S.cnt);
    hipLaunchKernelGGL(chunk_scan_kernel, dim3(1), dim3(256), 0, side, S.cnt, a.seqlen_kv);
    hipLaunchKernelGGL(chunk_fill_kernel, dim3(gx), dim3(256), 0, side, a.idx, b, a.seqlen_q, a.seqlen_kv, a.topk, q0,
                       nq, (const int32_t*)S.cnt, S.cur, S.pslot);
    hipError_t r = hipGetLastError();
    if (r == hipSuccess && overlap) r = hipEventRecord(ev->idx[c & 1], side);
    return r;
  };
  e = build_index(0);
  if (e == hipSuccess && total > 1) e = build_index(1);
  for (int c = 0; c < total && e == hipSuccess; ++c) {
    const Set& S = set[c & 1];
    if (overlap) e = hipStreamWaitEvent(st, ev->idx[c & 1], 0);
    if (e != hipSuccess) break;
    p.b = chunk_b(c);
    p.q0 = chunk_q0(c);
    p.pslot = S.pslot;
    p.contrib = S.contrib;
    hipLaunchKernelGGL(dsa_bwd256_kernel, dim3(chunk_nq(c), a.h_kv * n_hb), dim3(256), 0, st, p);
    e = hipGetLastError();
    if (e == hipSuccess && overlap) {
      e = hipEventRecord(ev->main[c & 1], st);
      if (e == hipSuccess) e = hipStreamWaitEvent(side, ev->main[c & 1], 0);
    }
    if (e != hipSuccess) break;
    hipLaunchKernelGGL(chunk_reduce_kernel, dim3(a.seqlen_kv, a.h_kv), dim3(64), 0, side, (const uint16_t*)S.contrib,
                       (const int32_t*)S.cnt, G, n_hb, a.dk, a.sdk, a.dv, a.sdv, chunk_b(c));
    e = hipGetLastError();
    if (e == hipSuccess && c + 2 < total) e = build_index(c + 2);
  }
  if (e == hipSuccess && overlap) {
    // the caller's stream waits for the last reduction (the side stream runs
    // every earlier one before it)
    e = hipEventRecord(ev->end, side);
    if (e == hipSuccess) e = hipStreamWaitEvent(st, ev->end, 0);
  }
  return e;
}

}  // namespace hca
