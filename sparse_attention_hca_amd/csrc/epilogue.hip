// Attention-output epilogue (ERNIE 5.5 Flash Base pages: mirrorspeed page,
// section "More structural improvements, data, and infrastructure"; besthub
// page, section "Core Architectural Innovations"): the output gate computed
// from the layer's low-rank query latent, and Virtual Head Attention's
// low-rank cross-head mixing with an identity skip, in one kernel:
//   y[b,t,h,e] = sigmoid(<c[b,t,:], W_g[h*d_v + e, :]>) * (o[b,t,h,e] + sum_h' (U V)[h,h'] o[b,t,h',e])
//
// gate_vha_kernel is a bf16 MFMA GEMM (v_mfma_f32_32x32x16_bf16, fp32
// accumulation) of the gate pre-activations G = C W_g^T whose epilogue applies
// the sigmoid, the head mixing and the product, so G never leaves registers:
//   * Workgroup tile: 256 tokens x 256 gate columns, 8 waves of 64 x 128 (two
//     per SIMD).  The 256 columns are every head's weights for a slice of
//     256 / H dims, ordered so that each lane ends with, for each of its
//     tokens, all H heads of 64 / H consecutive dims: the mixing over heads
//     is then a per-lane computation with no exchange.
//   * K (the latent, d_c) is streamed in chunks of 32 through a 5-stage LDS
//     ring (four chunks in flight, the whole 160 KB) by 16-byte LDS DMA; LDS
//     rows are 64 bytes with the four 16-byte chunks of row r XOR-swizzled by
//     (r / 4) % 4, which keeps the 16-byte operand reads of 16 consecutive
//     rows on distinct bank groups while each DMA instruction still fills one
//     contiguous kilobyte.  The product is formed transposed (weight rows as
//     the A operand), so the accumulator rows are gate columns.
//   * The workgroups one XCD runs at once take a 4 x 8 block of tiles
//     (tokens x dim slices): they share latent and weight rows in that XCD's
//     L2, and the 8 neighbouring dim slices cover whole 256-byte runs of o
//     and y.
//   * The tile's o rows (256 tokens x every head's 256 / H dims) follow the
//     last K chunk into the ring as four extra chunks, so they load under the
//     last MFMAs; each lane mixes its dims in LDS in place and the tile's y
//     leaves as whole per-head pieces.  U and V sit in the stage left free.
#include "device_common.h"
#include "launchers.h"
#include "mfma_asm.h"

namespace hca {
namespace {

constexpr int GM = 256, GN = 256, GK = 32;  // workgroup tile and K chunk
constexpr int G_WAVES = 8;                  // 4 (tokens) x 2 (columns) waves of 64 x 128
constexpr int A_ST = GM * 64, B_ST = GN * 64, G_STAGE = A_ST + B_ST;
constexpr int G_NST = 5;  // ring stages: chunk kc + 4 is issued while chunk kc is consumed

struct EpiParams {
  const uint16_t* c;  // latent: token (b, t) at c + b*scb + t*scs, d_c contiguous
  int64_t scb, scs;
  const uint16_t* w;  // W_g [H * d_v, d_c] contiguous
  const uint16_t* o;  // attention output [B, S, H, d_v]
  LStrides so;
  uint16_t* y;  // result [B, S, H, d_v]
  LStrides sy;
  const float* u;  // U [H, r]
  const float* v;  // V [r, H]
  int seqlen, M, d_c, d_v, r;
  int m_tiles, n_tiles;
};

// LDS offset of 16-byte chunk `ch` (0..3) of row r in a swizzled 64-byte-row tile.
__device__ __forceinline__ uint32_t swz(int r, int ch) { return (uint32_t)(r * 64 + 16 * (ch ^ ((r >> 2) & 3))); }

// Tile of workgroup `bid`.  Workgroups are dispatched to the 8 XCDs round
// robin, so when the count is a multiple of 8, XCD x is given the contiguous
// range x * (count / 8) .. of linear tiles; linear tiles then walk groups of 4
// token tiles, 4 consecutive tiles being the 4 token tiles of one dim slice.
__device__ __forceinline__ void tile_of(int bid, int m_tiles, int n_tiles, int& mt, int& nt) {
  const int nblk = m_tiles * n_tiles;
  const int T = (nblk & 7) ? bid : (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int g = T / (4 * n_tiles);
  const int gm = min(4, m_tiles - 4 * g);
  const int idx = T - g * 4 * n_tiles;
  mt = 4 * g + idx % gm;
  nt = idx / gm;
}

// NE consecutive bf16 of one head's row of o, as loaded.
template <int NE>
struct Raw;
template <>
struct Raw<8> {
  using T = u32x4;
};
template <>
struct Raw<4> {
  using T = u32x2;
};
template <>
struct Raw<2> {
  using T = uint32_t;
};
template <>
struct Raw<1> {
  using T = uint16_t;
};

template <int NE>
__device__ __forceinline__ float unpack(const typename Raw<NE>::T& x, int i) {
  if constexpr (NE == 1) {
    return __uint_as_float((uint32_t)x << 16);
  } else if constexpr (NE == 2) {
    return __uint_as_float(i ? (x & 0xffff0000u) : (x << 16));
  } else {
    const uint32_t d = x[i >> 1];
    return __uint_as_float((i & 1) ? (d & 0xffff0000u) : (d << 16));
  }
}

template <int NE>
__device__ __forceinline__ typename Raw<NE>::T pack(const float* f) {
  typename Raw<NE>::T x;
  if constexpr (NE == 1) {
    x = (uint16_t)(pack_bf16x2(f[0], 0.f) & 0xffffu);
  } else if constexpr (NE == 2) {
    x = pack_bf16x2(f[0], f[1]);
  } else {
#pragma unroll
    for (int i = 0; i < NE / 2; ++i) x[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  }
  return x;
}

// R: the rank rounded up to 4, 8 or 16 (U, V zero-padded in LDS).
template <int H, int R>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gate_vha_kernel(EpiParams p) {
  constexpr int EW = GN / H;  // dims of every head in one tile
  constexpr int NE = 64 / H;  // consecutive dims of every head in one lane (per token)
  using RawT = typename Raw<NE>::T;
  // the 160 KB ring; at the end of the K loop it takes the tile's o rows and U and V
  __shared__ __attribute__((aligned(16))) unsigned char smem[G_NST * G_STAGE];
  static_assert(2 * H * R * 4 <= G_STAGE, "U and V do not fit in one ring stage");
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int col = lane & 31, hf = lane >> 5;
  const int M = p.M;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)smem;

  // U and V, zero-padded to rank R (stored to LDS after the K loop)
  constexpr int UV_PER = (H * R + 511) / 512;
  float ureg[UV_PER], vreg[UV_PER];
#pragma unroll
  for (int k = 0; k < UV_PER; ++k) {
    const int i = tid + 512 * k;
    const int h = i / R, j = i % R;
    const bool ok = i < H * R && j < p.r;
    ureg[k] = ok ? p.u[h * p.r + j] : 0.f;
    vreg[k] = ok ? p.v[j * H + h] : 0.f;
  }

  int mt, nt;
  tile_of(blockIdx.x, p.m_tiles, p.n_tiles, mt, nt);
  const int m0 = mt * GM, e0 = nt * EW;
  const int ln = lane;

  // Source rows of this wave's four DMA instructions per chunk (16 rows of 64
  // bytes each): instructions w and w + 8 fill latent rows, w + 16 and w + 24
  // weight rows.  Weight row r of the tile feeds accumulator row rho = r % 128
  // of wave column r / 128; rho = 32 j + 8 q + 4 hf + c is slot s = 16 j + 4 q
  // + c of lane half hf, which holds head s % H, dim s / H of that half's dims.
  const uint16_t* src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ins = w + G_WAVES * i;
    const int r = 16 * (ins & 15) + (ln >> 2);
    const int ch = (ln & 3) ^ ((r >> 2) & 3);  // the global chunk this LDS slot holds
    if (i < 2) {
      const int m = min(m0 + r, M - 1);
      const int b = m / p.seqlen, t = m - b * p.seqlen;
      src[i] = p.c + b * p.scb + (int64_t)t * p.scs + 8 * ch;
    } else {
      const int rho = r & 127, wr = r >> 7;
      const int s = 16 * (rho >> 5) + 4 * ((rho >> 3) & 3) + (rho & 3);
      const int h = s % H;
      const int e = e0 + (128 / H) * wr + (64 / H) * ((rho >> 2) & 1) + s / H;
      src[i] = p.w + (int64_t)(h * p.d_v + e) * p.d_c + 8 * ch;
    }
  }
  auto issue = [&](int kc, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ins = w + G_WAVES * i;
      dma16_m0(src[i] + kc * GK, lds0 + st * G_STAGE + (i < 2 ? 0 : A_ST) + 1024 * (ins & 15));
    }
  };

  // acc[j][i]: gate columns 128 wn + 32 j .. (rows) x tokens 64 wm + 32 i .. (columns)
  f32x16 acc[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

  auto step = [&](int kc) __attribute__((always_inline)) {
    const unsigned char* sa = smem + (kc % G_NST) * G_STAGE;
    const unsigned char* sb = sa + A_ST;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = 2 * ks + hf;
      bf16x8 af[2], bfr[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 64 * wm + 32 * i + col;
        af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sa + swz(r, ch)));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 128 * wn + 32 * j + col;
        bfr[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sb + swz(r, ch)));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[j][i], 0, 0, 0);
    }
  };

  // The tile's o rows -- 256 tokens x 512 bytes (every head's 256 / H dims)
  // -- come into the ring by LDS DMA as four quarters of 64 tokens, one ring
  // stage each: piece (token t, head h) of PB bytes at row t % 64 of quarter
  // t / 64, byte (h ^ (t % H)) * PB (the XOR spreads a lane column's reads
  // over the banks).  With 16-byte pieces or wider, the quarters ride the
  // ring as four extra chunks behind the last K chunk (quarter q in stage
  // (nk + q) % G_NST), so they load under the last MFMAs; otherwise they
  // load into stages 0..3 after the loop.
  constexpr int PB = 512 / H;                 // bytes of one head's dims in one token row
  constexpr int DB = PB >= 16 ? 16 : 4;       // bytes per lane of one o DMA
  constexpr int SB = PB >= 16 ? 16 : PB;      // bytes per lane of one y store
  constexpr bool OVIRT = DB == 16;
  const int nk = p.d_c / GK;
  auto oq_stage = [&](int q) __attribute__((always_inline)) { return OVIRT ? (nk + q) % G_NST : q; };
  auto piece_src = [&](int off, int& t, int& h, int& pin) __attribute__((always_inline)) {
    t = off >> 9;
    const int within = off & 511;
    h = (within / PB) ^ (t & (H - 1));
    pin = within % PB;
  };
  auto token_off = [&](int t, const LStrides& st) __attribute__((always_inline)) {
    const int m = min(m0 + t, M - 1);
    const int b = m / p.seqlen, tt = m - b * p.seqlen;
    return b * st.b + (int64_t)tt * st.s;
  };
  // one quarter: 32 KB, 32 instructions of 1 KB (4 per wave, like a K chunk) at DB = 16
  auto issue_oq = [&](int q) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 32 * 1024 / (64 * DB) / G_WAVES; ++k) {
      const int ins = w + G_WAVES * k;
      int t, h, pin;
      piece_src(q * 32768 + ins * 64 * DB + ln * DB, t, h, pin);
      const uint16_t* g = p.o + token_off(t, p.so) + (int64_t)h * p.so.h + e0 + pin / 2;
      const uint32_t dst = lds0 + oq_stage(q) * G_STAGE + ins * 64 * DB;
      if constexpr (DB == 16) dma16_m0(g, dst);
      else dma4_m0(g, dst);
    }
  };
  auto issue_v = [&](int v) __attribute__((always_inline)) {
    if (v < nk) issue(v, v % G_NST);
    else if (OVIRT && v < nk + 4) issue_oq(v - nk);
  };

#pragma unroll
  for (int k = 0; k < G_NST - 1; ++k) issue_v(k);
  if constexpr (OVIRT) {
    // chunk kc landed once at most the three newer (virtual) chunks' DMAs, 4 per wave each, are in flight
    for (int kc = 0; kc < nk; ++kc) {
      asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");
      issue_v(kc + 4);
      step(kc);
    }
    // the o quarters landed; every wave is done with the ring's K stages
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  } else {
    int kc = 0;
    for (; kc + 3 < nk; ++kc) {
      asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");
      if (kc + 4 < nk) issue(kc + 4, (kc + 4) % G_NST);
      step(kc);
    }
    if (kc + 2 < nk) {
      asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
      step(kc);
      ++kc;
    }
    if (kc + 1 < nk) {
      asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
      step(kc);
      ++kc;
    }
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    step(kc);
    asm volatile("s_barrier" ::: "memory");  // every wave is done with the ring
#pragma unroll
    for (int q = 0; q < 4; ++q) issue_oq(q);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  // U and V in the stage the o quarters leave free
  float* su = reinterpret_cast<float*>(smem + (OVIRT ? (nk + 4) % G_NST : 4) * G_STAGE);
  float* sv = su + H * R;
#pragma unroll
  for (int k = 0; k < UV_PER; ++k) {
    const int i = tid + 512 * k;
    if (i < H * R) {
      const int h = i / R, j = i % R;
      su[i] = ureg[k];
      sv[j * H + h] = vreg[k];
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // Epilogue: each lane mixes its tokens' dims in place (o in, y out: every
  // element is read and written by one lane only), then the tile goes out as
  // whole pieces.
  const int ebl = (128 / H) * wn + (64 / H) * hf;  // the lane's first dim within the tile's slice
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    // U and V are re-read from LDS for each token rather than held across both
    asm volatile("" ::: "memory");
    const int tl = 64 * wm + 32 * i + col;  // the lane's token within the tile
    unsigned char* row = smem + oq_stage(tl >> 6) * G_STAGE + (tl & 63) * 512 + 2 * ebl;
    auto at = [&](int h) __attribute__((always_inline)) {
      return reinterpret_cast<RawT*>(row + (h ^ (tl & (H - 1))) * PB);
    };
    // the token's accumulators become its gates
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = __builtin_amdgcn_rcpf(1.f + __expf(-acc[j][i][r]));
    float pr[R][NE];
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
      for (int el = 0; el < NE; ++el) pr[rr][el] = 0.f;
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const RawT x = *at(h);
#pragma unroll
      for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int el = 0; el < NE; ++el) pr[rr][el] = fmaf(sv[rr * H + h], unpack<NE>(x, el), pr[rr][el]);
    }
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const RawT x = *at(h);
      float z[NE];
#pragma unroll
      for (int el = 0; el < NE; ++el) {
        float a = unpack<NE>(x, el);
#pragma unroll
        for (int rr = 0; rr < R; ++rr) a = fmaf(su[h * R + rr], pr[rr][el], a);
        const int sl = el * H + h;  // the lane's slot of (head h, dim el)
        z[el] = acc[sl >> 4][i][sl & 15] * a;
      }
      *at(h) = pack<NE>(z);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll 4
  for (int k = 0; k < 256 * 512 / (64 * SB) / G_WAVES; ++k) {
    const int off = (w + G_WAVES * k) * 64 * SB + ln * SB;
    int t, h, pin;
    piece_src(off, t, h, pin);
    const unsigned char* l = smem + oq_stage(t >> 6) * G_STAGE + (off & 32767);
    if (m0 + t < M) {
      uint16_t* g = p.y + token_off(t, p.sy) + (int64_t)h * p.sy.h + e0 + pin / 2;
      if constexpr (SB == 16) *reinterpret_cast<u32x4*>(g) = *reinterpret_cast<const u32x4*>(l);
      else if constexpr (SB == 8) *reinterpret_cast<u32x2*>(g) = *reinterpret_cast<const u32x2*>(l);
    }
  }
}

template <int H>
hipError_t launch_gate_vha(const EpiParams& ep, hipStream_t st) {
  const dim3 grid(ep.m_tiles * ep.n_tiles), block(64 * G_WAVES);
  if (ep.r <= 4) hipLaunchKernelGGL((gate_vha_kernel<H, 4>), grid, block, 0, st, ep);
  else if (ep.r <= 8) hipLaunchKernelGGL((gate_vha_kernel<H, 8>), grid, block, 0, st, ep);
  else hipLaunchKernelGGL((gate_vha_kernel<H, 16>), grid, block, 0, st, ep);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_output_epilogue(const void* o, LStrides so, const void* c, int64_t scb, int64_t scs,
                                       const void* w_g, const float* u, const float* v, void* y, LStrides sy,
                                       int batch, int seqlen, int h, int d_v, int d_c, int r, hipStream_t st) {
  EpiParams ep;
  ep.c = (const uint16_t*)c;
  ep.scb = scb;
  ep.scs = scs;
  ep.w = (const uint16_t*)w_g;
  ep.o = (const uint16_t*)o;
  ep.so = so;
  ep.y = (uint16_t*)y;
  ep.sy = sy;
  ep.u = u;
  ep.v = v;
  ep.seqlen = seqlen;
  ep.M = batch * seqlen;
  ep.d_c = d_c;
  ep.d_v = d_v;
  ep.r = r;
  ep.m_tiles = (ep.M + GM - 1) / GM;
  ep.n_tiles = d_v / (GN / h);
  switch (h) {
    case 8: return launch_gate_vha<8>(ep, st);
    case 16: return launch_gate_vha<16>(ep, st);
    case 32: return launch_gate_vha<32>(ep, st);
    case 64: return launch_gate_vha<64>(ep, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hca
