// Decode-time upkeep of the HCA raw-row ring (ERNIE 5.5 Flash Base pages:
// mirrorspeed page, "Hybrid sparse attention" section -- the most recent
// tokens stay uncompressed next to the 128-to-1 compressed entries).
//
// The ring holds 2R rows per (sequence, KV head).  The row of position t is
// written to rows t mod R and t mod R + R, so the rows of any run of up to R
// consecutive positions lo .. t sit contiguously from row lo mod R: a decode
// window is read straight from the ring, and a block that just closed is
// compressed from it by the block-compression kernel.
#include "device_common.h"
#include "launchers.h"

namespace hca {
namespace {

struct RingParams {
  const unsigned char* kn;  // new K rows [batch, 1, h_kv, d]
  const unsigned char* vn;
  unsigned char* kr;        // rings [batch, 2R, h_kv, d]
  unsigned char* vr;
  LStrides skn, svn, skr, svr;  // element strides
  int64_t slot0, slot1;         // t mod R and t mod R + R
  int es, chunks;               // bytes per element, 16-byte chunks per row
};

// One workgroup per (sequence, KV head): 16-byte copies of the K and V rows
// into both mirror slots.
__global__ __launch_bounds__(64) void ring_write_kernel(RingParams p) {
  const int64_t b = blockIdx.x, h = blockIdx.y;
  const int64_t es = p.es;
  const unsigned char* ks = p.kn + (b * p.skn.b + h * p.skn.h) * es;
  const unsigned char* vs = p.vn + (b * p.svn.b + h * p.svn.h) * es;
  unsigned char* k0 = p.kr + (b * p.skr.b + p.slot0 * p.skr.s + h * p.skr.h) * es;
  unsigned char* k1 = p.kr + (b * p.skr.b + p.slot1 * p.skr.s + h * p.skr.h) * es;
  unsigned char* v0 = p.vr + (b * p.svr.b + p.slot0 * p.svr.s + h * p.svr.h) * es;
  unsigned char* v1 = p.vr + (b * p.svr.b + p.slot1 * p.svr.s + h * p.svr.h) * es;
  for (int c = threadIdx.x; c < p.chunks; c += 64) {
    const u32x4 kx = ld16(ks + 16 * c), vx = ld16(vs + 16 * c);
    st16(k0 + 16 * c, kx);
    st16(k1 + 16 * c, kx);
    st16(v0 + 16 * c, vx);
    st16(v1 + 16 * c, vx);
  }
}

}  // namespace

hipError_t launch_ring_write(int dt, const void* k_new, LStrides skn, const void* v_new, LStrides svn, void* k_ring,
                             LStrides skr, void* v_ring, LStrides svr, int ring, int64_t t, int batch, int h_kv,
                             int head_dim, hipStream_t st) {
  RingParams p;
  p.kn = (const unsigned char*)k_new;
  p.vn = (const unsigned char*)v_new;
  p.kr = (unsigned char*)k_ring;
  p.vr = (unsigned char*)v_ring;
  p.skn = skn;
  p.svn = svn;
  p.skr = skr;
  p.svr = svr;
  p.slot0 = t % ring;
  p.slot1 = p.slot0 + ring;
  p.es = dt == 1 ? 2 : 4;
  p.chunks = head_dim * p.es / 16;
  hipLaunchKernelGGL(ring_write_kernel, dim3(batch, h_kv), dim3(64), 0, st, p);
  return hipGetLastError();
}

}  // namespace hca
