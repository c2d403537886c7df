// Inline-asm building blocks of the 512-wide MFMA attention kernels (gfx950):
// 16-byte LDS DMA and v_mfma_f32_32x32x16_bf16 with explicit accumulator
// register classes and wait states.
#pragma once
#include "device_common.h"

namespace hca {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// 16-byte LDS DMA of one wave: lane l copies 16 bytes from g (per lane) to LDS
// byte address lds + 16 l (lds travels in M0).  Written as asm so that the
// compiler does not track it as an LDS store (it would wait for it before
// unrelated LDS reads); the explicit vmcnt wait and barrier of each tile order
// DMA and reads.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

// dma16 with one wait state ahead of the load: an LDS DMA reads M0, which the
// compiler writes right before the asm, and an M0 write needs a wait state
// before an LDS DMA.
__device__ __forceinline__ void dma16_m0(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

// The two products are written as inline asm so that S^T accumulates in VGPRs
// (the softmax reads it) while O^T accumulates in AGPRs: O^T takes all 256
// AGPRs, and the compiler would otherwise put every MFMA accumulator in AGPRs
// and spill.  The compiler does not see these as MFMAs, so the wait states
// the ISA requires around them are explicit: after the last S^T step (its
// result is read by VALU), before the first O^T step of a tile (P^T was just
// written by VALU), before an MFMA that reads a VALU-written operand and
// before O^T is read back.  Back-to-back MFMAs on the same accumulator need
// none.
__device__ __forceinline__ void mfma_s_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_last(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 15\n\ts_nop 15" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_o(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void zero_o(f32x16& acc, const bf16x8& z) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=&a"(acc) : "v"(z));
}
__device__ __forceinline__ void mfma_o_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// 4-byte LDS DMA of one wave: lane l copies 4 bytes from g to LDS byte address
// lds + 4 l (same ordering rules as dma16).
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

// dma4 with the wait state an M0 write needs before an LDS DMA (see dma16_m0).
__device__ __forceinline__ void dma4_m0(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

// Transposing LDS read of the A operand of a 32x32x16 step whose rows are the
// contiguous axis of a row-major LDS tile: `p` already holds the lane offset
// (see the kernels); the second half comes from 8 rows further down.
__device__ __forceinline__ bf16x8 ld_tr_a(const unsigned char* p, int row_bytes) {
  const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  const s16x4 hi4 =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p + 8 * row_bytes));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace hca
