// Device helpers of the bf16 grouped GEMM kernels: explicit memory-counter waits, the
// direct-to-LDS 16-byte load, and the 32x32x16 bf16 MFMA on 16-byte fragments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_byte;

// s_waitcnt vmcnt(n) with expcnt and lgkmcnt left at their maxima
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
// lgkmcnt(0) with vmcnt and expcnt left at their maxima; as a builtin (not inline asm)
// the compiler sees that every earlier LDS access has completed
__device__ __forceinline__ void wait_lgkmcnt_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void block_barrier() { __asm__ volatile("s_barrier" ::: "memory"); }

// 16 bytes per lane from global memory into LDS at lds_base + 16 * lane.  Issued as
// inline assembly so that the compiler adds no wait of its own before later LDS reads;
// every wait for these loads is explicit.  M0 holds the LDS base; one wait state
// separates its write from the load that reads it.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  __asm__ volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gptr), "s"(lds_base)
      : "memory", "m0");
}

// The same load with a uniform 64-bit base in SGPRs and a 32-bit per-lane byte offset
// (address = sbase + voff: no 64-bit address arithmetic per lane), into LDS at lds_part +
// LDS_OFF (a constant added in the instruction stream, so the compiler keeps one LDS base
// per buffer live instead of one per load).  The add writes SCC, which is declared.
template <uint32_t LDS_OFF>
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_part) {
  __asm__ volatile(
      "s_add_u32 m0, %2, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_part), "n"(LDS_OFF)
      : "memory", "m0", "scc");
}

// The lane index, computed where it is used (v_mbcnt in volatile assembly): a value the
// compiler can neither hoist nor keep live, so it is never spilled and reloaded.  A reload
// is a memory load the compiler waits for with vmcnt, and that count includes the
// direct-to-LDS loads in flight.
__device__ __forceinline__ uint32_t opaque_lane() {
  uint32_t l;
  __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// 4 bytes per lane into LDS at lds_part + LDS_OFF + 4 * lane (a gather: each lane its own
// address sbase + voff)
template <uint32_t LDS_OFF>
__device__ __forceinline__ void dma4s(const void* sbase, uint32_t voff, uint32_t lds_part) {
  __asm__ volatile(
      "s_add_u32 m0, %2, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_part), "n"(LDS_OFF)
      : "memory", "m0", "scc");
}

// D += A * B^T on one 32x32 block over 16 k: lane l supplies row l % 32, k 8 * (l / 32) ..
// + 7 of both operands (any permutation of k applied to both operands alike is allowed)
__device__ __forceinline__ f32x16_t mma_bf16(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

}  // namespace moe
