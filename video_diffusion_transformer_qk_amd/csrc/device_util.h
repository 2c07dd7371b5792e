// Small device helpers shared by the gfx950 kernels: bf16 packing, vector types, direct LDS loads,
// cross-lane combines.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3attn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// bf16 bits -> float (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// Direct global -> LDS load (gfx950 global_load_lds_dwordx4): 16 bytes per lane from
// sbase + voff to the LDS byte address lds + 16 * lane; sbase (a 64-bit base held in scalar
// registers) and lds are wave-uniform, voff is the lane's unsigned 32-bit byte offset, so moving
// to the next tile is a scalar add and the per-lane offsets stay fixed. No register receives the
// data. The load is counted by vmcnt like any global load: wait_dma before the LDS is read.
//
// It is issued from an asm block: through the compiler builtin, the compiler put a vmcnt(0) wait in
// front of LDS reads issued while such a load is in flight, also where they read another buffer
// (a tile is computed while the next one arrives). The block has no output that the load writes;
// it saves and restores M0 (which the load takes its LDS address from), with the one wait state
// the hardware needs between writing M0 and the load.
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds));
}

// Waits for all of this wave's direct loads. It is asm, not the s_waitcnt builtin: the compiler's
// wait pass does not know of the loads issued by lds_dma16_s and dropped a builtin wait it took
// for redundant. For the same reason the compiler's own waits (for loads it issued itself) must
// not be left open across a direct load: a kernel waits for its ordinary loads with the builtin
// before its first lds_dma16_s (wait_own_loads), so that no compiler wait inside the tile loop
// counts the direct loads.
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_own_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// LDS byte address of a pointer into shared memory
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// LDS transpose read of 4 x 16-bit values (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane i receives element (i % 4) of the 8-byte chunks addressed by lanes 4*s + i/4, s = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(const_cast<void*>(lds_ptr)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine the values of lane l and lane l^32 without an LDS round trip, using
// v_permlane32_swap_b32 on two copies of x: between them the two results hold, in every lane,
// the lane's own value and its partner's, so a symmetric combine of the pair is exact.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace h3attn
