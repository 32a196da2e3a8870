// Shared device-side definitions for the gfx950 MLA decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cfloat>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(1))) const uint8_t gbl_u8;
// Constant address space: uniform loads through it become scalar (s_load) reads.
typedef __attribute__((address_space(4))) const int32_t const_i32;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Fixed geometry of the latent cache row (DeepSeek-V2/V3: kv_lora_rank 512,
// qk_rope_head_dim 64, qk_nope_head_dim 128, v_head_dim 128).
constexpr int DC = 512;
constexpr int DR = 64;
constexpr int DROW = DC + DR;          // 576 values per cached token
constexpr int DNOPE = 128;
constexpr int DV = 128;
constexpr int PAGE = 64;               // tokens per cache page
constexpr int ROW_BYTES = DROW * 2;    // bf16 row: 1152 bytes
constexpr int FP8_ROW_BYTES = 656;     // 512 codes | 64 bf16 | 4 fp32 scales

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 (gfx950 converts in hardware).
__device__ __forceinline__ __bf16 to_bf16(float f) { return static_cast<__bf16>(f); }

__device__ __forceinline__ uint16_t bf16_bits(__bf16 v) { return __builtin_bit_cast(uint16_t, v); }

// Round-to-nearest-even float -> IEEE half (bits).  Finite only below 65520.
__device__ __forceinline__ uint16_t f16_bits(float f) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f)); }

__device__ __forceinline__ float bf16_round_f32(float f) {
  return static_cast<float>(static_cast<__bf16>(f));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] in bits [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14));
}

// 16-byte global -> LDS copy per lane (global_load_lds_dwordx4): lane i's 16
// bytes land at LDS byte address lds_base + 16 i.  lds_base must be
// wave-uniform.  Issued through asm so that the compiler's own wait insertion
// does not treat every later LDS read as dependent on it; callers order the
// copies with explicit wait_vmcnt<> and barriers.  The asm has no register
// outputs, so no register is written asynchronously.
__device__ __forceinline__ void dma16(const void *gsrc, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gsrc), "s"(lds_base)
      : "memory", "m0");
}

// The same copy with a wave-uniform 64-bit base (SGPR pair) and a 32-bit
// per-lane byte offset: the per-copy address arithmetic stays scalar.
__device__ __forceinline__ void dma16_s(uint32_t voff, const void *sbase, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t *)p));
}

// Workgroup barrier without the memory fence __syncthreads() adds (the fence
// would wait for every outstanding global->LDS load, not just the ones the
// caller already waited for).  The empty asm keeps the compiler from moving
// memory operations across it.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Workgroup barrier after this wave's LDS writes have completed (lgkmcnt 0),
// so that they are visible to every wave past the barrier; outstanding
// global->LDS copies are not waited for.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

}  // namespace mla
