// common.h -- types and small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// bfloat16 pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bfloat16 pattern, round to nearest, ties to even (the hardware
// conversion, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two fp32 -> two packed bfloat16 patterns (low half = a), one conversion
// instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Element loads that widen either storage type to fp32.
__device__ __forceinline__ float load_as_f32(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_as_f32(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }

__device__ __forceinline__ void store_from_f32(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_from_f32(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }

// D = A * B + C on a 16x16 output tile with K = 32 (bf16 operands, fp32
// accumulation).  Lane l holds A[l % 16][8 (l / 16) + e] and
// B[8 (l / 16) + e][l % 16] in element e, and D[4 (l / 16) + j][l % 16] in
// element j.  Only the pairing of A's and B's k positions matters to the
// product, so callers may permute the k order as long as both sides agree.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

// LDS (address space 3) pointers, and the operand type of the transposing
// LDS read ds_read_b64_tr_b16.
#define AS3 __attribute__((address_space(3)))
typedef short tr_vec __attribute__((vector_size(8)));

// One wave-wide DMA of 64 x 16 bytes from global memory into LDS
// (global_load_lds_dwordx4): lane l reads sbase + voff[l] (a uniform 64-bit
// base in SGPRs plus a per-lane 32-bit offset) and writes lds_base + 16 l.
// Issued by hand so that the compiler does not serialise DMA rings with
// conservative waits; callers track completion with explicit vmcnt waits.
// No output registers are involved; M0 (the LDS base of the DMA) is saved
// and restored around it.
__device__ __forceinline__ void lds_dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(voff), "s"(sbase)
      : "memory");
}

// Wave-wide reductions over lanes that differ in the given xor bit(s).
__device__ __forceinline__ float xor_sum(float v, int mask) {
  return v + __shfl_xor(v, mask, 64);
}

}  // namespace mla
