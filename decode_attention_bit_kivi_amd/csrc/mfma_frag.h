// MFMA fragments for gfx950's v_mfma_f32_16x16x32_f16 and the bit-to-operand
// expansion shared by the score and attention kernels.
//
// Operand layout of the 16x16x32 instruction (wave64): lane l holds 8 float16
// of A for row l % 16 and 8 float16 of B for column l % 16, both in k-group
// l / 16; A's slot j in a k-group multiplies B's slot j of the same k-group.
// The 16x16 float32 result puts element (m, n) in lane n + 16 * (m / 4),
// register m % 4.
//
// A 1-bit code b of an element with scale s contributes s * (2b - 1) / 2
// around the group's midpoint, so the operand value is +-s: the code bit
// becomes the float16 sign bit of s (a set bit gives -s, so the operand is
// -(2b - 1) s and the kernels scale its products by -1/2).  The packed layout keeps the two
// elements of an operand dword 16 bit positions apart, so a shift moves both
// bits into the two sign positions and one and-or attaches the magnitudes;
// one 64-bit shift serves two code words, so the expansion costs three VALU
// operations per four elements, and every product with a float16 query
// element is exact in the float32 accumulator.
#pragma once

#include "common.h"

namespace specache {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

union Frag {
  half8_t h;
  uint4 v;
  uint32_t u[4];
};

__device__ __forceinline__ f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.h, b.h, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.0f, 0.0f, 0.0f, 0.0f}; }

// Elements whose bits sit at positions p and p + 16 of w0 and of w1, with shift = 15 - p: the
// float16 pairs (+-mag0.lo, +-mag0.hi) and (+-mag1.lo, +-mag1.hi).  Shifting the pair (w1:w0) left
// by shift <= 15 moves bits p and p + 16 of each word to bits 15 and 31 of its own half; what w0
// pushes into the high half lands below bit `shift`, where the mask drops it.
__device__ __forceinline__ void signed_pairs2(uint32_t w0, uint32_t w1, int shift, uint32_t mag0, uint32_t mag1,
                                              uint32_t& out0, uint32_t& out1) {
  const uint64_t x = ((((uint64_t)w1) << 32) | (uint64_t)w0) << shift;
  out0 = ((uint32_t)x & 0x80008000u) | mag0;
  out1 = ((uint32_t)(x >> 32) & 0x80008000u) | mag1;
}

// Two floats to a float16 pair, each rounded to nearest even (gfx950: one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
  typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
  typedef float float2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){lo, hi}, half2_t));
}

template <int NW>
struct Words {
  uint32_t w[NW];
};

// NW consecutive 32-bit words from a 4*NW-byte aligned address.
template <int NW>
__device__ __forceinline__ Words<NW> load_words(const uint32_t* p) {
  Words<NW> r;
  if constexpr (NW == 8) {
    const uint4 a = reinterpret_cast<const uint4*>(p)[0];
    const uint4 b = reinterpret_cast<const uint4*>(p)[1];
    r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
    r.w[4] = b.x; r.w[5] = b.y; r.w[6] = b.z; r.w[7] = b.w;
  } else if constexpr (NW == 4) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
  } else if constexpr (NW == 2) {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    r.w[0] = a.x; r.w[1] = a.y;
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) r.w[i] = p[i];
  }
  return r;
}

// Raw buffer over `bytes` bytes at `p` (gfx9 descriptor: untyped, no swizzle).  A load through it
// adds a wave-uniform byte offset (scalar register) to a per-lane byte offset, so the address
// arithmetic of a loop whose base moves uniformly stays off the VALU; bytes past the end read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// NW consecutive 32-bit words at byte voff + soff of the buffer (4*NW-byte aligned).
template <int NW>
__device__ __forceinline__ Words<NW> buffer_words(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  Words<NW> w;
  if constexpr (NW == 8 || NW == 4) {
#pragma unroll
    for (int h = 0; h < NW / 4; ++h) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(voff + 16 * h), (int)soff, 0);
      w.w[4 * h] = x[0]; w.w[4 * h + 1] = x[1]; w.w[4 * h + 2] = x[2]; w.w[4 * h + 3] = x[3];
    }
  } else if constexpr (NW == 2) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
    w.w[0] = x[0]; w.w[1] = x[1];
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) w.w[i] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(voff + 4 * i), (int)soff, 0);
  }
  return w;
}

__device__ __forceinline__ uint2 load_u2(const void* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ uint4 load_u4(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Reductions over the four k-groups of a wave (lanes l, l^16, l^32, l^48) on gfx950's
// cross-row swaps, with no LDS round trip.  Swapping a register with a copy of itself leaves
// the values of lanes l and l^16 (permlane16) or l and l^32 (permlane32) in the two registers
// (in a lane-dependent order), so a symmetric operation of the pair reduces over the partners.
// Written as inline assembly: the compiler's builtins for these swaps fold the second result
// away when it is combined with the first.  The wait states around the swap are those the
// compiler itself places next to it.
#define SPECACHE_SWAP_OP(SWAP, OP) "s_nop 1\n\t" SWAP " %0, %1\n\ts_nop 1\n\t" OP " %0, %0, %1"
__device__ __forceinline__ float max_over_groups(float x) {
  float y = x;
  asm(SPECACHE_SWAP_OP("v_permlane16_swap_b32", "v_max_f32") : "+v"(x), "+v"(y));
  y = x;
  asm(SPECACHE_SWAP_OP("v_permlane32_swap_b32", "v_max_f32") : "+v"(x), "+v"(y));
  return x;
}
// The maximum over k-groups g and g ^ 1 (lanes l and l ^ 16) only.
__device__ __forceinline__ float max_over_group_pairs(float x) {
  float y = x;
  asm(SPECACHE_SWAP_OP("v_permlane16_swap_b32", "v_max_f32") : "+v"(x), "+v"(y));
  return x;
}
__device__ __forceinline__ float sum_over_groups(float x) {
  float y = x;
  asm(SPECACHE_SWAP_OP("v_permlane16_swap_b32", "v_add_f32") : "+v"(x), "+v"(y));
  y = x;
  asm(SPECACHE_SWAP_OP("v_permlane32_swap_b32", "v_add_f32") : "+v"(x), "+v"(y));
  return x;
}
#undef SPECACHE_SWAP_OP

}  // namespace specache
