// Shared device helpers for the gfx950 attention kernels: vector types, MFMA
// wrappers, bf16 packing and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Lazy rescaling of the online softmax: the running output is rescaled only
// when a row max exceeds the reference by more than this many log2 units.
constexpr float kLazyRescale = 8.f;

// D = A(32x16) * B(16x32) + C, bf16 inputs, fp32 accumulate.  Lane l holds
// row (A) / column (B) l % 32 and eight contraction elements; C lane l holds
// column l % 32, rows 8*(i/4) + 4*(l/32) + i%4 for i in 0..15.
__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(bf16x8 a, bf16x8 b,
                                                     f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16-bit input elements: bf16 (the workloads' type) and fp16.  The kernels
// are written once against these traits: the 8-element MFMA operand vector,
// the 32x32x16 and 16x16x32 products with fp32 accumulation, and the
// round-to-nearest-even conversion of two fp32 values to a packed pair.
template <typename T>
struct Elem16;

template <>
struct Elem16<__bf16> {
  typedef __bf16 x8 __attribute__((ext_vector_type(8)));
  typedef __bf16 x2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 mma32(x8 a, x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(x8 a, x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
};

template <>
struct Elem16<_Float16> {
  typedef _Float16 x8 __attribute__((ext_vector_type(8)));
  typedef _Float16 x2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 mma32(x8 a, x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(x8 a, x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
};

// Rotary position embedding (half-split pairs (x[i], x[i + D/2]), angle
// p * base^(-2i/D)): the rate of each pair in turns per position,
// base^(-2i/D) / (2 pi), computed on the host in fp64 and passed by value.
struct RopeRates {
  double r[64];
};

// Rotate the pair (x1, x2) by the angle of position pos at rate r (turns per
// position).  The turn count is reduced to [0, 1) in fp64, so long positions
// keep their accuracy; sin and cos of the fraction come from v_sin_f32 /
// v_cos_f32, which take their argument in turns; the rotation is fp32.
__device__ __forceinline__ void rope_pair(float& x1, float& x2, int pos,
                                          double r) {
  const double t = (double)pos * r;
  const float f = (float)(t - floor(t));
  const float c = __builtin_amdgcn_cosf(f), s = __builtin_amdgcn_sinf(f);
  const float y1 = x1 * c - x2 * s;
  x2 = x1 * s + x2 * c;
  x1 = y1;
}

// fp32 variant: one contraction element per lane (lane half l/32 picks it).
__device__ __forceinline__ f32x16 mfma_32x32x2_f32(float a, float b,
                                                   f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float fast_log2(float x) {
  return __builtin_amdgcn_logf(x);
}

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Cross-lane moves inside rows of 16 lanes (DPP; no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(
      0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within 16

// Sum over aligned groups of N lanes (N = 8 or 16); every lane gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  if constexpr (N == 16) x += dpp<kDppMirror>(x);
  return x;
}

// Exchange with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}
// x combined with its value in the other half of the wave (lane ^ 32) by
// max or +, with one v_permlane32_swap (no LDS traffic).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(
      __builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
      false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]),
               __builtin_bit_cast(float, (unsigned)r[1]));
}

// s_waitcnt vmcnt(N): at most N vector-memory loads of this wave in flight
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// LDS operand reads issued as inline assembly, for loops that keep
// direct-to-LDS loads in flight on purpose: the compiler treats LDS reads it
// can see as possibly aliasing every such load and would wait for all of
// them.  The caller waits with lds_wait_all() and then passes each result
// through lds_tie(), which orders its uses after the wait.  Addresses are
// LDS byte addresses; OFF is an immediate byte offset.
template <int OFF = 0>
__device__ __forceinline__ void lds_read_b128_async(u32x4& v, unsigned addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2"
               : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
}
template <int OFF = 0>
__device__ __forceinline__ void lds_read_tr16_async(u32x2& v, unsigned addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
               : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
}
__device__ __forceinline__ void lds_wait_all() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
template <typename T>
__device__ __forceinline__ void lds_tie(T& v) {
  asm volatile("" : "+v"(v));
}
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) void*)p;
}

}  // namespace attn
