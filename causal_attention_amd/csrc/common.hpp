// Shared device helpers for the gfx950 attention kernels: vector types, MFMA
// wrappers, bf16 packing and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Lazy rescaling of the online softmax: the running output is rescaled only
// when a row max exceeds the reference by more than this many log2 units.
constexpr float kLazyRescale = 8.f;

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
