// KV-cache append for the decode loop: the kv_cache_store step of the
// operator table in "手写Triton kernel重构Qwen3.5-0.8B" (section 2.2, row 18:
// write the new k/v into the KV cache), in the form the CUDA Graph section
// of that page needs (sections 4.1-4.5: preallocated buffers, positions kept
// on the device so that one captured graph can be replayed step after step).
//
// Cache layout ("padded"): kcache, vcache [B, Hkv, cap, D]; sequence b holds
// seqlens[b] valid rows per KV head.  One workgroup per sequence copies the
// new token's k and v ([B, Hkv, D]) into row seqlens[b] of every KV head and
// then advances seqlens[b], so the decode launched after it on the same
// stream attends to the new token.  A sequence whose cache is full (or whose
// length is negative) is left unchanged.
#pragma once

#include "common.hpp"

namespace attn {

constexpr int kAppendThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kAppendThreads) void attn_kv_append_kernel(
    const T* __restrict__ k_new, const T* __restrict__ v_new,
    T* __restrict__ kcache, T* __restrict__ vcache, int* __restrict__ seqlens,
    int Hkv, int cap) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  const int b = blockIdx.x;
  const int L = seqlens[b];                  // read by every thread first
  if (L < 0 || L >= cap) return;
  for (int i = threadIdx.x; i < Hkv * CPR; i += kAppendThreads) {
    const int g = i / CPR, c = i % CPR;
    const size_t src = ((size_t)b * Hkv + g) * D + 8 * c;
    const size_t dst = (((size_t)b * Hkv + g) * cap + L) * D + 8 * c;
    *reinterpret_cast<u32x4*>(kcache + dst) =
        *reinterpret_cast<const u32x4*>(k_new + src);
    *reinterpret_cast<u32x4*>(vcache + dst) =
        *reinterpret_cast<const u32x4*>(v_new + src);
  }
  __syncthreads();                           // every thread has read L
  if (threadIdx.x == 0) seqlens[b] = L + 1;
}

}  // namespace attn
