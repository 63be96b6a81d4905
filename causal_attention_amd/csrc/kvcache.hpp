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
// length is negative) is left unchanged.  With RoPE on, k is rotated to its
// position seqlens[b] as it is stored (the k_rope step of the same table,
// row 5, fused into the store the way its section 1.2 fuses RoPE into the
// loads), so the cache holds rotated keys.
#pragma once

#include "common.hpp"

namespace attn {

constexpr int kAppendThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kAppendThreads) void attn_kv_append_kernel(
    const T* __restrict__ k_new, const T* __restrict__ v_new,
    T* __restrict__ kcache, T* __restrict__ vcache, int* __restrict__ seqlens,
    int Hkv, int cap, int use_rope, RopeRates rope) {
  using E = Elem16<T>;
  typedef typename E::x8 x8;
  constexpr int HC = D / 16;                 // 16-byte chunk pairs per row
  __shared__ double rates[D / 2];
  if (use_rope)
    for (int i = threadIdx.x; i < D / 2; i += kAppendThreads)
      rates[i] = rope.r[i];
  __syncthreads();
  const int b = blockIdx.x;
  const int L = seqlens[b];                  // read by every thread first
  if (L < 0 || L >= cap) return;
  // thread i: KV head g, chunks c and c + D/16 (dims 8c.. and D/2 + 8c..),
  // the two halves of RoPE's pairs
  for (int i = threadIdx.x; i < Hkv * HC; i += kAppendThreads) {
    const int g = i / HC, c = i % HC;
    const size_t src = ((size_t)b * Hkv + g) * D + 8 * c;
    const size_t dst = (((size_t)b * Hkv + g) * cap + L) * D + 8 * c;
    x8 k1 = *reinterpret_cast<const x8*>(k_new + src);
    x8 k2 = *reinterpret_cast<const x8*>(k_new + src + D / 2);
    if (use_rope) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x1 = (float)k1[e], x2 = (float)k2[e];
        rope_pair(x1, x2, L, rates[8 * c + e]);
        k1[e] = (T)x1;
        k2[e] = (T)x2;
      }
    }
    *reinterpret_cast<x8*>(kcache + dst) = k1;
    *reinterpret_cast<x8*>(kcache + dst + D / 2) = k2;
    *reinterpret_cast<u32x4*>(vcache + dst) =
        *reinterpret_cast<const u32x4*>(v_new + src);
    *reinterpret_cast<u32x4*>(vcache + dst + D / 2) =
        *reinterpret_cast<const u32x4*>(v_new + src + D / 2);
  }
  __syncthreads();                           // every thread has read L
  if (threadIdx.x == 0) seqlens[b] = L + 1;
}

}  // namespace attn
