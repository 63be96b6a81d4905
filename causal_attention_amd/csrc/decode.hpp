// Decode kernels: one query row per sequence against its packed KV cache,
// split over the cache length, then a log-sum-exp combine.
//
// Method ("Attention三算子融合实战：从Triton到CUDA的推理加速优化"): the decode
// setting of section 1.3 (one query row, K and V as long as the history), the
// key split of section 4.4 (large key chunks handled by separate blocks, each
// running the online softmax of section 2.2, merged across blocks
// afterwards), and the partial-buffer-plus-reduce-kernel pattern of
// "手写Triton kernel重构Qwen3.5-0.8B" section 3.3 (a separate small reduce
// kernel rather than atomics).  GQA (section 2.1 of that page): the Hq/Hkv
// query heads of one KV head are handled by the same workgroup, so each K/V
// byte is read from HBM once, not once per query head.
//
// This path is bound by HBM bandwidth (about 4 FLOP per byte), so it uses no
// MFMA.  A "lane group" of D/8 lanes owns one key row at a time, each lane
// holding 8 dims loaded as one 16-byte vector, so one load instruction of a
// wave covers 64/(D/8) consecutive key rows: one contiguous run of memory.  Each lane
// group runs its own online softmax over its keys (the merge order does not
// matter), so the loop has no cross-group communication; the groups are
// merged once at the end of the split through LDS.  All loads of a batch of
// UNR keys per group are issued before any arithmetic so that every lane
// keeps 2*UNR 16-byte loads in flight.
#pragma once

#include "common.hpp"

namespace attn {

constexpr int kDecodeThreads = 128;    // 2 waves
constexpr int kDecodeMinChunk = 64;    // smallest split, in keys

// Keys of split s for a sequence of L keys: [s*chunk, min(L, (s+1)*chunk)).
__device__ __forceinline__ int decode_chunk(int L, int ns) {
  return max((L + ns - 1) / ns, kDecodeMinChunk);
}

template <int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void attn_decode_split_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ Kc,
    const __bf16* __restrict__ Vc, const int* __restrict__ seqlens,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, int Hkv, int ns,
    float scale_log2) {
  constexpr int GL = D / 8;                   // lanes per key row
  constexpr int NG = kDecodeThreads / GL;     // lane groups per workgroup
  constexpr int UNR = 8;                      // keys per group per batch

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Hq = Hkv * G;
  const int L = max(seqlens[b], 0);
  const int chunk = decode_chunk(L, ns);
  const long long start = (long long)s * chunk;
  if (start >= L) return;                     // uniform over the workgroup
  const int kbeg = (int)start;
  const int kend = min(L, kbeg + chunk);

  const int tid = threadIdx.x;
  const int grp = tid / GL, gl = tid % GL;

  // Element offset of sequence b's cache block: Hkv*D*sum(L_0..L_{b-1}).
  __shared__ long long red[kDecodeThreads / 64];
  long long part = 0;
  for (int i = tid; i < b; i += kDecodeThreads) part += max(seqlens[i], 0);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
  if ((tid & 63) == 0) red[tid >> 6] = part;
  __syncthreads();
  long long prefix = 0;
#pragma unroll
  for (int i = 0; i < kDecodeThreads / 64; ++i) prefix += red[i];
  const size_t base =
      ((size_t)prefix * Hkv + (size_t)g * L) * D + (size_t)gl * 8;
  const __bf16* Kp = Kc + base;
  const __bf16* Vp = Vc + base;

  // This lane's 8 query dims of each head in the group, pre-scaled so the
  // dot product is already a log2-domain score.
  float q[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const u32x4 w4 = *reinterpret_cast<const u32x4*>(
        Q + ((size_t)(b * Hq + g * G + h)) * D + gl * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      q[h][2 * e] = bf16_lo(w4[e]) * scale_log2;
      q[h][2 * e + 1] = bf16_hi(w4[e]) * scale_log2;
    }
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  for (int k0 = kbeg; k0 < kend; k0 += NG * UNR) {
    u32x4 kr[UNR], vr[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int key = k0 + grp + NG * u;
      if (key < kend) {
        kr[u] = *reinterpret_cast<const u32x4*>(Kp + (size_t)key * D);
        vr[u] = *reinterpret_cast<const u32x4*>(Vp + (size_t)key * D);
      } else {
        kr[u] = u32x4{};
        vr[u] = u32x4{};
      }
    }
    float sc[G][UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float kf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = bf16_lo(kr[u][e]);
        kf[2 * e + 1] = bf16_hi(kr[u][e]);
      }
      const bool ok = k0 + grp + NG * u < kend;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(q[h][e], kf[e], d);
        d = group_sum<GL>(d);
        sc[h][u] = ok ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = sc[h][0];
#pragma unroll
      for (int u = 1; u < UNR; ++u) mx = fmaxf(mx, sc[h][u]);
      const float m_new = fmaxf(m[h], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m[h] - m_use);
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        sc[h][u] = fast_exp2(sc[h][u] - m_use);
        psum += sc[h][u];
      }
      l[h] = l[h] * alpha + psum;
      m[h] = m_new;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v0 = bf16_lo(vr[u][e]), v1 = bf16_hi(vr[u][e]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h][2 * e] = fmaf(sc[h][u], v0, acc[h][2 * e]);
          acc[h][2 * e + 1] = fmaf(sc[h][u], v1, acc[h][2 * e + 1]);
        }
      }
    }
  }

  // Merge the NG lane groups of this workgroup (LSE algebra), then write
  // this split's normalised output and natural-log LSE.
  __shared__ float sm_m[NG][G], sm_l[NG][G];
  __shared__ float sm_acc[NG][G][D];
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_acc[grp][h][gl * 8 + e] = acc[h][e];
    if (gl == 0) {
      sm_m[grp][h] = m[h];
      sm_l[grp][h] = l[h];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kDecodeThreads) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < NG; ++j) M = fmaxf(M, sm_m[j][h]);
    float W = 0.f, o = 0.f;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const float wj = fast_exp2(sm_m[j][h] - M);   // 0 for an empty group
      W = fmaf(wj, sm_l[j][h], W);
      o = fmaf(wj, sm_acc[j][h][d], o);
    }
    const size_t row = ((size_t)(b * Hq + g * G + h)) * ns + s;
    ws_o[row * D + d] = o / W;
    if (d == 0) ws_lse[row] = (M + fast_log2(W)) * kLn2;
  }
}

// Combine the active splits of each (sequence, query head):
// M = max_s lse_s, w_s = exp(lse_s - M), o = sum w_s o_s / sum w_s,
// lse = M + ln(sum w_s).  A sequence with no keys gives o = 0, lse = -inf.
template <int D>
__global__ __launch_bounds__(D) void attn_decode_combine_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
    const int* __restrict__ seqlens, __bf16* __restrict__ O,
    float* __restrict__ LSE, int Hq, int ns) {
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int d = threadIdx.x;
  const int L = max(seqlens[b], 0);
  const int chunk = decode_chunk(L, ns);
  const int nact = (L + chunk - 1) / chunk;
  const float* lse_p = ws_lse + (size_t)bh * ns;
  const float* o_p = ws_o + (size_t)bh * ns * D;

  float M = -INFINITY;
  for (int s = 0; s < nact; ++s) M = fmaxf(M, lse_p[s]);
  float W = 0.f, o = 0.f;
  for (int s = 0; s < nact; ++s) {
    const float w = fast_exp2((lse_p[s] - M) * kLog2e);
    W += w;
    o = fmaf(w, o_p[(size_t)s * D + d], o);
  }
  const float res = nact > 0 ? o / W : 0.f;
  O[(size_t)bh * D + d] = (__bf16)res;
  if (LSE != nullptr && d == 0)
    LSE[bh] = nact > 0 ? M + logf(W) : -INFINITY;
}

}  // namespace attn
