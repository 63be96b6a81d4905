// Prefill kernels: one workgroup per (batch, query head, 128-row query tile),
// streaming K/V tiles of the matching KV head through LDS.
//
// Method ("Attention三算子融合实战：从Triton到CUDA的推理加速优化"): sections
// 2.2-2.3 (online softmax over key blocks, output rescaled by exp(m - m_new),
// divided by l once at the end as in the CUDA skeleton of section 4.2),
// section 4.3 (causal mask: key blocks wholly above the diagonal are skipped,
// the diagonal block is masked elementwise with -inf) and section 6.1 (a
// ragged tail block is loaded as zeros and its scores set to -inf).
//
// gfx950 mapping.  Each of the 4 waves owns 32 query rows.  Scores are formed
// transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K rows are the A
// operand (read from LDS), Q^T is the B operand (kept in VGPRs for the whole
// tile), and the accumulator leaves each lane with ONE query (lane % 32) and
// 16 keys per 32-key block.  Row max and row sum are then an in-lane
// reduction plus one exchange with the other wave half.  The probabilities
// P^T are re-used in place as the B operand of O^T = V^T P^T (a contraction
// over keys accepts any key order, as long as the A operand V^T reads V in the
// same order), so P never leaves registers.  V is stored transposed in LDS so
// that each lane's eight keys for one output dimension are two 8-byte runs.
// Softmax runs in the exp2 domain with scale*log2(e) folded in.
#pragma once

#include "common.hpp"

namespace attn {

constexpr int kPrefillThreads = 256;   // 4 waves
constexpr int kPrefillBM = 128;        // query rows per workgroup

// Block index -> (batch, KV head, query head, query tile).  Consecutive block
// indices walk over (batch, KV head) pairs first so that, when the pair count
// is a multiple of 8, every block of one pair lands on the same XCD (blocks
// are dealt to the 8 XCDs round-robin) and its K/V stay in that XCD's L2.
// Query tiles are issued heaviest first (most key tiles under the causal
// mask) so the short diagonal tiles fill the tail of the launch.
struct TileCoord {
  int b, g, hq, qt;
};

__device__ __forceinline__ TileCoord tile_coord(int bid, int B, int Hq,
                                                int Hkv, int n_qtiles) {
  const int G = Hq / Hkv;
  const int P = B * Hkv;
  const int pair = bid % P;
  const int rest = bid / P;
  TileCoord c;
  c.b = pair / Hkv;
  c.g = pair % Hkv;
  c.hq = c.g * G + rest % G;
  c.qt = n_qtiles - 1 - rest / G;
  return c;
}

// Online-softmax update of one 32-query x (16*NKB)-key transposed score block
// held as NKB accumulators.  x are log2-domain scores (masked = -inf).  Returns
// alpha (the rescale factor of the old state) and overwrites x with p.
template <int NKB>
__device__ __forceinline__ float softmax_step(f32x16 (&x)[NKB], float& m_i,
                                              float& l_i) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, x[kb][i]);
  mx = fmaxf(mx, swap_halves(mx));
  const float m_new = fmaxf(m_i, mx);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = fast_exp2(m_i - m_use);
  float sum = 0.f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(x[kb][i] - m_use);
      x[kb][i] = p;
      sum += p;
    }
  l_i = l_i * alpha + sum;   // lane-partial: this half's keys only
  m_i = m_new;
  return alpha;
}

// Scale to the log2 domain and apply the causal / tail mask.  key(kb, i) is
// the key index of accumulator element i of block kb for this lane.
template <int NKB, bool CAUSAL>
__device__ __forceinline__ void scale_and_mask(f32x16 (&x)[NKB], float c,
                                               int j0, int hh, int query,
                                               int S, bool need_mask) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = x[kb][i] * c;
      if (need_mask) {
        const int key = j0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
        const bool dead = (key >= S) || (CAUSAL && key > query);
        v = dead ? -INFINITY : v;
      }
      x[kb][i] = v;
    }
}

// ---------------------------------------------------------------- bf16 path

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kPrefillThreads) void attn_prefill_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
    const __bf16* __restrict__ V, __bf16* __restrict__ O,
    float* __restrict__ LSE, int B, int Hq, int Hkv, int S, float scale_log2,
    int n_qtiles) {
  constexpr int BM = kPrefillBM, BN = 64, NKB = BN / 32, NDB = D / 32;
  constexpr int KT = D / 16;                  // MFMA k-steps over D
  constexpr int KSTR = D + 8;                 // K tile row stride (elements)
  constexpr int VSTR = BN + 4;                // V^T tile row stride
  constexpr int DCH = D / 8;                  // 16-byte chunks per row
  constexpr int KCH = BN * DCH / kPrefillThreads;      // K chunks per thread
  constexpr int VTASKS = (BN / 4) * DCH;      // 4-key x 8-dim V blocks
  static_assert(KCH >= 1 && VTASKS <= kPrefillThreads, "tile shape");

  __shared__ __attribute__((aligned(16))) __bf16 Ks[BN * KSTR];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[D * VSTR];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const TileCoord tc = tile_coord(blockIdx.x, B, Hq, Hkv, n_qtiles);
  const __bf16* Qp = Q + (size_t)(tc.b * Hq + tc.hq) * S * D;
  const __bf16* Kp = K + (size_t)(tc.b * Hkv + tc.g) * S * D;
  const __bf16* Vp = V + (size_t)(tc.b * Hkv + tc.g) * S * D;

  const int q_lo = tc.qt * BM;
  const int q_hi = min(S, q_lo + BM);
  const int wq0 = q_lo + 32 * w;          // first query row of this wave
  const int query = wq0 + r;              // this lane's query row
  const int kv_end = CAUSAL ? q_hi : S;
  const int n_kv = (kv_end + BN - 1) / BN;

  // Q^T as the MFMA B operand: lane holds query `query`, dims 16t+8hh..+7.
  bf16x8 qB[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    if (query < S)
      qB[t] = *reinterpret_cast<const bf16x8*>(Qp + (size_t)query * D +
                                               16 * t + 8 * hh);
    else
      qB[t] = bf16x8{};
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_i = -INFINITY, l_i = 0.f;

  // Global -> register staging of one K/V tile (prefetched one tile ahead).
  u32x4 kreg[KCH];
  u32x4 vreg[4];
  const int vtask = tid;                       // valid if < VTASKS
  const int vc = vtask % DCH, vkq = vtask / DCH;
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * kPrefillThreads;
      const int row = j0 + c / DCH, col = c % DCH;
      kreg[i] = (row < S) ? *reinterpret_cast<const u32x4*>(
                                Kp + (size_t)row * D + col * 8)
                          : u32x4{};
    }
    if (vtask < VTASKS) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int row = j0 + 4 * vkq + u;
        vreg[u] = (row < S) ? *reinterpret_cast<const u32x4*>(
                                  Vp + (size_t)row * D + vc * 8)
                            : u32x4{};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * kPrefillThreads;
      *reinterpret_cast<u32x4*>(&Ks[(c / DCH) * KSTR + (c % DCH) * 8]) =
          kreg[i];
    }
    if (vtask < VTASKS) {
      // Transpose a 4-key x 8-dim block: dim e of keys 4vkq..4vkq+3 becomes
      // one 8-byte run of row (8vc + e) of V^T.
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wd = e >> 1;
        uint32_t k0 = vreg[0][wd], k1 = vreg[1][wd], k2 = vreg[2][wd],
                 k3 = vreg[3][wd];
        if (e & 1) {
          k0 >>= 16; k1 >>= 16; k2 >>= 16; k3 >>= 16;
        }
        u32x2 pr;
        pr[0] = (k0 & 0xffffu) | (k1 << 16);
        pr[1] = (k2 & 0xffffu) | (k3 << 16);
        *reinterpret_cast<u32x2*>(&Vt[(8 * vc + e) * VSTR + 4 * vkq]) = pr;
      }
    }
  };

  if (n_kv > 0) load_tile(0);
  for (int jt = 0; jt < n_kv; ++jt) {
    const int j0 = jt * BN;
    __syncthreads();              // every wave is done with the previous tile
    store_tile();
    __syncthreads();              // tile visible to all waves
    if (jt + 1 < n_kv) load_tile(j0 + BN);

    // Waves whose rows all lie above this tile's first key skip it (all of
    // its scores would be masked).
    if (CAUSAL && j0 > wq0 + 31) continue;

    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &Ks[(kb * 32 + r) * KSTR + 16 * t + 8 * hh]);
        sacc[kb] = mfma_32x32x16_bf16(a, qB[t], sacc[kb]);
      }
    }
    const bool need_mask = (j0 + BN > S) || (CAUSAL && j0 + BN - 1 > wq0);
    scale_and_mask<NKB, CAUSAL>(sacc, scale_log2, j0, hh, query, S,
                                need_mask);
    const float alpha = softmax_step<NKB>(sacc, m_i, l_i);
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;

#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 pb;
#pragma unroll
        for (int s = 0; s < 8; ++s) pb[s] = (__bf16)sacc[kb][8 * u + s];
        // Slot s of this lane holds key kb*32 + 16u + 4hh + (s&3) + 8*(s>>2).
        const int kcol = kb * 32 + 16 * u + 4 * hh;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const __bf16* vrow = &Vt[(db * 32 + r) * VSTR + kcol];
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 8);
          const bf16x8 a = {lo[0], lo[1], lo[2], lo[3],
                            hi[0], hi[1], hi[2], hi[3]};
          oacc[db] = mfma_32x32x16_bf16(a, pb, oacc[db]);
        }
      }
  }

  // Epilogue: O = acc / l (bf16, RNE) and LSE = (m + log2 l) * ln 2.
  const float l_tot = l_i + swap_halves(l_i);
  if (query < S) {
    const float inv = 1.f / l_tot;
    __bf16* orow = O + (size_t)(tc.b * Hq + tc.hq) * S * D + (size_t)query * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 pr;
        pr[0] = pack_bf16x2(oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv);
        pr[1] = pack_bf16x2(oacc[db][4 * a + 2] * inv,
                            oacc[db][4 * a + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * a + 4 * hh) = pr;
      }
    if (LSE != nullptr && hh == 0)
      LSE[(size_t)(tc.b * Hq + tc.hq) * S + query] =
          (m_i + fast_log2(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------- fp32 path
//
// Same tiling with v_mfma_f32_32x32x2_f32 (one contraction element per lane
// half).  Lane half hh owns dims [hh*D/2, hh*D/2 + D/2) of the S^T
// contraction, so Q^T and K are read as contiguous half rows.  For O^T the
// fp32 probabilities are used directly: accumulator element i of block kb is
// the B operand of one k-step whose two keys (one per lane half) are
// kb*32 + 8*(i/4) + 4*hh + i%4, and V is read untransposed from LDS.

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kPrefillThreads) void attn_prefill_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K,
    const float* __restrict__ V, float* __restrict__ O,
    float* __restrict__ LSE, int B, int Hq, int Hkv, int S, float scale_log2,
    int n_qtiles) {
  constexpr int BM = kPrefillBM, BN = 32, NKB = BN / 32, NDB = D / 32;
  constexpr int HD = D / 2;                   // contraction elems per half
  constexpr int STR = D + 4;                  // LDS row stride (floats)
  constexpr int DCH = D / 4;                  // 16-byte chunks per row
  constexpr int CH = BN * DCH / kPrefillThreads;
  static_assert(CH >= 1, "tile shape");

  __shared__ __attribute__((aligned(16))) float Ks[BN * STR];
  __shared__ __attribute__((aligned(16))) float Vs[BN * STR];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const TileCoord tc = tile_coord(blockIdx.x, B, Hq, Hkv, n_qtiles);
  const float* Qp = Q + (size_t)(tc.b * Hq + tc.hq) * S * D;
  const float* Kp = K + (size_t)(tc.b * Hkv + tc.g) * S * D;
  const float* Vp = V + (size_t)(tc.b * Hkv + tc.g) * S * D;

  const int q_lo = tc.qt * BM;
  const int q_hi = min(S, q_lo + BM);
  const int wq0 = q_lo + 32 * w;
  const int query = wq0 + r;
  const int kv_end = CAUSAL ? q_hi : S;
  const int n_kv = (kv_end + BN - 1) / BN;

  float qB[HD];
#pragma unroll
  for (int t = 0; t < HD; t += 4) {
    f32x4 v4 = f32x4{};
    if (query < S)
      v4 = *reinterpret_cast<const f32x4*>(Qp + (size_t)query * D + hh * HD +
                                           t);
    qB[t] = v4[0]; qB[t + 1] = v4[1]; qB[t + 2] = v4[2]; qB[t + 3] = v4[3];
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_i = -INFINITY, l_i = 0.f;

  f32x4 kreg[CH], vreg[CH];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + i * kPrefillThreads;
      const int row = j0 + c / DCH, col = c % DCH;
      const bool ok = row < S;
      kreg[i] = ok ? *reinterpret_cast<const f32x4*>(Kp + (size_t)row * D +
                                                     col * 4)
                   : f32x4{};
      vreg[i] = ok ? *reinterpret_cast<const f32x4*>(Vp + (size_t)row * D +
                                                     col * 4)
                   : f32x4{};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + i * kPrefillThreads;
      const int off = (c / DCH) * STR + (c % DCH) * 4;
      *reinterpret_cast<f32x4*>(&Ks[off]) = kreg[i];
      *reinterpret_cast<f32x4*>(&Vs[off]) = vreg[i];
    }
  };

  if (n_kv > 0) load_tile(0);
  for (int jt = 0; jt < n_kv; ++jt) {
    const int j0 = jt * BN;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (jt + 1 < n_kv) load_tile(j0 + BN);
    if (CAUSAL && j0 > wq0 + 31) continue;

    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = f32x16{};
      const float* krow = &Ks[(kb * 32 + r) * STR + hh * HD];
#pragma unroll
      for (int t = 0; t < HD; t += 4) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(krow + t);
        sacc[kb] = mfma_32x32x2_f32(a4[0], qB[t], sacc[kb]);
        sacc[kb] = mfma_32x32x2_f32(a4[1], qB[t + 1], sacc[kb]);
        sacc[kb] = mfma_32x32x2_f32(a4[2], qB[t + 2], sacc[kb]);
        sacc[kb] = mfma_32x32x2_f32(a4[3], qB[t + 3], sacc[kb]);
      }
    }
    const bool need_mask = (j0 + BN > S) || (CAUSAL && j0 + BN - 1 > wq0);
    scale_and_mask<NKB, CAUSAL>(sacc, scale_log2, j0, hh, query, S,
                                need_mask);
    const float alpha = softmax_step<NKB>(sacc, m_i, l_i);
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;

#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          oacc[db] = mfma_32x32x2_f32(Vs[key * STR + db * 32 + r],
                                      sacc[kb][i], oacc[db]);
      }
  }

  const float l_tot = l_i + swap_halves(l_i);
  if (query < S) {
    const float inv = 1.f / l_tot;
    float* orow = O + (size_t)(tc.b * Hq + tc.hq) * S * D + (size_t)query * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 o4 = {oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv,
                    oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * a + 4 * hh) = o4;
      }
    if (LSE != nullptr && hh == 0)
      LSE[(size_t)(tc.b * Hq + tc.hq) * S + query] =
          (m_i + fast_log2(l_tot)) * kLn2;
  }
}

}  // namespace attn
