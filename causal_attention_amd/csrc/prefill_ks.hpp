// Key-split prefill for launches too small to fill the GPU.
//
// In the 4-wave kernel every wave of a workgroup walks all key tiles of its
// query tile, so a launch with few workgroups lasts as long as the key chain
// of its last query rows (the batch-1, 12-head, seq-512 launch: 48
// workgroups for 256 compute units, eight 64-key tiles one after another).
// Here the four waves of a workgroup share 32 query rows and split the key
// tiles between them (wave w takes tiles w, w+4, ...), each with its own
// online-softmax state (attention-fusion page, section 2.2), and the four
// states are merged at the end with their maxima and sums: the merge of key
// ranges of section 4.4 of the same page, done in LDS.  The grid has four
// times as many workgroups and each key chain is a quarter as long.
//
// Per wave: Q^T as the MFMA B operand in VGPRs (as in the 4-wave kernel),
// its own double-buffered K/V ring in LDS filled by direct loads (no
// barrier inside the loop: no wave reads another wave's tiles), tiles of 64
// keys at head dim 64 and 32 keys at head dim 128 (8 KB each for K and V;
// 128 KB of LDS per workgroup, one workgroup per compute unit).
#pragma once

#include "prefill.hpp"

namespace attn {

template <int D>
struct KsLayout {
  static constexpr int BN = D == 64 ? 64 : 32;   // keys per tile
  static constexpr int NKB = BN / 32;            // 32-key MFMA blocks
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;           // rows per load instr
  static constexpr int NLI = BN / RPI;           // load instrs per K tile
  static constexpr int TILE = BN * D;            // elements of one K tile
  static_assert(NLI == 8 && TILE * 2 == 8192, "8 KB tiles, 8 loads");
};

template <typename T, int D, bool CAUSAL, bool RMS = false>
__global__ __launch_bounds__(kPrefillThreads, 1) void attn_prefill_ks_kernel(
    const T* __restrict__ Q, const T* __restrict__ K,
    const T* __restrict__ V, T* __restrict__ O,
    float* __restrict__ LSE, int B, int Hq, int Hkv, int S,
    float scale_log2, RmsEpilogue<T> rms) {
  using L = KsLayout<D>;
  constexpr int BN = L::BN, NKB = L::NKB, CPR = L::CPR, RPI = L::RPI;
  constexpr int TILE = L::TILE;
  constexpr int NDB = D / 32, KT = D / 16;
  using E = Elem16<T>;
  typedef typename E::x8 x8;

  // [wave][buffer][K, V][TILE]
  __shared__ __attribute__((aligned(1024))) T smem[4 * 2 * 2 * TILE];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r = lane & 31, hh = lane >> 5;

  // Block -> (batch, query head, 32-row block), heaviest row blocks first.
  const int BH = B * Hq;
  const int nrb = (S + 31) / 32;
  const int bid = blockIdx.x;
  const int rb = CAUSAL ? nrb - 1 - bid / BH : bid / BH;
  const int b = (bid % BH) / Hq, hq = (bid % BH) % Hq;
  const int g = hq / (Hq / Hkv);
  const size_t q_row0 = (size_t)(b * Hq + hq) * S;
  const size_t kv_row0 = (size_t)(b * Hkv + g) * S;
  const T* Qp = Q + q_row0 * D;
  const T* Kp = K + kv_row0 * D;
  const T* Vp = V + kv_row0 * D;

  const int q0 = rb * 32;
  const int query = q0 + r;
  const int kv_end = CAUSAL ? min(S, q0 + 32) : S;
  const int n_kv = (kv_end + BN - 1) / BN;
  // tiles below every row of the block and inside S need no mask
  const int n_full = min(min(n_kv, S / BN), CAUSAL ? (q0 + 1) / BN : n_kv);

  x8 qB[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t)
    qB[t] = query < S ? *reinterpret_cast<const x8*>(Qp + (size_t)query * D +
                                                     16 * t + 8 * hh)
                      : x8{};

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_i = -INFINITY, l_i = 0.f;

  // Direct loads of one whole tile by this wave: load i fills LDS rows
  // i*RPI .. i*RPI+RPI-1 (1 KB), lanes in order; chunks XOR-swizzled on the
  // memory side as in the 4-wave kernel.  Two runs of four loads, M0 once
  // per run (the immediate offset i*1024 advances both addresses).
  unsigned koffb[8], voffb[8], koffr[8], voffr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = i * RPI + lane / CPR, pos = lane % CPR;
    koffb[i] = (row * D + 8 * swz_k<CPR>(row, pos)) * 2;
    voffb[i] = (row * D + 8 * swz_v<CPR>(row, pos)) * 2;
    koffr[i] = koffb[i] - (i & 3) * 1024;
    voffr[i] = voffb[i] - (i & 3) * 1024;
  }
  const u32x4 krs = buffer_rsrc(Kp), vrs = buffer_rsrc(Vp);
  T* const ring = smem + w * 4 * TILE;           // this wave's 2 x (K, V)
  auto issue_tile = [&](int jt, int buf) {
    T* Kd = ring + buf * 2 * TILE;
    T* Vd = Kd + TILE;
    const int j0 = jt * BN;
    const unsigned soff = (unsigned)j0 * D * 2;
    if (j0 + BN <= S) {
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        const unsigned ko[4] = {koffr[4 * run], koffr[4 * run + 1],
                                koffr[4 * run + 2], koffr[4 * run + 3]};
        const unsigned vo[4] = {voffr[4 * run], voffr[4 * run + 1],
                                voffr[4 * run + 2], voffr[4 * run + 3]};
        lds_buffer_load16_run<4>(krs, ko, soff, Kd + run * 4 * RPI * D);
        lds_buffer_load16_run<4>(vrs, vo, soff, Vd + run * 4 * RPI * D);
      }
    } else {
      // rows past the end load row S-1 (their scores are masked)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = i * RPI + lane / CPR;
        const int back = (min(j0 + row, S - 1) - (j0 + row)) * D * 2;
        lds_buffer_load16(krs, koffb[i] + back, soff, Kd + i * RPI * D);
        lds_buffer_load16(vrs, voffb[i] + back, soff, Vd + i * RPI * D);
      }
    }
  };

  const int grp = lane >> 4, jl = lane & 15;
  const int vrow_off = 4 * (grp >> 1) + (jl >> 2);
  const int vcol_off = 16 * (grp & 1) + 4 * (jl & 3);
  auto qk_sub = [&](const T* Kt, int kb) {
    f32x16 acc = f32x16{};
    const int row = kb * 32 + r;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const x8 a = *reinterpret_cast<const x8*>(
          Kt + row * D + 8 * swz_k<CPR>(row, 2 * t + hh));
      acc = E::mma32(a, qB[t], acc);
    }
    return acc;
  };
  auto pv_sub = [&](const T* Vt, int kb, const x8 (&pb)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row0 = kb * 32 + 16 * u + vrow_off;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = db * 32 + vcol_off;
        const int c = col >> 3, e = col & 7;
        const u32x2 lo = lds_read_tr16(Vt + row0 * D +
                                       8 * swz_v<CPR>(row0, c) + e);
        const u32x2 hi = lds_read_tr16(Vt + (row0 + 8) * D +
                                       8 * swz_v<CPR>(row0 + 8, c) + e);
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
        oacc[db] = E::mma32(__builtin_bit_cast(x8, a), pb[u], oacc[db]);
      }
    }
  };
  // One tile, its 32-key blocks in turn: scores, mask, row max (lazy
  // rescale), probabilities, P V.  A wave's first tiles may hold no key a
  // row can see (wave w starts at tile w): such rows keep m = -inf and get
  // p = 0 until their first visible key.
  auto tile_body = [&](bool mask, int j0, const T* Kt, const T* Vt) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 s = qk_sub(Kt, kb);
      if (mask) apply_mask_block<CAUSAL>(s, j0 + 32 * kb, hh, query, S);
      float t5[5];
#pragma unroll
      for (int q = 0; q < 5; ++q)
        t5[q] = fmaxf(fmaxf(s[3 * q], s[3 * q + 1]), s[3 * q + 2]);
      const float mx =
          max_halves(fmaxf(fmaxf(fmaxf(t5[0], t5[1]), t5[2]),
                           fmaxf(fmaxf(t5[3], t5[4]), s[15]))) *
          scale_log2;
      if (mx > m_i + kLazyRescale) {
        const float alpha = fast_exp2(m_i - mx);
        l_i *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        m_i = mx;
      }
      const float neg_m = m_i == -INFINITY ? 0.f : -m_i;
      x8 pb[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = fast_exp2(fmaf(s[8 * u + i], scale_log2, neg_m));
          l_i += p;
          pb[u][i] = (T)p;
        }
      pv_sub(Vt, kb, pb);
    }
  };

  // This wave's tiles w, w+4, ...; the next one in flight while the
  // current one is multiplied (16 loads per tile).
  if (w < n_kv) issue_tile(w, 0);
  for (int jt = w, i = 0; jt < n_kv; jt += 4, ++i) {
    if (jt + 4 < n_kv) {
      issue_tile(jt + 4, (i + 1) & 1);
      wait_vmem_le<16>();
    } else {
      wait_vmem();
    }
    // no LDS read of this tile may be placed above the wait (there is no
    // barrier here to order them)
    asm volatile("" ::: "memory");
    const T* Kt = ring + (i & 1) * 2 * TILE;
    tile_body(jt >= n_full, jt * BN, Kt, Kt + TILE);
  }

  // Merge: waves 1-3 leave (O, m, l) in LDS, lane by lane (the same lane
  // holds the same query row and accumulator elements in every wave);
  // wave 0 combines with M = max m_w and weights 2^(m_w - M), then writes.
  constexpr int NV = NDB * 16 + 2;               // values per lane
  static_assert(3 * NV * 64 * 4 <= (int)sizeof(smem), "merge area");
  float* st = reinterpret_cast<float*>(smem);
  __syncthreads();                               // every wave's tiles done
  if (w > 0) {
    float* s0 = st + (size_t)(w - 1) * NV * 64 + lane;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) s0[(db * 16 + e) * 64] = oacc[db][e];
    s0[(NV - 2) * 64] = m_i;
    s0[(NV - 1) * 64] = l_i;
  }
  __syncthreads();
  if (w != 0) return;
  float mw[3], aw[3];
  float M = m_i;                 // finite: every row sees key 0 (tile 0)
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    mw[x] = st[((size_t)x * NV + NV - 2) * 64 + lane];
    M = fmaxf(M, mw[x]);
  }
  const float a0 = fast_exp2(m_i - M);
  float l = a0 * l_i;
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    aw[x] = fast_exp2(mw[x] - M);                // 0 for m = -inf
    l = fmaf(aw[x], st[((size_t)x * NV + NV - 1) * 64 + lane], l);
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float o = a0 * oacc[db][e];
#pragma unroll
      for (int x = 0; x < 3; ++x)
        o = fmaf(aw[x], st[((size_t)x * NV + db * 16 + e) * 64 + lane], o);
      oacc[db][e] = o;
    }
  const float l_tot = l + swap_halves(l);
  if constexpr (RMS) {
    // residual add + RMSNorm of the merged row
    const bool live = query < S;
    rms_epilogue_row<T, NDB>(oacc, 1.f / l_tot, live,
                             q_row0 + (live ? query : 0), hh, O, rms);
    if (live && LSE != nullptr && hh == 0)
      LSE[q_row0 + query] = (M + fast_log2(l_tot)) * kLn2;
  } else if (query < S) {
    const float inv = 1.f / l_tot;
    T* orow = O + (q_row0 + query) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 pr;
        pr[0] = E::pack2(oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv);
        pr[1] = E::pack2(oacc[db][4 * a + 2] * inv,
                         oacc[db][4 * a + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * a + 4 * hh) = pr;
      }
    if (LSE != nullptr && hh == 0)
      LSE[q_row0 + query] = (M + fast_log2(l_tot)) * kLn2;
  }
}

}  // namespace attn

namespace attn {

// The fp32 sibling of the key-split kernel (the fp32 prefill's steps: one
// query row per lane of v_mfma_f32_32x32x2_f32, probabilities kept in fp32).
// Each wave loads its own 32-key tiles through registers into its own LDS
// rows (padded by 4 floats against bank conflicts), one tile at a time.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kPrefillThreads, 1) void attn_prefill_f32_ks_kernel(
    const float* __restrict__ Q, const float* __restrict__ K,
    const float* __restrict__ V, float* __restrict__ O,
    float* __restrict__ LSE, int B, int Hq, int Hkv, int S,
    float scale_log2) {
  constexpr int BN = 32, NKB = 1, NDB = D / 32;
  constexpr int HD = D / 2;                   // contraction elems per half
  constexpr int STR = D + 4;                  // LDS row stride (floats)
  constexpr int DCH = D / 4;                  // 16-byte chunks per row
  constexpr int CH = BN * DCH / 64;           // chunks per lane per tile
  constexpr int HALF = D == 128 ? 2 : 1;      // K, V staged in turn at 128

  __shared__ __attribute__((aligned(16))) float smem[4 * 2 * BN * STR];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r = lane & 31, hh = lane >> 5;

  const int BH = B * Hq;
  const int nrb = (S + 31) / 32;
  const int bid = blockIdx.x;
  const int rb = CAUSAL ? nrb - 1 - bid / BH : bid / BH;
  const int b = (bid % BH) / Hq, hq = (bid % BH) % Hq;
  const int g = hq / (Hq / Hkv);
  const size_t q_row0 = (size_t)(b * Hq + hq) * S;
  const float* Qp = Q + q_row0 * D;
  const float* Kp = K + (size_t)(b * Hkv + g) * S * D;
  const float* Vp = V + (size_t)(b * Hkv + g) * S * D;

  const int q0 = rb * 32;
  const int query = q0 + r;
  const int kv_end = CAUSAL ? min(S, q0 + 32) : S;
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

  float* const Ks = smem + w * 2 * BN * STR;
  float* const Vs = Ks + BN * STR;
  // rows past S load as zeros (their scores are masked)
  auto stage = [&](const float* src, float* dst, int j0) {
    constexpr int CHH = CH / HALF;
#pragma unroll
    for (int h = 0; h < HALF; ++h) {
      f32x4 reg[CHH];
#pragma unroll
      for (int i = 0; i < CHH; ++i) {
        const int c = lane + (h * CHH + i) * 64;
        const int row = j0 + c / DCH, col = c % DCH;
        reg[i] = row < S ? *reinterpret_cast<const f32x4*>(
                               src + (size_t)row * D + col * 4)
                         : f32x4{};
      }
#pragma unroll
      for (int i = 0; i < CHH; ++i) {
        const int c = lane + (h * CHH + i) * 64;
        *reinterpret_cast<f32x4*>(&dst[(c / DCH) * STR + (c % DCH) * 4]) =
            reg[i];
      }
    }
  };

  for (int jt = w; jt < n_kv; jt += 4) {
    const int j0 = jt * BN;
    stage(Kp, Ks, j0);
    stage(Vp, Vs, j0);
    f32x16 sacc[NKB];
    sacc[0] = f32x16{};
    const float* krow = &Ks[r * STR + hh * HD];
#pragma unroll
    for (int t = 0; t < HD; t += 4) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(krow + t);
      sacc[0] = mfma_32x32x2_f32(a4[0], qB[t], sacc[0]);
      sacc[0] = mfma_32x32x2_f32(a4[1], qB[t + 1], sacc[0]);
      sacc[0] = mfma_32x32x2_f32(a4[2], qB[t + 2], sacc[0]);
      sacc[0] = mfma_32x32x2_f32(a4[3], qB[t + 3], sacc[0]);
    }
    if ((j0 + BN > S) || (CAUSAL && j0 + BN - 1 > q0))
      apply_mask<NKB, CAUSAL>(sacc, j0, hh, query, S);
    softmax_step<NKB, NDB>(sacc, scale_log2, m_i, l_i, oacc);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 8 * (i >> 2) + 4 * hh + (i & 3);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = mfma_32x32x2_f32(Vs[key * STR + db * 32 + r], sacc[0][i],
                                    oacc[db]);
    }
  }

  // Merge through LDS as in the 16-bit key-split kernel.
  constexpr int NV = NDB * 16 + 2;
  static_assert(3 * NV * 64 * 4 <= (int)sizeof(smem), "merge area");
  float* st = smem;
  __syncthreads();
  if (w > 0) {
    float* s0 = st + (size_t)(w - 1) * NV * 64 + lane;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) s0[(db * 16 + e) * 64] = oacc[db][e];
    s0[(NV - 2) * 64] = m_i;
    s0[(NV - 1) * 64] = l_i;
  }
  __syncthreads();
  if (w != 0) return;
  float mw[3], aw[3];
  float M = m_i;
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    mw[x] = st[((size_t)x * NV + NV - 2) * 64 + lane];
    M = fmaxf(M, mw[x]);
  }
  const float a0 = fast_exp2(m_i - M);
  float l = a0 * l_i;
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    aw[x] = fast_exp2(mw[x] - M);
    l = fmaf(aw[x], st[((size_t)x * NV + NV - 1) * 64 + lane], l);
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float o = a0 * oacc[db][e];
#pragma unroll
      for (int x = 0; x < 3; ++x)
        o = fmaf(aw[x], st[((size_t)x * NV + db * 16 + e) * 64 + lane], o);
      oacc[db][e] = o;
    }
  const float l_tot = l + swap_halves(l);
  if (query < S) {
    const float inv = 1.f / l_tot;
    float* orow = O + (q_row0 + query) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 o4 = {oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv,
                    oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * a + 4 * hh) = o4;
      }
    if (LSE != nullptr && hh == 0)
      LSE[q_row0 + query] = (M + fast_log2(l_tot)) * kLn2;
  }
}

}  // namespace attn
