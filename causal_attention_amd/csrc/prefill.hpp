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
// transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (_f16 for fp16
// inputs): K rows are the A
// operand (read from LDS), Q^T is the B operand (kept in VGPRs for the whole
// tile), and the accumulator leaves each lane with ONE query (lane % 32) and
// 16 keys per 32-key block.  Row max and row sum are then an in-lane
// reduction plus one exchange with the other wave half.  The probabilities
// P^T are re-used in place as the B operand of O^T = V^T P^T (a contraction
// over keys accepts any key order, as long as the A operand V^T reads V in the
// same order), so P never leaves registers.  V is stored transposed in LDS so
// that each lane's eight keys for one output dimension are two 8-byte runs.
// Softmax runs in the exp2 domain with scale*log2(e) folded into the exp2
// argument (the scale must be positive).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace attn {

constexpr int kPrefillThreads = 256;   // 4 waves

constexpr int kPrefillBM = 128;        // query rows per workgroup

// Block index -> (batch, KV head, query head, query tile).
//
// Work order: query tiles heaviest first (most key tiles under the causal
// mask), so short tiles fill the tail of the launch.  Blocks are dealt to
// the GPU in "rounds" of one block per CU (n_cu blocks); rounds with an odd
// index are reversed (in groups of 8, see below), so the two blocks that
// share a CU in the first wave of the launch are a heavy and a light one and
// every CU starts with about the same total work ("snake" order).
//
// XCD locality: consecutive work indices walk over (batch, KV head) pairs
// first, and blocks are dealt to the 8 XCDs round-robin, so when the pair
// count is a multiple of 8 every block of one pair lands on the same XCD
// and its K/V stay in that XCD's L2.  Reversing a round by whole groups of
// 8 block indices keeps each block on the XCD of its pair.
struct TileCoord {
  int b, g, hq, qt;
};

__device__ __forceinline__ TileCoord tile_coord(int bid, int nblocks, int B,
                                                int Hq, int Hkv, int n_qtiles,
                                                int n_cu) {
  int idx = bid;
  const int round = bid / n_cu;
  if ((round & 1) && (round + 1) * n_cu <= nblocks && (n_cu & 7) == 0) {
    const int pos = bid - round * n_cu;
    idx = round * n_cu + (n_cu / 8 - 1 - pos / 8) * 8 + (pos & 7);
  }
  const int G = Hq / Hkv;
  const int P = B * Hkv;
  const int pair = idx % P;
  const int rest = idx / P;
  TileCoord c;
  c.b = pair / Hkv;
  c.g = pair % Hkv;
  c.hq = c.g * G + rest % G;
  c.qt = n_qtiles - 1 - rest / G;
  return c;
}

// Online-softmax update of one 32-query x (16*NKB)-key transposed score block
// held as NKB accumulators of RAW scores q.k (masked = -inf).  With
// c = scale*log2(e) > 0 the log2-domain score is x*c, so the row max is taken
// on the raw scores and the scale is folded into the exp2 argument
// (p = exp2(x*c - m_ref), one FMA per score); x is overwritten with p.
//
// The running output is rescaled only when the row max exceeds the
// reference m_ref by more than kLazyRescale (2^8): the result is unchanged
// because the final division by l cancels any common reference, and the
// bound keeps p <= 256 (finite in fp32, same relative precision in bf16).  On
// the first visible block m_ref is -inf and the rescale factor is 0.
template <int NKB, int NDB>
__device__ __forceinline__ void softmax_step(f32x16 (&x)[NKB], float c,
                                             float& m_ref, float& l_i,
                                             f32x16 (&oacc)[NDB]) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, x[kb][i]);
  mx = fmaxf(mx, swap_halves(mx)) * c;
  if (mx > m_ref + kLazyRescale) {
    const float alpha = fast_exp2(m_ref - mx);
    l_i *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    m_ref = mx;
  }
  // A row with no visible key yet keeps m_ref = -inf and gets p = 0.
  const float neg_m = (m_ref == -INFINITY) ? 0.f : -m_ref;
  float sum = 0.f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(fmaf(x[kb][i], c, neg_m));
      x[kb][i] = p;
      sum += p;
    }
  l_i += sum;   // lane-partial: this half's keys only
}

// Causal / tail mask of a raw score block: key(kb, i) is the key index of
// accumulator element i of block kb for this lane (lane half hh).
template <int NKB, bool CAUSAL>
__device__ __forceinline__ void apply_mask(f32x16 (&x)[NKB], int j0, int hh,
                                           int query, int S) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = j0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
      const bool dead = (key >= S) || (CAUSAL && key > query);
      x[kb][i] = dead ? -INFINITY : x[kb][i];
    }
}

// Causal / tail mask of one 32-key block (key base j0) of raw scores.
template <bool CAUSAL>
__device__ __forceinline__ void apply_mask_block(f32x16& x, int j0, int hh,
                                                 int query, int S) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int key = j0 + 8 * (i >> 2) + 4 * hh + (i & 3);
    const bool dead = (key >= S) || (CAUSAL && key > query);
    x[i] = dead ? -INFINITY : x[i];
  }
}

// ------------------------------------------------- bf16 / fp16 path
//
// K and V tiles go global -> LDS with gfx950's direct loads
// (buffer_load_dwordx4 ... lds: no VGPR staging, each wave instruction fills
// 1 KB of LDS in lane order), double-buffered so that the next tile streams in
// while the current one is multiplied; one barrier per tile.  Rows are
// stored with their 16-byte chunks XOR-swizzled so the MFMA operand reads
// hit distinct LDS banks.  V stays row-major in LDS and its transposed MFMA
// operand comes from ds_read_b64_tr_b16: in each group of 16 lanes, lane j
// points at 4 dims of key row j/4 and lane i receives dim i of those 4 keys.

// LDS chunk position of 16-byte chunk c of row `row` (CPR chunks per row).
template <int CPR>
__device__ __forceinline__ int swz_k(int row, int c) {
  // A-operand reads: 16 consecutive rows, same chunk -> distinct banks.
  return CPR == 16 ? (c ^ (row & 15)) : (c ^ ((row >> 1) & 7));
}
template <int CPR>
__device__ __forceinline__ int swz_v(int row, int c) {
  // transposed reads: 4 consecutive rows x 4 aligned chunks -> distinct
  // banks; XOR by a multiple of 4 keeps aligned chunk quads together.
  return CPR == 16 ? (c ^ ((row & 3) << 2)) : (c ^ (((row >> 1) & 1) << 2));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposed 8-byte LDS read of 16-bit elements (any 16-bit type).
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// gfx9 raw buffer descriptor: 48-bit base, stride 0, no range limit.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base) {
  const size_t a = reinterpret_cast<size_t>(base);
  return u32x4{(unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)a),
               (unsigned)__builtin_amdgcn_readfirstlane(
                   (int)((a >> 32) & 0xffff)),
               0xffffffffu, 0x00020000u};
}

// One direct-to-LDS load, buffer_load_dwordx4 ... lds: lane i's 16 bytes at
// base + soff + voff go to LDS at l + 16 i (1 KB per wave instruction; l and
// soff are wave-uniform).  The descriptor and the tile offset sit in SGPRs,
// so a load costs no 64-bit address arithmetic per lane.  It is issued as
// inline assembly: the compiler takes a direct load it can see as possibly
// aliasing every later LDS read and puts s_waitcnt vmcnt(0) before the first
// transposed V read of the tile, i.e. it would wait for the NEXT tile's loads
// (a memory round trip when K/V come from HBM) although they fill the other
// buffer.  The loop waits for its loads itself (wait_vmem before the barrier
// of each step), and no load is left in flight when the loop ends.
// A wave's IPW loads of one tile, into consecutive 1 KB LDS blocks from l,
// with M0 set once: load i carries the immediate offset i*1024, which the
// hardware adds to both the LDS and the memory address, so voff[i] holds
// lane offset of load i minus i*1024 (never negative: the wave's rows of
// load i start i KB into the tile).
template <int IPW>
__device__ __forceinline__ void lds_buffer_load16_run(const u32x4& rsrc,
                                                      const unsigned (&voff)[IPW],
                                                      unsigned soff, void* l) {
  const unsigned m = __builtin_amdgcn_readfirstlane(lds_addr(l));
  const unsigned so = __builtin_amdgcn_readfirstlane(soff);
  static_assert(IPW == 2 || IPW == 4, "loads per wave");
  if constexpr (IPW == 4)
    asm volatile("s_mov_b32 m0, %4\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %0, %5, %6 offen lds\n\t"
                 "buffer_load_dwordx4 %1, %5, %6 offen offset:1024 lds\n\t"
                 "buffer_load_dwordx4 %2, %5, %6 offen offset:2048 lds\n\t"
                 "buffer_load_dwordx4 %3, %5, %6 offen offset:3072 lds"
                 :: "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]),
                    "s"(m), "s"(rsrc), "s"(so) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %0, %3, %4 offen lds\n\t"
                 "buffer_load_dwordx4 %1, %3, %4 offen offset:1024 lds"
                 :: "v"(voff[0]), "v"(voff[1]),
                    "s"(m), "s"(rsrc), "s"(so) : "memory", "m0");
}
__device__ __forceinline__ void lds_buffer_load16(const u32x4& rsrc,
                                                  unsigned voff, unsigned soff,
                                                  void* l) {
  const unsigned m = __builtin_amdgcn_readfirstlane(lds_addr(l));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\t"
               "buffer_load_dwordx4 %0, %1, %3 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(m),
                  "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory", "m0");
}

// s_waitcnt vmcnt(0): this wave's direct-to-LDS loads have landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kPrefillThreads, 2) void attn_prefill_kernel(
    const T* __restrict__ Q, const T* __restrict__ K,
    const T* __restrict__ V, T* __restrict__ O,
    float* __restrict__ LSE, int B, int Hq, int Hkv, int S_all,
    float scale_log2, int n_qtiles, int n_cu, int use_rope, RopeRates rope,
    const int* __restrict__ cu_seqlens, const int* __restrict__ seq_lens) {
  constexpr int BM = kPrefillBM, BN = 64, NKB = BN / 32, NDB = D / 32;
  constexpr int KT = D / 16;                  // MFMA k-steps over D
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;               // rows per wave load instr
  constexpr int IPW = BN / RPI / 4;           // load instrs per wave per tile
  constexpr int TILE = BN * D;                // elements per K or V tile
  static_assert(IPW >= 1, "tile shape");
  using E = Elem16<T>;
  typedef typename E::x8 x8;

  // [buffer][K, V][TILE]
  __shared__ __attribute__((aligned(1024))) T smem[4 * TILE];

  const int tid = threadIdx.x;
  // wave index as a uniform (scalar) value, so per-wave branches are scalar
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const TileCoord tc =
      tile_coord(blockIdx.x, gridDim.x, B, Hq, Hkv, n_qtiles, n_cu);
  // Length of this sequence and the first row of (batch, head) in Q / O /
  // LSE and in K / V: dense [B, H, S, D]; or a ragged batch (cu_seqlens:
  // sequence b is a [H, S_b, D] block at row offset H * cu[b]); or a dense
  // batch padded to S_all (seq_lens: the first L_b rows of sequence b are
  // valid; keys past L_b are masked, query rows past it get o = 0 and
  // lse = -inf).
  int S = S_all;
  size_t q_row0 = (size_t)(tc.b * Hq + tc.hq) * S_all;
  size_t kv_row0 = (size_t)(tc.b * Hkv + tc.g) * S_all;
  if (cu_seqlens != nullptr) {
    const int c0 = cu_seqlens[tc.b];
    S = cu_seqlens[tc.b + 1] - c0;
    if (tc.qt * kPrefillBM >= S) return;   // query tile past this sequence
    q_row0 = (size_t)c0 * Hq + (size_t)tc.hq * S;
    kv_row0 = (size_t)c0 * Hkv + (size_t)tc.g * S;
  } else if (seq_lens != nullptr) {
    S = min(max(seq_lens[tc.b], 0), S_all);
  }
  // Padding rows [S, S_all) of this query tile: o = 0, lse = -inf (a row of
  // 32 lanes x two halves per wave, D/2 elements per lane).
  auto pad_row = [&](int row) {
    T* orow = O + (q_row0 + row) * D + hh * (D / 2);
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      *reinterpret_cast<u32x4*>(orow + 8 * c) = u32x4{};
    if (LSE != nullptr && hh == 0) LSE[q_row0 + row] = -INFINITY;
  };
  if (seq_lens != nullptr && tc.qt * kPrefillBM >= S) {
    const int row = tc.qt * kPrefillBM + 32 * w + r;
    if (row < S_all) pad_row(row);
    return;                                 // whole tile is padding
  }
  const T* Qp = Q + q_row0 * D;
  const T* Kp = K + kv_row0 * D;
  const T* Vp = V + kv_row0 * D;

  const int q_lo = tc.qt * BM;
  const int q_hi = min(S, q_lo + BM);
  const int wq0 = q_lo + 32 * w;          // first query row of this wave
  const int query = wq0 + r;              // this lane's query row
  const int kv_end = CAUSAL ? q_hi : S;
  const int n_kv = (kv_end + BN - 1) / BN;

  // Q^T as the MFMA B operand: lane holds query `query`, dims 16t+8hh..+7.
  x8 qB[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    if (query < S)
      qB[t] = *reinterpret_cast<const x8*>(Qp + (size_t)query * D +
                                               16 * t + 8 * hh);
    else
      qB[t] = x8{};
  }
  // RoPE on load: the pair of dim d = 16t + 8hh + e (t < KT/2) is
  // d + D/2, held by the same lane in register t + KT/2.
  if (use_rope) {
#pragma unroll
    for (int t = 0; t < KT / 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x1 = (float)qB[t][e], x2 = (float)qB[t + KT / 2][e];
        const double r = hh ? rope.r[16 * t + 8 + e] : rope.r[16 * t + e];
        rope_pair(x1, x2, query, r);
        qB[t][e] = (T)x1;
        qB[t + KT / 2][e] = (T)x2;
      }
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_i = -INFINITY, l_i = 0.f;

  // Issue the direct loads of key tile jt into (Kd, Vd).  Rows past the end
  // of the sequence load row S-1 (their scores are masked to -inf, so their
  // values are multiplied by p = 0).
  unsigned koffb[IPW], voffb[IPW], koffr[IPW], voffr[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int row = (w * IPW + i) * RPI + lane / CPR, pos = lane % CPR;
    koffb[i] = (row * D + 8 * swz_k<CPR>(row, pos)) * 2;
    voffb[i] = (row * D + 8 * swz_v<CPR>(row, pos)) * 2;
    koffr[i] = koffb[i] - i * 1024;
    voffr[i] = voffb[i] - i * 1024;
  }
  const u32x4 krs = buffer_rsrc(Kp), vrs = buffer_rsrc(Vp);
  auto issue_tile = [&](int jt, T* Kd, T* Vd) {
    const int j0 = jt * BN;
    const unsigned soff = (unsigned)j0 * D * 2;   // tile offset in bytes
    if (j0 + BN <= S) {
      static_assert(RPI * D * 2 == 1024, "1 KB per load");
      lds_buffer_load16_run<IPW>(krs, koffr, soff, Kd + w * IPW * RPI * D);
      lds_buffer_load16_run<IPW>(vrs, voffr, soff, Vd + w * IPW * RPI * D);
    } else {
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int r0 = (w * IPW + i) * RPI;
        const int row = r0 + lane / CPR;
        const int back = (min(j0 + row, S - 1) - (j0 + row)) * D * 2;
        lds_buffer_load16(krs, koffb[i] + back, soff, Kd + r0 * D);
        lds_buffer_load16(vrs, voffb[i] + back, soff, Vd + r0 * D);
      }
    }
  };

  // One 64-key tile as two 32-key sub-blocks, each with its own row max and
  // lazy-rescale check (the online softmax accepts any blocking), ordered so
  // that independent MFMA and VALU work sit next to each other:
  //   S0 = K0 Q^T;  [S1 = K1 Q^T  ||  P0 = exp2(S0)];  [O += V0^T P0  ||
  //   P1 = exp2(S1)];  rescale O if S1 raised the max;  O += V1^T P1.
  // P0 is accumulated with the reference it was computed against before
  // any rescale for S1 is applied, so O, l and P stay consistent.
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
  // p = exp2(s*c + neg_m) as two x8 B operands; returns the lane sum.
  auto exp_sub = [&](const f32x16& sv, float neg_m, x8 (&pb)[2]) {
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = fast_exp2(fmaf(sv[8 * u + i], scale_log2, neg_m));
        sum += p;
        pb[u][i] = (T)p;
      }
    return sum;
  };
  auto rowmax = [&](const f32x16& sv) {
    float t[5];
#pragma unroll
    for (int g = 0; g < 5; ++g)
      t[g] = fmaxf(fmaxf(sv[3 * g], sv[3 * g + 1]), sv[3 * g + 2]);
    const float mx = fmaxf(fmaxf(fmaxf(t[0], t[1]), t[2]),
                           fmaxf(fmaxf(t[3], t[4]), sv[15]));
    return max_halves(mx) * scale_log2;
  };
  auto rescale = [&](float m_new) {
    const float alpha = fast_exp2(m_i - m_new);
    l_i *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    m_i = m_new;
  };

  auto tile_body = [&](auto mask_tag, int j0, const T* Kt,
                       const T* Vt) {
    constexpr bool MASK = decltype(mask_tag)::value;
    f32x16 s0 = qk_sub(Kt, 0);
    if constexpr (MASK) apply_mask_block<CAUSAL>(s0, j0, hh, query, S);
    const float mx0 = rowmax(s0);
    if (mx0 > m_i + kLazyRescale) rescale(mx0);
    // Every row sees key 0, so m is finite from the first sub-block on.
    const float neg_m0 = -m_i;

    f32x16 s1 = qk_sub(Kt, 1);
    x8 pb0[2];
    l_i += exp_sub(s0, neg_m0, pb0);

    if constexpr (MASK)
      apply_mask_block<CAUSAL>(s1, j0 + 32, hh, query, S);
    const float mx1 = rowmax(s1);
    const bool up = mx1 > m_i + kLazyRescale;
    const float neg_m1 = up ? -mx1 : -m_i;

    pv_sub(Vt, 0, pb0);
    x8 pb1[2];
    const float sum1 = exp_sub(s1, neg_m1, pb1);
    if (up) rescale(mx1);
    l_i += sum1;
    pv_sub(Vt, 1, pb1);
  };
  // Tile jt lives in buffer jt & 1.  The leading tiles need no mask for any
  // row of the workgroup; the rest (the causal diagonal and a ragged tail,
  // at most three tiles) run a second loop with the elementwise mask.  Every
  // wave computes every tile of the range: a wave whose rows all lie above
  // a tile's keys gets p = 0 from the mask.
  const int n_full = min(min(n_kv, S / BN), CAUSAL ? (q_lo + 1) / BN : n_kv);
  auto step = [&](auto mask_tag, int jt, int buf) {
    wait_vmem();                  // this wave's loads of tile jt landed
    __syncthreads();              // everyone's landed; tile jt-1 consumed
    T* cur = smem + buf * 2 * TILE;
    T* nxt = smem + (buf ^ 1) * 2 * TILE;
    if (jt + 1 < n_kv) issue_tile(jt + 1, nxt, nxt + TILE);
    tile_body(mask_tag, jt * BN, cur, cur + TILE);
  };
  if (n_kv > 0) issue_tile(0, smem, smem + TILE);
  // Two tiles per iteration so that the buffer of each is a constant.
  int jt = 0;
  for (; jt < n_full; jt += 2) {
    step(std::false_type{}, jt, 0);
    if (jt + 1 < n_full) step(std::false_type{}, jt + 1, 1);
  }
  for (jt = n_full; jt < n_kv; ++jt) step(std::true_type{}, jt, jt & 1);

  // Epilogue: O = acc / l (input type, RNE) and LSE = (m_ref + log2 l) * ln 2.
  const float l_tot = l_i + swap_halves(l_i);
  if (query < S) {
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
      LSE[q_row0 + query] =
          (m_i + fast_log2(l_tot)) * kLn2;
  } else if (seq_lens != nullptr && query < S_all) {
    pad_row(query);
  }
}

// RoPE of whole rows: x, y [rows, D] with row i at position i % S (the
// [B, H, S, D] layout), y = x rotated (y may be x).  One thread per pair of
// 16-byte chunks (c, c + D/16); the rates sit in LDS.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_rope_rows_kernel(
    const T* __restrict__ x, T* __restrict__ y, long long rows, int S,
    RopeRates rope) {
  using E = Elem16<T>;
  typedef typename E::x8 x8;
  constexpr int HC = D / 16;                 // chunk pairs per row
  __shared__ double rates[D / 2];
  for (int i = threadIdx.x; i < D / 2; i += 256) rates[i] = rope.r[i];
  __syncthreads();
  const long long id = (long long)blockIdx.x * 256 + threadIdx.x;
  if (id >= rows * HC) return;
  const long long row = id / HC;
  const int c = (int)(id % HC);
  const int pos = (int)(row % S);
  const T* xr = x + row * D;
  T* yr = y + row * D;
  x8 a = *reinterpret_cast<const x8*>(xr + 8 * c);
  x8 b = *reinterpret_cast<const x8*>(xr + D / 2 + 8 * c);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float x1 = (float)a[e], x2 = (float)b[e];
    rope_pair(x1, x2, pos, rates[8 * c + e]);
    a[e] = (T)x1;
    b[e] = (T)x2;
  }
  *reinterpret_cast<x8*>(yr + 8 * c) = a;
  *reinterpret_cast<x8*>(yr + D / 2 + 8 * c) = b;
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
    int n_qtiles, int n_cu) {
  constexpr int BM = kPrefillBM, BN = 32, NKB = BN / 32, NDB = D / 32;
  constexpr int HD = D / 2;                   // contraction elems per half
  constexpr int STR = D + 4;                  // LDS row stride (floats)
  constexpr int DCH = D / 4;                  // 16-byte chunks per row
  constexpr int CH = BN * DCH / kPrefillThreads;
  static_assert(CH >= 1, "tile shape");

  __shared__ __attribute__((aligned(16))) float Ks[BN * STR];
  __shared__ __attribute__((aligned(16))) float Vs[BN * STR];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const TileCoord tc =
      tile_coord(blockIdx.x, gridDim.x, B, Hq, Hkv, n_qtiles, n_cu);
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
    if ((j0 + BN > S) || (CAUSAL && j0 + BN - 1 > wq0))
      apply_mask<NKB, CAUSAL>(sacc, j0, hh, query, S);
    softmax_step<NKB, NDB>(sacc, scale_log2, m_i, l_i, oacc);

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
