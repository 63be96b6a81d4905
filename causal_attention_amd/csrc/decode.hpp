// Decode kernels: one query row per sequence against its KV cache (packed or
// padded), split over the keys of the whole batch, then a log-sum-exp combine
// of the pieces of each (sequence, query head) that were split.
//
// Method ("Attention三算子融合实战：从Triton到CUDA的推理加速优化"): the decode
// setting of section 1.3 (one query row, K and V as long as the history), the
// key split of section 4.4 (key chunks handled by separate blocks, each
// running the online softmax of section 2.2, merged afterwards), and the
// partial-buffer-plus-reduce-kernel pattern of "手写Triton kernel重构
// Qwen3.5-0.8B" section 3.3 (a separate small reduce kernel rather than
// atomics).  GQA (section 2.1 of that page): the G = Hq/Hkv query heads of
// one KV head are handled together, so each K/V byte is read from HBM once,
// not once per query head.
//
// gfx950 mapping.  The path is bound by HBM bandwidth (about 4 FLOP per
// byte), so the design goal is a steady stream of large, contiguous loads on
// every CU from the first microsecond to the last:
//  * Work split ("stream-K"): the caches are cut into 32-key blocks and the
//    blocks of all (sequence, KV head) segments, in that order, are divided
//    into P equal contiguous ranges, one per single-wave workgroup (P = two
//    per CU by default).  Every workgroup gets the same number of blocks
//    whatever the length mix, and all of them start together.  A segment
//    that lies wholly in one range is finished by its workgroup; a segment
//    cut by range boundaries leaves one partial (normalised output and LSE)
//    per piece, and the range holding its first block records which ranges
//    hold the others, for the combine kernel.
//  * Each wave streams its blocks in order through a double-buffered LDS
//    ring: K and V (and, with a piece's first block, the segment's G query
//    rows) arrive by gfx950's direct loads (global_load_lds_dwordx4, 1 KB
//    contiguous per instruction), and the next block's loads (across
//    segment ends too) are issued before the current one is multiplied.
//    A deeper ring (four buffers) measured no faster: the kernel streams
//    at about 5.7 TB/s once running, and its time on the C4 workload is
//    dominated by the fixed latency of a launch (length scan, first load,
//    tail), not by loads in flight.
//  * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 (_f16 for
//    fp16 inputs; the heads are MFMA columns, the other columns are zero):
//    K rows are the A operand, V^T comes from transposed LDS reads
//    (ds_read_b64_tr_b16), the query rows are read once per piece (and
//    rotated there when RoPE is on), and the probabilities stay in registers
//    as the B operand of the second product.  The running output is rescaled
//    only when the row max grows by more than 2^8 (exact: the final division
//    by l cancels any common reference).
//  * The caches are either packed per sequence or padded to a per-sequence
//    capacity (the serving-loop layout of attn_kv_append); only the address
//    of a segment's first row differs.
#pragma once

#include "common.hpp"

namespace attn {

constexpr int kDecodeBlock = 32;                  // keys per block


// T blocks cut into P equal contiguous ranges: range i starts at
// floor(i*T/P) = q*i + floor(r*i/P) with T = q*P + r (r*i < P*P, so the
// second division is 32-bit).  The two 64-bit quotients below (q, and the
// range holding a block) come from one double-precision division each,
// corrected by one step: for T < 2^40 and P <= 4096 the numerators are
// exact doubles and the rounded quotient is within one of the true one.
// (A binary search over lo() cost about a microsecond per segment end,
// on one lane, in the middle of a range's stream.)
struct Ranges {
  long long T, q;
  int r, P;
  __host__ __device__ __forceinline__ Ranges(long long T_, int P_)
      : T(T_), P(P_) {
    q = (long long)((double)T_ / (double)P_);
    if (q * P_ > T_) --q;
    else if ((q + 1) * P_ <= T_) ++q;
    r = (int)(T_ - q * P_);
  }
  __host__ __device__ __forceinline__ long long lo(int i) const {
    return q * i + (unsigned)(r * i) / (unsigned)P;
  }
  // The range holding block x (0 <= x < T): the largest i with lo(i) <= x,
  // which is floor(((x + 1) P - 1) / T).
  __host__ __device__ __forceinline__ int owner(long long x) const {
    const long long num = (x + 1) * P - 1;
    long long i = (long long)((double)num / (double)T);
    if (i * T > num) --i;
    else if ((i + 1) * T <= num) ++i;
    return (int)i;
  }
};

// Inclusive prefix sum of x over the 64 lanes of the wave by DPP: shifts
// by 1, 2, 4 and 8 within each row of 16 lanes (lanes shifted in from
// outside the row add 0), then lane 15 of rows 0 and 2 added to rows 1 and
// 3, then lane 31 to rows 2 and 3.
__device__ __forceinline__ int wave_scan_add(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Lane l's value of v as a wave-uniform (scalar) value.
__device__ __forceinline__ long long lane_i64(long long v, int l) {
  const int lo = __builtin_amdgcn_readlane((int)(v & 0xffffffffLL), l);
  const int hi = __builtin_amdgcn_readlane((int)(v >> 32), l);
  return ((long long)hi << 32) | (unsigned)lo;
}

// 64 consecutive sequences [base, base+64), one per lane: L (clamped to
// [0, cap] when cap > 0, else to >= 0), its 32-key block count, and the
// exclusive prefix sums of keys and of blocks over all sequences before it.
// kend / bend: the inclusive totals at the end of the chunk (wave-uniform).
struct SeqChunk {
  int base;
  int L, nb;
  long long kx, bx;
  long long kend, bend;
};

__device__ __forceinline__ SeqChunk load_chunk(const int* __restrict__ seqlens,
                                               int B, int cap, int base,
                                               long long k0, long long b0,
                                               int lane) {
  SeqChunk c;
  c.base = base;
  const int b = base + lane;
  c.L = (b < B) ? max(seqlens[b], 0) : 0;
  if (cap > 0) c.L = min(c.L, cap);
  c.nb = (c.L + kDecodeBlock - 1) / kDecodeBlock;
  long long ki, bi;
  if (__ballot(c.L >= (1 << 24)) == 0) {
    // every length below 2^24, so 64 of them sum below 2^30: 32-bit DPP
    // scans (this is on every workgroup's path before its first load)
    ki = wave_scan_add(c.L);
    bi = wave_scan_add(c.nb);
  } else {
    ki = c.L;
    bi = c.nb;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long kt = __shfl_up(ki, off, 64);
      const long long bt = __shfl_up(bi, off, 64);
      if (lane >= off) {
        ki += kt;
        bi += bt;
      }
    }
  }
  c.kx = k0 + ki - c.L;
  c.bx = b0 + bi - c.nb;
  c.kend = k0 + lane_i64(ki, 63);
  c.bend = b0 + lane_i64(bi, 63);
  return c;
}

// One (sequence b, KV head g) segment, as a range [s0, s0 + nb) in the global
// block order (segment-major: b*Hkv + g), with key offset kx of sequence b
// and the part [a, e) of it that this workgroup processes.  Wave-uniform.
struct DecodeSeg {
  int b, g, L, nb;
  long long kx, s0, a, e;
  bool valid;
};

__device__ __forceinline__ DecodeSeg make_seg(const SeqChunk& c, int lane_b,
                                              int g, int Hkv, long long lo,
                                              long long hi) {
  DecodeSeg s;
  s.b = c.base + lane_b;
  s.g = g;
  s.L = __builtin_amdgcn_readlane(c.L, lane_b);
  s.nb = __builtin_amdgcn_readlane(c.nb, lane_b);
  s.kx = lane_i64(c.kx, lane_b);
  s.s0 = lane_i64(c.bx, lane_b) * Hkv + (long long)g * s.nb;
  s.a = max(lo, s.s0);
  s.e = min(hi, s.s0 + s.nb);
  s.valid = s.a < s.e;
  return s;
}

// K rows in LDS: 16-byte chunk c of row r at chunk position c ^ f(r), so the
// 16 rows read by one A-operand load hit distinct banks.
template <int D>
__device__ __forceinline__ int dec_swz_k(int row, int c) {
  return D == 128 ? (c ^ (row & 15)) : (c ^ ((row >> 1) & 7));
}
// V rows: the 16 rows of one transposed load hit distinct banks (f is even,
// which keeps the chunk pairs of a transposed read together).
template <int D>
__device__ __forceinline__ int dec_swz_v(int row, int c) {
  return D == 128 ? (c ^ ((row & 7) << 1)) : (c ^ (((row >> 1) & 3) << 1));
}

__device__ __forceinline__ void dec_lds_load16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(
      g, (__attribute__((address_space(3))) void*)(l), 16, 0, 0);
}

template <int D, int G>
struct DecodeLayout {
  static constexpr int KT = D / 32;             // QK k-steps (32 dims)
  static constexpr int NDB = D / 16;            // PV output blocks (16 dims)
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;          // rows per load instruction
  static constexpr int NKI = kDecodeBlock / RPI;     // instrs per K (or V)
  static constexpr int QBYTES = (G * D * 2 + 1023) / 1024 * 1024;
  static constexpr int NQI = QBYTES / 1024;          // instrs for Q
  static constexpr int GROUP = 2 * NKI + NQI;        // instrs per block
  static constexpr int KBYTES = kDecodeBlock * D * 2;
  static constexpr int BUF = 2 * KBYTES + QBYTES;    // K | V | Q
  static constexpr int LDS = 2 * BUF;                // double buffer
};

// One wave per workgroup, one key range per wave.
template <typename T, int D, int G>
__global__ __launch_bounds__(64) void attn_decode_split_kernel(
    const T* __restrict__ Q, const T* __restrict__ Kc,
    const T* __restrict__ Vc, const int* __restrict__ seqlens,
    T* __restrict__ O, float* __restrict__ LSE,
    float* __restrict__ ws_o, float* __restrict__ ws_lse,
    int2* __restrict__ ws_seg, long long* __restrict__ ws_total, int B,
    int Hkv, int P, int cap, float scale_log2, int use_rope,
    RopeRates rope) {
  using Lay = DecodeLayout<D, G>;
  constexpr int KT = Lay::KT, NDB = Lay::NDB, CPR = Lay::CPR;
  constexpr int RPI = Lay::RPI, NKI = Lay::NKI, NQI = Lay::NQI;
  constexpr int BUF = Lay::BUF, KBYTES = Lay::KBYTES;
  static_assert(G <= 16, "heads are MFMA columns");
  using E = Elem16<T>;
  typedef typename E::x8 x8;

  __shared__ __attribute__((aligned(1024))) unsigned char lds[Lay::LDS];
  __shared__ double s_rates[D / 2];          // RoPE rates (when use_rope)

  const int lane = threadIdx.x;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int Hq = Hkv * G;
  const int wg = blockIdx.x;

  // The key blocks of every (sequence, KV head) segment, in order, and this
  // wave's range [lo, hi) of them.  For B <= 64 the first chunk of sequence
  // lengths is kept for the search below.
  SeqChunk ch = load_chunk(seqlens, B, cap, 0, 0, 0, lane);
  long long nblk = ch.bend;
  for (int base = 64; base < B; base += 64)
    nblk = load_chunk(seqlens, B, cap, base, 0, nblk, lane).bend;
  const long long total = nblk * Hkv;
  const Ranges rg(total, P);
  const long long lo = rg.lo(wg), hi = rg.lo(wg + 1);

  // Workgroup 0: the block total for the combine kernel, and sequences
  // without keys (o = 0, lse = -inf, nothing to combine).
  if (wg == 0) {
    if (lane == 0) *ws_total = total;
    for (int base = 0; base < B; base += 64) {
      const int b = base + lane;
      if (b < B && seqlens[b] <= 0) {
        for (int i = 0; i < Hq * D; i += 8)
          *reinterpret_cast<u32x4*>(O + (size_t)b * Hq * D + i) = u32x4{};
        if (LSE != nullptr)
          for (int h = 0; h < Hq; ++h) LSE[(size_t)b * Hq + h] = -INFINITY;
        for (int g = 0; g < Hkv; ++g) ws_seg[(size_t)b * Hkv + g] = int2{1, 0};
      }
    }
  }
  if (lo >= hi) return;

  // The segment holding block lo.
  int lb = 0, g0 = 0;
  for (;;) {
    const long long s = ch.bx * Hkv, e = (ch.bx + ch.nb) * Hkv;
    const unsigned long long hit =
        __ballot(ch.base + lane < B && s <= lo && lo < e);
    if (hit) {
      lb = __builtin_ctzll(hit);
      const long long sb = lane_i64(ch.bx, lb) * Hkv;
      const int nbb = __builtin_amdgcn_readlane(ch.nb, lb);
      const long long into = lo - sb;    // < Hkv * nbb
      g0 = into <= 0x7fffffffLL ? (int)((unsigned)into / (unsigned)nbb)
                                : (int)(into / nbb);
      break;
    }
    ch = load_chunk(seqlens, B, cap, ch.base + 64, ch.kend, ch.bend, lane);
  }
  DecodeSeg cur = make_seg(ch, lb, g0, Hkv, lo, hi);

  // The segment after `s` (next KV head, else the next sequence with keys),
  // or an invalid one when `s` reaches the end of the range.
  auto next_seg = [&](const DecodeSeg& s) {
    if (s.e >= hi) {
      DecodeSeg n = s;
      n.valid = false;
      return n;
    }
    if (s.g + 1 < Hkv) return make_seg(ch, lb, s.g + 1, Hkv, lo, hi);
    for (;;) {
      const unsigned long long more =
          __ballot(lane > lb && ch.base + lane < B && ch.nb > 0);
      if (more) {
        lb = __builtin_ctzll(more);
        return make_seg(ch, lb, 0, Hkv, lo, hi);
      }
      // blocks remain in the range, so a later chunk holds them
      ch = load_chunk(seqlens, B, cap, ch.base + 64, ch.kend, ch.bend,
                      lane);
      lb = -1;
    }
  };

  // Per-lane byte offsets of the direct loads: K / V row i*RPI + lane/CPR
  // of a block with its chunks swizzled, and element lane*8 (+512 per
  // instruction) of the query rows.
  unsigned koff[NKI], voff[NKI], qoff[NQI];
#pragma unroll
  for (int i = 0; i < NKI; ++i) {
    const int row = i * RPI + lane / CPR, pos = lane % CPR;
    koff[i] = (row * D + 8 * dec_swz_k<D>(row, pos)) * 2;
    voff[i] = (row * D + 8 * dec_swz_v<D>(row, pos)) * 2;
  }
#pragma unroll
  for (int i = 0; i < NQI; ++i) qoff[i] = min((i * 64 + lane) * 8, G * D - 8) * 2;

  // Direct loads of block blk of segment s into buffer buf: K and V rows
  // (past the end of the sequence: row L-1, whose score is masked) and the
  // segment's G query rows.
  auto issue = [&](const DecodeSeg& s, long long blk, int buf) {
    const int k0 = (int)(blk - s.s0) * kDecodeBlock;
    // packed: sequence b at key offset kx, head g after g*L rows; padded
    // (cap > 0): sequence b, head g at row (b*Hkv + g)*cap
    const size_t seg_off =
        cap > 0 ? ((size_t)s.b * Hkv + s.g) * (size_t)cap * D
                : ((size_t)s.kx * Hkv + (size_t)s.g * s.L) * D;
    const char* Kp = reinterpret_cast<const char*>(Kc + seg_off);
    const char* Vp = reinterpret_cast<const char*>(Vc + seg_off);
    unsigned char* kb = lds + buf * BUF;
    if (k0 + kDecodeBlock <= s.L) {
      const char* Kb = Kp + (size_t)k0 * D * 2;
      const char* Vb = Vp + (size_t)k0 * D * 2;
#pragma unroll
      for (int i = 0; i < NKI; ++i) {
        dec_lds_load16(Kb + koff[i], kb + i * 1024);
        dec_lds_load16(Vb + voff[i], kb + KBYTES + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NKI; ++i) {
        const int row = i * RPI + lane / CPR;
        const int d = (min(k0 + row, s.L - 1) - (k0 + row)) * D * 2;
        const char* Kb = Kp + (size_t)k0 * D * 2 + d;
        const char* Vb = Vp + (size_t)k0 * D * 2 + d;
        dec_lds_load16(Kb + koff[i], kb + i * 1024);
        dec_lds_load16(Vb + voff[i], kb + KBYTES + i * 1024);
      }
    }
    // the query rows only with a piece's first block (compute reads them
    // there once and keeps them in registers)
    if (blk == s.a) {
      const char* Qp = reinterpret_cast<const char*>(
          Q + ((size_t)s.b * Hq + (size_t)s.g * G) * D);
#pragma unroll
      for (int i = 0; i < NQI; ++i)
        dec_lds_load16(Qp + qoff[i], kb + 2 * KBYTES + i * 1024);
    }
  };

  // Online-softmax state of head c16: reference max (log2 domain),
  // lane-partial sum, O^T rows 16db + 4g4 + i.
  f32x4 oacc[NDB];
  float m_ref = -INFINITY, l_i = 0.f;
  // This piece's query rows as the B operand (read from LDS on the piece's
  // first block, rotated there when RoPE is on, then kept).
  u32x4 qkeep[KT];
  if (use_rope)
    for (int i = lane; i < D / 2; i += 64) s_rates[i] = rope.r[i];

  const unsigned lds_base = lds_addr(lds);
  // One block: keys k0 .. k0+31 of segment s, in buffer buf.
  auto compute = [&](const DecodeSeg& s, long long blk, int buf) {
    const unsigned kb = lds_base + buf * BUF;
    const int k0 = (int)(blk - s.s0) * kDecodeBlock;
    // Q^T (B operand): column c16 = head c16 (zero for c16 >= G), dims
    // 32t + 8g4 .. +7.  K (A operand): rows 16kh + c16, same dims.
    u32x4 kv[2][KT];
    const int qh = min(c16, G - 1);
    const bool fresh = blk == s.a;           // first block of this piece
    if (fresh) {
#pragma unroll
      for (int t = 0; t < KT; ++t)
        lds_read_b128_async(qkeep[t], kb + 2 * KBYTES + qh * D * 2 +
                                          (32 * t + 8 * g4) * 2);
    }
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const int row = 16 * kh + c16;
        lds_read_b128_async(kv[kh][t],
                            kb + row * D * 2 +
                                16 * dec_swz_k<D>(row, 4 * t + g4));
      }
    // V^T (A operand): lane group g4 reads keys 4g4..+3 and 16+4g4..+3 (the
    // key order of P^T), dims 16db + (lane & 15).
    u32x2 vlo[NDB], vhi[NDB];
    const int r0 = 4 * g4 + (c16 >> 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int col = 16 * db + 4 * (c16 & 3);
      const int cc = col >> 3, e = col & 7;
      lds_read_tr16_async(vlo[db], kb + KBYTES + r0 * D * 2 +
                                       16 * dec_swz_v<D>(r0, cc) + 2 * e);
      lds_read_tr16_async(vhi[db], kb + KBYTES + (r0 + 16) * D * 2 +
                                       16 * dec_swz_v<D>(r0 + 16, cc) + 2 * e);
    }
    lds_wait_all();
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      lds_tie(kv[0][t]);
      lds_tie(kv[1][t]);
    }
    if (fresh) {
#pragma unroll
      for (int t = 0; t < KT; ++t) lds_tie(qkeep[t]);
      // RoPE of the query at its position L - 1 (the newest token): the
      // pair of dim d = 32t + 8g4 + e (t < KT/2) is d + D/2, held by the
      // same lane in register t + KT/2.
      if (use_rope) {
#pragma unroll
        for (int t = 0; t < KT / 2; ++t) {
          x8 a = __builtin_bit_cast(x8, qkeep[t]);
          x8 b = __builtin_bit_cast(x8, qkeep[t + KT / 2]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float x1 = (float)a[e], x2 = (float)b[e];
            rope_pair(x1, x2, s.L - 1, s_rates[32 * t + 8 * g4 + e]);
            a[e] = (T)x1;
            b[e] = (T)x2;
          }
          qkeep[t] = __builtin_bit_cast(u32x4, a);
          qkeep[t + KT / 2] = __builtin_bit_cast(u32x4, b);
        }
      }
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      lds_tie(vlo[db]);
      lds_tie(vhi[db]);
    }

    f32x4 sacc[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      sacc[kh] = f32x4{};
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const x8 qb = (c16 < G) ? __builtin_bit_cast(x8, qkeep[t])
                                    : x8{};
        sacc[kh] = E::mma16(__builtin_bit_cast(x8, kv[kh][t]),
                                      qb, sacc[kh]);
      }
    }
    // lane holds head c16, keys k0 + 16kh + 4g4 + i (raw q.k; masked = -inf)
    float x[8];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 16 * kh + 4 * g4 + i;
        x[4 * kh + i] = (key < s.L) ? sacc[kh][i] : -INFINITY;
      }
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
    if (mx > m_ref + kLazyRescale) {
      // new reference (every block has a live key, so on a segment's first
      // block m_ref is -inf, mx is finite and the rescale factor is 0)
      const float alpha = fast_exp2(m_ref - mx);
      l_i *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;
      m_ref = mx;
    }
    const float neg_m = -m_ref;
    x8 pB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = fast_exp2(fmaf(x[i], scale_log2, neg_m));
      l_i += p;
      pB[i] = (T)p;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x4 a = {vlo[db][0], vlo[db][1], vhi[db][0], vhi[db][1]};
      oacc[db] = E::mma16(__builtin_bit_cast(x8, a), pB,
                                    oacc[db]);
    }
  };

  // This wave's blocks lo .. hi-1 in order; the next one is put in flight
  // before the current one is multiplied, across segment ends too.
  issue(cur, lo, 0);
  int n = 0;                          // blocks multiplied so far
  for (;;) {
    const DecodeSeg nxt = next_seg(cur);
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = f32x4{};
    m_ref = -INFINITY;
    l_i = 0.f;
    for (long long blk = cur.a; blk < cur.e; ++blk) {
      if (blk + 1 < cur.e) {
        issue(cur, blk + 1, (n + 1) & 1);     // not a piece's first block
        wait_vmem_le<2 * NKI>();
      } else if (nxt.valid) {
        issue(nxt, nxt.a, (n + 1) & 1);       // K, V and the query rows
        wait_vmem_le<Lay::GROUP>();
      } else {
        wait_vmem_le<0>();
      }
      compute(cur, blk, n & 1);
      ++n;
    }
    // Segment end: the final output when the whole segment is in this
    // range, else this piece's normalised output and LSE.
    l_i += __shfl_xor(l_i, 16, 64);
    l_i += __shfl_xor(l_i, 32, 64);
    if (c16 < G) {
      const float inv = 1.f / l_i;
      const float lse = (m_ref + fast_log2(l_i)) * kLn2;
      if (cur.s0 >= lo && cur.s0 + cur.nb <= hi) {
        const size_t row = (size_t)cur.b * Hq + (size_t)cur.g * G + c16;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          u32x2 pr;
          pr[0] = E::pack2(oacc[db][0] * inv, oacc[db][1] * inv);
          pr[1] = E::pack2(oacc[db][2] * inv, oacc[db][3] * inv);
          *reinterpret_cast<u32x2*>(O + row * D + 16 * db + 4 * g4) = pr;
        }
        if (LSE != nullptr && g4 == 0) LSE[row] = lse;
      } else {
        const size_t row =
            ((size_t)wg + (size_t)cur.b * Hkv + cur.g) * G + c16;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          *reinterpret_cast<f32x4*>(ws_o + row * D + 16 * db + 4 * g4) =
              oacc[db] * inv;
        if (g4 == 0) ws_lse[row] = lse;
      }
    }
    // The range holding a segment's first block records which ranges hold
    // its pieces (one range: finished here).
    if (lane == 0 && cur.a == cur.s0)
      ws_seg[(size_t)cur.b * Hkv + cur.g] =
          int2{wg, rg.owner(cur.s0 + cur.nb - 1)};
    if (!nxt.valid) break;
    cur = nxt;
  }
}

// Combine the pieces of each (sequence, KV head) segment that range
// boundaries cut: M = max lse_i, w_i = exp(lse_i - M),
// o = sum w_i o_i / sum w_i, lse = M + ln(sum w_i).  One workgroup of D
// threads per (sequence, query head).  The split kernel recorded the ranges
// holding the pieces; a segment finished in one range, or a sequence without
// keys, needs nothing here.  Pieces are taken 16 at a time, with their LSEs
// and partial rows all in flight together.
template <typename T, int D, int G>
__global__ __launch_bounds__(D) void attn_decode_combine_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
    const int2* __restrict__ ws_seg, const long long* __restrict__ ws_total,
    T* __restrict__ O, float* __restrict__ LSE, int Hkv, int P) {
  constexpr int TB = 16;
  __shared__ float s_m[TB];
  const int j = blockIdx.x / G, h = blockIdx.x % G;
  const int d = threadIdx.x;
  const int Hq = Hkv * G;
  const int2 sg = ws_seg[j];
  if (sg.x >= sg.y) return;
  const Ranges rg(*ws_total, P);
  const size_t orow = (size_t)(j / Hkv) * Hq + (size_t)(j % Hkv) * G + h;

  float M = -INFINITY, W = 0.f, o = 0.f;
  for (int c0 = sg.x; c0 <= sg.y; c0 += TB) {
    const int n = min(TB, sg.y - c0 + 1);
    // piece d's LSE (empty ranges hold no piece: -inf), and this thread's
    // dimension of all n pieces, issued together
    float lse_d = -INFINITY;
    if (d < n && rg.lo(c0 + d) < rg.lo(c0 + d + 1))
      lse_d = ws_lse[((size_t)(c0 + d) + j) * G + h];
    float v[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t)
      v[t] = t < n ? ws_o[(((size_t)c0 + t + j) * G + h) * D + d] : 0.f;
    __syncthreads();                   // previous round's s_w / s_m read
    if (d < TB) s_m[d] = lse_d;
    __syncthreads();
    float mc = -INFINITY;
#pragma unroll
    for (int t = 0; t < TB; ++t) mc = fmaxf(mc, s_m[t]);
    const float Mn = fmaxf(M, mc);
    const float a = fast_exp2((M - Mn) * kLog2e);       // 0 on first round
    W *= a;
    o *= a;
    M = Mn;
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const float w = fast_exp2((s_m[t] - Mn) * kLog2e);   // 0 when empty
      W += w;
      o = fmaf(w, w > 0.f ? v[t] : 0.f, o);
    }
  }
  O[orow * D + d] = (T)(o / W);
  if (LSE != nullptr && d == 0) LSE[orow] = M + logf(W);
}

}  // namespace attn
