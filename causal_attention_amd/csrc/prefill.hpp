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

#include <climits>
#include <type_traits>

#include "common.hpp"

namespace attn {

#ifdef ATTN_DEBUG_TRACE
// Debug builds only (libattn_debug.so): the online-softmax state of one
// chosen query row after every key tile of the 4-wave and fp32 prefill
// kernels, for comparison with the reference's state at the same key count
// (the debugging practice of the attention-fusion page, section 6.3).
// Record jt of the target row holds {keys covered so far, m in natural-log
// units of the scaled scores, l = sum of exp(s - m) over those keys}.
struct TraceTarget {
  float* buf;      // device, 3 * cap floats; NULL: tracing off
  int b, h, row, cap;
};
__device__ TraceTarget g_trace;

// Called by every lane after tile jt (the exchange of the lane-partial sum
// needs both halves of the wave); only the target row's lane writes.
__device__ __forceinline__ void trace_tile(int b, int h, int row, int hh,
                                           int jt, int keys, float m_log2,
                                           float l_lane) {
  const float l = l_lane + __shfl_xor(l_lane, 32, 64);
  const TraceTarget t = g_trace;
  if (t.buf != nullptr && hh == 0 && b == t.b && h == t.h && row == t.row &&
      jt < t.cap) {
    float* r = t.buf + 3 * (size_t)jt;
    r[0] = (float)keys;
    r[1] = m_log2 * 0.6931471805599453f;
    r[2] = l;
  }
}
#define ATTN_TRACE_TILE(...) trace_tile(__VA_ARGS__)
#else
#define ATTN_TRACE_TILE(...) ((void)0)
#endif

constexpr int kPrefillThreads = 256;   // 4 waves

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

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

// Tile queue (register-blocked kernel, causal launches of several rounds,
// when the caller passes a workspace): each workgroup takes the next work
// index from a counter in the workspace instead of deriving it from its
// block index, and the indices run heaviest tile first with no snake.  A
// compute unit that finishes early, or an XCD that runs faster than the
// others, then takes the next heaviest tile, so the launch is list-scheduled
// longest first over the whole GPU.  With hardware dispatch alone every XCD
// receives a fixed eighth of the blocks: measured on MI355X (B1, 8/2 heads,
// S = 32768), the XCDs of one KV head ran their tiles 4% slower than the
// others and finished up to 90 us after them, and the queue took the launch
// from 1813-1822 to 1720 us.
//
// The counter (64 bits) is zero between launches: the workgroup that draws
// the launch's last index puts it back to zero, by a compare-and-swap that
// succeeds only if nobody has drawn since (every other workgroup of the
// launch has drawn by then).  An index is the draw modulo the block count.
// Whatever the counter held at the start, each launch's draws are then a
// permutation of its blocks: without a reset they are nblocks consecutive
// values; with one, the values drawn before it run from the start value c
// up to nblocks - 1 and those after it from 0 up to c - 1.  A nonzero start
// only rotates the order.
__device__ __forceinline__ int queue_take(unsigned long long* ctr,
                                          unsigned nblocks) {
  const unsigned long long v = __hip_atomic_fetch_add(
      ctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (v == nblocks - 1ull) {
    unsigned long long expected = nblocks;
    __hip_atomic_compare_exchange_strong(ctr, &expected, 0ull,
                                         __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
  }
  return (int)(v % nblocks);
}

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

// The same mask as one per-lane limit compared with immediates: key
// j0 + 8(e/4) + 4 hh + e%4 is dead when it exceeds the last visible key
// (the query row when causal, S - 1 always).  Computing the limit per tile
// keeps the compiler from hoisting sixteen comparisons out of a loop.
// Each element takes -inf through a bit select on the sign of
// lim - offset, so no lane-mask (SGPR) comparisons are kept alive.
template <bool CAUSAL>
__device__ __forceinline__ void apply_mask_lim(f32x16& x, int j0, int hh,
                                               int query, int S) {
  const int last = CAUSAL ? min(query, S - 1) : S - 1;
  const int lim = last - j0 - 4 * hh;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const unsigned dead = (unsigned)((lim - (8 * (e >> 2) + (e & 3))) >> 31);
    // (through a scalar: a bit cast of the vector element itself reads
    // element 0 with this compiler)
    const float xe = x[e];
    const unsigned bits = __builtin_bit_cast(unsigned, xe);
    x[e] = __builtin_bit_cast(float, (bits & ~dead) | (0xff800000u & dead));
  }
}

// apply_mask_lim on elements e0 .. e0+3 only.
template <bool CAUSAL>
__device__ __forceinline__ void apply_mask_lim4(f32x16& x, int e0, int j0,
                                                int hh, int query, int S) {
  const int last = CAUSAL ? min(query, S - 1) : S - 1;
  const int lim = last - j0 - 4 * hh;
#pragma unroll
  for (int e = e0; e < e0 + 4; ++e) {
    const unsigned dead = (unsigned)((lim - (8 * (e >> 2) + (e & 3))) >> 31);
    const float xe = x[e];
    const unsigned bits = __builtin_bit_cast(unsigned, xe);
    x[e] = __builtin_bit_cast(float, (bits & ~dead) | (0xff800000u & dead));
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

// Load i of a wave's run (see lds_buffer_load16_run) on its own: M0 = l,
// immediate offset i*1024 on both addresses.
template <int I>
__device__ __forceinline__ void lds_buffer_load16_at(const u32x4& rsrc,
                                                     unsigned voff,
                                                     unsigned soff, void* l) {
  const unsigned m = __builtin_amdgcn_readfirstlane(lds_addr(l));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\t"
               "buffer_load_dwordx4 %0, %2, %3 offen offset:%4 lds"
               :: "v"(voff), "s"(m), "s"(rsrc),
                  "s"(__builtin_amdgcn_readfirstlane(soff)), "i"(I * 1024)
               : "memory", "m0");
}

// s_waitcnt vmcnt(0): this wave's direct-to-LDS loads have landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Residual add and RMSNorm fused into the 16-bit kernels' epilogue (the
// fused RMSNorm-with-residual of the "triton-optimization" page, section
// 3.2, applied to each query row of one head, the next extension named by
// section 6.3 of the attention-fusion page): x = o + residual with o the
// attention row before rounding, y = x / sqrt(mean(x^2) + eps) * w.  y goes
// to O and x back into the residual buffer, both rounded to nearest even.
template <typename T>
struct RmsEpilogue {
  T* resid;        // [B, Hq, S, D]: read, then overwritten with x
  const T* w;      // [D]
  float eps;
};

// The epilogue of one query row in the transposed-output layout shared by
// the 16-bit kernels: the lane holding the row (hh = 0) and its partner in
// the other wave half (hh = 1) hold its D = 32 NDB values between them,
// element 4a + e of accumulator db being dim 32db + 8a + 4hh + e.  acc holds
// the unnormalised output, inv = 1 / l.  Both lanes must call it (the
// squared sums are exchanged); a row past the end (live false) only skips
// memory.  Writes y to O's row and x to the residual's row.
template <typename T, int NDB>
__device__ __forceinline__ void rms_epilogue_row(f32x16 (&acc)[NDB],
                                                 float inv, bool live,
                                                 size_t row, int hh,
                                                 T* __restrict__ O,
                                                 const RmsEpilogue<T>& rms) {
  using E = Elem16<T>;
  typedef T t4 __attribute__((ext_vector_type(4)));
  constexpr int D = NDB * 32;
  T* xrow = rms.resid + row * D;
  float ss = 0.f;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      u32x2 rr = u32x2{};
      if (live)
        rr = *reinterpret_cast<const u32x2*>(xrow + db * 32 + 8 * a + 4 * hh);
      const t4 r4 = __builtin_bit_cast(t4, rr);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = acc[db][4 * a + e] * inv + (float)r4[e];
        acc[db][4 * a + e] = x;
        ss = fmaf(x, x, ss);
      }
    }
  ss += __shfl_xor(ss, 32, 64);
  const float rs = 1.f / sqrtf(ss * (1.f / D) + rms.eps);
  if (!live) return;
  T* orow = O + row * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int col = db * 32 + 8 * a + 4 * hh;
      const t4 w4 = __builtin_bit_cast(t4,
                                       *reinterpret_cast<const u32x2*>(
                                           rms.w + col));
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * a + e];
      u32x2 py, px;
      py[0] = E::pack2(x[0] * rs * (float)w4[0], x[1] * rs * (float)w4[1]);
      py[1] = E::pack2(x[2] * rs * (float)w4[2], x[3] * rs * (float)w4[3]);
      px[0] = E::pack2(x[0], x[1]);
      px[1] = E::pack2(x[2], x[3]);
      *reinterpret_cast<u32x2*>(orow + col) = py;
      *reinterpret_cast<u32x2*>(xrow + col) = px;
    }
}

template <typename T, int D, bool CAUSAL, bool RMS = false>
__global__ __launch_bounds__(kPrefillThreads, 2) void attn_prefill_kernel(
    const T* __restrict__ Q, const T* __restrict__ K,
    const T* __restrict__ V, T* __restrict__ O,
    float* __restrict__ LSE, int B, int Hq, int Hkv, int S_all,
    float scale_log2, int n_qtiles, int n_cu, int use_rope, RopeRates rope,
    const int* __restrict__ cu_seqlens, const int* __restrict__ seq_lens,
    RmsEpilogue<T> rms) {
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
    ATTN_TRACE_TILE(tc.b, tc.hq, query, hh, jt, min((jt + 1) * BN, S), m_i,
                    l_i);
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
  if constexpr (RMS) {
    const bool live = query < S;
    rms_epilogue_row<T, NDB>(oacc, 1.f / l_tot, live,
                             q_row0 + (live ? query : 0), hh, O, rms);
    if (live && LSE != nullptr && hh == 0)
      LSE[q_row0 + query] = (m_i + fast_log2(l_tot)) * kLn2;
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
      LSE[q_row0 + query] =
          (m_i + fast_log2(l_tot)) * kLn2;
  } else if (seq_lens != nullptr && query < S_all) {
    pad_row(query);
  }
}

// ------------------------------------------------- shared helpers

// Keep a value computed before this point: the compiler otherwise sinks
// pure arithmetic past a barrier to the phase that uses it.
template <typename V>
__device__ __forceinline__ void pin(V& v) {
  asm volatile("" : "+v"(v));
}

// s_barrier that the scheduler moves nothing across.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ------------------------------------- register-blocked prefill kernel
//
// One wave per SIMD, each owning 64 query rows as two 32-row blocks, so
// every K or V operand read from LDS feeds two MFMAs (half the LDS traffic
// per MFMA of a 32-row wave).  With a whole SIMD's 512 registers per lane,
// Q and the output accumulators live in the accumulation registers (AGPRs),
// which only MFMAs read; scores, probabilities and the K / V operands are
// VGPRs.  The QK^T products are issued as inline assembly so that the
// scores land in VGPRs (the compiler otherwise puts every MFMA result in
// AGPRs and copies the scores back).  Two forms: four query heads of one KV
// head per 256-thread workgroup (one wave per head, the same 64 rows; one
// workgroup per compute unit), or two waves of one head (128 rows; two
// workgroups per compute unit).
//
// Fixed reference.  Each row keeps the max of its first key tile (every row
// sees it) as the reference m of the online softmax of section 2.2 of the
// attention-fusion page, and never rescales: later probabilities
// p = 2^(x - m) may exceed 1, and O / l and LSE = m + log2 l are exact for
// any reference.  While every score stays below m + h, p < 2^h: h = 15 for
// fp16 probabilities (largest finite value 65504), 32 for bf16 (fp32 sums
// of p v then overflow only for |v| beyond 2^70).  After a pass, a row whose
// sum l went past 2^h makes the workgroup run its tile again with
// m + log2 l, an upper bound of the row's scores (see the pass loop).
// Without a rescale no VALU ever touches the accumulators inside the loop.
//
// Each wave overlaps its own softmax with its MFMAs through a software
// pipeline across 32-key tiles (scores double-buffered); per tile i:
//   A(i): 16 MFMAs of S(i+1) = K(i+1) Q^T, each followed by the
//         exponentials of one pair of scores of tile i and the packing of
//         the previous pair; the loads of K(i+5) and V(i+4) spread over
//         the slots
//   B(i): 16 MFMAs of O^T += V(i)^T P(i)^T, each followed by a slice of the
//         row sums of P(i), of the mask of S(i+1) (last tiles only) and of
//         x(i+1) = S(i+1) c - m; the V(i+1) and K(i+2) operand reads
// then a wait for this wave's loads of the tiles read next, an LDS wait and
// one barrier (every wave's loads visible, every wave's reads of the ring
// slots about to be refilled done).
//
// The QK^T products being assembly, the wait states the hardware needs
// between their results and a VALU read are inserted here (s_nop), with
// margin over what the compiler emits for the same dependency; the build's
// assembly is checked for AGPR operands rewritten right after such an MFMA.
constexpr int kRBRing = 4;
constexpr int kRBMaxPasses = 8;
// log2 headroom over the reference for probabilities of type T
template <typename T>
constexpr float rb_headroom() {
  return std::is_same<T, _Float16>::value ? 15.f : 32.f;
}

template <typename T>
struct MfmaAsm;
template <>
struct MfmaAsm<__bf16> {
  // d (VGPR) = a (VGPR) b (AGPR), and d += a b
  static __device__ __forceinline__ void qk0(f32x16& d, const u32x4& a,
                                             const u32x4& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                 : "=&v"(d) : "v"(a), "a"(b));
  }
  static __device__ __forceinline__ void qk(f32x16& d, const u32x4& a,
                                            const u32x4& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                 : "+v"(d) : "v"(a), "a"(b));
  }
};
template <>
struct MfmaAsm<_Float16> {
  static __device__ __forceinline__ void qk0(f32x16& d, const u32x4& a,
                                             const u32x4& b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0"
                 : "=&v"(d) : "v"(a), "a"(b));
  }
  static __device__ __forceinline__ void qk(f32x16& d, const u32x4& a,
                                            const u32x4& b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0"
                 : "+v"(d) : "v"(a), "a"(b));
  }
};

// Wait states after an MFMA result before a VALU reads it (19).  The two
// score blocks the assembly MFMAs wrote pass through the statement: every
// read of them then depends on it (none is scheduled above the wait), and
// their registers hold them until it, so no other value is placed there
// while the MFMAs, unseen by the compiler, still write back.
__device__ __forceinline__ void mfma_to_valu_wait(f32x16& s0, f32x16& s1) {
  asm volatile("s_nop 15\n\ts_nop 2" : "+v"(s0), "+v"(s1));
}

// Balanced causal schedule of the four-heads form, for launches whose
// 64-row query tiles all run at once (one workgroup per compute unit).
// Query tile t needs n_t key tiles, growing with t, so with one tile per
// compute unit the launch lasts as long as its last tile.  Instead tiles
// l and nq-1-l are paired and their n_l + n_h key tiles are cut about
// evenly between two workgroups: A runs key tiles 0 .. c-1 of the heavy
// tile h, c = (n_h - n_l) / 2 - kRBCutShift (at least 0; A's fixed costs are
// the larger), leaves that partial state (unnormalised O, reference
// m, row sums l, lane by lane) in the workspace and then runs tile l whole;
// B runs key tiles c .. n_h-1 of tile h and merges A's part into its own
// before it writes tile h (two key ranges of one row merged with their
// maxima and sums, as in section 4.4 of the attention-fusion page).  With
// nq odd the middle tile runs alone: its key tiles equal half a pair's.
//
// Hand-off: flag word p of the workspace is 0 between launches.  A writes
// its part, waits until the stores are acknowledged, then sets the flag
// 0 -> 1.  B polls it for a bounded time; on time-out it sets 0 -> 2 and
// runs tile h whole itself, and A, finding 2, puts back 0.  Both compare-
// and-swaps hit the same word, so exactly one of the two orders happens,
// and in each the flag ends 0: no workgroup ever waits without bound and
// the next launch starts from zeros.  Part and flag travel with
// device-coherent (agent-scope) accesses, which bypass the per-XCD L2s
// (A and B may sit on different XCDs), instead of a release / acquire pair,
// whose L2 write-back and invalidation cost several microseconds each.
// Device-coherent 16-byte stores and loads (agent scope: past the per-XCD
// L2, to the level all XCDs share), as assembly: the compiler has no
// 16-byte atomic access.  The store ends with a wait state, so that its
// data registers may be rewritten at once.
__device__ __forceinline__ void coherent_store16(float* p, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1"
               :
               : "v"(p), "v"(v)
               : "memory");
}
// Sixteen device-coherent 16-byte loads, chunk c (c = 0 .. 15) at
// p + c * 1024 bytes, and the wait for all of them in one statement (no
// result register is read or copied before its data has arrived); the
// second form also loads chunk 16 from q.
__device__ __forceinline__ void coherent_load16x16(f32x4 (&v)[16],
                                                   const float* p) {
  const char* b = reinterpret_cast<const char*>(p);
  asm volatile(
      "global_load_dwordx4 %0, %16, off offset:0 sc1\n\tglobal_load_dwordx4 %1, %16, off offset:1024 sc1\n\tglobal_load_dwordx4 %2, %16, off offset:2048 sc1\n\tglobal_load_dwordx4 %3, %16, off offset:3072 sc1\n\tglobal_load_dwordx4 %4, %17, off offset:0 sc1\n\tglobal_load_dwordx4 %5, %17, off offset:1024 sc1\n\tglobal_load_dwordx4 %6, %17, off offset:2048 sc1\n\tglobal_load_dwordx4 %7, %17, off offset:3072 sc1\n\tglobal_load_dwordx4 %8, %18, off offset:0 sc1\n\tglobal_load_dwordx4 %9, %18, off offset:1024 sc1\n\tglobal_load_dwordx4 %10, %18, off offset:2048 sc1\n\tglobal_load_dwordx4 %11, %18, off offset:3072 sc1\n\tglobal_load_dwordx4 %12, %19, off offset:0 sc1\n\tglobal_load_dwordx4 %13, %19, off offset:1024 sc1\n\tglobal_load_dwordx4 %14, %19, off offset:2048 sc1\n\tglobal_load_dwordx4 %15, %19, off offset:3072 sc1\n\ts_waitcnt vmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]),
        "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]),
        "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]),
        "=&v"(v[14]), "=&v"(v[15])
      : "v"(b), "v"(b + 4096), "v"(b + 8192), "v"(b + 12288)
      : "memory");
}
__device__ __forceinline__ void coherent_load16x17(f32x4 (&v)[17],
                                                   const float* p,
                                                   const float* q) {
  const char* b = reinterpret_cast<const char*>(p);
  asm volatile(
      "global_load_dwordx4 %0, %17, off offset:0 sc1\n\tglobal_load_dwordx4 %1, %17, off offset:1024 sc1\n\tglobal_load_dwordx4 %2, %17, off offset:2048 sc1\n\tglobal_load_dwordx4 %3, %17, off offset:3072 sc1\n\tglobal_load_dwordx4 %4, %18, off offset:0 sc1\n\tglobal_load_dwordx4 %5, %18, off offset:1024 sc1\n\tglobal_load_dwordx4 %6, %18, off offset:2048 sc1\n\tglobal_load_dwordx4 %7, %18, off offset:3072 sc1\n\tglobal_load_dwordx4 %8, %19, off offset:0 sc1\n\tglobal_load_dwordx4 %9, %19, off offset:1024 sc1\n\tglobal_load_dwordx4 %10, %19, off offset:2048 sc1\n\tglobal_load_dwordx4 %11, %19, off offset:3072 sc1\n\tglobal_load_dwordx4 %12, %20, off offset:0 sc1\n\tglobal_load_dwordx4 %13, %20, off offset:1024 sc1\n\tglobal_load_dwordx4 %14, %20, off offset:2048 sc1\n\tglobal_load_dwordx4 %15, %20, off offset:3072 sc1\n\tglobal_load_dwordx4 %16, %21, off sc1\n\ts_waitcnt vmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]),
        "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]),
        "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]),
        "=&v"(v[14]), "=&v"(v[15]), "=&v"(v[16])
      : "v"(b), "v"(b + 4096), "v"(b + 8192), "v"(b + 12288), "v"(q)
      : "memory");
}

struct SplitCoord {
  int b, g, hgrp, pair, role;   // role 0: A, 1: B, 2: the middle tile alone
};

// Workgroups walk (batch, KV head) fastest, then head groups of that KV
// head, then pair slots (A and B of a pair adjacent).
__device__ __forceinline__ SplitCoord split_coord(int bid, int B, int Hgrp,
                                                  int Hkv, int nq) {
  const int P = B * Hkv;
  const int bg = bid % P;
  const int rest = bid / P;
  const int Gg = Hgrp / Hkv;
  SplitCoord c;
  c.b = bg / Hkv;
  c.g = bg % Hkv;
  c.hgrp = c.g * Gg + rest % Gg;
  const int slot = rest / Gg;
  c.pair = slot >> 1;
  c.role = ((nq & 1) && slot == nq - 1) ? 2 : (slot & 1);
  return c;
}

// Causal key tiles (32 keys) of 64-row query tile t.
__host__ __device__ __forceinline__ int rb_causal_tiles(int t, int S) {
  const int hi = 64 * t + 64 < S ? 64 * t + 64 : S;
  return (hi + 31) / 32;
}

// Workspace of the balanced schedule: a fixed region of flag words (one
// per pair, at most kRBMaxPairs; the same place for every launch, so one
// workspace serves launches of any sizes), then per pair, wave and 16-byte
// chunk (32 of O, one of m and l) the 64 lanes' values.
constexpr int kRBDumpChunks = 33;
// Key tiles moved from A's share of the heavy tile to B's: besides its key
// tiles, A pays a second job start and its part's stores (about 6 us on
// MI355X), B the wait and the merge (about 4 us), so an even cut leaves A
// last.  Measured on the batch-4 seq-2048 launch (bf16, 8/2 heads): shifts
// 0 / 1 / 2 / 3 / 4 ran 52.4 / 51.3 / 51.0 / 51.6 / 52.3 us mean.
constexpr int kRBCutShift = 2;
constexpr int kRBFlagBytes = 4096;
constexpr int kRBMaxPairs = kRBFlagBytes / 4;
__host__ __device__ __forceinline__ size_t rb_split_bytes(long long np) {
  return (size_t)kRBFlagBytes + (size_t)np * 4 * kRBDumpChunks * 64 * 16;
}

// GQ = 1: one query head per workgroup, 2 waves x 64 rows (128-row query
// tiles, two workgroups per compute unit).  GQ = 4: four query heads of one
// KV head per workgroup, one wave per head on the same 64 rows (64-row
// query tiles, one workgroup per compute unit): every K / V tile loaded
// into LDS feeds 256 query rows instead of 128, and all waves share one
// causal diagonal.
template <typename T, int D, bool CAUSAL, int GQ, bool SPLIT = false,
          bool RMS = false>
__global__ __launch_bounds__(GQ == 4 ? 256 : 128, GQ == 4 ? 1 : 2)
void attn_prefill_rb_kernel(
    const T* __restrict__ Q, const T* __restrict__ K,
    const T* __restrict__ V, T* __restrict__ O,
    float* __restrict__ LSE, int B, int Hq, int Hkv, int S_all,
    float scale_log2, int n_qtiles, int n_cu, int use_rope, RopeRates rope,
    const int* __restrict__ cu_seqlens, const int* __restrict__ seq_lens,
    void* __restrict__ ws, int wait_ticks, RmsEpilogue<T> rms) {
  static_assert(D == 128, "64 rows per wave at head dim 128");
  static_assert(!(RMS && SPLIT), "the fused epilogue has no split form");
  static_assert(GQ == 1 || GQ == 4, "heads per workgroup");
  static_assert(!SPLIT || (GQ == 4 && CAUSAL), "balanced causal schedule");
  constexpr int WAVES = GQ == 4 ? 4 : 2;
  constexpr int BM = GQ == 4 ? 64 : 128;      // query rows per head
  constexpr int TK = 32;                      // keys per tile
  constexpr int KT = D / 16;                  // QK k-steps
  constexpr int NDB = D / 32;                 // PV output blocks
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;               // rows per 1 KB load
  constexpr int TILE = TK * D * 2;            // 8 KB per K (or V) tile
  constexpr int IPW = TILE / 1024 / WAVES;    // loads per wave and tile
  constexpr int NB = kRBRing;
  constexpr int SLOT = 2 * TILE;
  using E = Elem16<T>;
  using M = MfmaAsm<T>;
  typedef typename E::x8 x8;

  __shared__ __attribute__((aligned(1024))) unsigned char smem[NB * SLOT];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r = lane & 31, hh = lane >> 5;
  // (batch, KV head, head group, query tile); this wave's query head.  The
  // balanced schedule (SPLIT) takes dense inputs without RoPE.
  const unsigned long long t_start =
      SPLIT ? __builtin_amdgcn_s_memrealtime() : 0ull;
  if constexpr (SPLIT) {
    use_rope = 0;
    cu_seqlens = nullptr;
    seq_lens = nullptr;
  }
  TileCoord tc;
  SplitCoord sc{};
  if constexpr (SPLIT) {
    sc = split_coord(blockIdx.x, B, Hq / GQ, Hkv, n_qtiles);
    tc.b = sc.b;
    tc.g = sc.g;
    tc.hq = sc.hgrp;
    tc.qt = sc.pair;
  } else if (ws != nullptr) {
    // tile queue: dense causal launches only (the host passes no workspace
    // to the other forms of this kernel)
    __shared__ int s_idx;
    if (tid == 0)
      s_idx = queue_take(static_cast<unsigned long long*>(ws), gridDim.x);
    __syncthreads();
    tc = tile_coord(s_idx, gridDim.x, B, Hq / GQ, Hkv, n_qtiles, INT_MAX);
  } else {
    tc = tile_coord(blockIdx.x, gridDim.x, B, Hq / GQ, Hkv, n_qtiles, n_cu);
  }
  const int hq = tc.hq * GQ + (GQ == 4 ? w : 0);

  int S = S_all;
  size_t q_row0 = (size_t)(tc.b * Hq + hq) * S_all;
  size_t kv_row0 = (size_t)(tc.b * Hkv + tc.g) * S_all;
  if (cu_seqlens != nullptr) {
    const int c0 = cu_seqlens[tc.b];
    S = cu_seqlens[tc.b + 1] - c0;
    if (tc.qt * BM >= S) return;
    q_row0 = (size_t)c0 * Hq + (size_t)hq * S;
    kv_row0 = (size_t)c0 * Hkv + (size_t)tc.g * S;
  } else if (seq_lens != nullptr) {
    S = min(max(seq_lens[tc.b], 0), S_all);
  }
  // o = 0, lse = -inf for a padding row (one half row per lane half).
  auto pad_row = [&](int row) {
    T* orow = O + (q_row0 + row) * D + hh * (D / 2);
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      *reinterpret_cast<u32x4*>(orow + 8 * c) = u32x4{};
    if (LSE != nullptr && hh == 0) LSE[q_row0 + row] = -INFINITY;
  };
  if (seq_lens != nullptr && tc.qt * BM >= S) {
    const int wq = tc.qt * BM + (GQ == 4 ? 0 : 64 * w);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      if (wq + 32 * rb + r < S_all) pad_row(wq + 32 * rb + r);
    return;
  }
  const T* Qp = Q + q_row0 * D;

  // The current job: query tile q_lo / BM against key tiles
  // kbase / TK .. kbase / TK + n - 1 (all tiles counted from kbase on).
  int q_lo = 0, wq0 = 0;      // first row of the tile, of this wave
  int kbase = 0, n = 0;       // first key, key tiles (>= 1)
  int n_full = 0;             // leading tiles that need no mask
  int n_plain = 0;            // ... whose loads five tiles on are full
  int s_rel = 0, jmax = 0;    // keys from kbase on, last tile holding keys
  u32x4 krs, vrs;             // K, V from row kbase of this KV head
  u32x4 qB[2][KT];            // Q^T B operands of both row blocks (AGPRs)
  auto setup_job = [&](int qt, int jlo, int jhi) {
    q_lo = qt * BM;
    wq0 = q_lo + (GQ == 4 ? 0 : 64 * w);
    const int q_hi = min(S, q_lo + BM);
    const int n_abs = ((CAUSAL ? q_hi : S) + TK - 1) / TK;
    kbase = jlo * TK;
    n = min(jhi, n_abs) - jlo;
    s_rel = S - kbase;
    const int s_tiles = s_rel / TK;
    n_full = max(0, min(min(n, s_tiles), CAUSAL ? (q_lo + 1) / TK - jlo : n));
    n_plain = min(n_full, s_tiles - 5);
    jmax = (s_rel - 1) / TK;
    krs = buffer_rsrc(K + (kv_row0 + kbase) * D);
    vrs = buffer_rsrc(V + (kv_row0 + kbase) * D);
  };
  // Q^T operands of the job's rows, loaded before the job's first K / V
  // loads.  Loaded later, inside the pass, the compiler no longer keeps
  // them in their own AGPRs for the whole job but copies each into a
  // shared one right after the (assembly) MFMA that read the previous one.
  auto load_q = [&]() {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int query = wq0 + 32 * rb + r;
      x8 qv[KT];
#pragma unroll
      for (int t = 0; t < KT; ++t)
        qv[t] = query < S ? *reinterpret_cast<const x8*>(
                                Qp + (size_t)query * D + 16 * t + 8 * hh)
                          : x8{};
      if (use_rope) {
#pragma unroll
        for (int t = 0; t < KT / 2; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float x1 = (float)qv[t][e], x2 = (float)qv[t + KT / 2][e];
            const double rr =
                hh ? rope.r[16 * t + 8 + e] : rope.r[16 * t + e];
            rope_pair(x1, x2, query, rr);
            qv[t][e] = (T)x1;
            qv[t + KT / 2][e] = (T)x2;
          }
      }
#pragma unroll
      for (int t = 0; t < KT; ++t)
        qB[rb][t] = __builtin_bit_cast(u32x4, qv[t]);
    }
  };

  // Direct loads: wave w fills 1 KB blocks IPW w .. IPW w + IPW-1 of a tile.
  unsigned koffr[IPW], voffr[IPW];
#pragma unroll
  for (int ii = 0; ii < IPW; ++ii) {
    const int row = (w * IPW + ii) * RPI + lane / CPR, pos = lane % CPR;
    koffr[ii] = (row * D + 8 * swz_k<CPR>(row, pos)) * 2 - ii * 1024;
    voffr[ii] = (row * D + 8 * swz_v<CPR>(row, pos)) * 2 - ii * 1024;
  }
  // Load II of this wave's share of K (kv = 0) or V (kv = 1) tile j of the
  // job (key tile kbase / TK + j) into ring slot j % NB.  A tile past the
  // last one holding keys loads that one instead (its slot is not read
  // again); rows past S load row S - 1 (their scores are masked).
  auto issue1 = [&](int kv, int j, auto ii_c, auto full_c) {
    constexpr int II = decltype(ii_c)::value;
    if constexpr (decltype(full_c)::value) {   // tile j known full
      unsigned char* dst = smem + (j % NB) * SLOT + kv * TILE + w * IPW * 1024;
      lds_buffer_load16_at<II>(kv ? vrs : krs, kv ? voffr[II] : koffr[II],
                               (unsigned)j * (TK * D * 2), dst);
      return;
    }
    const int j0 = min(j, jmax) * TK;
    const unsigned soff = (unsigned)j0 * D * 2;
    unsigned char* dst = smem + (j % NB) * SLOT + kv * TILE + w * IPW * 1024;
    const u32x4& rs = kv ? vrs : krs;
    const unsigned voff = kv ? voffr[II] : koffr[II];
    if (j0 + TK <= s_rel) {
      lds_buffer_load16_at<II>(rs, voff, soff, dst);
    } else {
      const int row = (w * IPW + II) * RPI + lane / CPR;
      const int back = (min(j0 + row, s_rel - 1) - (j0 + row)) * D * 2;
      lds_buffer_load16(rs, voff + II * 1024 + back, soff, dst + II * 1024);
    }
  };
  auto issue = [&](int kv, int j) {
    static_for<IPW>([&](auto ii) { issue1(kv, j, ii, std::false_type{}); });
  };

  u32x4 kreg[KT];                      // K operands of the next QK
  u32x4 vop[2][2 * NDB];               // V operands, double-buffered
  const int grp = lane >> 4, jl = lane & 15;
  const int vrow_off = 4 * (grp >> 1) + (jl >> 2);
  const int vcol_off = 16 * (grp & 1) + 4 * (jl & 3);
  auto read_k1 = [&](auto slot_c, int t) {
    constexpr int SL = decltype(slot_c)::value;
    kreg[t] = *reinterpret_cast<const u32x4*>(
        smem + SL * SLOT + (r * D + 8 * swz_k<CPR>(r, 2 * t + hh)) * 2);
  };
  // Half h (keys 8h .. 8h+7 of its k-step) of V operand x (k-step x / NDB,
  // output block x % NDB) of slot SL.
  auto read_vh = [&](auto slot_c, auto buf_c, int x, int h) {
    constexpr int SL = decltype(slot_c)::value;
    constexpr int VB = decltype(buf_c)::value;
    const T* Vt = reinterpret_cast<const T*>(smem + SL * SLOT + TILE);
    const int u = x / NDB, db = x % NDB;
    const int row = u * 16 + vrow_off + 8 * h;
    const int col = db * 32 + vcol_off;
    const int c = col >> 3, e = col & 7;
    const u32x2 v = lds_read_tr16(Vt + row * D + 8 * swz_v<CPR>(row, c) + e);
    vop[VB][x][2 * h] = v[0];
    vop[VB][x][2 * h + 1] = v[1];
  };

  f32x16 oacc[2][NDB];
  float m_ref[2], l_i[2];
  f32x16 sbuf[2][2];                   // [buffer][row block]
  u32x4 pP[2][2];                      // [row block][k-step], packed pairs

  // QK^T slot s of a tile: k-step s/2 of row block s%2 (consecutive slots
  // are independent MFMAs; a row block's chain advances every other slot).
  auto qk_slot = [&](auto buf_c, int s) {
    constexpr int SB = decltype(buf_c)::value;
    const int t = s >> 1, rb = s & 1;
    if (t == 0) M::qk0(sbuf[SB][rb], kreg[0], qB[rb][0]);
    else M::qk(sbuf[SB][rb], kreg[t], qB[rb][t]);
  };
  // Causal / tail mask of elements e0 .. e0+3 of row block rb of buffer SB
  // for key tile i.
  auto mask4 = [&](auto buf_c, int rb, int e0, int i) {
    constexpr int SB = decltype(buf_c)::value;
    apply_mask_lim4<CAUSAL>(sbuf[SB][rb], e0, kbase + i * TK, hh,
                            wq0 + 32 * rb + r, S);
  };
  // Row max (log2 domain) of one row block of buffer SB.
  auto rowmax = [&](auto buf_c, int rb) {
    constexpr int SB = decltype(buf_c)::value;
    const f32x16& sv = sbuf[SB][rb];
    float t0 = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
    float t1 = fmaxf(fmaxf(sv[3], sv[4]), sv[5]);
    float t2 = fmaxf(fmaxf(sv[6], sv[7]), sv[8]);
    float t3 = fmaxf(fmaxf(sv[9], sv[10]), sv[11]);
    float t4 = fmaxf(fmaxf(sv[12], sv[13]), sv[14]);
    const float mx =
        fmaxf(fmaxf(fmaxf(t0, t1), t2), fmaxf(fmaxf(t3, t4), sv[15]));
    return max_halves(mx) * scale_log2;
  };
  // x = s c - m for elements e0 .. e0+3 of row block rb.
  auto fma4 = [&](auto buf_c, int rb, int e0, float neg_m) {
    constexpr int SB = decltype(buf_c)::value;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      sbuf[SB][rb][e0 + e] = fmaf(sbuf[SB][rb][e0 + e], scale_log2, neg_m);
  };
  // Pair p of a tile: elements 2(p%8), 2(p%8)+1 of row block p/8.  The
  // probabilities replace the scores in place (summed into l later).
  auto exp_pair = [&](auto buf_c, int p, float& e0, float& e1) {
    constexpr int SB = decltype(buf_c)::value;
    const int rb = p >> 3, e = 2 * (p & 7);
    e0 = sbuf[SB][rb][e] = fast_exp2(sbuf[SB][rb][e]);
    e1 = sbuf[SB][rb][e + 1] = fast_exp2(sbuf[SB][rb][e + 1]);
  };
  auto use_pair = [&](int p, float e0, float e1) {
    const int rb = p >> 3, e = 2 * (p & 7);
    pP[rb][e >> 3][(e & 7) >> 1] = E::pack2(e0, e1);
  };
  // l += pair p of buffer SB (fp32 probabilities).
  auto sum_pair = [&](auto buf_c, int p) {
    constexpr int SB = decltype(buf_c)::value;
    const int rb = p >> 3, e = 2 * (p & 7);
    l_i[rb] = (l_i[rb] + sbuf[SB][rb][e]) + sbuf[SB][rb][e + 1];
  };

  // One pass over the key tiles with reference m_ref: each row's first-tile
  // max in pass 0, the bound computed after the previous pass otherwise.
  using B0 = std::integral_constant<int, 0>;
  auto run_pass = [&](int pass, const float (&m_next)[2]) {
    // ---- prologue: K0 K1 V0 K2 V1 K3 V2 V3 in flight, then S(0), then K4
    // into K0's slot; K(1) and V(0) in registers.  From here on tile t
    // loads K(t+5) and V(t+4) (every load is issued, past the end too, so
    // the counts of loads in flight are fixed).
    issue(0, 0);
    issue(0, 1);
    issue(1, 0);
    issue(0, 2);
    issue(1, 1);
    issue(0, 3);
    issue(1, 2);
    issue(1, 3);
    wait_vmem_le<7 * IPW>();                  // K0
    __syncthreads();
#pragma unroll
    for (int t = 0; t < KT; ++t) read_k1(B0{}, t);
#pragma unroll
    for (int s = 0; s < 16; ++s) qk_slot(B0{}, s);
    mfma_to_valu_wait(sbuf[0][0], sbuf[0][1]);
    if (0 >= n_full) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int e0 = 0; e0 < 16; e0 += 4) mask4(B0{}, rb, e0, 0);
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      m_ref[rb] = pass == 0 ? rowmax(B0{}, rb) : m_next[rb];
#pragma unroll
      for (int e0 = 0; e0 < 16; e0 += 4) fma4(B0{}, rb, e0, -m_ref[rb]);
      l_i[rb] = 0.f;
    }
    // K(1), V(0) now; K(2), V(1) in the first tile
    wait_vmem_le<3 * IPW>();                  // K1, V0, K2, V1
    __syncthreads();
    issue(0, 4);
#pragma unroll
    for (int x = 0; x < 2 * NDB; ++x) {
      read_vh(B0{}, B0{}, x, 0);
      read_vh(B0{}, B0{}, x, 1);
    }
#pragma unroll
    for (int t = 0; t < KT; ++t)
      read_k1(std::integral_constant<int, 1>{}, t);   // stale when n == 1
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[rb][db] = f32x16{};

    // ---- main loop (unrolled by the ring size so slots are immediates).
    // Each MFMA is followed by at most about one MFMA's duration of VALU
    // work: a second MFMA issued while the first still runs stalls the
    // wave, and with it the VALU work queued behind it.  The loads of a
    // tile are spread over its QK slots: issued back to back, they stall
    // the wave for several hundred cycles.
    // FULL: the tiles this one loads (K(i+5), V(i+3)) are full tiles.
    auto tile = [&](auto u_c, auto masked_c, auto full_c, int i) {
      constexpr int U = decltype(u_c)::value;
      constexpr bool MASKED = decltype(masked_c)::value;
      using Bc = std::integral_constant<int, U & 1>;
      using Bn = std::integral_constant<int, (U + 1) & 1>;
      using Vn = std::integral_constant<int, (U + 1) & 1>;
      using Sv = std::integral_constant<int, (U + 1) % NB>;
      using Sk = std::integral_constant<int, (U + 2) % NB>;
      // A(i): 16 QK MFMAs of S(i+1), each followed by the exponentials of
      // one pair of scores of tile i and the packing of the previous pair;
      // 2 IPW evenly spaced ones also by this wave's loads of K(i+5) and
      // V(i+4).
      float pe0, pe1;
      exp_pair(Bc{}, 0, pe0, pe1);
      static_for<16>([&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
        qk_slot(Bn{}, s);                      // stale on the last tile
        __builtin_amdgcn_sched_barrier(0);
        float ne0 = 0.f, ne1 = 0.f;
        if (s + 1 < 16) exp_pair(Bc{}, s + 1, ne0, ne1);
        use_pair(s, pe0, pe1);
        pe0 = ne0;
        pe1 = ne1;
        constexpr int GAP = 16 / (2 * IPW);     // slots per load
        if constexpr (s % GAP == GAP - 1) {
          constexpr int q = s / GAP;
          if constexpr (q < IPW)
            issue1(0, i + 5, std::integral_constant<int, q>{}, full_c);
          else
            issue1(1, i + 4, std::integral_constant<int, q - IPW>{}, full_c);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        pin(sbuf[U & 1][rb]);
        pin(pP[rb][0]);
        pin(pP[rb][1]);
      }
      // B(i): 16 PV MFMAs (V operands read in the previous tile), each
      // followed by a slice of the row sums of P(i), of the mask of S(i+1)
      // (tiles that need one) and of x(i+1) = S(i+1) c - m; the first eight
      // by the V(i+1) operand reads, slots 4 .. 11 by the K(i+2) reads.
      const float nm0 = -m_ref[0], nm1 = -m_ref[1];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int u = k >> 3, db = (k >> 1) & 3, rb = k & 1;
        oacc[rb][db] = E::mma32(__builtin_bit_cast(x8, vop[U & 1][u * NDB + db]),
                                __builtin_bit_cast(x8, pP[rb][u]),
                                oacc[rb][db]);
        __builtin_amdgcn_sched_barrier(0);
        // S(i+1) complete (the wait overlaps this MFMA)
        if (k == 0) mfma_to_valu_wait(sbuf[(U + 1) & 1][0],
                                      sbuf[(U + 1) & 1][1]);
        // LDS reads end by slot 11, so that the wait for them before the
        // barrier finds them done
        if (k < 8) {
          read_vh(Sv{}, Vn{}, k, 0);            // stale at the end
          read_vh(Sv{}, Vn{}, k, 1);
        }
        if (k >= 4 && k < 12) read_k1(Sk{}, k - 4);   // stale at the end
        sum_pair(Bc{}, k);
        if constexpr (MASKED) {
          if (k >= 1 && k < 9) {
            const int j = k - 1;               // 8 slices of 4 elements
            mask4(Bn{}, j >> 2, 4 * (j & 3), i + 1);
          }
          if (k >= 8) {
            const int j = k - 8;
            fma4(Bn{}, j >> 2, 4 * (j & 3), (j >> 2) ? nm1 : nm0);
          }
        } else {
          if (k >= 1 && k < 9) {
            const int j = k - 1;
            fma4(Bn{}, j >> 2, 4 * (j & 3), (j >> 2) ? nm1 : nm0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        pin(l_i[rb]);
        pin(sbuf[(U + 1) & 1][rb]);
      }
      // Before the barrier: this wave's loads of the tiles read next
      // (V(i+2), K(i+3), issued two tiles ago; the loads of the last two
      // tiles may still run) have landed and its LDS reads of V(i+1) and
      // K(i+2) are complete; after it, their slots may be refilled.
      wait_vmem_le<4 * IPW>();
      __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0)
      wg_barrier();
    };
    // Tiles whose successor needs no mask and whose loads are full tiles
    // run in a loop without mask or tail code; the last few (the diagonal,
    // a ragged tail, loads past the end) in one that always masks, so that
    // no branch in either loop rewrites the scores.
    static_assert(NB == 4, "the loop is unrolled by the ring size");
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;
    using Plain = std::false_type;
    using Masked = std::true_type;
    using Full = std::true_type;
    using Any = std::false_type;
    int it = 0;
    for (; it + 4 < n_plain; it += 4) {
      tile(C0{}, Plain{}, Full{}, it);
      tile(C1{}, Plain{}, Full{}, it + 1);
      tile(C2{}, Plain{}, Full{}, it + 2);
      tile(C3{}, Plain{}, Full{}, it + 3);
    }
    for (; it < n; it += 4) {
      tile(C0{}, Masked{}, Any{}, it);
      if (it + 1 < n) tile(C1{}, Masked{}, Any{}, it + 1);
      if (it + 2 < n) tile(C2{}, Masked{}, Any{}, it + 2);
      if (it + 3 < n) tile(C3{}, Masked{}, Any{}, it + 3);
    }
    wait_vmem();
  };
  // Passes.  After a pass, a row whose sum l outgrew 2^h (or overflowed
  // fp32) had a probability above the headroom: the workgroup runs its tile
  // again (the two waves agree through LDS; every load has landed and every
  // LDS read is done at the loop's last barrier) with m = m + log2 l, which
  // bounds every score of the row from above (l >= each p), so that p <= 1;
  // after an fp32 overflow (some p >= 2^128 / S), m + 100 is still below the
  // row's max.  Rows within the headroom take the new m as well.
  constexpr float kLimit = (float)(1ull << (int)rb_headroom<T>());
  // The job's passes; at the end every load has landed and every LDS read
  // is done (the loop's last barrier).
  auto run_job = [&]() {
    float m_next[2] = {0.f, 0.f};
    for (int pass = 0; pass < kRBMaxPasses; ++pass) {
      run_pass(pass, m_next);
      bool over = false;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float l_tot = l_i[rb] + swap_halves(l_i[rb]);
        const bool inf = l_tot == INFINITY;
        over = over || inf || l_tot > kLimit;
        m_next[rb] = m_ref[rb] + (inf ? 100.f : fast_log2(l_tot));
      }
      int* flag = reinterpret_cast<int*>(smem);
      const int any = __ballot(over) != 0;    // with every lane active
      if (lane == 0) flag[w] = any;
      __syncthreads();
      int any_w = 0;
#pragma unroll
      for (int x = 0; x < WAVES; ++x) any_w |= flag[x];
      const bool again = any_w != 0;
      __syncthreads();
      if (!again) break;
    }
  };

  // Jobs: the whole tile, or under the balanced schedule A's part of the
  // heavy tile (kept in the workspace) and then the light tile, B's part of
  // the heavy tile merged with A's, or the middle tile.
  enum { kFinal = 0, kPart = 1, kMerge = 2 };
  int jq = tc.qt, jlo = 0, jhi = 1 << 30, jmode = kFinal;
  // pair index, heavy tile, flag words and this lane's part of the pair
  // (the SPLIT instantiation only; ws is non-null there)
  const int np_bg = n_qtiles / 2;       // pairs per (batch, head group)
  const int pidx = (sc.b * (Hq / GQ) + sc.hgrp) * np_bg + sc.pair;
  const int qt_h = n_qtiles - 1 - sc.pair;
  int* const flags = static_cast<int*>(ws);
  // wave-uniform base (scalar registers); value q of chunk c of lane l at
  // (c * 64 + l) * 4 + q
  float* const dump = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                               kRBFlagBytes) +
                      ((size_t)pidx * WAVES + w) * (kRBDumpChunks * 64 * 4);
  if constexpr (SPLIT) {
    {
      const int c = sc.role == 2
                        ? 0
                        : max(0, (rb_causal_tiles(qt_h, S) -
                                  rb_causal_tiles(sc.pair, S)) / 2 -
                                     kRBCutShift);
      if (sc.role == 0 && c > 0) {
        jq = qt_h;
        jhi = c;
        jmode = kPart;
      } else if (sc.role == 1) {
        jq = qt_h;
        jlo = c;
        jmode = c > 0 ? kMerge : kFinal;
      }
    }
  }

  while (true) {
    setup_job(jq, jlo, jhi);
    load_q();
    run_job();
    if constexpr (SPLIT) {
      if (jmode == kPart) {
        // A: the part, then flag 0 -> 1 (or 2 -> 0 when B gave up on it).
        // Part and flag are written with device-coherent (agent-scope)
        // accesses, which go past this XCD's L2 to memory, so no cache
        // write-back is needed: every wave waits for its stores to be
        // acknowledged before the barrier, and only then is the flag set.
        // The lane index passes through an empty statement so that the
        // addresses are formed here, not hoisted out of the job loop (33 of
        // them would not fit in registers).
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a)
              coherent_store16(
                  dump + (((rb * NDB + db) * 4 + a) * 64 + ln) * 4,
                  f32x4{oacc[rb][db][4 * a], oacc[rb][db][4 * a + 1],
                        oacc[rb][db][4 * a + 2], oacc[rb][db][4 * a + 3]});
        coherent_store16(dump + (32 * 64 + ln) * 4,
                         f32x4{m_ref[0], m_ref[1], l_i[0], l_i[1]});
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) {
          int expected = 0;
          if (!__hip_atomic_compare_exchange_strong(
                  flags + pidx, &expected, 1, __ATOMIC_RELAXED,
                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            __hip_atomic_store(flags + pidx, 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        jq = sc.pair;
        jlo = 0;
        jhi = 1 << 30;
        jmode = kFinal;
        continue;
      }
      if (jmode == kMerge) {
        // B: wait for A's part, at most twice as long as this workgroup
        // has run so far plus 20 us, or wait_ticks if >= 0 (real-time
        // counter, 100 MHz)
        int* got_s = reinterpret_cast<int*>(smem) + 8;
        if (tid == 0) {
          const unsigned long long now = __builtin_amdgcn_s_memrealtime();
          const unsigned long long deadline =
              now + (wait_ticks >= 0 ? (unsigned long long)wait_ticks
                                     : 2 * (now - t_start) + 2000);
          int got = 0;
          while (true) {
            // device-coherent polls (an acquire would also invalidate the
            // L2 each time)
            if (__hip_atomic_load(flags + pidx, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT) == 1) {
              got = 1;
              break;
            }
            if (__builtin_amdgcn_s_memrealtime() > deadline) {
              int expected = 0;
              got = __hip_atomic_compare_exchange_strong(
                        flags + pidx, &expected, 2, __ATOMIC_RELAXED,
                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                        ? 0
                        : 1;           // A posted meanwhile
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
          if (got)
            __hip_atomic_store(flags + pidx, 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          *got_s = got;
        }
        __syncthreads();
        const int got = __builtin_amdgcn_readfirstlane(*got_s);
        __syncthreads();
        if (!got) {                    // run the heavy tile whole
          jlo = 0;
          jmode = kFinal;
          continue;
        }
        // the part is read with device-coherent loads, issued after the
        // flag was seen (the barrier above), so they see A's stores
        // the part in two batches of loads in flight together: m and l
        // with O chunks 0 .. 15, then chunks 16 .. 31 (addresses formed
        // here, as for the stores)
        int ln = lane;
        asm volatile("" : "+v"(ln));
        float fa[2], fb[2];
        {
          f32x4 part[17];
          coherent_load16x17(part, dump + ln * 4, dump + (32 * 64 + ln) * 4);
          const f32x4 ml = part[16];
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const float mx = fmaxf(ml[rb], m_ref[rb]);
            fa[rb] = fast_exp2(ml[rb] - mx);
            fb[rb] = fast_exp2(m_ref[rb] - mx);
            l_i[rb] = fa[rb] * ml[2 + rb] + fb[rb] * l_i[rb];
            m_ref[rb] = mx;
          }
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const int rb = c >> 4, db = (c >> 2) & 3, a = c & 3;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              oacc[rb][db][4 * a + q] =
                  fa[rb] * part[c][q] + fb[rb] * oacc[rb][db][4 * a + q];
          }
        }
        {
          f32x4 part[16];
          coherent_load16x16(part, dump + (16 * 64 + ln) * 4);
#pragma unroll
          for (int c = 16; c < 32; ++c) {
            const int rb = c >> 4, db = (c >> 2) & 3, a = c & 3;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              oacc[rb][db][4 * a + q] = fa[rb] * part[c - 16][q] +
                                        fb[rb] * oacc[rb][db][4 * a + q];
          }
        }
      }
    }
    break;
  }

  // ---- epilogue: O = acc / l, LSE = (m_ref + log2 l) ln 2
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int query = wq0 + 32 * rb + r;
    const float l_tot = l_i[rb] + swap_halves(l_i[rb]);
    if constexpr (RMS) {
      // residual add + RMSNorm (dense launches only)
      const bool live = query < S;
      rms_epilogue_row<T, NDB>(oacc[rb], 1.f / l_tot, live,
                               q_row0 + (live ? query : 0), hh, O, rms);
      if (live && LSE != nullptr && hh == 0)
        LSE[q_row0 + query] = (m_ref[rb] + fast_log2(l_tot)) * kLn2;
      continue;
    }
    if (query < S) {
      const float inv = 1.f / l_tot;
      T* orow = O + (q_row0 + query) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          u32x2 pr;
          pr[0] = E::pack2(oacc[rb][db][4 * a] * inv,
                           oacc[rb][db][4 * a + 1] * inv);
          pr[1] = E::pack2(oacc[rb][db][4 * a + 2] * inv,
                           oacc[rb][db][4 * a + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * a + 4 * hh) = pr;
        }
      if (LSE != nullptr && hh == 0)
        LSE[q_row0 + query] = (m_ref[rb] + fast_log2(l_tot)) * kLn2;
    } else if (seq_lens != nullptr && query < S_all) {
      pad_row(query);
    }
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
    ATTN_TRACE_TILE(tc.b, tc.hq, query, hh, jt, min(j0 + BN, S), m_i, l_i);

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
