// Decode kernels: one query row per sequence against its packed KV cache,
// split over the cache length, then a log-sum-exp combine.
//
// Method ("Attention三算子融合实战：从Triton到CUDA的推理加速优化"): the decode
// setting of section 1.3 (one query row, K and V as long as the history), the
// key split of section 4.4 (large key chunks handled by separate blocks, each
// running the online softmax of section 2.2, merged across blocks
// afterwards), and the partial-buffer-plus-reduce-kernel pattern of
// "手写Triton kernel重构Qwen3.5-0.8B" section 3.3 (a separate small reduce
// kernel rather than atomics).  GQA (section 2.1 of that page): the G = Hq/Hkv
// query heads of one KV head are handled by the same workgroup, so each K/V
// byte is read from HBM once, not once per query head.
//
// gfx950 mapping.  The path is bound by HBM bandwidth (about 4 FLOP per
// byte); the arithmetic is put on v_mfma_f32_16x16x32_bf16 only so that it
// costs almost no issue slots next to the loads.  Each wave takes 32-key
// blocks of its split and keeps the next block's loads in flight while it
// multiplies the current one:
//  * S^T = K Q^T: the A operand is read straight from the cache into VGPRs
//    (lane l holds key l%16 of a 16-key half, 8 consecutive dims), Q^T is the
//    B operand with the G heads as columns (the other columns are zero).  The
//    accumulator leaves lane l with head l%16 and keys 4*(l/16)..+3 of each
//    half.
//  * Those probabilities are re-used as the B operand of O^T = V^T P^T (key
//    slot s of lane group l/16 is key 4*(l/16)+s of half 0 for s < 4, of half
//    1 otherwise), so P never leaves registers.  V goes global -> LDS with
//    gfx950's direct loads into a per-wave double buffer, and the A operand
//    V^T comes from transposed LDS reads (ds_read_b64_tr_b16).
//  * The row max and sum are per head, over the 4 lane groups: two cross-lane
//    exchanges per block.  The running output is rescaled only when the max
//    grows by more than 2^8 (exact: the final division by l cancels any
//    common reference value; the bound keeps p <= 256).
// The waves of a workgroup merge their (m, l, O) through LDS at the end and
// write the split's normalised output and natural-log LSE to the workspace;
// a second small kernel merges the splits of each (sequence, head).  (Doing
// that merge in the last split to finish would need device-scope fences,
// which on this 8-XCD part write back and invalidate a whole L2 per
// workgroup: far slower than one more launch.)
#pragma once

#include "common.hpp"

namespace attn {

constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = 64 * kDecodeWaves;
constexpr int kDecodeBlock = 32;                          // keys per wave step
constexpr int kDecodeMinChunk = kDecodeWaves * kDecodeBlock;

// Keys of split s for a sequence of L keys: [s*chunk, min(L, (s+1)*chunk)),
// chunk a multiple of 32 and at least one block per wave.
__device__ __forceinline__ int decode_chunk(int L, int ns) {
  int c = max((L + ns - 1) / ns, kDecodeMinChunk);
  return (c + kDecodeBlock - 1) / kDecodeBlock * kDecodeBlock;
}

__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(bf16x8 a, bf16x8 b,
                                                    f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Wave-wide sum of a 64-bit value.
__device__ __forceinline__ long long wave_sum64(long long x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Direct global -> LDS load of 16 bytes per lane (lane order in LDS) and
// the transposed LDS read (in each group of 16 lanes, lane j points at 4
// dims of key row j/4; lane i receives dim i of those 4 keys).
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void dec_lds_load16(const void* g, __bf16* l) {
  __builtin_amdgcn_global_load_lds(
      g, (__attribute__((address_space(3))) void*)(l), 16, 0, 0);
}
__device__ __forceinline__ bf16x4 dec_lds_read_tr16(const __bf16* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// V block rows in LDS: 16-byte chunk c of key row r is stored at chunk
// position c ^ f(r), so the 16 rows read by one transposed load hit distinct
// banks (f is even, which keeps chunk pairs together).
template <int D>
__device__ __forceinline__ int dec_swz(int row, int c) {
  return D == 128 ? (c ^ ((row & 7) << 1)) : (c ^ (((row >> 1) & 3) << 1));
}

// One 32-key block of one wave: K in registers as two 16-key MFMA A
// operands; V goes straight to the wave's LDS buffer.
template <int D>
struct DecodeK {
  bf16x8 ka[2][D / 32];
};

// Issue the loads of the block at key j0 (keys >= kend: K reads as zero,
// V rows clamp to the last live key and are multiplied by p = 0).
template <int D>
__device__ __forceinline__ void decode_load(DecodeK<D>& blk, __bf16* vdst,
                                            const __bf16* Kp,
                                            const __bf16* Vp, int j0,
                                            int kend, int lane) {
  constexpr int KT = D / 32;
  constexpr int CPR = D / 8;                 // chunks per row
  constexpr int RPI = 64 / CPR;              // rows per load instruction
  const int c16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const int key = j0 + 16 * kh + c16;
#pragma unroll
    for (int t = 0; t < KT; ++t)
      blk.ka[kh][t] = (key < kend) ? *reinterpret_cast<const bf16x8*>(
                                         Kp + (size_t)key * D + 32 * t + 8 * g4)
                                   : bf16x8{};
  }
#pragma unroll
  for (int i = 0; i < kDecodeBlock / RPI; ++i) {
    const int row = i * RPI + lane / CPR, pos = lane % CPR;
    const int key = min(j0 + row, kend - 1);
    dec_lds_load16(Vp + (size_t)key * D + 8 * dec_swz<D>(row, pos),
                   vdst + i * RPI * D);
  }
}

// s_waitcnt vmcnt(N): at most N vector-memory loads of this wave in flight.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Online-softmax step of one wave over one 32-key block whose V rows are in
// vsrc (its loads are the only ones this wave has in flight).
template <int D>
__device__ __forceinline__ void decode_step(const DecodeK<D>& blk,
                                            const bf16x8 (&qB)[D / 32],
                                            const __bf16* vsrc, int j0,
                                            int kend, int lane, float c,
                                            float& m_ref, float& l_i,
                                            f32x4 (&oacc)[D / 16]) {
  constexpr int KT = D / 32;
  constexpr int NDB = D / 16;
  const int c16 = lane & 15, g4 = lane >> 4;

  f32x4 sacc[2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    sacc[kh] = f32x4{};
#pragma unroll
    for (int t = 0; t < KT; ++t)
      sacc[kh] = mfma_16x16x32_bf16(blk.ka[kh][t], qB[t], sacc[kh]);
  }
  // lane holds head c16, keys j0 + 16kh + 4g4 + i (raw q.k; masked = -inf)
  float x[8];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = j0 + 16 * kh + 4 * g4 + i;
      x[4 * kh + i] = (key < kend) ? sacc[kh][i] : -INFINITY;
    }
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
  if (mx > m_ref + kLazyRescale) {
    // new reference (taken on the first block with a live key: m_ref is
    // -inf there and the rescale factor is 0)
    const float alpha = fast_exp2(m_ref - mx);
    l_i *= alpha;
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;
    m_ref = mx;
  }
  const float neg_m = (m_ref == -INFINITY) ? 0.f : -m_ref;
  bf16x8 pB;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = fast_exp2(fmaf(x[i], c, neg_m));
    l_i += p;
    pB[i] = (__bf16)p;
  }

  wait_vmem_le<0>();               // this block's V rows have landed
  // O^T += V^T P^T: lane group g4 reads keys 4g4..+3 and 16+4g4..+3 (the
  // key order of P^T), dims 16db + (lane & 15).
  const int r0 = 4 * g4 + (c16 >> 2);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int col = 16 * db + 4 * (c16 & 3);
    const int ch = col >> 3, e = col & 7;
    const bf16x4 lo = dec_lds_read_tr16(vsrc + r0 * D +
                                        8 * dec_swz<D>(r0, ch) + e);
    const bf16x4 hi = dec_lds_read_tr16(vsrc + (r0 + 16) * D +
                                        8 * dec_swz<D>(r0 + 16, ch) + e);
    const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    oacc[db] = mfma_16x16x32_bf16(a, pB, oacc[db]);
  }
}

template <int D, int G>
__global__ __launch_bounds__(kDecodeThreads, 4) void attn_decode_split_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ Kc,
    const __bf16* __restrict__ Vc, const int* __restrict__ seqlens,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, int Hkv, int ns,
    float scale_log2) {
  constexpr int KT = D / 32;          // QK k-steps (32 dims each)
  constexpr int NDB = D / 16;         // PV output blocks (16 dims each)
  static_assert(G <= 16, "heads are MFMA columns");

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;
  const int Hq = Hkv * G;

  // L_b and the cache offset sum(L_0..L_{b-1}) from one load per lane.
  long long prefix = 0;
  int L = 0;
  for (int base = 0; base <= b; base += 64) {
    const int i = base + lane;
    const int x = (i <= b) ? max(seqlens[i], 0) : 0;
    if (b - base < 64) L = __shfl(x, b - base, 64);
    prefix += wave_sum64(i < b ? x : 0);
  }
  const int chunk = decode_chunk(L, ns);
  const int nact = (L + chunk - 1) / chunk;    // splits with keys
  if (s >= nact) return;        // uniform over the workgroup (also L == 0)
  const int kbeg = s * chunk;
  const int kend = min(L, kbeg + chunk);
  const __bf16* Kp = Kc + ((size_t)prefix * Hkv + (size_t)g * L) * D;
  const __bf16* Vp = Vc + ((size_t)prefix * Hkv + (size_t)g * L) * D;

  // Q^T as the B operand: column c16 is head g*G + c16 (zero if c16 >= G),
  // k-step t covers dims 32t + 8*g4 .. +7.
  bf16x8 qB[KT];
  const __bf16* qrow = Q + (size_t)(b * Hq + g * G + min(c16, G - 1)) * D;
#pragma unroll
  for (int t = 0; t < KT; ++t)
    qB[t] = (c16 < G) ? *reinterpret_cast<const bf16x8*>(qrow + 32 * t +
                                                         8 * g4)
                      : bf16x8{};

  // Per-wave LDS buffer of one V block; after the key loop the same memory
  // holds the cross-wave merge.
  constexpr int VBYTES = kDecodeWaves * kDecodeBlock * D * 2;
  constexpr int MBYTES = kDecodeWaves * (32 + G * D) * 4;
  static_assert(MBYTES <= VBYTES, "merge fits in the V buffers");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[VBYTES];
  __bf16* vbuf = reinterpret_cast<__bf16*>(lds) + w * kDecodeBlock * D;

  f32x4 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x4{};
  float m_ref = -INFINITY;   // reference max (log2 domain) of head c16
  float l_i = 0.f;           // lane-partial sum for head c16

  // This wave's blocks start at kbeg + 32w and step by 128.  Each block's K
  // (registers) and V (LDS) loads are issued together and waited for once:
  // with 16 resident waves per CU every wave has one block in flight.
  DecodeK<D> blk;
  for (int j0 = kbeg + w * kDecodeBlock; j0 < kend;
       j0 += kDecodeWaves * kDecodeBlock) {
    decode_load<D>(blk, vbuf, Kp, Vp, j0, kend, lane);
    decode_step<D>(blk, qB, vbuf, j0, kend, lane, scale_log2, m_ref, l_i,
                   oacc);
  }

  // Per-wave state of head c16: m_ref, l (sum over the 4 lane groups),
  // O^T rows 16db + 4g4 + i.  Merge the waves through LDS.
  l_i += __shfl_xor(l_i, 16, 64);
  l_i += __shfl_xor(l_i, 32, 64);
  __syncthreads();                       // every wave is done with its V
  float* sm_m = reinterpret_cast<float*>(lds);            // [waves][16]
  float* sm_l = sm_m + kDecodeWaves * 16;                 // [waves][16]
  float* sm_o = sm_l + kDecodeWaves * 16;                 // [waves][G][D]
  if (g4 == 0) {
    sm_m[w * 16 + c16] = m_ref;
    sm_l[w * 16 + c16] = l_i;
  }
  if (c16 < G) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sm_o[(w * G + c16) * D + 16 * db + 4 * g4 + i] = oacc[db][i];
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kDecodeThreads) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kDecodeWaves; ++j) M = fmaxf(M, sm_m[j * 16 + h]);
    float W = 0.f, o = 0.f;
#pragma unroll
    for (int j = 0; j < kDecodeWaves; ++j) {
      const float wj = fast_exp2(sm_m[j * 16 + h] - M);  // 0 for an idle wave
      W = fmaf(wj, sm_l[j * 16 + h], W);
      o = fmaf(wj, sm_o[(j * G + h) * D + d], o);
    }
    const size_t row = ((size_t)(b * Hq + g * G + h)) * ns + s;
    ws_o[row * D + d] = o / W;
    if (d == 0) ws_lse[row] = (M + fast_log2(W)) * kLn2;
  }

}


// Combine the active splits of each (sequence, query head):
// M = max_s lse_s, w_s = exp(lse_s - M), o = sum w_s o_s / sum w_s,
// lse = M + ln(sum w_s).  A sequence with no keys gives o = 0, lse = -inf.
// One workgroup of D threads per (sequence, head); the split weights are
// formed once in LDS and the partial rows are read 8 at a time.
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

  __shared__ float wgt[256];
  __shared__ float red[D / 64];
  float mloc = -INFINITY;
  for (int s = d; s < nact; s += D) mloc = fmaxf(mloc, lse_p[s]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
    mloc = fmaxf(mloc, __shfl_xor(mloc, off, 64));
  if ((d & 63) == 0) red[d >> 6] = mloc;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int i = 1; i < D / 64; ++i) M = fmaxf(M, red[i]);
  for (int s = d; s < nact; s += D)
    wgt[s] = fast_exp2((lse_p[s] - M) * kLog2e);
  __syncthreads();

  float W = 0.f, o = 0.f;
  int s = 0;
  for (; s + 8 <= nact; s += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = o_p[(size_t)(s + u) * D + d];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      W += wgt[s + u];
      o = fmaf(wgt[s + u], v[u], o);
    }
  }
  for (; s < nact; ++s) {
    W += wgt[s];
    o = fmaf(wgt[s], o_p[(size_t)s * D + d], o);
  }
  const float res = nact > 0 ? o / W : 0.f;
  O[(size_t)bh * D + d] = (__bf16)res;
  if (LSE != nullptr && d == 0)
    LSE[bh] = nact > 0 ? M + logf(W) : -INFINITY;
}

}  // namespace attn
