// C-ABI entry points of libattn.so: host-side validation, tile choice and
// kernel launches.  Declarations and the contract live in include/attn.h.
#include "attn.h"
#include "attn_debug.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <math.h>
#include <stdint.h>

#include "decode.hpp"
#include "kvcache.hpp"
#include "prefill.hpp"
#include "prefill_ks.hpp"

namespace {

using attn::kPrefillBM;
using attn::kPrefillThreads;

// Compute units of the current device (cached per device; 256 if the query
// fails).  Orders prefill blocks and sizes the decode split.
int device_cu_count() {
  // per-device cache; concurrent callers may both query, and store the same
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount,
                              dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Common shape checks of both prefill entry points.
// Largest S * D of one head's rows (2^30 elements: 2 GB of 16-bit data).
constexpr long long kMaxHeadElems = 1LL << 30;

int check_prefill(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, int B, int Hq, int Hkv, int S, int D,
                  float scale, bool* empty) {
  *empty = false;
  if (B < 0 || S < 0 || Hq < 0 || Hkv < 0 || D < 0) return ATTN_ERR_SHAPE;
  if (Hq == 0 || Hkv == 0 || Hq % Hkv != 0) return ATTN_ERR_GQA;
  if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if (!isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_SCALE;
  // Grid size: one workgroup per (batch, query head, 128-row tile).
  const long long tiles = ((long long)S + kPrefillBM - 1) / kPrefillBM;
  if ((long long)B * Hq * tiles > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  // The K and V rows of one (batch, KV head) are addressed with 32-bit byte
  // offsets from their first row.
  if ((long long)S * D > kMaxHeadElems) return ATTN_ERR_SHAPE;
  if (B == 0 || S == 0) {
    *empty = true;
    return ATTN_OK;
  }
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(o, 16) || !aligned(lse, 4))
    return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

// Per-pair RoPE rates in turns per position, base^(-2i/D) / (2 pi), in fp64
// (base = 0: RoPE off, all rates 0).
attn::RopeRates rope_rates(double base, int D) {
  attn::RopeRates r = {};
  if (base > 0.0)
    for (int i = 0; i < D / 2 && i < 64; ++i)
      r.r[i] = pow(base, -2.0 * i / D) / (2.0 * M_PI);
  return r;
}

bool rope_base_ok(float base) { return isfinite(base) && base >= 0.f; }

template <typename T, template <int, bool> class Launcher>
int launch_prefill(const T* q, const T* k, const T* v, T* o, float* lse,
                   int B, int Hq, int Hkv, int S, int D, float scale,
                   int causal, void* stream, int use_rope = 0,
                   const attn::RopeRates& rope = attn::RopeRates{},
                   const int* cu_seqlens = nullptr,
                   const int* seq_lens = nullptr, void* split_ws = nullptr,
                   void* queue_ws = nullptr) {
  const int n_qtiles = (S + kPrefillBM - 1) / kPrefillBM;
  const dim3 grid((unsigned)(B * Hq * n_qtiles));
  const dim3 block(kPrefillThreads);
  const float sl2 = scale * attn::kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int ncu = device_cu_count();
  if (D == 64) {
    if (causal)
      Launcher<64, true>::run(grid, block, st, q, k, v, o, lse, B, Hq, Hkv, S,
                              sl2, n_qtiles, ncu, use_rope, rope,
                              cu_seqlens, seq_lens, split_ws, queue_ws);
    else
      Launcher<64, false>::run(grid, block, st, q, k, v, o, lse, B, Hq, Hkv,
                               S, sl2, n_qtiles, ncu, use_rope, rope,
                              cu_seqlens, seq_lens, split_ws, queue_ws);
  } else {
    if (causal)
      Launcher<128, true>::run(grid, block, st, q, k, v, o, lse, B, Hq, Hkv,
                               S, sl2, n_qtiles, ncu, use_rope, rope,
                              cu_seqlens, seq_lens, split_ws, queue_ws);
    else
      Launcher<128, false>::run(grid, block, st, q, k, v, o, lse, B, Hq, Hkv,
                                S, sl2, n_qtiles, ncu, use_rope, rope,
                              cu_seqlens, seq_lens, split_ws, queue_ws);
  }
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// Prefill kernels for 16-bit inputs:
//   rb: attn_prefill_rb_kernel (head dim 128; one wave per SIMD, 64 query
//       rows per wave; four query heads of a KV head per workgroup when the
//       group size is a multiple of 4, else 2 waves of one head);
//   w4: attn_prefill_kernel (4 waves of 32 rows, two workgroups per CU).
// rb runs more MFMA work per cycle but in coarser workgroups; w4 balances
// small launches better.  Measured on MI355X (causal, bf16, D = 128, group
// sizes 1 and 4), rb is ahead once the launch holds about 5e8 score
// elements (B Hq S^2 / 2) and behind by 5-18% below about 3e8; the table
// switches at 4e8.  attn_prefill_select() overrides the table.
std::atomic<int> g_prefill_kernel{ATTN_PREFILL_AUTO};

bool prefill_use_rb(int B, int Hq, int S, int D, int causal) {
  if (D != 128) return false;
  const int sel = g_prefill_kernel.load(std::memory_order_relaxed);
  if (sel != ATTN_PREFILL_AUTO) return sel == ATTN_PREFILL_RB;
  const double work = (double)B * Hq * S * (causal ? 0.5 * (S + 1) : S);
  return work >= 4e8;
}

// The key-split kernel (attn_prefill_ks_kernel: four waves share 32 query
// rows and split their key tiles) for dense launches too small to fill the
// GPU, where the other kernels' launches last as long as the key chain of
// their last query rows: its grid, B Hq ceil(S/32) workgroups of one per
// compute unit, must fit in two rounds.  Measured on MI355X (bf16, mean of
// 300 launches, us, key-split against the automatic choice before it):
// B1 12/12 S512 D64 causal 10.3 / 13.6 (full 9.9 / 12.9); B1 12/12 S1024
// D64 14.9 / 20.5; B2 12/12 S512 D64 13.0 / 13.8; B1 8/2 S512 D128 11.9 /
// 16.7; B1 8/2 S1024 D128 16.3 / 24.9; B2 8/2 S1024 D128 21.8 / 25.5;
// B1 8/2 S2048 D128 30.4 / 41.6 (the balanced schedule); B1 32/8 S512 D128
// 17.4 / 17.4 (two rounds); B4 8/2 S1024 D128, four rounds, 40.1 / 28.4.
// It takes precedence over the balanced schedule.  ATTN_PREFILL_KS forces
// it (dense calls without RoPE; the others then take the 4-wave kernel).
bool prefill_use_ks(int B, int Hq, int S, int D, int causal) {
  (void)causal;
  if (D != 64 && D != 128) return false;
  const long long ks_grid = (long long)B * Hq * ((S + 31) / 32);
  const int sel = g_prefill_kernel.load(std::memory_order_relaxed);
  // forced: wherever the grid is addressable (else the 4-wave kernel)
  if (sel == ATTN_PREFILL_KS) return ks_grid <= 0x7fffffffLL;
  if (sel != ATTN_PREFILL_AUTO) return false;
  return ks_grid <= 2LL * device_cu_count();
}

// Bound of the balanced schedule's wait for a partner's part, in ticks of
// the 100 MHz real-time counter (-1: the kernel's own rule).
std::atomic<int> g_split_wait{-1};

// Pairs of the balanced causal schedule of the register-blocked kernel
// (four query heads per workgroup), 0 where it does not apply: causal, head
// dim 128, group size a multiple of 4, at least two 64-row query tiles, and
// all of the launch's workgroups resident at once (one per compute unit),
// where the unbalanced schedule lasts as long as its last query tile.  The
// automatic choice takes it from S = 2048 on: measured on MI355X (causal,
// bf16, 8/2 heads), 5% ahead of the 4-wave kernel at B = 4, S = 2048, level
// at B = 1, S = 2048, 21-29% ahead at S = 4096 and 8192, and behind at
// S <= 1024, where each workgroup's 17 or fewer key tiles do not repay the
// second job's start and the hand-off.  ATTN_PREFILL_RB takes it wherever
// it applies.
constexpr int kSplitMinS = 2048;
long long prefill_split_pairs(int B, int Hq, int Hkv, int S, int D,
                              int causal) {
  if (!causal || D != 128 || Hkv <= 0 || Hq % Hkv != 0 ||
      (Hq / Hkv) % 4 != 0 || B <= 0 || S <= 0)
    return 0;
  const int sel = g_prefill_kernel.load(std::memory_order_relaxed);
  if (sel == ATTN_PREFILL_W4 || sel == ATTN_PREFILL_KS) return 0;
  if (sel == ATTN_PREFILL_AUTO && S < kSplitMinS) return 0;
  if (prefill_use_ks(B, Hq, S, D, causal)) return 0;   // small launches
  const long long nq = (S + 63) / 64;
  if (nq < 2) return 0;
  if ((long long)B * (Hq / 4) * nq > device_cu_count()) return 0;
  const long long np = (long long)B * (Hq / 4) * (nq / 2);
  return np <= attn::kRBMaxPairs ? np : 0;
}

// Whether a dense causal 16-bit launch given a workspace runs the
// register-blocked kernel (four query heads per workgroup) with the tile
// queue: where that kernel is chosen, the balanced schedule is not, and the
// launch holds more workgroups than compute units (in one round every
// workgroup is resident from the start and the queue would only add its
// atomic round trip).  The queue counter is the workspace's first 8 bytes.
bool prefill_queue_applies(int B, int Hq, int Hkv, int S, int D,
                           int causal) {
  if (!causal || D != 128 || B <= 0 || S <= 0 || Hkv <= 0 ||
      Hq % Hkv != 0 || (Hq / Hkv) % 4 != 0)
    return false;
  if (prefill_use_ks(B, Hq, S, D, causal)) return false;
  if (!prefill_use_rb(B, Hq, S, D, causal)) return false;
  if ((long long)B * (Hq / 4) * ((S + 63) / 64) <= device_cu_count())
    return false;
  return prefill_split_pairs(B, Hq, Hkv, S, D, causal) == 0;
}

// 16-bit inputs (bf16 or fp16): the MFMA kernels for element type T.
template <typename T>
struct Half16Prefill {
  template <int D, bool C>
  struct L {
    static void run(dim3 g, dim3 b, hipStream_t st, const T* q, const T* k,
                    const T* v, T* o, float* lse, int B, int Hq, int Hkv,
                    int S, float sl2, int nq, int ncu, int use_rope,
                    const attn::RopeRates& rope, const int* cu_seqlens,
                    const int* seq_lens, void* split_ws, void* queue_ws) {
      if constexpr (D == 128) {
        if constexpr (C) {
          if (split_ws != nullptr) {
            // balanced causal schedule, four query heads per workgroup
            const int nq4 = (S + 63) / 64;
            hipLaunchKernelGGL((attn::attn_prefill_rb_kernel<T, D, C, 4, true>),
                               dim3((unsigned)(B * (Hq / 4) * nq4)),
                               dim3(256), 0, st, q, k, v, o, lse, B, Hq, Hkv,
                               S, sl2, nq4, ncu, 0, rope, nullptr, nullptr,
                               split_ws,
                               g_split_wait.load(std::memory_order_relaxed),
                               attn::RmsEpilogue<T>{});
            return;
          }
        }
      }
      if (use_rope == 0 && cu_seqlens == nullptr && seq_lens == nullptr &&
          prefill_use_ks(B, Hq, S, D, C)) {
        hipLaunchKernelGGL((attn::attn_prefill_ks_kernel<T, D, C>),
                           dim3((unsigned)((long long)B * Hq * ((S + 31) / 32))),
                           dim3(kPrefillThreads), 0, st, q, k, v, o, lse, B,
                           Hq, Hkv, S, sl2, attn::RmsEpilogue<T>{});
        return;
      }
      if constexpr (D == 128) {
        if (prefill_use_rb(B, Hq, S, D, C)) {
          if ((Hq / Hkv) % 4 == 0) {
            // four query heads of a KV head per workgroup, 64-row tiles
            const int nq4 = (S + 63) / 64;
            // (with a workspace, dense causal launches take their tiles
            // from the tile queue)
            hipLaunchKernelGGL((attn::attn_prefill_rb_kernel<T, D, C, 4>),
                               dim3((unsigned)(B * (Hq / 4) * nq4)),
                               dim3(256), 0, st, q, k, v, o, lse, B, Hq, Hkv,
                               S, sl2, nq4, ncu, use_rope, rope, cu_seqlens,
                               seq_lens, queue_ws, -1, attn::RmsEpilogue<T>{});
          } else {
            hipLaunchKernelGGL((attn::attn_prefill_rb_kernel<T, D, C, 1>), g,
                               dim3(128), 0, st, q, k, v, o, lse, B, Hq, Hkv,
                               S, sl2, nq, ncu, use_rope, rope, cu_seqlens,
                               seq_lens, nullptr, -1, attn::RmsEpilogue<T>{});
          }
          return;
        }
      }
      hipLaunchKernelGGL((attn::attn_prefill_kernel<T, D, C>), g, b, 0, st, q,
                         k, v, o, lse, B, Hq, Hkv, S, sl2, nq, ncu, use_rope,
                         rope, cu_seqlens, seq_lens, attn::RmsEpilogue<T>{});
    }
  };
};

template <int D, bool C>
struct F32Prefill {
  static void run(dim3 g, dim3 b, hipStream_t st, const float* q,
                  const float* k, const float* v, float* o, float* lse, int B,
                  int Hq, int Hkv, int S, float sl2, int nq, int ncu,
                  int /*use_rope*/, const attn::RopeRates& /*rope*/,
                  const int* /*cu_seqlens*/, const int* /*seq_lens*/,
                  void* /*split_ws*/, void* /*queue_ws*/) {
    if (prefill_use_ks(B, Hq, S, D, C)) {
      hipLaunchKernelGGL((attn::attn_prefill_f32_ks_kernel<D, C>),
                         dim3((unsigned)((long long)B * Hq * ((S + 31) / 32))),
                         dim3(kPrefillThreads), 0, st, q, k, v, o, lse, B, Hq,
                         Hkv, S, sl2);
      return;
    }
    hipLaunchKernelGGL((attn::attn_prefill_f32_kernel<D, C>), g, b, 0, st, q,
                       k, v, o, lse, B, Hq, Hkv, S, sl2, nq, ncu);
  }
};

// ------------------------------------------------------------------ decode

// Default number of key-block ranges for decode: two per compute unit (each
// range is one single-wave workgroup).
int auto_splits(int B, int Hkv) {
  (void)B;
  (void)Hkv;
  const int n = 2 * device_cu_count();
  return n < ATTN_MAX_SPLITS ? n : ATTN_MAX_SPLITS;
}

int check_decode_sizes(int B, int Hq, int Hkv, int D, int num_splits) {
  if (B < 0 || Hq < 0 || Hkv < 0 || D < 0) return ATTN_ERR_SHAPE;
  if (Hq == 0 || Hkv == 0 || Hq % Hkv != 0) return ATTN_ERR_GQA;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return ATTN_ERR_GQA;
  if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if (num_splits < 0 || num_splits > ATTN_MAX_SPLITS) return ATTN_ERR_SPLITS;
  if ((long long)B * Hq > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

// Workspace layout: P + B*Hkv partial slots of G heads each (slot i + j holds
// range i's piece of segment j = b*Hkv + g): fp32 outputs [slots, G, D], fp32
// LSEs [slots, G], the ranges holding each segment's pieces [B*Hkv] (int2),
// and the block total (int64), each part starting on a 16-byte boundary.
struct DecodeWorkspace {
  size_t o_off, lse_off, seg_off, total_off, bytes;
};

DecodeWorkspace decode_workspace(int B, int Hq, int Hkv, int D, int P) {
  auto up16 = [](size_t x) { return (x + 15) / 16 * 16; };
  const size_t rows = ((size_t)P + (size_t)B * Hkv) * (size_t)(Hq / Hkv);
  DecodeWorkspace w;
  w.o_off = 0;
  w.lse_off = up16(rows * D * sizeof(float));
  w.seg_off = w.lse_off + up16(rows * sizeof(float));
  w.total_off = w.seg_off + up16((size_t)B * Hkv * sizeof(int2));
  w.bytes = w.total_off + 16;
  return w;
}

template <typename T, int D, int G>
void launch_decode_dg(const T* q, const T* kc, const T* vc,
                      const int* seqlens, T* o, float* lse, float* ws_o,
                      float* ws_lse, int2* ws_seg, long long* ws_total, int B,
                      int Hkv, int P, int cap, float sl2, int use_rope,
                      const attn::RopeRates& rope, hipStream_t st) {
  hipLaunchKernelGGL((attn::attn_decode_split_kernel<T, D, G>), dim3(P),
                     dim3(64), 0, st, q, kc, vc, seqlens, o, lse, ws_o, ws_lse,
                     ws_seg, ws_total, B, Hkv, P, cap, sl2, use_rope, rope);
  hipLaunchKernelGGL((attn::attn_decode_combine_kernel<T, D, G>),
                     dim3(B * Hkv * G), dim3(D), 0, st, ws_o, ws_lse, ws_seg,
                     ws_total, o, lse, Hkv, P);
}

template <typename T, int D>
void launch_decode_d(int G, const T* q, const T* kc, const T* vc,
                     const int* seqlens, T* o, float* lse, float* ws_o,
                     float* ws_lse, int2* ws_seg, long long* ws_total, int B,
                     int Hkv, int P, int cap, float sl2, int use_rope,
                     const attn::RopeRates& rope, hipStream_t st) {
  switch (G) {
    case 1: launch_decode_dg<T, D, 1>(q, kc, vc, seqlens, o, lse, ws_o, ws_lse,
                                      ws_seg, ws_total, B, Hkv, P, cap, sl2,
                                      use_rope, rope, st);
      break;
    case 2: launch_decode_dg<T, D, 2>(q, kc, vc, seqlens, o, lse, ws_o, ws_lse,
                                      ws_seg, ws_total, B, Hkv, P, cap, sl2,
                                      use_rope, rope, st);
      break;
    case 4: launch_decode_dg<T, D, 4>(q, kc, vc, seqlens, o, lse, ws_o, ws_lse,
                                      ws_seg, ws_total, B, Hkv, P, cap, sl2,
                                      use_rope, rope, st);
      break;
    default: launch_decode_dg<T, D, 8>(q, kc, vc, seqlens, o, lse, ws_o,
                                       ws_lse, ws_seg, ws_total, B, Hkv, P,
                                       cap, sl2, use_rope, rope, st);
      break;
  }
}

// Shared body of the bf16 and fp16 prefill entry points.
// A workspace (nullable) enables the balanced causal schedule where it
// applies; it is ignored elsewhere.
template <typename T>
int prefill16(const void* q, const void* k, const void* v, void* o,
              float* lse, int B, int Hq, int Hkv, int S, int D, float scale,
              int causal, void* stream, void* workspace = nullptr,
              size_t workspace_bytes = 0) {
  bool empty;
  const int st = check_prefill(q, k, v, o, lse, B, Hq, Hkv, S, D, scale,
                               &empty);
  if (st != ATTN_OK || empty) return st;
  void* split_ws = nullptr;
  void* queue_ws = nullptr;
  if (workspace != nullptr) {
    const long long np = prefill_split_pairs(B, Hq, Hkv, S, D, causal);
    if (np > 0) {
      if (!aligned(workspace, 16)) return ATTN_ERR_ALIGN;
      if (workspace_bytes < attn::rb_split_bytes(np))
        return ATTN_ERR_WORKSPACE;
      split_ws = workspace;
    } else if (prefill_queue_applies(B, Hq, Hkv, S, D, causal)) {
      if (!aligned(workspace, 16)) return ATTN_ERR_ALIGN;
      if (workspace_bytes < (size_t)attn::kRBFlagBytes)
        return ATTN_ERR_WORKSPACE;
      queue_ws = workspace;
    }
  }
  return launch_prefill<T, Half16Prefill<T>::template L>(
      static_cast<const T*>(q), static_cast<const T*>(k),
      static_cast<const T*>(v), static_cast<T*>(o), lse, B, Hq, Hkv, S, D,
      scale, causal, stream, 0, attn::RopeRates{}, nullptr, nullptr,
      split_ws, queue_ws);
}

// Prefill with the residual-add + RMSNorm epilogue: the plain dense
// prefill's kernel (key-split, register-blocked or 4-wave, without the
// balanced schedule) with its RMS flag, any shape the prefill accepts.
template <typename T>
int prefill16_rms(const void* q, const void* k, const void* v,
                  void* residual, const void* weight, void* out, float* lse,
                  int B, int Hq, int Hkv, int S, int D, float scale,
                  int causal, float eps, void* stream) {
  bool empty;
  const int st = check_prefill(q, k, v, out, lse, B, Hq, Hkv, S, D, scale,
                               &empty);
  if (st != ATTN_OK) return st;
  if (!isfinite(eps) || !(eps >= 0.f)) return ATTN_ERR_SCALE;
  if (empty) return ATTN_OK;
  if (!residual || !weight) return ATTN_ERR_NULL;
  if (!aligned(residual, 16) || !aligned(weight, 16)) return ATTN_ERR_ALIGN;
  if (residual == out) return ATTN_ERR_SHAPE;   // x and y need their own rows
  const int nq = (S + kPrefillBM - 1) / kPrefillBM;
  const dim3 g((unsigned)(B * Hq * nq)), b(kPrefillThreads);
  const float sl2 = scale * attn::kLog2e;
  const int ncu = device_cu_count();
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const T *qt = static_cast<const T*>(q), *kt = static_cast<const T*>(k),
          *vt = static_cast<const T*>(v);
  T* ot = static_cast<T*>(out);
  const attn::RmsEpilogue<T> rms{static_cast<T*>(residual),
                                 static_cast<const T*>(weight), eps};
  const attn::RopeRates rope{};
  // the kernel table of the plain dense prefill, without the balanced
  // schedule (no workspace here)
  const bool ks = prefill_use_ks(B, Hq, S, D, causal);
  const bool rb = !ks && prefill_use_rb(B, Hq, S, D, causal);
  const dim3 gks((unsigned)((long long)B * Hq * ((S + 31) / 32)));
#define ATTN_RMS_LAUNCH(DD, CC)                                               \
  if (ks)                                                                     \
    hipLaunchKernelGGL((attn::attn_prefill_ks_kernel<T, DD, CC, true>), gks, \
                       b, 0, hs, qt, kt, vt, ot, lse, B, Hq, Hkv, S, sl2,     \
                       rms);                                                  \
  else                                                                        \
    hipLaunchKernelGGL((attn::attn_prefill_kernel<T, DD, CC, true>), g, b, 0,\
                       hs, qt, kt, vt, ot, lse, B, Hq, Hkv, S, sl2, nq, ncu,  \
                       0, rope, nullptr, nullptr, rms)
  if (D == 64) {
    if (causal) { ATTN_RMS_LAUNCH(64, true); } else { ATTN_RMS_LAUNCH(64, false); }
  } else if (rb && (Hq / Hkv) % 4 == 0) {
    const int nq4 = (S + 63) / 64;
    const dim3 g4((unsigned)(B * (Hq / 4) * nq4));
    if (causal)
      hipLaunchKernelGGL((attn::attn_prefill_rb_kernel<T, 128, true, 4, false,
                                                       true>),
                         g4, dim3(256), 0, hs, qt, kt, vt, ot, lse, B, Hq,
                         Hkv, S, sl2, nq4, ncu, 0, rope, nullptr, nullptr,
                         nullptr, -1, rms);
    else
      hipLaunchKernelGGL((attn::attn_prefill_rb_kernel<T, 128, false, 4,
                                                       false, true>),
                         g4, dim3(256), 0, hs, qt, kt, vt, ot, lse, B, Hq,
                         Hkv, S, sl2, nq4, ncu, 0, rope, nullptr, nullptr,
                         nullptr, -1, rms);
  } else if (rb) {
    if (causal)
      hipLaunchKernelGGL((attn::attn_prefill_rb_kernel<T, 128, true, 1, false,
                                                       true>),
                         g, dim3(128), 0, hs, qt, kt, vt, ot, lse, B, Hq, Hkv,
                         S, sl2, nq, ncu, 0, rope, nullptr, nullptr, nullptr,
                         -1, rms);
    else
      hipLaunchKernelGGL((attn::attn_prefill_rb_kernel<T, 128, false, 1,
                                                       false, true>),
                         g, dim3(128), 0, hs, qt, kt, vt, ot, lse, B, Hq, Hkv,
                         S, sl2, nq, ncu, 0, rope, nullptr, nullptr, nullptr,
                         -1, rms);
  } else {
    if (causal) { ATTN_RMS_LAUNCH(128, true); } else { ATTN_RMS_LAUNCH(128, false); }
  }
#undef ATTN_RMS_LAUNCH
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// Shared body of the decode entry points; cap = 0 for the packed cache, else
// the per-sequence capacity of the padded cache.
template <typename T>
int decode16(const void* q, const void* kcache, const void* vcache,
             const int* seqlens, void* o, int B, int Hq, int Hkv, int D,
             int cap, float scale, int num_splits, float* lse,
             void* workspace, size_t workspace_bytes, void* stream,
             float rope_base = 0.f) {
  if (!rope_base_ok(rope_base)) return ATTN_ERR_SCALE;
  const attn::RopeRates rope = rope_rates(rope_base, D);
  const int use_rope = rope_base > 0.f;
  int st = check_decode_sizes(B, Hq, Hkv, D, num_splits);
  if (st != ATTN_OK) return st;
  if (!isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_SCALE;
  if (B == 0) return ATTN_OK;
  if (!q || !kcache || !vcache || !seqlens || !o || !workspace)
    return ATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(kcache, 16) || !aligned(vcache, 16) ||
      !aligned(o, 16) || !aligned(seqlens, 4) || !aligned(lse, 4) ||
      !aligned(workspace, 16))
    return ATTN_ERR_ALIGN;
  const int P = num_splits == 0 ? auto_splits(B, Hkv) : num_splits;
  const DecodeWorkspace wl = decode_workspace(B, Hq, Hkv, D, P);
  if (workspace_bytes < wl.bytes) return ATTN_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  float* ws_o = reinterpret_cast<float*>(ws + wl.o_off);
  float* ws_lse = reinterpret_cast<float*>(ws + wl.lse_off);
  int2* ws_seg = reinterpret_cast<int2*>(ws + wl.seg_off);
  long long* ws_total = reinterpret_cast<long long*>(ws + wl.total_off);
  const int G = Hq / Hkv;
  const float sl2 = scale * attn::kLog2e;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const T* qb = static_cast<const T*>(q);
  const T* kb = static_cast<const T*>(kcache);
  const T* vb = static_cast<const T*>(vcache);
  T* ob = static_cast<T*>(o);
  if (D == 64)
    launch_decode_d<T, 64>(G, qb, kb, vb, seqlens, ob, lse, ws_o, ws_lse,
                           ws_seg, ws_total, B, Hkv, P, cap, sl2, use_rope,
                           rope, hs);
  else
    launch_decode_d<T, 128>(G, qb, kb, vb, seqlens, ob, lse, ws_o, ws_lse,
                            ws_seg, ws_total, B, Hkv, P, cap, sl2, use_rope,
                           rope, hs);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// Prefill with RoPE: K rotated once into k_rot by a first launch (every
// query tile of its head reads it), q rotated on load by the attention
// kernel.
template <typename T>
int prefill_rope16(const void* q, const void* k, const void* v, void* o,
                   float* lse, void* k_rot, int B, int Hq, int Hkv, int S,
                   int D, float scale, int causal, float rope_base,
                   void* stream) {
  bool empty;
  const int st = check_prefill(q, k, v, o, lse, B, Hq, Hkv, S, D, scale,
                               &empty);
  if (st != ATTN_OK) return st;
  if (!rope_base_ok(rope_base) || !(rope_base > 0.f)) return ATTN_ERR_SCALE;
  if (empty) return ATTN_OK;
  if (!k_rot) return ATTN_ERR_NULL;
  if (!aligned(k_rot, 16)) return ATTN_ERR_ALIGN;
  const attn::RopeRates rope = rope_rates(rope_base, D);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const long long rows = (long long)B * Hkv * S;
  const long long threads = rows * (D / 16);
  const dim3 grid((unsigned)((threads + 255) / 256));
  const T* kb = static_cast<const T*>(k);
  T* kr = static_cast<T*>(k_rot);
  if (D == 64)
    hipLaunchKernelGGL((attn::attn_rope_rows_kernel<T, 64>), grid, dim3(256),
                       0, hs, kb, kr, rows, S, rope);
  else
    hipLaunchKernelGGL((attn::attn_rope_rows_kernel<T, 128>), grid, dim3(256),
                       0, hs, kb, kr, rows, S, rope);
  if (hipGetLastError() != hipSuccess) return ATTN_ERR_LAUNCH;
  return launch_prefill<T, Half16Prefill<T>::template L>(
      static_cast<const T*>(q), kr, static_cast<const T*>(v),
      static_cast<T*>(o), lse, B, Hq, Hkv, S, D, scale, causal, stream, 1,
      rope);
}

template <typename T>
int prefill_varlen16(const void* q, const void* k, const void* v, void* o,
                     float* lse, const int* cu_seqlens, int B, int max_seqlen,
                     int Hq, int Hkv, int D, float scale, int causal,
                     void* stream) {
  bool empty;
  const int st = check_prefill(q, k, v, o, lse, B, Hq, Hkv, max_seqlen, D,
                               scale, &empty);
  if (st != ATTN_OK || empty) return st;
  if (!cu_seqlens) return ATTN_ERR_NULL;
  if (!aligned(cu_seqlens, 4)) return ATTN_ERR_ALIGN;
  return launch_prefill<T, Half16Prefill<T>::template L>(
      static_cast<const T*>(q), static_cast<const T*>(k),
      static_cast<const T*>(v), static_cast<T*>(o), lse, B, Hq, Hkv,
      max_seqlen, D, scale, causal, stream, 0, attn::RopeRates{}, cu_seqlens);
}

template <typename T>
int prefill_padded16(const void* q, const void* k, const void* v, void* o,
                     float* lse, const int* seqlens, int B, int Hq, int Hkv,
                     int S, int D, float scale, int causal, void* stream) {
  bool empty;
  const int st =
      check_prefill(q, k, v, o, lse, B, Hq, Hkv, S, D, scale, &empty);
  if (st != ATTN_OK || empty) return st;
  if (!seqlens) return ATTN_ERR_NULL;
  if (!aligned(seqlens, 4)) return ATTN_ERR_ALIGN;
  return launch_prefill<T, Half16Prefill<T>::template L>(
      static_cast<const T*>(q), static_cast<const T*>(k),
      static_cast<const T*>(v), static_cast<T*>(o), lse, B, Hq, Hkv, S, D,
      scale, causal, stream, 0, attn::RopeRates{}, nullptr, seqlens);
}

template <typename T>
int decode_padded16(const void* q, const void* kcache, const void* vcache,
                    const int* seqlens, void* o, int B, int Hq, int Hkv, int D,
                    int cap, float scale, int num_splits, float* lse,
                    float rope_base, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (cap <= 0) return B == 0 ? ATTN_OK : ATTN_ERR_SHAPE;
  if ((long long)B * Hkv * cap > 0x7fffffffffffLL) return ATTN_ERR_SHAPE;
  return decode16<T>(q, kcache, vcache, seqlens, o, B, Hq, Hkv, D, cap, scale,
                     num_splits, lse, workspace, workspace_bytes, stream,
                     rope_base);
}

// KV-cache append for element type T (the RoPE rotation reads and writes T).
template <typename T>
int kv_append16(const void* k_new, const void* v_new, void* kcache,
                void* vcache, int* seqlens, int B, int Hkv, int D, int cap,
                float rope_base, void* stream) {
  if (B < 0 || Hkv < 0 || cap < 0) return ATTN_ERR_SHAPE;
  if (!rope_base_ok(rope_base)) return ATTN_ERR_SCALE;
  const attn::RopeRates rope = rope_rates(rope_base, D);
  const int use_rope = rope_base > 0.f;
  if (Hkv == 0) return ATTN_ERR_GQA;
  if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if (B == 0) return ATTN_OK;
  if (cap == 0) return ATTN_ERR_SHAPE;
  if (!k_new || !v_new || !kcache || !vcache || !seqlens) return ATTN_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(kcache, 16) ||
      !aligned(vcache, 16) || !aligned(seqlens, 4))
    return ATTN_ERR_ALIGN;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const T* kn = static_cast<const T*>(k_new);
  const T* vn = static_cast<const T*>(v_new);
  T* kc = static_cast<T*>(kcache);
  T* vc = static_cast<T*>(vcache);
  if (D == 64)
    hipLaunchKernelGGL((attn::attn_kv_append_kernel<T, 64>), dim3(B),
                       dim3(attn::kAppendThreads), 0, hs, kn, vn, kc, vc,
                       seqlens, Hkv, cap, use_rope, rope);
  else
    hipLaunchKernelGGL((attn::attn_kv_append_kernel<T, 128>), dim3(B),
                       dim3(attn::kAppendThreads), 0, hs, kn, vn, kc, vc,
                       seqlens, Hkv, cap, use_rope, rope);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// ------------------------------------------------- no-allocation decode
//
// The decode workspace of attn_decode_noalloc: a fixed array in device
// memory, one copy per GPU, held until the process ends.  In host code the
// name `scratch` stands for the symbol, not for a device address: every use
// goes through the address hipGetSymbolAddress returns for the current
// device, taken once per device and kept.
constexpr size_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of `scratch` on the current device (nullptr when the
// lookup fails).  Concurrent first calls may both look it up and store the
// same address.
void* scratch_address() {
  static std::atomic<void*> addr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess)
      return nullptr;
    addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

int attn_prefill(const void* q, const void* k, const void* v, void* o,
                 float* lse, int B, int Hq, int Hkv, int S, int D,
                 float scale, int causal, void* stream) {
  return prefill16<__bf16>(q, k, v, o, lse, B, Hq, Hkv, S, D, scale, causal,
                           stream);
}

int attn_prefill_f16(const void* q, const void* k, const void* v, void* o,
                     float* lse, int B, int Hq, int Hkv, int S, int D,
                     float scale, int causal, void* stream) {
  return prefill16<_Float16>(q, k, v, o, lse, B, Hq, Hkv, S, D, scale, causal,
                             stream);
}

size_t attn_prefill_workspace_size(int B, int Hq, int Hkv, int S, int D,
                                   int causal) {
  if (B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return 0;
  const long long np = prefill_split_pairs(B, Hq, Hkv, S, D, causal);
  if (np > 0) return attn::rb_split_bytes(np);
  return prefill_queue_applies(B, Hq, Hkv, S, D, causal)
             ? (size_t)attn::kRBFlagBytes
             : 0;
}

int attn_prefill_schedule(int B, int Hq, int Hkv, int S, int D, int causal) {
  if (B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return ATTN_SCHEDULE_STATIC;
  if (prefill_split_pairs(B, Hq, Hkv, S, D, causal) > 0)
    return ATTN_SCHEDULE_BALANCED;
  return prefill_queue_applies(B, Hq, Hkv, S, D, causal)
             ? ATTN_SCHEDULE_QUEUE
             : ATTN_SCHEDULE_STATIC;
}

int attn_prefill_ws(const void* q, const void* k, const void* v, void* o,
                    float* lse, int B, int Hq, int Hkv, int S, int D,
                    float scale, int causal, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return prefill16<__bf16>(q, k, v, o, lse, B, Hq, Hkv, S, D, scale, causal,
                           stream, workspace, workspace_bytes);
}

int attn_prefill_ws_f16(const void* q, const void* k, const void* v, void* o,
                        float* lse, int B, int Hq, int Hkv, int S, int D,
                        float scale, int causal, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return prefill16<_Float16>(q, k, v, o, lse, B, Hq, Hkv, S, D, scale,
                             causal, stream, workspace, workspace_bytes);
}

int attn_prefill_rope(const void* q, const void* k, const void* v, void* o,
                      float* lse, void* k_rot, int B, int Hq, int Hkv, int S,
                      int D, float scale, int causal, float rope_base,
                      void* stream) {
  return prefill_rope16<__bf16>(q, k, v, o, lse, k_rot, B, Hq, Hkv, S, D,
                                scale, causal, rope_base, stream);
}

int attn_prefill_rope_f16(const void* q, const void* k, const void* v,
                          void* o, float* lse, void* k_rot, int B, int Hq,
                          int Hkv, int S, int D, float scale, int causal,
                          float rope_base, void* stream) {
  return prefill_rope16<_Float16>(q, k, v, o, lse, k_rot, B, Hq, Hkv, S, D,
                                  scale, causal, rope_base, stream);
}

int attn_prefill_varlen(const void* q, const void* k, const void* v, void* o,
                        float* lse, const int* cu_seqlens, int B,
                        int max_seqlen, int Hq, int Hkv, int D, float scale,
                        int causal, void* stream) {
  return prefill_varlen16<__bf16>(q, k, v, o, lse, cu_seqlens, B, max_seqlen,
                                  Hq, Hkv, D, scale, causal, stream);
}

int attn_prefill_varlen_f16(const void* q, const void* k, const void* v,
                            void* o, float* lse, const int* cu_seqlens, int B,
                            int max_seqlen, int Hq, int Hkv, int D,
                            float scale, int causal, void* stream) {
  return prefill_varlen16<_Float16>(q, k, v, o, lse, cu_seqlens, B,
                                    max_seqlen, Hq, Hkv, D, scale, causal,
                                    stream);
}

int attn_prefill_padded(const void* q, const void* k, const void* v, void* o,
                        float* lse, const int* seqlens, int B, int Hq,
                        int Hkv, int S, int D, float scale, int causal,
                        void* stream) {
  return prefill_padded16<__bf16>(q, k, v, o, lse, seqlens, B, Hq, Hkv, S, D,
                                  scale, causal, stream);
}

int attn_prefill_padded_f16(const void* q, const void* k, const void* v,
                            void* o, float* lse, const int* seqlens, int B,
                            int Hq, int Hkv, int S, int D, float scale,
                            int causal, void* stream) {
  return prefill_padded16<_Float16>(q, k, v, o, lse, seqlens, B, Hq, Hkv, S,
                                    D, scale, causal, stream);
}

int attn_prefill_residual_rmsnorm(const void* q, const void* k,
                                  const void* v, void* residual,
                                  const void* weight, void* out, float* lse,
                                  int B, int Hq, int Hkv, int S, int D,
                                  float scale, int causal, float eps,
                                  void* stream) {
  return prefill16_rms<__bf16>(q, k, v, residual, weight, out, lse, B, Hq,
                               Hkv, S, D, scale, causal, eps, stream);
}

int attn_prefill_residual_rmsnorm_f16(const void* q, const void* k,
                                      const void* v, void* residual,
                                      const void* weight, void* out,
                                      float* lse, int B, int Hq, int Hkv,
                                      int S, int D, float scale, int causal,
                                      float eps, void* stream) {
  return prefill16_rms<_Float16>(q, k, v, residual, weight, out, lse, B, Hq,
                                 Hkv, S, D, scale, causal, eps, stream);
}

int attn_prefill_f32(const float* q, const float* k, const float* v, float* o,
                     float* lse, int B, int Hq, int Hkv, int S, int D,
                     float scale, int causal, void* stream) {
  bool empty;
  const int st = check_prefill(q, k, v, o, lse, B, Hq, Hkv, S, D, scale,
                               &empty);
  if (st != ATTN_OK || empty) return st;
  return launch_prefill<float, F32Prefill>(q, k, v, o, lse, B, Hq, Hkv, S, D,
                                           scale, causal, stream);
}

int attn_decode_auto_splits(int B, int Hkv) { return auto_splits(B, Hkv); }

int attn_prefill_kernel_for(int B, int Hq, int S, int D, int causal) {
  if (prefill_use_ks(B, Hq, S, D, causal)) return ATTN_PREFILL_KS;
  return prefill_use_rb(B, Hq, S, D, causal) ? ATTN_PREFILL_RB
                                             : ATTN_PREFILL_W4;
}

int attn_prefill_split_wait(int ticks) {
  if (ticks < -1) return ATTN_ERR_SHAPE;
  return g_split_wait.exchange(ticks);
}

int attn_prefill_select(int kernel) {
  if (kernel != ATTN_PREFILL_AUTO && kernel != ATTN_PREFILL_W4 &&
      kernel != ATTN_PREFILL_RB && kernel != ATTN_PREFILL_KS)
    return ATTN_ERR_SHAPE;
  return g_prefill_kernel.exchange(kernel);
}

size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int D,
                                  int num_splits) {
  if (check_decode_sizes(B, Hq, Hkv, D, num_splits) != ATTN_OK) return 0;
  const int P = num_splits == 0 ? auto_splits(B, Hkv) : num_splits;
  return decode_workspace(B, Hq, Hkv, D, P).bytes;
}

int attn_decode(const void* q, const void* kcache, const void* vcache,
                const int* seqlens, void* o, int B, int Hq, int Hkv, int D,
                float scale, int num_splits, float* lse, void* workspace,
                size_t workspace_bytes, void* stream) {
  return decode16<__bf16>(q, kcache, vcache, seqlens, o, B, Hq, Hkv, D, 0,
                          scale, num_splits, lse, workspace, workspace_bytes,
                          stream);
}

int attn_decode_f16(const void* q, const void* kcache, const void* vcache,
                    const int* seqlens, void* o, int B, int Hq, int Hkv, int D,
                    float scale, int num_splits, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return decode16<_Float16>(q, kcache, vcache, seqlens, o, B, Hq, Hkv, D, 0,
                            scale, num_splits, lse, workspace, workspace_bytes,
                            stream);
}

int attn_decode_noalloc(const void* q, const void* kcache,
                        const void* vcache, const int* seqlens, void* o, int B,
                        int Hq, int Hkv, int D, float scale, int num_splits,
                        float* lse, void* stream) {
  const int st = check_decode_sizes(B, Hq, Hkv, D, num_splits);
  if (st != ATTN_OK) return st;
  const int P = num_splits == 0 ? auto_splits(B, Hkv) : num_splits;
  if (B > 0 && decode_workspace(B, Hq, Hkv, D, P).bytes > kScratchBytes)
    return ATTN_ERR_WORKSPACE;
  void* ws = B > 0 ? scratch_address() : nullptr;
  if (B > 0 && ws == nullptr) return ATTN_ERR_LAUNCH;
  return decode16<__bf16>(q, kcache, vcache, seqlens, o, B, Hq, Hkv, D, 0,
                          scale, num_splits, lse, ws, kScratchBytes, stream);
}

int attn_decode_padded(const void* q, const void* kcache, const void* vcache,
                       const int* seqlens, void* o, int B, int Hq, int Hkv,
                       int D, int cap, float scale, int num_splits, float* lse,
                       float rope_base, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return decode_padded16<__bf16>(q, kcache, vcache, seqlens, o, B, Hq, Hkv, D,
                                 cap, scale, num_splits, lse, rope_base,
                                 workspace, workspace_bytes, stream);
}

int attn_decode_padded_f16(const void* q, const void* kcache,
                           const void* vcache, const int* seqlens, void* o,
                           int B, int Hq, int Hkv, int D, int cap, float scale,
                           int num_splits, float* lse, float rope_base,
                           void* workspace, size_t workspace_bytes,
                           void* stream) {
  return decode_padded16<_Float16>(q, kcache, vcache, seqlens, o, B, Hq, Hkv,
                                   D, cap, scale, num_splits, lse, rope_base,
                                   workspace, workspace_bytes, stream);
}

int attn_kv_append(const void* k_new, const void* v_new, void* kcache,
                   void* vcache, int* seqlens, int B, int Hkv, int D, int cap,
                   float rope_base, void* stream) {
  return kv_append16<__bf16>(k_new, v_new, kcache, vcache, seqlens, B, Hkv, D,
                             cap, rope_base, stream);
}

int attn_kv_append_f16(const void* k_new, const void* v_new, void* kcache,
                       void* vcache, int* seqlens, int B, int Hkv, int D,
                       int cap, float rope_base, void* stream) {
  return kv_append16<_Float16>(k_new, v_new, kcache, vcache, seqlens, B, Hkv,
                               D, cap, rope_base, stream);
}

#ifdef ATTN_DEBUG_TRACE
int attn_debug_trace(int b, int h, int row, float* buf, int capacity) {
  if (buf != nullptr && (b < 0 || h < 0 || row < 0 || capacity < 0))
    return ATTN_ERR_SHAPE;
  if (!aligned(buf, 4)) return ATTN_ERR_ALIGN;
  const attn::TraceTarget t{buf, b, h, row, capacity};
  return hipMemcpyToSymbol(HIP_SYMBOL(attn::g_trace), &t, sizeof t) ==
                 hipSuccess
             ? ATTN_OK
             : ATTN_ERR_LAUNCH;
}
#endif

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_NULL: return "ATTN_ERR_NULL";
    case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE";
    case ATTN_ERR_GQA: return "ATTN_ERR_GQA";
    case ATTN_ERR_HEAD_DIM: return "ATTN_ERR_HEAD_DIM";
    case ATTN_ERR_ALIGN: return "ATTN_ERR_ALIGN";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_SPLITS: return "ATTN_ERR_SPLITS";
    case ATTN_ERR_LAUNCH: return "ATTN_ERR_LAUNCH";
    case ATTN_ERR_SCALE: return "ATTN_ERR_SCALE";
    default: return "ATTN_ERR_UNKNOWN";
  }
}

}  // extern "C"
