/*
 * attn.h -- fused scaled-dot-product attention on MI355X (gfx950), C ABI.
 *
 * The operation is the attention chain of "Attention三算子融合实战：从Triton到
 * CUDA的推理加速优化" (section 1.1): scores S = Q K^T times a scale, a row-wise
 * softmax P of S, and O = P V, computed in one kernel with the online softmax
 * of section 2.2 (running row max m and sum l, old terms rescaled by
 * exp(m - m_new)) so that S and P never reach device memory (section 2.3).
 * The causal mask is that of section 4.3: query row i sees key j only when
 * j <= i.  Grouped-query attention follows "手写Triton kernel重构Qwen3.5-0.8B"
 * (section 2.1: two KV heads serve eight query heads): query head h reads KV
 * head h / (Hq / Hkv).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller, contiguous
 *    row-major, 16-byte aligned (lse: 4-byte aligned).  The library never
 *    allocates, frees or synchronises; it only enqueues kernels on `stream`
 *    (a hipStream_t; NULL means the default stream) and returns.
 *  - Every argument check runs on the host before any HIP call; a failed
 *    check returns a negative attn_status and enqueues nothing.  Errors are
 *    never printed or raised.  ATTN_ERR_LAUNCH reports a failed kernel launch.
 *  - Empty work (B == 0, or S == 0 for prefill) returns ATTN_OK and enqueues
 *    nothing.
 *  - Outputs must not alias inputs.  The library holds no state between
 *    calls: calls on different streams are independent, and a call may be
 *    captured into a HIP graph.
 *  - Accumulation is fp32 throughout (running m, l and the output
 *    accumulator); bf16 results are rounded to nearest even.
 *  - Results are deterministic: no atomics, fixed reduction order.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,      /* a required pointer is NULL */
  ATTN_ERR_SHAPE = -2,     /* a negative size, or a size too large to index */
  ATTN_ERR_GQA = -3,       /* Hq or Hkv <= 0, Hq % Hkv != 0, or an
                              unsupported group size Hq / Hkv */
  ATTN_ERR_HEAD_DIM = -4,  /* D is not 64 or 128 */
  ATTN_ERR_ALIGN = -5,     /* a pointer is not aligned as required */
  ATTN_ERR_WORKSPACE = -6, /* workspace smaller than required */
  ATTN_ERR_SPLITS = -7,    /* num_splits < 0 or > ATTN_MAX_SPLITS */
  ATTN_ERR_LAUNCH = -8,    /* the HIP runtime rejected a kernel launch */
  ATTN_ERR_SCALE = -9      /* scale is not a finite positive number (or a
                              RoPE base or an RMSNorm eps is negative or
                              not finite) */
} attn_status;

/* Largest num_splits attn_decode accepts. */
#define ATTN_MAX_SPLITS 4096

/*
 * Prefill attention, bf16 storage.
 *   q, o : [B, Hq,  S, D] bf16     k, v : [B, Hkv, S, D] bf16
 *   lse  : [B, Hq,  S]    fp32     natural-log log-sum-exp of each scaled,
 *                                   masked score row (m + ln l; the form of
 *                                   the "triton-optimization" page, section
 *                                   3.5); may be NULL to skip it.
 *   scale: multiplier of Q K^T, finite and > 0 (1/sqrt(D) in the usual
 *          setting; the fused Triton kernel of the attention-fusion page,
 *          section 3.2, applies it to qk before the softmax).
 *   causal: nonzero for the causal mask j <= i, zero for no mask.
 * Any S >= 0 with S * D <= 2^30 is accepted (tail tiles are masked, as
 * section 6.1 of the attention-fusion page requires); the rows of one head
 * are addressed with 32-bit byte offsets, so a larger S is ATTN_ERR_SHAPE.
 * D must be 64 or 128.
 */
int attn_prefill(const void* q, const void* k, const void* v, void* o,
                 float* lse, int B, int Hq, int Hkv, int S, int D,
                 float scale, int causal, void* stream);

/*
 * Bytes of device workspace that let attn_prefill_ws (and _ws_f16) run a
 * causal launch with the balanced schedule or the tile queue (below), 0
 * where neither applies.  The balanced schedule applies to causal launches
 * with D = 128, Hq / Hkv a multiple of 4, S > 64, and at most one workgroup
 * of B (Hq/4) ceil(S/64) per compute unit of the current device; under ATTN_PREFILL_AUTO from
 * S = 2048 on (below that the 4-wave kernel was measured faster), under
 * ATTN_PREFILL_RB for any such S, under ATTN_PREFILL_W4 never.
 * Query tile t needs a number of key tiles growing with t, so when every
 * tile has its own compute unit the launch otherwise lasts as long as its
 * last tile; the balanced schedule pairs tile t with tile nq-1-t and cuts
 * the pair's key tiles evenly between two workgroups, the second merging
 * the first's part of the longer row range with its own (the merge of key
 * ranges by their maxima and sums, attention-fusion page, section 4.4, with
 * the partial buffer of the Qwen page, section 3.3).
 * The tile queue (4096 bytes) applies to the other causal launches of the
 * register-blocked kernel with four query heads per workgroup (D = 128,
 * Hq / Hkv a multiple of 4, the kernel chosen by the table or by
 * ATTN_PREFILL_RB): launches of more workgroups than compute units, which
 * run in rounds.  Each workgroup then takes the next query tile, heaviest
 * first, from a counter in the workspace, so compute units and XCDs that
 * finish early take more of the work (list scheduling, longest first) where
 * hardware dispatch alone gives every XCD a fixed share of the tiles.  Both
 * sizes depend on the device's compute-unit count: query them with that
 * device current.
 */
size_t attn_prefill_workspace_size(int B, int Hq, int Hkv, int S, int D,
                                   int causal);

/* Schedules of a 16-bit attn_prefill_ws launch given a workspace. */
#define ATTN_SCHEDULE_STATIC 0   /* no workspace used */
#define ATTN_SCHEDULE_BALANCED 1 /* paired tiles, split and merged */
#define ATTN_SCHEDULE_QUEUE 2    /* tiles taken from the tile queue */

/*
 * The schedule attn_prefill_ws runs for these sizes when it is given a
 * workspace of attn_prefill_workspace_size bytes, under the current kernel
 * setting and device (one of ATTN_SCHEDULE_*; STATIC for invalid sizes).
 */
int attn_prefill_schedule(int B, int Hq, int Hkv, int S, int D, int causal);

/*
 * attn_prefill / attn_prefill_f16 with a caller-owned device workspace
 * (16-byte aligned) for the balanced schedule or the tile queue.  workspace
 * NULL, or a launch neither applies to: the same launch as attn_prefill.
 * Where one applies, workspace_bytes below attn_prefill_workspace_size is
 * ATTN_ERR_WORKSPACE.  Its first 4096 bytes hold one flag word per pair of
 * query tiles (balanced schedule) or the queue counter (first 8 bytes):
 * they must be zero before the workspace's first use, and every call leaves
 * them zero, so one workspace serves calls of any sizes in turn (the rest of
 * the workspace may hold anything).  The output is the same, bit for bit,
 * with or without the tile queue: it changes only which workgroup computes a
 * tile (a nonzero counter still gives every tile to exactly one workgroup;
 * it only changes their order).  Calls that share
 * a workspace must not overlap in time (launch them on one stream).  A workgroup waits for its partner's part
 * for a bounded time only, then computes the part itself, so a launch
 * always completes.  Other arguments and errors as attn_prefill.
 */
int attn_prefill_ws(const void* q, const void* k, const void* v, void* o,
                    float* lse, int B, int Hq, int Hkv, int S, int D,
                    float scale, int causal, void* workspace,
                    size_t workspace_bytes, void* stream);
int attn_prefill_ws_f16(const void* q, const void* k, const void* v, void* o,
                        float* lse, int B, int Hq, int Hkv, int S, int D,
                        float scale, int causal, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Prefill attention, fp16 storage.  Same arguments and layouts as
 * attn_prefill with q, k, v, o in IEEE fp16.  The mixed-precision rule of
 * the attention-fusion page, section 5.5, holds as for bf16: fp16 only in
 * the stored tensors and the MFMA inputs (P is rounded to fp16 for the PV
 * product), fp32 for the QK^T and PV accumulation and for every
 * cross-iteration state (m, l, acc).  Errors as attn_prefill.
 */
int attn_prefill_f16(const void* q, const void* k, const void* v, void* o,
                     float* lse, int B, int Hq, int Hkv, int S, int D,
                     float scale, int causal, void* stream);

/*
 * Prefill attention with rotary position embedding (RoPE) on q and k, bf16.
 * Arguments as attn_prefill, plus:
 *   k_rot    : [B, Hkv, S, D] bf16 output, owned by the caller: k rotated to
 *              positions 0..S-1 (what a KV cache stores), then read by the
 *              attention kernel.  Must not alias q, k, v or o.
 *   rope_base: > 0 (e.g. 10000).  Pair i = (x[i], x[i + D/2]) of a head
 *              vector at position p turns by p * rope_base^(-2i/D): the
 *              half-split rotation of the "triton-optimization" page,
 *              section 3.4, with the usual angle (the pages print none).
 *              Otherwise ATTN_ERR_SCALE.
 * q is rotated on load inside the attention kernel (the Qwen3.5-0.8B page,
 * section 1.2: RoPE computed in fp32 while q and k are loaded, no cos/sin
 * tensor); k is rotated once by a first launch into k_rot, because every
 * query tile of its head reads it.  Angles are reduced to a fraction of a
 * turn in fp64 and sin/cos taken in fp32; rotated values are rounded to bf16
 * for the MFMA.  Two launches on `stream`.
 */
int attn_prefill_rope(const void* q, const void* k, const void* v, void* o,
                      float* lse, void* k_rot, int B, int Hq, int Hkv, int S,
                      int D, float scale, int causal, float rope_base,
                      void* stream);

/*
 * attn_prefill_rope with fp16 storage: q, k, v, o and k_rot in IEEE fp16
 * (fp32 rotation and accumulation, as for attn_prefill_f16).  Same
 * arguments, layouts and errors.
 */
int attn_prefill_rope_f16(const void* q, const void* k, const void* v,
                          void* o, float* lse, void* k_rot, int B, int Hq,
                          int Hkv, int S, int D, float scale, int causal,
                          float rope_base, void* stream);

/*
 * Prefill attention over a ragged batch (variable sequence lengths), bf16:
 * the padding mask of the attention-fusion page, section 4.3, and the
 * dynamic shapes of its section 6.1, with no padding stored at all.
 *   cu_seqlens: DEVICE int32 [B + 1], non-decreasing, cu[0] = 0: sequence b
 *               has S_b = cu[b+1] - cu[b] tokens.
 *   q, o      : sequence b is a [Hq, S_b, D] bf16 block at element offset
 *               Hq * D * cu[b]        (the packed layout of attn_decode's
 *   k, v      : [Hkv, S_b, D] blocks at Hkv * D * cu[b]   caches)
 *   lse       : [Hq, S_b] fp32 blocks at offset Hq * cu[b], or NULL.
 *   max_seqlen: an upper bound of every S_b, known on the host; it sizes the
 *               grid (rows past it are not computed).
 * Each sequence is attended on its own (causal or full), exactly as
 * attn_prefill with B = 1 and S = S_b.  Other arguments and errors as
 * attn_prefill (with S = max_seqlen); cu_seqlens NULL: ATTN_ERR_NULL.
 */
int attn_prefill_varlen(const void* q, const void* k, const void* v, void* o,
                        float* lse, const int* cu_seqlens, int B,
                        int max_seqlen, int Hq, int Hkv, int D, float scale,
                        int causal, void* stream);

/*
 * attn_prefill_varlen with fp16 storage (q, k, v, o in IEEE fp16).  Same
 * arguments, layouts and errors.
 */
int attn_prefill_varlen_f16(const void* q, const void* k, const void* v,
                            void* o, float* lse, const int* cu_seqlens, int B,
                            int max_seqlen, int Hq, int Hkv, int D,
                            float scale, int causal, void* stream);

/*
 * Prefill attention over a padded batch, bf16: the padding mask of the
 * attention-fusion page, section 4.3, on the dense layout of attn_prefill
 * (every sequence stored with S rows, the first L_b of them valid).
 *   q, o : [B, Hq, S, D] bf16   k, v : [B, Hkv, S, D] bf16
 *   lse  : [B, Hq, S] fp32, or NULL.
 *   seqlens: DEVICE int32 [B]; L_b = seqlens[b] clamped to [0, S].
 * Rows i < L_b of sequence b attend keys j < L_b (and j <= i when causal),
 * exactly as attn_prefill on the first L_b rows alone; the padding rows
 * i >= L_b get o = 0 and lse = -inf.  Padding K / V rows are never read.
 * Other arguments and errors as attn_prefill; seqlens NULL: ATTN_ERR_NULL,
 * not 4-byte aligned: ATTN_ERR_ALIGN.
 */
int attn_prefill_padded(const void* q, const void* k, const void* v, void* o,
                        float* lse, const int* seqlens, int B, int Hq,
                        int Hkv, int S, int D, float scale, int causal,
                        void* stream);

/*
 * attn_prefill_padded with fp16 storage (q, k, v, o in IEEE fp16).  Same
 * arguments, layouts and errors.
 */
int attn_prefill_padded_f16(const void* q, const void* k, const void* v,
                            void* o, float* lse, const int* seqlens, int B,
                            int Hq, int Hkv, int S, int D, float scale,
                            int causal, void* stream);

/*
 * Prefill attention with a fused residual add and RMSNorm on its output, bf16
 * storage: the fused RMSNorm-with-residual of the "triton-optimization" page
 * (section 3.2; the same forward as "第 6 讲：核函数与 Triton", section 9.1)
 * applied in the attention kernel's epilogue, the extension named by the
 * attention-fusion page, section 6.3.  For each query row of each head, with
 * o the attention output row (fp32, before rounding):
 *   x = o + residual[b, h, i, :]
 *   out[b, h, i, :] = x / sqrt(mean_d(x^2) + eps) * weight
 *   residual[b, h, i, :] = x            (in place, for the next layer)
 *   q, out, residual : [B, Hq, S, D] bf16    k, v : [B, Hkv, S, D] bf16
 *   weight : [D] bf16    lse : [B, Hq, S] fp32 (the attention's), or NULL
 *   eps    : >= 0 and finite (the pages' default is 1e-6; with eps = 0 an
 *            all-zero row x gives NaN)
 * The row normalised is one head's D values.  The kernel is the one
 * attn_prefill would take without a workspace (attn_prefill_kernel_for);
 * other arguments as attn_prefill.  Errors as attn_prefill, plus:
 * residual or weight NULL -> ATTN_ERR_NULL; either not 16-byte aligned ->
 * ATTN_ERR_ALIGN; eps negative or not finite -> ATTN_ERR_SCALE; residual ==
 * out -> ATTN_ERR_SHAPE.
 */
int attn_prefill_residual_rmsnorm(const void* q, const void* k,
                                  const void* v, void* residual,
                                  const void* weight, void* out, float* lse,
                                  int B, int Hq, int Hkv, int S, int D,
                                  float scale, int causal, float eps,
                                  void* stream);

/*
 * attn_prefill_residual_rmsnorm with fp16 storage (q, k, v, residual, weight
 * and out in IEEE fp16).  Same arguments, layouts and errors.
 */
int attn_prefill_residual_rmsnorm_f16(const void* q, const void* k,
                                      const void* v, void* residual,
                                      const void* weight, void* out,
                                      float* lse, int B, int Hq, int Hkv,
                                      int S, int D, float scale, int causal,
                                      float eps, void* stream);

/*
 * Prefill attention, fp32 storage.  Same arguments and layouts as
 * attn_prefill with every tensor fp32.  The probabilities P stay fp32 (the
 * accuracy setting of the attention-fusion page, sections 3.3 and 5.5).
 * Launches small enough for the key-split rule of attn_prefill_select (or
 * under ATTN_PREFILL_KS) take the fp32 key-split kernel, the others the
 * fp32 kernel.
 */
int attn_prefill_f32(const float* q, const float* k, const float* v, float* o,
                     float* lse, int B, int Hq, int Hkv, int S, int D,
                     float scale, int causal, void* stream);

/*
 * Which kernel the 16-bit prefill entry points (attn_prefill*, bf16 and
 * fp16) launch, process-wide: ATTN_PREFILL_AUTO picks from the shape (the
 * key-split kernel for dense launches whose B Hq ceil(S/32) workgroups fit
 * in one round of the compute units, the register-blocked kernel for head
 * dim 128 and large launches, the 4-wave kernel otherwise);
 * ATTN_PREFILL_W4, ATTN_PREFILL_RB and ATTN_PREFILL_KS force one (RB
 * applies to head dim 128 only, D = 64 then uses W4; KS applies to the
 * dense entry points without RoPE, the ragged, padded and RoPE entry points
 * then use W4).  All compute the same function; they differ in rounding
 * order only.  For tuning and testing.  Returns the previous setting, or
 * ATTN_ERR_SHAPE for another value (the setting is then unchanged).
 * Launches already issued keep their kernel; calls racing with launches on
 * other threads pick either.
 */
#define ATTN_PREFILL_AUTO 0
#define ATTN_PREFILL_W4 1
#define ATTN_PREFILL_RB 2
#define ATTN_PREFILL_KS 3
int attn_prefill_select(int kernel);

/* The kernel (ATTN_PREFILL_W4, ATTN_PREFILL_RB or ATTN_PREFILL_KS) a dense
   16-bit prefill launch with these sizes would use under the current
   setting, without a workspace (with one, the balanced schedule or the tile
   queue runs the RB kernel, four heads per workgroup, wherever
   attn_prefill_workspace_size is nonzero).  W4 launches B Hq ceil(S/128) workgroups of 256 threads; RB
   launches B (Hq/4) ceil(S/64) workgroups of 256 threads when Hq/Hkv is a
   multiple of 4, else B Hq ceil(S/128) of 128 threads; KS launches
   B Hq ceil(S/32) workgroups of 256 threads. */
int attn_prefill_kernel_for(int B, int Hq, int S, int D, int causal);

/*
 * How long, in ticks of the GPU's 100 MHz real-time counter, a workgroup of
 * the balanced schedule waits for its partner's part before computing that
 * part itself: -1 (the default) waits twice as long as the workgroup has
 * run so far plus 20 us; 0 gives up at once.  Process-wide, for testing the
 * give-up path and for tuning; the results are the same either way up to
 * rounding order.  Returns the previous setting, or ATTN_ERR_SHAPE for a
 * value below -1 (the setting is then unchanged).
 */
int attn_prefill_split_wait(int ticks);

/*
 * Bytes of device workspace attn_decode needs for these sizes
 * (num_splits == 0 selects the same automatic split count attn_decode uses).
 * Returns 0 when the sizes are invalid.
 */
size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int D,
                                  int num_splits);

/* The split count attn_decode uses for num_splits == 0: twice the number of
   compute units of the current device (512 when it cannot be queried;
   nothing is read back from the device, and B and Hkv do not change it). */
int attn_decode_auto_splits(int B, int Hkv);

/*
 * Decode attention: one query row per sequence against its whole KV cache
 * (the decode setting of the attention-fusion page, section 1.3: Q has one
 * row while K and V grow with the history), split over the keys and merged
 * with a log-sum-exp combine (section 4.4: key chunks handled by separate
 * blocks and merged afterwards; section 2.2: the merge order does not matter
 * once m and l are kept).
 *   q, o     : [B, Hq, D] bf16
 *   kcache,
 *   vcache   : packed per sequence: sequence b is a [Hkv, L_b, D] bf16 block
 *              at element offset Hkv * D * (L_0 + ... + L_{b-1}).
 *   seqlens  : DEVICE int32 [B], L_b = number of cached keys the query of
 *              sequence b attends to (its own key included).  L_b <= 0 gives
 *              o = 0 and lse = -inf for that sequence.
 *   num_splits: 1..ATTN_MAX_SPLITS, or 0 for attn_decode_auto_splits(B, Hkv).
 *              The caches are cut into 32-key blocks; the blocks of all
 *              (sequence, KV head) pairs, in that order, are divided into
 *              num_splits equal contiguous ranges, one per workgroup, so the
 *              work per workgroup does not depend on the length mix.
 *   scale    : multiplier of q.k, finite and > 0.
 *   lse      : [B, Hq] fp32 natural-log LSE, or NULL.
 *   workspace: DEVICE scratch of at least
 *              attn_decode_workspace_size(B, Hq, Hkv, D, num_splits) bytes,
 *              16-byte aligned, owned by the caller; its contents on entry
 *              do not matter and are overwritten.  Calls in flight at the
 *              same time must not share a workspace.
 * Two launches on `stream`: the split kernel streams each range, finishes
 * every (sequence, KV head) pair whose blocks all lie in one range, and for
 * a pair cut by range boundaries writes one normalised partial output and
 * LSE per piece (plus which ranges hold them) to the workspace; the combine
 * kernel merges those pieces (log-sum-exp combine).
 * Supported group sizes Hq / Hkv: 1, 2, 4, 8.
 */
int attn_decode(const void* q, const void* kcache, const void* vcache,
                const int* seqlens, void* o, int B, int Hq, int Hkv, int D,
                float scale, int num_splits, float* lse, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * Decode attention, fp16 storage: attn_decode with q, kcache, vcache and o
 * in IEEE fp16 (attention-fusion page, section 5.5: fp16 storage, fp32
 * accumulation and state).  Same layouts, workspace and errors.
 */
int attn_decode_f16(const void* q, const void* kcache, const void* vcache,
                    const int* seqlens, void* o, int B, int Hq, int Hkv, int D,
                    float scale, int num_splits, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Size of the device-resident workspace of attn_decode_noalloc (8 MiB). */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

/*
 * attn_decode without a caller workspace, for callers that cannot allocate
 * device memory or pass scratch (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same q, kcache, vcache,
 * seqlens, o, sizes, scale, num_splits, lse and stream as attn_decode, and
 * the same kernels and results.  The workspace is a fixed
 * ATTN_NOALLOC_SCRATCH_BYTES array in device memory that the library holds
 * on each GPU it runs on until the process ends; the library looks up its
 * address once per device, on the first call made with that device current
 * (the stream must belong to the current device).  No call allocates or
 * frees memory.
 * Errors: as attn_decode, plus ATTN_ERR_WORKSPACE when
 * attn_decode_workspace_size(B, Hq, Hkv, D, num_splits) exceeds
 * ATTN_NOALLOC_SCRATCH_BYTES, and ATTN_ERR_LAUNCH when the array's address
 * cannot be obtained.
 * Every call on one GPU uses that GPU's one array: calls that may overlap in
 * time on the same GPU (different streams, or host threads) race on it and
 * must be serialised by the caller.  Nothing in the array needs clearing
 * between calls (its contents on entry do not matter).
 */
int attn_decode_noalloc(const void* q, const void* kcache,
                        const void* vcache, const int* seqlens, void* o, int B,
                        int Hq, int Hkv, int D, float scale, int num_splits,
                        float* lse, void* stream);

/*
 * KV-cache append: the kv_cache_store step of the operator table of the
 * Qwen3.5-0.8B page ("手写Triton kernel重构Qwen3.5-0.8B", section 2.2, row 18:
 * write the new k/v into the KV cache), shaped for the CUDA Graph decode of
 * that page's section 4 (preallocated buffers, positions on the device).
 *   k_new, v_new  : [B, Hkv, D] bf16, 16-byte aligned (v is copied bit for
 *                   bit; k too unless it is rotated)
 *   kcache, vcache: [B, Hkv, cap, D] bf16, the "padded" cache:
 *                   sequence b holds seqlens[b] valid rows per KV head
 *   seqlens       : DEVICE int32 [B].  For every b with
 *                   0 <= seqlens[b] < cap, row seqlens[b] of each KV head of
 *                   sequence b receives k_new / v_new and seqlens[b] is
 *                   incremented; a full sequence is left unchanged.
 *   rope_base     : 0 for a plain copy; > 0 to store k rotated by RoPE at
 *                   its position seqlens[b] (the k_rope step of the same
 *                   table, row 5, fused into the store), see
 *                   attn_prefill_rope for the rotation.  Negative or
 *                   non-finite: ATTN_ERR_SCALE.
 * One launch on `stream`; nothing is read back to the host, so a decode step
 * (append, then attn_decode_padded) can be captured once in a hipGraph and
 * replayed step after step.  D must be 64 or 128; cap >= 1 when B > 0.
 */
int attn_kv_append(const void* k_new, const void* v_new, void* kcache,
                   void* vcache, int* seqlens, int B, int Hkv, int D, int cap,
                   float rope_base, void* stream);

/*
 * attn_kv_append for fp16 caches: k_new, v_new [B, Hkv, D] and kcache,
 * vcache [B, Hkv, cap, D] in IEEE fp16 (a rotated k is computed in fp32 and
 * rounded to fp16).  Same arguments and errors.
 */
int attn_kv_append_f16(const void* k_new, const void* v_new, void* kcache,
                       void* vcache, int* seqlens, int B, int Hkv, int D,
                       int cap, float rope_base, void* stream);

/*
 * Decode attention over the padded cache of attn_kv_append: attn_decode with
 * kcache, vcache [B, Hkv, cap, D] bf16 and L_b = min(seqlens[b], cap).  Same
 * q, o, lse, num_splits, workspace (attn_decode_workspace_size) and errors;
 * cap <= 0 with B > 0 is ATTN_ERR_SHAPE.
 *   rope_base: 0 for none; > 0 rotates each query by RoPE at its position
 *              L_b - 1 (it is the newest token) inside the kernel, as the
 *              Qwen3.5-0.8B page (section 1.2) applies RoPE while loading q;
 *              the cached keys are expected already rotated
 *              (attn_kv_append with the same base).
 */
int attn_decode_padded(const void* q, const void* kcache, const void* vcache,
                       const int* seqlens, void* o, int B, int Hq, int Hkv,
                       int D, int cap, float scale, int num_splits, float* lse,
                       float rope_base, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * attn_decode_padded for fp16 caches (the ones attn_kv_append_f16 fills):
 * q, o, kcache, vcache in IEEE fp16.  Same arguments, workspace and errors.
 */
int attn_decode_padded_f16(const void* q, const void* kcache,
                           const void* vcache, const int* seqlens, void* o,
                           int B, int Hq, int Hkv, int D, int cap, float scale,
                           int num_splits, float* lse, float rope_base,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/* A static description of a status code ("ATTN_OK", ...). */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
