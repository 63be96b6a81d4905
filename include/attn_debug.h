/*
 * attn_debug.h -- the per-tile softmax trace of the debug build of the
 * library (libattn_debug.so, compiled with ATTN_DEBUG_TRACE; the release
 * libattn.so does not export it).
 *
 * The attention-fusion page ("Attention三算子融合实战：从Triton到CUDA的推理加速优化",
 * section 6.3) debugs a fused kernel by printing the running row max m_i and
 * row sum l_i after every key block and comparing them with the reference's
 * values at the same positions.  This is that aid for the 4-wave and fp32
 * prefill kernels: after every key tile, the state of one chosen query row is
 * written to a device buffer instead of printed.
 */
#ifndef ATTN_DEBUG_H_
#define ATTN_DEBUG_H_

#ifdef __cplusplus
extern "C" {
#endif

#ifdef ATTN_DEBUG_TRACE
/*
 * Trace query row `row` of batch entry `b`, query head `h` in the prefill
 * launches enqueued after this call returns (until the next call).
 *   buf      : DEVICE float[3 * capacity], owned by the caller; NULL turns
 *              tracing off.  Record t (t-th key tile of the kernel: 64 keys
 *              for the 16-bit 4-wave kernel, 32 for the fp32 kernel) holds
 *              {keys covered so far (min((t + 1) * tile, S)), m, l}: m is the
 *              row's reference max in natural-log units of the scaled scores
 *              and l the sum of exp(s - m) over the visible keys so far, so
 *              m + ln l is the log-sum-exp of the scores seen.  Tiles past
 *              `capacity`, and tiles a causal kernel skips, write nothing.
 *   The traced kernels are the 4-wave 16-bit kernel and the fp32 kernel:
 *   call attn_prefill_select(ATTN_PREFILL_W4) first for 16-bit inputs.
 * The target is copied to the device synchronously (the null stream).
 * Errors: a negative index or capacity with buf != NULL -> ATTN_ERR_SHAPE;
 * buf not 4-byte aligned -> ATTN_ERR_ALIGN; the copy failed ->
 * ATTN_ERR_LAUNCH.
 */
int attn_debug_trace(int b, int h, int row, float* buf, int capacity);
#endif

#ifdef __cplusplus
}
#endif

#endif  /* ATTN_DEBUG_H_ */
