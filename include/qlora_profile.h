/*
 * qlora_profile.h -- opt-in per-kernel timing of libqlora.so (a tracing aid;
 * it has no counterpart on the method's pages and changes no result).
 *
 * Between qlora_profile_begin() and qlora_profile_end(), every kernel the
 * library enqueues is bracketed by two HIP events recorded on the stream it
 * is launched on.  qlora_profile_end() stops recording, waits for those
 * events (host-blocking) and sums the elapsed times per kernel name; the
 * summary stays readable until the next qlora_profile_begin().  Host memory
 * only; the returned name pointers stay valid until then.  Recording adds a
 * little time between kernels, so time end-to-end throughput separately.
 */
#ifndef QLORA_PROFILE_H_
#define QLORA_PROFILE_H_

#include <stdint.h>

typedef struct ihipStream_t *hipStream_t;

#ifdef __cplusplus
extern "C" {
#endif

int qlora_profile_begin(void);  /* clear the summary and start recording; QLORA_OK        */
int qlora_profile_end(void);    /* stop, wait, summarize; QLORA_ERR_HIP if an event failed  */
int qlora_profile_count(void);  /* number of distinct kernel names in the summary          */
/* Entry i of the summary: kernel name, number of launches, summed milliseconds.
 * QLORA_ERR_BAD_SHAPE (-2) when i is out of range. */
int qlora_profile_entry(int i, const char **name, int64_t *launches, double *total_ms);

/* The attainable BF16 matrix-core rate, as a denominator beside the 2.5
 * PFLOP/s spec peak: enqueue on `stream` one kernel of `workgroups` 4-wave
 * workgroups in which every wave issues v_mfma_f32_16x16x32_bf16 (the tile
 * kernels' instruction) back to back on 8 independent accumulator tiles,
 * `iters` rounds, no memory traffic; `out` (device, workgroups * 256 floats)
 * receives the accumulators, `*flops` the kernel's flop count.  The caller
 * times it with events on `stream`.  QLORA_ERR_BAD_SHAPE / QLORA_ERR_HIP. */
/* The forward of qlora_linear_fwd with the frozen weight already in BF16
 * (W_bf16 [n, k] device, e.g. qlora_dequant_bf16's output) on the same
 * kernels: the adapter product H, then the same tile kernel reading the BF16
 * tile instead of expanding NF4 codes (no block-scale table, no expansion).
 * The 16-bit baseline against which the NF4 dequantization's cost is
 * measured ("QLoRA Paper Breakdown", Engineering Limitations: dequantizing
 * on every use costs time against 16-bit LoRA).  Given W_bf16 = w_hat, Y and
 * H equal qlora_linear_fwd's bit for bit.  Arguments, workspace and status
 * as qlora_linear_fwd; one contraction split at every shape. */
int qlora_profile_linear_fwd_bf16w(const uint16_t *W_bf16, int64_t n, int64_t k, const uint16_t *X, int64_t M,
                                   const uint16_t *A, const uint16_t *B, int r, float alpha, uint16_t *Y, float *H_out,
                                   void *ws, size_t ws_bytes, hipStream_t stream);

int qlora_profile_mfma_peak(int64_t iters, int32_t workgroups, float *out, double *flops, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_PROFILE_H_ */
