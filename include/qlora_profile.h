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

#ifdef __cplusplus
extern "C" {
#endif

int qlora_profile_begin(void);  /* clear the summary and start recording; QLORA_OK        */
int qlora_profile_end(void);    /* stop, wait, summarize; QLORA_ERR_HIP if an event failed  */
int qlora_profile_count(void);  /* number of distinct kernel names in the summary          */
/* Entry i of the summary: kernel name, number of launches, summed milliseconds.
 * QLORA_ERR_BAD_SHAPE (-2) when i is out of range. */
int qlora_profile_entry(int i, const char **name, int64_t *launches, double *total_ms);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_PROFILE_H_ */
