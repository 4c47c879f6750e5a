/*
 * qlora_nf4_timing.h -- kernel timing of libqlora_nf4_timing.so, a
 * measurement build of the same sources as libqlora_nf4.so (identical
 * kernels and entry points, declared in qlora_nf4.h). It is not part of the
 * method and not in the product library: libqlora_nf4.so exports none of
 * these symbols and keeps no mutable host state.
 *
 * In the timing build, between qlora_profile_begin(cap, mask) and
 * qlora_profile_end(), every launch of a kernel whose id bit is set in
 * `mask` (bit QLORA_K_*; 0 = all kernels) is bracketed by two hipEvents
 * recorded on the launch stream, up to `cap` launches; other launches get no
 * events. qlora_profile_query waits for the recorded events and returns the
 * number of launches of kernel `kernel_id` (QLORA_K_*) and their summed
 * duration in milliseconds. The event table is process-global state of the
 * timing build: calls are not thread-safe (one benchmarking thread), begin()
 * creates the events (host allocation) and release() destroys them.
 * Returns QLORA_ERR_INVALID_ARG for cap < 1 or NULL outputs, QLORA_ERR_HIP
 * if creating, waiting for or reading an event fails (begin() then leaves no
 * events behind).
 */
#ifndef QLORA_NF4_TIMING_H
#define QLORA_NF4_TIMING_H

#include "qlora_nf4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Ids 8 and 10 name no kernel of this library (their reductions are folded
 * into the producing kernels); they stay reserved so the other ids are stable. */
enum {
  QLORA_K_QUANTIZE = 0, QLORA_K_DOUBLE_QUANT = 1, QLORA_K_DEQUANTIZE = 2,
  QLORA_K_GEMM_FWD = 3, QLORA_K_GEMM_DX = 4, QLORA_K_GEMV = 5, QLORA_K_GEMV_EPILOGUE = 6,
  QLORA_K_LORA_DOWN = 7, QLORA_K_LORA_REDUCE = 8, QLORA_K_LORA_COLACC = 9,
  QLORA_K_LORA_COLACC_REDUCE = 10, QLORA_K_MERGE = 11, QLORA_K_LAYOUT = 12,
  QLORA_K_ADAMW = 13, QLORA_K_LOFTQ_PRODUCT = 14, QLORA_K_LOFTQ_SMALL = 15,
  QLORA_K_RESIDUAL = 16, QLORA_K_COUNT = 17
};
QLORA_API qlora_status qlora_profile_begin(int32_t cap, uint32_t mask);
QLORA_API qlora_status qlora_profile_end(void);
QLORA_API qlora_status qlora_profile_query(int32_t kernel_id, int32_t *count, double *total_ms);
QLORA_API qlora_status qlora_profile_release(void);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_TIMING_H */
