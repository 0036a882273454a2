/*
 * ah_instrument.h -- measurement hooks of libah.so.
 *
 * Not part of the search path (include/ah.h): a benchmark or a profiler uses
 * these to time the dominant scan kernel on its own, to read the scan's own
 * counters after a call, and to measure the HBM read rate that a plain stream
 * of 16-byte loads reaches on this GPU (the measured reference for the code
 * scan's bytes per second).  Conventions as in ah.h: device pointers owned by
 * the caller, every call only enqueues on `stream`, AH_OK or a negative
 * AH_ERR_* status checked on the host before anything is enqueued.
 */
#ifndef AH_INSTRUMENT_H
#define AH_INSTRUMENT_H

#include "ah.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ah_scan_topk with two caller-created hipEvent_t handles (either may be NULL)
 * recorded on `stream` immediately before and after the main scan kernel (the
 * leaf inversion, threshold warm-up and final selection run outside the pair).
 * Arguments, results and errors are those of ah_scan_topk. */
int ah_scan_topk_timed(const int8_t* lut_i8, int64_t nq, int32_t B, const uint8_t* codes,
                       int32_t code_stride, int64_t n, const int32_t* ids,
                       const int64_t* leaf_offsets, int32_t L, const int32_t* leaves, int32_t nl,
                       int32_t R, int32_t* cand_ids_out, int32_t* cand_scores_out, void* workspace,
                       size_t workspace_bytes, void* stream, void* main_start_event,
                       void* main_stop_event);

/* Byte offsets, inside a workspace of ah_scan_workspace_bytes(nq, B, n, L, nl,
 * R) bytes, of the scan's counters as the last ah_scan_topk call on that
 * workspace left them (read them after the stream has finished the call):
 *   appended_offset: uint32 [nq], rows appended to each query's candidate list
 *                    (every row whose sum reached the query's running threshold);
 *   control_offset:  uint32 [16]; word 1 = queries whose candidate list
 *                    overflowed and were recomputed by the exact fallback.
 * Errors: AH_ERR_NULL (an output pointer), AH_ERR_SHAPE (sizes as for
 * ah_scan_workspace_bytes). */
int ah_scan_workspace_counters(int64_t nq, int32_t B, int64_t n, int32_t L, int32_t nl, int32_t R,
                               size_t* appended_offset, size_t* control_offset);

/* Reads `bytes` of device memory at `data` once, with nontemporal 16-byte
 * loads in a grid-stride loop (blocks_per_cu x 256 workgroups of 256 threads,
 * four loads in flight per thread), and writes sink[0] only if the XOR of every word read
 * equals a fixed improbable value (so the loads cannot be dropped).  Bytes per
 * second of this call are the plain-stream HBM read rate.
 * Errors: AH_ERR_NULL (data or sink with bytes > 0), AH_ERR_SHAPE (bytes not
 * a multiple of 16, blocks_per_cu outside 1..64), AH_ERR_UNSUPPORTED (data not
 * 16-byte aligned).  bytes == 0 is a no-op. */
int ah_hbm_read_probe(const void* data, size_t bytes, int32_t blocks_per_cu, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AH_INSTRUMENT_H */
