/*
 * pace_measure.h -- measurement kernels that bound what one decode launch can achieve on
 * this device.  They are not part of the method; bench.py times them beside the decode
 * kernel so that its bandwidth fraction can be read against ceilings measured on the same
 * box, in the same launch shape and the same graph conditions.
 *
 * Built into bit_recurrent_state_amd/libpace_measure.so.  Plain C; pointers are device
 * pointers owned by the caller; nothing allocates or synchronises.  Every call returns
 * 0 (hipSuccess) or the HIP error of its launch, and -1 for invalid arguments (nothing
 * launched).
 */
#ifndef PACE_MEASURE_H
#define PACE_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A kernel that does nothing, launched as grid (gx, gy) x `threads` threads: the fixed
 * cost of a launch of that shape (dispatch, start-up and end of kernel) inside a graph.
 * Errors: -1 for gx, gy < 1 or threads not a multiple of 64 in [64, 1024]. */
int pace_measure_empty(int32_t gx, int32_t gy, int32_t threads, void* stream);

/* Read-only stream in the decode kernel's launch shape: grid (gx, gy) of `threads`
 * threads, workgroup w = y * gx + x reads bytes_per_wg contiguous bytes starting at
 * src + w * bytes_per_wg with 16-byte non-temporal vector loads (as the decode kernel reads
 * its packed state), folds them with XOR and writes one 4-byte word per workgroup to
 * sink[w].  Moves gx * gy * bytes_per_wg bytes: an upper bound for the decode launch's
 * own memory stream in the same shape.
 * src: at least gx * gy * bytes_per_wg bytes, 16-byte aligned; sink: gx * gy words.
 * Errors: -1 for null pointers, misaligned src, bytes_per_wg not a positive multiple of 16,
 * or a bad shape (as above). */
int pace_measure_stream(const void* src, size_t bytes_per_wg, int32_t gx, int32_t gy,
                        int32_t threads, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PACE_MEASURE_H */
