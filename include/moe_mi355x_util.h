/*
 * moe_mi355x_util.h -- measurement kernels exported by the same library.
 *
 * The denominators of the bandwidth figures are measured, not assumed: the
 * warp-decode post (hardware-efficiency section) rates its decode against a
 * copy kernel reading contiguous memory on the same GPU, and so do we.
 * Conventions as in moe_mi355x.h (device pointers, async on `stream`).
 */
#ifndef MOE_MI355X_UTIL_H
#define MOE_MI355X_UTIL_H

#include <stddef.h>
#include <stdint.h>

#include "moe_mi355x.h"

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0:bytes) = src[0:bytes): one 16-byte load and store per thread over a
 * grid that covers the buffer.  bytes must be a multiple of 16 and both
 * pointers 16-byte aligned; MOE_ERR_UNSUPPORTED past (2^31-1)*256
 * elements (the same limit holds for the read and the fill below). */
moe_status moe_util_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Reads src[0:bytes) (one 16-byte load per thread) and may write one float
 * per workgroup to sink[0:moe_util_read_sink_len()) (index taken modulo that
 * length), a store that depends on the loaded words so the loads stay live. */
moe_status moe_util_read(const void* src, size_t bytes, float* sink, void* stream);
int32_t moe_util_read_sink_len(void);

/* Writes `value` to every 32-bit word of dst[0:bytes), one 16-byte store per
 * thread: evicts caches between timed calls.  bytes must be a multiple of 16
 * and dst 16-byte aligned. */
moe_status moe_util_fill(void* dst, size_t bytes, uint32_t value, void* stream);

/* Compute units of the current device (cached). */
int32_t moe_util_num_cus(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_UTIL_H */
