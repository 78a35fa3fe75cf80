/*
 * rga_measure.h — measurement helpers of the same library. They are not part
 * of the gated-residual / modulation path; the bench uses them to measure the
 * attainable HBM bandwidth on the same device (a plain copy moves a known
 * number of bytes, which also calibrates the HBM traffic counters) and to
 * evict the device's caches before a cold timing.
 *
 * Same conventions as rga.h: device pointers, caller-owned buffers,
 * asynchronous on `stream`, RGA_* status codes.
 */
#ifndef RGA_MEASURE_H
#define RGA_MEASURE_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * dst[i] = src[i] for nbytes bytes with 128-bit loads and stores.
 * nbytes must be a multiple of 16 and both pointers 16-byte aligned
 * (RGA_ERR_UNSUPPORTED); the ranges must not overlap (RGA_ERR_ALIAS);
 * NULL with nbytes > 0 or nbytes < 0 is RGA_ERR_INVALID_ARG.
 */
int rga_copy(const void* src, void* dst, int64_t nbytes, hipStream_t stream);

/*
 * Writes nbytes of dst (every 32-bit word set to `value`) with 128-bit
 * plain stores. Same argument rules as rga_copy (no source).
 */
int rga_fill(void* dst, int64_t nbytes, uint32_t value, hipStream_t stream);

/*
 * Reads all nbytes of src with plain, cache-allocating 128-bit loads and
 * XORs every 16-byte word of src into the 16 bytes at sink (device memory,
 * 16-byte aligned; the caller initialises it). Reading a buffer larger than
 * the caches evicts earlier data while leaving only clean lines, which makes
 * it the cache flush of a cold timing. nbytes must be a multiple of 16;
 * sink must not overlap src (RGA_ERR_ALIAS).
 */
int rga_read(const void* src, int64_t nbytes, void* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RGA_MEASURE_H */
