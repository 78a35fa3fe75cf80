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

/*
 * Stream ceiling of one read:write mix: nsrc source streams (0 to 3) of
 * nbytes each, read in full, and, when dst is not NULL, one destination
 * stream of nbytes written in full with dst[i] = XOR of the sources' word i
 * (a fixed pattern when nsrc == 0). The access shape is the gate-add
 * kernels': 64-lane workgroups, nontemporal 128-bit loads and stores, lane t
 * of a workgroup on consecutive words, words_per_lane (1, 2 or 4) words per
 * lane strided by 64 words. It times what a mix of nsrc reads and one write
 * of the same size can reach on the device, apart from any arithmetic.
 *   - src: array of nsrc device pointers (may be NULL when nsrc == 0).
 *   - dst == NULL makes a read-only stream (nsrc >= 1): the XOR of all words
 *     is then folded per lane and written to the 16 bytes at sink only if it
 *     equals a fixed 128-bit pattern (so no load can be dropped); sink is a
 *     16-byte aligned device word the caller owns, otherwise unused.
 *   - dst == src[0] is the in-place form (each word is read, then written,
 *     by one lane); any other overlap of dst with a source, or of sink with
 *     any stream, is RGA_ERR_ALIAS.
 * Errors: nsrc outside 0..3, words_per_lane not 1, 2 or 4, nbytes < 0, a
 * NULL source, no destination with nsrc == 0, no sink for a read-only stream:
 * RGA_ERR_INVALID_ARG; nbytes % 16 != 0 or a pointer not 16-byte aligned:
 * RGA_ERR_UNSUPPORTED. nbytes == 0 is a no-op.
 */
int rga_stream(const void* const* src, int nsrc, void* dst, int64_t nbytes,
               int words_per_lane, void* sink, hipStream_t stream);

/* rga_stream's validation alone, on the host: the status rga_stream would
 * return before enqueueing anything (RGA_OK when it would launch). */
int rga_check_stream(const void* const* src, int nsrc, const void* dst, int64_t nbytes,
                     int words_per_lane, const void* sink);

/* Cache policy of the stores of rga_gate_add_variant. */
enum {
    RGA_STORE_NT = 0,     /* nontemporal (what every library kernel uses) */
    RGA_STORE_PLAIN = 1,  /* default policy: the lines stay dirty in the L2 */
    RGA_STORE_DEVICE = 2, /* device scope (SC1): written through the L2 into
                             the memory-side cache, which may hold them */
};

/*
 * The bf16 broadcast-gate add out = x + u * g of rga_residual_gate_add
 * (RGA_GATE_BCAST; same arithmetic, same result bit for bit) in a chosen
 * kernel shape, to measure the shapes the library does not use:
 *   - rows_per_wave (1, 2, 4 or 8): one wave takes a 64-pack column chunk
 *     of that many consecutive rows and loads its gate pack once for all of
 *     them (the row-tiled form of the residual-gate page's "B200 Nsight
 *     Compute check"); 1 is the library's shape;
 *   - store_policy: RGA_STORE_*.
 * Arguments, layout, aliasing and errors as rga_residual_gate_add with
 * gate_mode = RGA_GATE_BCAST (D % 8 == 0, 16-byte aligned pointers); a bad
 * rows_per_wave or store_policy is RGA_ERR_INVALID_ARG.
 */
int rga_gate_add_variant(const void* x, const void* u, const void* g, void* out,
                         int64_t B, int64_t L, int64_t D, int rows_per_wave,
                         int store_policy, hipStream_t stream);

/* rga_gate_add_variant's validation alone, on the host. */
int rga_check_gate_add_variant(const void* x, const void* u, const void* g, const void* out,
                               int64_t B, int64_t L, int64_t D, int rows_per_wave,
                               int store_policy);

/*
 * rga_rms_modulate_ex with row modulation (RGA_MOD_ROW) and
 * rga_gate_add_rms_modulate_ex with row modulation, with the number of
 * workgroups each CU may hold set by the caller: same kernels, arithmetic,
 * results and argument rules as those calls (plus wg_per_cu), to measure
 * the occupancy rule of the kernels that stage scale and shift rows in LDS
 * (two rows per workgroup; 2-byte storage). Those kernels ask for more LDS
 * than the staging needs so that only about a chosen amount of rows stays
 * on a CU: wg_per_cu > 0 asks for that many workgroups per CU, -1 for no cap
 * (the staging alone decides), 0 for the library's rule. Kernels that stage
 * nothing (binary32 rows, per-token modulation) ignore it.
 * wg_per_cu outside -1..16 is RGA_ERR_INVALID_ARG.
 */
int rga_modulate_occupancy(const void* x, const void* scale, const void* shift, float eps,
                           void* out, int64_t B, int64_t L, int64_t D, int dtype, int wg_per_cu,
                           hipStream_t stream);
int rga_fused_occupancy(const void* x, const void* u, const void* g, const void* scale,
                        const void* shift, float eps, void* x_out, void* y, int64_t B,
                        int64_t L, int64_t D, int gate_mode, int dtype, int wg_per_cu,
                        hipStream_t stream);

/* Their validation alone, on the host. */
int rga_check_modulate_occupancy(const void* x, const void* scale, const void* shift, float eps,
                                 const void* out, int64_t B, int64_t L, int64_t D, int dtype,
                                 int wg_per_cu);
int rga_check_fused_occupancy(const void* x, const void* u, const void* g, const void* scale,
                              const void* shift, float eps, const void* x_out, const void* y,
                              int64_t B, int64_t L, int64_t D, int gate_mode, int dtype,
                              int wg_per_cu);

/* Schedules of rga_modulate_variant and rga_fused_variant. */
enum {
    RGA_SCHED_LIBRARY = 0,     /* the library's own schedule */
    RGA_SCHED_LOADS_FIRST = 1, /* each row's loads issued before the workgroup
                                  stages its scale and shift rows (the
                                  modulation also reduces the row before the
                                  workgroup's barrier) */
    RGA_SCHED_ONE_PLUS = 2,    /* 1 + scale staged in LDS widened to binary32,
                                  two words per pack, beside the shift row */
    RGA_SCHED_TWO_ROWS = 3,    /* two rows per wave, one after the other */
    RGA_SCHED_PREFETCH = 4,    /* two rows per wave, the second row's loads
                                  issued before the first row is worked on */
};

/*
 * rms_modulate (bf16, row modulation) and rga_gate_add_rms_modulate (bf16,
 * RGA_GATE_BCAST) on rows of exactly 4096 elements, the workload's hidden
 * size, in a chosen schedule of the kernels that stage the batch's rows in
 * LDS (two rows, two waves, per workgroup; the library's occupancy rule),
 * to measure the schedules the library does not use. Every schedule
 * computes the same arithmetic in the same order: results equal the
 * library's bit for bit. Arguments, layout, aliasing and errors as
 * rms_modulate and rga_gate_add_rms_modulate (D % 8 == 0, 16-byte aligned
 * pointers), plus: D other than 4096 (and not 0) is RGA_ERR_UNSUPPORTED, a
 * schedule outside RGA_SCHED_* is RGA_ERR_INVALID_ARG.
 */
int rga_modulate_variant(const void* x, const void* scale, const void* shift, float eps,
                         void* out, int64_t B, int64_t L, int64_t D, int schedule,
                         hipStream_t stream);
int rga_fused_variant(const void* x, const void* u, const void* g, const void* scale,
                      const void* shift, float eps, void* x_out, void* y, int64_t B, int64_t L,
                      int64_t D, int schedule, hipStream_t stream);

/* Their validation alone, on the host. */
int rga_check_modulate_variant(const void* x, const void* scale, const void* shift, float eps,
                               const void* out, int64_t B, int64_t L, int64_t D, int schedule);
int rga_check_fused_variant(const void* x, const void* u, const void* g, const void* scale,
                            const void* shift, float eps, const void* x_out, const void* y,
                            int64_t B, int64_t L, int64_t D, int schedule);

#ifdef __cplusplus
}
#endif

#endif /* RGA_MEASURE_H */
