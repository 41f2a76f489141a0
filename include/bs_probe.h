/*
 * bs_probe.h -- C ABI of the measurement kernels (libbsprobe.so), built next
 * to the GEMV library and used by the benchmark only: they compute nothing of
 * the hot path.  They give, in the same process and on the same stream as
 * the GEMVs, the two hardware terms every GEMV time is read against:
 *   - the cost of launching a kernel that does nothing (the dispatch floor);
 *   - the time a plain streaming read of exactly a GEMV's weight bytes takes
 *     (the read ceiling of that shape: the GEMV streams the same bytes and
 *     must also compute and store).
 * "BitState / HSDR PoC Technical Brief - v0.5", section 9, names memory
 * bandwidth among the quantities to report and section 10 asks for the
 * limiting term to be isolated; these kernels isolate it.
 *
 * Status codes are those of bs.h (0 = OK, -3 = out of range, -5 = HIP).
 * Device pointers are caller-owned; calls enqueue on `stream` (hipStream_t
 * as void*, NULL = default stream) and return.
 */
#ifndef BS_PROBE_H
#define BS_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * bs_probe_read -- read `bytes` bytes at `src` once with 16-byte
 * non-temporal loads (workgroups of 256 threads, `per_thread` loads each:
 * 1, 2, 4 or 8), fold them with xor and store one int64 per thread to
 * `sink` (bs_probe_read_sink_count(bytes, per_thread) of them), so no load
 * is dead.  Loads past `bytes` read zero.
 *   src   device, 16-byte aligned;  1 <= bytes <= 2^31 - 16
 *   sink  device int64[bs_probe_read_sink_count(...)], 8-byte aligned
 * Errors: -1 (NULL), -3 (bytes, per_thread), -5 (launch).
 */
int64_t bs_probe_read_sink_count(uint64_t bytes, int32_t per_thread);
int32_t bs_probe_read(const void *src, uint64_t bytes, int32_t per_thread, int64_t *sink,
                      void *stream);

/*
 * bs_probe_read_strided -- the same read with a fixed grid: `blocks`
 * workgroups of 256 threads (1 <= blocks <= 65536), each reading 32 KB
 * contiguous per step and striding by the grid's span, then one int64 per
 * thread to `sink` (blocks * 256 of them).  For large buffers, where the
 * one-pass grid grows with the bytes.  Same limits on src and bytes.
 * Errors: -1 (NULL), -3 (bytes, blocks, alignment), -5 (launch).
 */
int32_t bs_probe_read_strided(const void *src, uint64_t bytes, int32_t blocks, int64_t *sink,
                              void *stream);

/*
 * bs_probe_empty -- launch `blocks` workgroups of `threads` threads
 * (1 <= blocks <= 2^20, threads 64..1024, a multiple of 64) that do nothing.
 * Errors: -3 (sizes), -5 (launch).
 */
int32_t bs_probe_empty(int32_t blocks, int32_t threads, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* BS_PROBE_H */
