/*
 * qli_probe.h - measured ceilings of the MI355X the library runs on, so that
 * achieved rates can be reported against what this GPU sustains as well as
 * against its published peaks (HBM3E 8 TB/s, dense INT8 MFMA 5.0 POP/s).
 *
 * Both entry points enqueue one kernel on `stream` and return at once; the
 * caller times them (HIP events on the same stream) and computes the rate:
 *   bytes / time for qli_probe_hbm_read,
 *   qli_probe_int8_mfma_ops(grid, iterations) / time for qli_probe_int8_mfma.
 * They allocate nothing.  Returns a qli_status (qli.h).
 */
#ifndef QLI_PROBE_H
#define QLI_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Stream `bytes` (a multiple of 16, > 0) of device memory at `buf` (16-B
 * aligned) with 16-byte non-temporal vector loads, spread over `grid`
 * workgroups (1..65536) of 256 threads in contiguous runs; the loaded data
 * is folded into one word per workgroup that is written to `sink` (device,
 * `grid` words) only if it equals an impossible value, so the loads cannot
 * be removed and nothing else is written. */
int qli_probe_hbm_read(const void* buf, size_t bytes, int grid, uint32_t* sink, void* stream);

/* `grid` workgroups (1..65536) of 256 threads; every wave issues
 * `iterations` (1..2^20) rounds of four independent v_mfma_i32_32x32x32_i8
 * on register operands (no memory traffic), then writes to `sink` (device,
 * `grid` words) only on an impossible value. */
int qli_probe_int8_mfma(int grid, int iterations, uint32_t* sink, void* stream);

/* INT8 operations (2 per multiply-add) one qli_probe_int8_mfma launch performs. */
double qli_probe_int8_mfma_ops(int grid, int iterations);

#ifdef __cplusplus
}
#endif

#endif /* QLI_PROBE_H */
