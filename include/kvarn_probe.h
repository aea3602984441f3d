/*
 * kvarn_probe.h -- measurement helper of the benchmark, not part of the KVarN ABI
 * (libkvarn_probe.so, built beside libkvarn.so).
 */
#ifndef KVARN_PROBE_H
#define KVARN_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` of device memory at src_dev once (16-byte nontemporal loads; `grid`
 * workgroups of 256 lanes, each reading a contiguous 1 / grid of the buffer) on `stream` (a hipStream_t as void*).
 * Each workgroup writes one checksum word to sink_dev[blockIdx] (uint32[grid], device).
 * The launch's bytes / duration is the streaming-read bandwidth the decode reports its
 * fraction of. Returns 0 on success, 1 for a NULL pointer, a grid outside [1, 65536], a size
 * that is not a multiple of 16 or a misaligned pointer (nothing enqueued), 4 if the launch
 * failed. bytes == 0 is a no-op. */
__attribute__((visibility("default"))) int kvarn_probe_stream_read(const void* src_dev,
                                                                   size_t bytes, void* sink_dev,
                                                                   int32_t grid, void* stream);

/* VALU issue calibration: `grid` workgroups of 256 lanes each run `rounds` rounds of 32
 * float32 FMAs (eight independent chains per lane) and store one float per lane to out_dev
 * (float[grid * 256], device). rounds * 32 * grid * 4 wave64 FMA instructions over 1024 SIMDs
 * and the launch's duration give the cycles per instruction at the clock of the run.
 * Returns 0, 1 (bad argument, nothing enqueued) or 4 (launch failed). */
__attribute__((visibility("default"))) int kvarn_probe_valu_fma(void* out_dev, int32_t grid,
                                                                int32_t rounds, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVARN_PROBE_H */
