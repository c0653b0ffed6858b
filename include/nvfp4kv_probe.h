/*
 * nvfp4kv_probe — measurement aid of the nvfp4kv benchmark (libnvfp4kv_probe.so).
 *
 * Not an operation of the NVFP4 KV cache: it gives the HBM read rate a plain
 * kernel reaches on the same device and the same number of bytes, the
 * ceiling against which the attention kernels' cache-read stream is judged.
 */
#ifndef NVFP4KV_PROBE_H
#define NVFP4KV_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes at device pointer `data` (16-byte aligned, bytes a
 * positive multiple of 16) with `grid` workgroups of 256 lanes, 16 bytes per
 * lane and load, and write one XOR fold per wave to `sink` (device, at least
 * grid * 16 bytes, 4-byte aligned). Asynchronous on `stream`. Returns 0, 1
 * for a bad argument (nothing launched) or 4 if the launch failed.
 */
int32_t nvfp4kv_probe_read_stream(const void* data, int64_t bytes, int32_t grid, void* sink, int64_t sink_bytes,
                                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4KV_PROBE_H */
