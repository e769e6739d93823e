/* Streaming-bandwidth probe (libts_stream_probe.so): measurement infrastructure
 * for bench.py, not part of the TokenSelect method.
 *
 * ts_stream_probe reads `bytes` bytes from device buffer `src` (16-byte aligned,
 * bytes a multiple of 16) with `grid` workgroups of 256 threads, each reading one
 * contiguous range with 16-byte nontemporal loads. With `write` nonzero it also
 * writes bytes / 16 bytes to device buffer `dst` (16-byte aligned, at least
 * bytes / 16 bytes long): 2 KB per 32 KB read, contiguous per workgroup, the
 * read/write mix of the decode step's scoring pass (2048 bytes of K read and 128
 * bytes of fp32 logits written per token at 32 query / 8 KV heads, d = 128, bf16).
 * The written values are meaningless. `sink` is a device uint32 the kernel may
 * write to keep its loads live. The launch is asynchronous on `stream`.
 * Returns 0 on success, -1 on an invalid argument (nothing launched), or the
 * hipError_t of the launch. The caller owns every buffer.
 */
#ifndef TS_STREAM_PROBE_H
#define TS_STREAM_PROBE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int ts_stream_probe(const void* src, size_t bytes, void* dst, int write, int grid, uint32_t* sink,
                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
