/* Streaming-bandwidth and chunk-attention phase probes (libts_stream_probe.so):
 * measurement infrastructure for bench.py, not part of the TokenSelect method.
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

/* Chunk-attention phase probe (phase_probe.hip): `grid` workgroups of 512 threads
 * repeat `iters` times the instruction mix of one phase of the bf16 chunk attention's
 * block loop (mode 0: the scores of the next block with this block's exp2; 1: the
 * P V products; 2: the two alternating per SIMD; 3: mode 0 without the exp2; 4: mode 0
 * without the matrix products) on LDS-resident data taken from `src` (device, 16-byte
 * aligned, src_bytes >= 40960). Each wave writes its start and end wall clock
 * (s_memrealtime, 100 MHz) to times[2 * (8 * workgroup + wave) + {0, 1}] (device,
 * 16 * grid u64) and one float per thread to out (device, 512 * grid floats; values
 * meaningless). Asynchronous on `stream`; returns 0, -1 on an invalid argument (nothing
 * launched), or the hipError_t of the launch. The caller owns every buffer. */
int ts_chunk_phase_probe(int mode, int iters, int grid, const void* src, size_t src_bytes, float* out,
                         unsigned long long* times, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
