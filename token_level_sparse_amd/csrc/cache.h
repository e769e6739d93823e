// Step 0 of the decode step: the Selection Cache test, as a device function.
//
// Source: TokenSelect deepnotes page, appendix Algorithm 1, and the blog page,
// section 3.2: reselect when there is no cached query yet or when the cosine of
// the current query with the cached one falls below theta; store the query (and,
// later in the step, the new TopK) only when reselecting; otherwise reuse the
// cached TopK. The query is every head's vector concatenated (H * d elements).
//
// A workgroup accumulates <Q, C_Q>, |Q|^2 and |C_Q|^2 in fp64 over the stored
// element values in a fixed order: every workgroup that evaluates a request gets
// the same bits, so the workgroups of the score kernel agree on the decision
// without exchanging it. The result differs from an fp64 reference only when
// |cos - theta| is at the 1e-15 level. A zero-norm query or cached query has no cosine and reselects.
#pragma once

#include "common.h"

namespace ts {

// 16-byte chunk of the concatenated query: 8 bf16 or 4 fp32 elements.
template <bool kBf16> struct QChunk;
template <> struct QChunk<true> {
  static constexpr int kElems = 8;
  static __device__ __forceinline__ void cvt(const uint4& w, double (&x)[8]) {
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = (double)bf16_lo(v[e]);
      x[2 * e + 1] = (double)bf16_hi(v[e]);
    }
  }
};
template <> struct QChunk<false> {
  static constexpr int kElems = 4;
  static __device__ __forceinline__ void cvt(const uint4& w, double (&x)[8]) {
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
  }
};

// The first kCachePre chunks of each thread (t, t + 256) of request r's query and
// cached query, requested ahead of the caller's other loads; cache_hit_wg adds them
// first, so the sums keep their order.
constexpr int kCachePre = 2;
// |cos| <= 1 (Cauchy-Schwarz); the fp64 quotient exceeds 1 by a few units of 2^-53 at most
constexpr double kCacheNeverHit = 1.0 + 0x1p-20;
struct CachePre {
  uint4 q[kCachePre], c[kCachePre];
};
template <bool kBf16>
__device__ __forceinline__ void cache_preload(const void* q, const void* cached_q, int r, int n, CachePre& pre) {
  const int64_t nchunks = n / QChunk<kBf16>::kElems;
  const int64_t cbase = (int64_t)r * nchunks;
#pragma unroll
  for (int u = 0; u < kCachePre; ++u) {
    const int64_t j = threadIdx.x + 256 * u;
    if (j < nchunks) {
      pre.q[u] = static_cast<const uint4*>(q)[cbase + j];
      pre.c[u] = static_cast<const uint4*>(cached_q)[cbase + j];
    }
  }
}

// Selection Cache decision for request r, evaluated by a whole 256-thread
// workgroup (every thread must call it: it holds two barriers). Thread t sums the
// 16-byte chunks t, t + 256, ...; the four wavefront sums are added in wave order,
// so every workgroup that decides request r gets the same bits. s_red is LDS
// scratch of 12 doubles. `pre`, if not null, holds request r's chunks loaded by
// cache_preload. Returns the decision to every thread.
template <bool kBf16>
__device__ int cache_hit_wg(const void* q, const void* cached_q, int r, int n, int valid,
                            double theta, double (*s_red)[4], const CachePre* pre = nullptr) {
  // theta above 1 (plus a margin well beyond the rounding of the cosine): the test
  // can never pass, and every request reselects without reading either query
  if (theta > kCacheNeverHit) return 0;
  using C = QChunk<kBf16>;
  const int64_t nchunks = n / C::kElems;
  const int64_t cbase = (int64_t)r * nchunks;
  double dot = 0.0, qq = 0.0, cc = 0.0;
  auto add = [&](const uint4& wq, const uint4& wc) {
    double a[8], c[8];
    C::cvt(wq, a);
    C::cvt(wc, c);
#pragma unroll
    for (int e = 0; e < C::kElems; ++e) {
      dot = fma(a[e], c[e], dot);
      qq = fma(a[e], a[e], qq);
      cc = fma(c[e], c[e], cc);
    }
  };
  int64_t j = threadIdx.x;
  if (pre) {
#pragma unroll
    for (int u = 0; u < kCachePre; ++u, j += 256)
      if (j < nchunks) add(pre->q[u], pre->c[u]);
  }
  for (; j < nchunks; j += 256)
    add(static_cast<const uint4*>(q)[cbase + j], static_cast<const uint4*>(cached_q)[cbase + j]);
  dot = wave_sum_d(dot);
  qq = wave_sum_d(qq);
  cc = wave_sum_d(cc);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & (kWave - 1)) == 0) { s_red[0][wave] = dot; s_red[1][wave] = qq; s_red[2][wave] = cc; }
  __syncthreads();
  dot = ((s_red[0][0] + s_red[0][1]) + s_red[0][2]) + s_red[0][3];
  qq = ((s_red[1][0] + s_red[1][1]) + s_red[1][2]) + s_red[1][3];
  cc = ((s_red[2][0] + s_red[2][1]) + s_red[2][2]) + s_red[2][3];
  __syncthreads();                                    // s_red free for the next call
  if (valid == 0 || !(qq > 0.0) || !(cc > 0.0)) return 0;
  return (dot / (sqrt(qq) * sqrt(cc)) >= theta) ? 1 : 0;
}

}  // namespace ts
