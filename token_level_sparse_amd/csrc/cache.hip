// Step 0 of the decode step: the Selection Cache test.
//
// Source: TokenSelect deepnotes page, appendix Algorithm 1, and the blog page,
// section 3.2: reselect when there is no cached query yet or when the cosine of
// the current query with the cached one falls below theta; store the query (and,
// later in the step, the new TopK) only when reselecting; otherwise reuse the
// cached TopK. The query is every head's vector concatenated (H * d elements).
//
// One workgroup per request accumulates <Q, C_Q>, |Q|^2 and |C_Q|^2 in fp64 over
// the stored element values, in a fixed order, so the decision is reproducible
// and differs from an fp64 reference only when |cos - theta| is at the 1e-15
// level. A zero-norm query or cached query has no cosine and reselects. The same
// workgroup writes C_Q <- Q and valid <- 1 on a miss, after every thread has
// finished reading C_Q, and clears that request's radix histograms for the
// TopK kernels that follow.
#include "common.h"
#include "kernels.h"

namespace ts {
namespace {

// 16-byte chunk of the concatenated query: 8 bf16 or 4 fp32 elements.
template <bool kBf16> struct Chunk;
template <> struct Chunk<true> {
  static constexpr int kElems = 8;
  static __device__ __forceinline__ void get(const void* base, int64_t chunk, double (&x)[8]) {
    const uint4 w = static_cast<const uint4*>(base)[chunk];
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = (double)bf16_lo(v[e]);
      x[2 * e + 1] = (double)bf16_hi(v[e]);
    }
  }
};
template <> struct Chunk<false> {
  static constexpr int kElems = 4;
  static __device__ __forceinline__ void get(const void* base, int64_t chunk, double (&x)[8]) {
    const float4 w = static_cast<const float4*>(base)[chunk];
    x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
  }
};

template <bool kBf16>
__global__ __launch_bounds__(256) void cache_check_kernel(CacheParams p) {
  __shared__ double s_part[3][4];
  __shared__ int s_hit;
  using C = Chunk<kBf16>;
  const int r = blockIdx.x;
  const int64_t n = (int64_t)p.H * p.d;            // multiple of 128
  const int64_t nchunks = n / C::kElems;
  const int64_t cbase = (int64_t)r * nchunks;
  double dot = 0.0, qq = 0.0, cc = 0.0;
#pragma unroll 2
  for (int64_t j = threadIdx.x; j < nchunks; j += blockDim.x) {
    double a[8], c[8];
    C::get(p.q, cbase + j, a);
    C::get(p.cached_q, cbase + j, c);
#pragma unroll
    for (int e = 0; e < C::kElems; ++e) {
      dot = fma(a[e], c[e], dot);
      qq = fma(a[e], a[e], qq);
      cc = fma(c[e], c[e], cc);
    }
  }
  dot = wave_sum_d(dot);
  qq = wave_sum_d(qq);
  cc = wave_sum_d(cc);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { s_part[0][wave] = dot; s_part[1][wave] = qq; s_part[2][wave] = cc; }
  __syncthreads();
  if (threadIdx.x == 0) {
    const double d = ((s_part[0][0] + s_part[0][1]) + s_part[0][2]) + s_part[0][3];
    const double a = ((s_part[1][0] + s_part[1][1]) + s_part[1][2]) + s_part[1][3];
    const double c = ((s_part[2][0] + s_part[2][1]) + s_part[2][2]) + s_part[2][3];
    int hit = 0;
    if (p.valid[r] != 0 && a > 0.0 && c > 0.0) hit = (d / (sqrt(a) * sqrt(c)) >= p.theta) ? 1 : 0;
    s_hit = hit;
    p.hit[r] = hit;
  }
  __syncthreads();
  if (s_hit) return;
  const uint4* src = static_cast<const uint4*>(p.q) + cbase;
  uint4* dst = static_cast<uint4*>(p.cached_q) + cbase;
  for (int64_t j = threadIdx.x; j < nchunks; j += blockDim.x) dst[j] = src[j];
  uint32_t* h = p.hist + (int64_t)r * 3 * kHistBins;
  for (int i = threadIdx.x; i < 3 * kHistBins; i += blockDim.x) h[i] = 0u;
  if (p.mass) {
    unsigned long long* m = p.mass + (int64_t)r * 3 * kHistBins;
    for (int i = threadIdx.x; i < 3 * kHistBins; i += blockDim.x) m[i] = 0ull;
  }
  if (threadIdx.x == 0) p.valid[r] = 1;
}

}  // namespace

hipError_t launch_cache_check(const CacheParams& p, hipStream_t s) {
  if (p.bf16)
    hipLaunchKernelGGL(cache_check_kernel<true>, dim3(p.b), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(cache_check_kernel<false>, dim3(p.b), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ts
