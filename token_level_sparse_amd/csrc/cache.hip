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

template <bool kBf16>
__device__ __forceinline__ double elem(const void* base, int64_t i) {
  if (kBf16) return (double)__uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[i] << 16);
  return (double)static_cast<const float*>(base)[i];
}

template <bool kBf16>
__global__ __launch_bounds__(256) void cache_check_kernel(CacheParams p) {
  __shared__ double s_part[3][4];
  __shared__ int s_hit;
  const int r = blockIdx.x;
  const int64_t n = (int64_t)p.H * p.d;
  const int64_t base = (int64_t)r * n;
  double dot = 0.0, qq = 0.0, cc = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const double a = elem<kBf16>(p.q, base + i);
    const double c = elem<kBf16>(p.cached_q, base + i);
    dot = fma(a, c, dot);
    qq = fma(a, a, qq);
    cc = fma(c, c, cc);
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
  if (kBf16) {
    const uint16_t* src = static_cast<const uint16_t*>(p.q) + base;
    uint16_t* dst = static_cast<uint16_t*>(p.cached_q) + base;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) dst[i] = src[i];
  } else {
    const float* src = static_cast<const float*>(p.q) + base;
    float* dst = static_cast<float*>(p.cached_q) + base;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) dst[i] = src[i];
  }
  uint32_t* h = p.hist + (int64_t)r * 3 * kHistBins;
  for (int i = threadIdx.x; i < 3 * kHistBins; i += blockDim.x) h[i] = 0u;
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
