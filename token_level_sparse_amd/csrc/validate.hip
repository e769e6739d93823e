// Checks of the device-side input contract of a batch (request lengths against
// their block-table rows, page ids against the pool; selections against their
// requests), for callers that want them before a step; the other kernels trust
// these inputs.
#include "common.h"
#include "kernels.h"

namespace ts {
namespace {

typedef unsigned long long u64;

__global__ void validate_init_kernel(u64* report) {
  if (threadIdx.x == 0) {
    report[0] = 0ull;            // violations
    report[1] = ~0ull;           // smallest (request << 32 | page) key of a violation
    report[2] = 0ull;            // requests whose length is outside [0, stride * 16]
    report[3] = 0ull;            // sum of the non-negative lengths
  }
}

// blockIdx.y = request; the x dimension strides over the request's block-table row.
__global__ __launch_bounds__(256) void validate_kernel(ValidateParams p) {
  const int r = blockIdx.y;
  const int32_t n = p.seq_lens[r];
  const int64_t cap = (int64_t)p.stride * kPage;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (n < 0 || n > cap) {
      atomicAdd(&p.report[0], 1ull);
      atomicAdd(&p.report[2], 1ull);
      atomicMin(&p.report[1], ((u64)r << 32) | 0xffffffffull);
    }
    if (n > 0) atomicAdd(&p.report[3], (u64)n);
  }
  // the pages the request reaches, never past its row
  const int64_t pages = n <= 0 ? 0 : ((int64_t)n + kPage - 1) / kPage;
  const int64_t reach = pages < p.stride ? pages : p.stride;
  const int32_t* row = p.block_table + (int64_t)r * p.stride;
  for (int64_t pi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; pi < reach;
       pi += (int64_t)gridDim.x * blockDim.x) {
    const int32_t v = row[pi];
    if (v < 0 || (int64_t)v >= p.pool_pages) {
      atomicAdd(&p.report[0], 1ull);
      atomicMin(&p.report[1], ((u64)r << 32) | (u64)pi);
    }
  }
}

// blockIdx.y = request; the x dimension strides over the request's TopK entries.
__global__ __launch_bounds__(256) void validate_selection_kernel(SelValidateParams p) {
  const int r = blockIdx.y;
  const int32_t n = p.seq_lens[r];
  const int32_t cnt = p.sel_count[r];
  const int32_t cap = min(p.top_k, max(n, 0));
  const bool count_ok = cnt >= 0 && cnt <= cap;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (!count_ok) {
      atomicAdd(&p.report[0], 1ull);
      atomicAdd(&p.report[2], 1ull);
      atomicMin(&p.report[1], ((u64)r << 32) | 0xffffffffull);
    } else {
      atomicAdd(&p.report[3], (u64)cnt);
    }
  }
  // the entries a consumer reads: the count, never past the row
  const int32_t m = count_ok ? cnt : min(max(cnt, 0), p.top_k);
  const int32_t* row = p.sel_idx + (int64_t)r * p.top_k;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < m; e += gridDim.x * blockDim.x) {
    const int32_t v = row[e];
    const bool in = v >= 0 && v < n;
    const bool asc = e == 0 || row[e - 1] < v;
    if (!in || !asc) {
      atomicAdd(&p.report[0], 1ull);
      atomicMin(&p.report[1], ((u64)r << 32) | (u64)e);
    }
  }
}

}  // namespace

hipError_t launch_validate_selection(const SelValidateParams& p, hipStream_t s) {
  hipLaunchKernelGGL(validate_init_kernel, dim3(1), dim3(64), 0, s, p.report);
  const int64_t chunks = ((int64_t)p.top_k + 255) / 256;
  const dim3 grid((unsigned)(chunks < 256 ? chunks : 256), (unsigned)p.b);
  hipLaunchKernelGGL(validate_selection_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_validate(const ValidateParams& p, hipStream_t s) {
  hipLaunchKernelGGL(validate_init_kernel, dim3(1), dim3(64), 0, s, p.report);
  const int64_t chunks = ((int64_t)p.stride + 255) / 256;
  const dim3 grid((unsigned)(chunks < 256 ? chunks : 256), (unsigned)p.b);
  hipLaunchKernelGGL(validate_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ts
