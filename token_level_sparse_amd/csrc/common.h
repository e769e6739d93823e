// Device helpers shared by the gfx950 kernels of the decode-step path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ts {

constexpr int kHeadDim = 128;     // the head dimension the kernels support
constexpr int kPage = 16;         // the page size (tokens) the kernels support
constexpr int kWave = 64;         // CDNA wavefront
constexpr int kXcds = 8;          // accelerator complex dies; workgroup i runs on XCD i % 8
constexpr int kMaxBatch = 1024;   // requests per call (LDS prefix tables)
constexpr int kMaxGroup = 8;      // query heads per KV head
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------- element types
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 2^x on the hardware exp unit; exp(x) = exp2(x * log2 e).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float exp_via2(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// ---------------------------------------------------------------- lane exchange
// DPP move inside a 16-lane row (row/bank masks full, out-of-row reads give 0).
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               kCtrl, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i inside each half row
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i inside each row

// Sum over the 16 lanes of a row; every lane of the row gets the total.
// The partner sets {^1}, {^2}, {^7}, {^15} span all 16 lanes.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  x += dpp_f<kDppMirror>(x);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ double wave_sum_d(double x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int wave_sum_i(int x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Merge two (max, sum of exp(x - max)) pairs; (-inf, 0) is the empty pair.
__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
  float mn = fmaxf(m, m2);
  if (mn == kNegInf) return;
  s = s * exp_via2(m - mn) + s2 * exp_via2(m2 - mn);
  m = mn;
}

// ---------------------------------------------------------------- ragged batch tables
// Fills s_tab[0..b] with the exclusive prefix of f(r) for r < b (s_tab[b] = total).
// Wave 0 does the work (each lane a run of requests, then a wave scan); every
// thread of the block must call it; ends with a barrier.
template <typename T, typename F>
__device__ void block_prefix(T* s_tab, int b, F f) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int per = (b + kWave - 1) / kWave;
    const int r0 = lane * per;
    const int r1 = min(b, r0 + per);
    T sum = 0;
    for (int r = r0; r < r1; ++r) sum += f(r);
    T inc = sum;
    for (int o = 1; o < kWave; o <<= 1) {
      T t = __shfl_up(inc, o);
      if (lane >= o) inc += t;
    }
    T run = inc - sum;
    for (int r = r0; r < r1; ++r) {
      s_tab[r] = run;
      run += f(r);
    }
    if (lane == kWave - 1) s_tab[b] = inc;
  }
  __syncthreads();
}

// Largest r in [0, b) with s_tab[r] <= x (s_tab ascending, s_tab[0] = 0 <= x).
template <typename T>
__device__ __forceinline__ int find_segment(const T* s_tab, int b, T x) {
  int lo = 0, hi = b - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_tab[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace ts
