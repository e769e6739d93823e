// Chunk-attention phase probe (libts_stream_probe.so): measurement infrastructure for
// bench.py --phase-probe, not part of the TokenSelect method.
//
// Each wave of 8-wave workgroups (two waves per SIMD, as the bf16 chunk attention
// runs) repeats the instruction mix of one phase of that kernel's 64-key block loop on
// LDS-resident data, with no staging and no barriers, and records its wall-clock time:
//   EXP: 16 K operand reads (ds_read_b128), 16 v_mfma_f32_32x32x16_bf16 (the next
//        block's scores) and, between them, the 32 probabilities of one row half
//        (fma, v_exp_f32, sum), as the attention kernel interleaves them;
//   PV:  32 transposed V reads (ds_read_b64_tr_b16), 16 cvt to bf16, 16 MFMAs.
// Modes: 0 EXP twice per iteration; 1 PV twice; 2 EXP then PV in waves 0-3 and PV then
// EXP in waves 4-7 (each SIMD runs one wave of each kind); 3 EXP with the exp2 replaced
// by its fma argument; 4 EXP with the MFMAs replaced by one add each. Comparing 0, 3
// and 4 shows whether v_exp_f32 overlaps the matrix cores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ts_stream_probe.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
constexpr int kRow = 256;                     // bytes of one 128-dim bf16 row
constexpr int kKeys = 64;                     // rows per LDS block
constexpr int kThreads = 512;
__device__ __forceinline__ int k_pos(int x, int c) { return c ^ (x & 15); }
__device__ __forceinline__ int v_pos(int x, int c) { return c ^ ((x & 3) << 1); }

template <bool kExp, bool kMfma>
__device__ __forceinline__ float exp_phase(const char* kb, const bf16x8_t (&q)[8], f32x16_t (&cur)[2],
                                           f32x16_t (&nxt)[2], int l32, int lg, float nm, float sl2) {
  f32x16_t a0 = {}, a1 = {};
  float psum = 0.f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const bf16x8_t k0 = *reinterpret_cast<const bf16x8_t*>(kb + l32 * kRow + 16 * k_pos(l32, 2 * ks + lg));
    const bf16x8_t k1 = *reinterpret_cast<const bf16x8_t*>(kb + (32 + l32) * kRow + 16 * k_pos(32 + l32, 2 * ks + lg));
    if (kMfma) a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, q[ks], a0, 0, 0, 0);
    else a0[ks] += (float)k0[0];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float x = cur[ks >> 2][4 * (ks & 3) + e];
      const float pr = kExp ? __builtin_amdgcn_exp2f(fmaf(x, sl2, nm)) : fmaf(x, sl2, nm);
      cur[ks >> 2][4 * (ks & 3) + e] = pr;
      psum += pr;
    }
    if (kMfma) a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, q[ks], a1, 0, 0, 0);
    else a1[ks] += (float)k1[0];
#pragma unroll
    for (int e = 2; e < 4; ++e) {
      const float x = cur[ks >> 2][4 * (ks & 3) + e];
      const float pr = kExp ? __builtin_amdgcn_exp2f(fmaf(x, sl2, nm)) : fmaf(x, sl2, nm);
      cur[ks >> 2][4 * (ks & 3) + e] = pr;
      psum += pr;
    }
  }
  nxt[0] = a0;
  nxt[1] = a1;
  return psum;
}

__device__ __forceinline__ void pv_phase(const char* vb, const f32x16_t (&p)[2], int l32, int lg, f32x16_t (&o)[4]) {
  const int s = threadIdx.x & 15, half = l32 >> 4;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int b8 = 8 * hh;
      const bf16x8_t pb = {(__bf16)p[t][b8], (__bf16)p[t][b8 + 1], (__bf16)p[t][b8 + 2], (__bf16)p[t][b8 + 3],
                           (__bf16)p[t][b8 + 4], (__bf16)p[t][b8 + 5], (__bf16)p[t][b8 + 6], (__bf16)p[t][b8 + 7]};
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int x = 32 * t + 16 * hh + 4 * lg + (s >> 2);        // x + 8 < kKeys
        const int c = 4 * dt + 2 * half + ((s & 3) >> 1), b = 8 * (s & 1);
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + x * kRow + 16 * v_pos(x, c) + b));
        const s16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + (x + 8) * kRow + 16 * v_pos(x + 8, c) + b));
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, o[dt], 0, 0, 0);
      }
    }
}

// src: at least kSrcVec 16-byte vectors (K block, V block, query operands).
constexpr int kBlockVec = kKeys * kRow / 16;                 // 1024
constexpr int kSrcVec = 2 * kBlockVec + 64 * 8;              // 2560

template <int kMode>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void phase_kernel(const uint4* src, float* out, unsigned long long* times, int iters) {
  __shared__ __align__(16) char s_k[kKeys * kRow];
  __shared__ __align__(16) char s_v[kKeys * kRow];
  for (int i = threadIdx.x; i < kBlockVec; i += kThreads) {
    reinterpret_cast<uint4*>(s_k)[i] = src[i];
    reinterpret_cast<uint4*>(s_v)[i] = src[kBlockVec + i];
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, lg = lane >> 5;
  bf16x8_t q[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) q[ks] = __builtin_bit_cast(bf16x8_t, src[2 * kBlockVec + lane * 8 + ks]);
  f32x16_t sa[2] = {}, sb[2] = {}, o[4] = {};
  float acc = 0.f;
  const float sl2 = 0.1275f, nm = -(float)(wave & 3);
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    if (kMode == 0 || kMode == 3 || kMode == 4) {
      constexpr bool kExp = kMode != 3, kMfma = kMode != 4;
      acc += exp_phase<kExp, kMfma>(s_k, q, sa, sb, l32, lg, nm, sl2);
      acc += exp_phase<kExp, kMfma>(s_k, q, sb, sa, l32, lg, nm, sl2);
    } else if (kMode == 1) {
      pv_phase(s_v, sa, l32, lg, o);
      pv_phase(s_v, sb, l32, lg, o);
    } else if (wave < 4) {
      acc += exp_phase<true, true>(s_k, q, sa, sb, l32, lg, nm, sl2);
      pv_phase(s_v, sa, l32, lg, o);
    } else {
      pv_phase(s_v, sb, l32, lg, o);
      acc += exp_phase<true, true>(s_k, q, sb, sa, l32, lg, nm, sl2);
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc += o[d][i];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc += sa[0][i] + sb[1][i];
  out[blockIdx.x * kThreads + threadIdx.x] = acc;
  if (lane == 0) {
    times[(blockIdx.x * 8 + wave) * 2] = t0;
    times[(blockIdx.x * 8 + wave) * 2 + 1] = t1;
  }
}

}  // namespace

extern "C" int ts_chunk_phase_probe(int mode, int iters, int grid, const void* src, size_t src_bytes, float* out,
                                    unsigned long long* times, hipStream_t stream) {
  if (mode < 0 || mode > 4 || iters < 1 || grid < 1 || !src || !out || !times ||
      src_bytes < (size_t)kSrcVec * 16 || ((uintptr_t)src & 15))
    return -1;
  const dim3 g(grid), b(kThreads);
  const uint4* s = static_cast<const uint4*>(src);
  switch (mode) {
    case 0: hipLaunchKernelGGL(phase_kernel<0>, g, b, 0, stream, s, out, times, iters); break;
    case 1: hipLaunchKernelGGL(phase_kernel<1>, g, b, 0, stream, s, out, times, iters); break;
    case 2: hipLaunchKernelGGL(phase_kernel<2>, g, b, 0, stream, s, out, times, iters); break;
    case 3: hipLaunchKernelGGL(phase_kernel<3>, g, b, 0, stream, s, out, times, iters); break;
    default: hipLaunchKernelGGL(phase_kernel<4>, g, b, 0, stream, s, out, times, iters); break;
  }
  return (int)hipGetLastError();
}
