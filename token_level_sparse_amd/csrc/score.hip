// Steps 1-2 of the decode step: paged Q.K scoring and per-head softmax statistics.
//
// Source: TokenSelect deepnotes page, appendix Algorithm 2 (Paged Dot Product
// Kernel: per head, the query is held on chip while blocks of paged keys are read
// once from HBM and their inner products written back), and the head soft vote
// equation (softmax of each head's raw inner products over all cached tokens).
//
// gfx950 design. The page pool is [page][H_kv][16][d], so one (page, KV head) is
// 16 contiguous token rows (4 KiB in bf16). One wavefront owns a run of pages of
// one KV head and reads each key row once for all G query heads of that group
// (the pages' kernel parallelises per query head, which under GQA would read
// every row G times). A 64-lane wave covers four token rows per 16-byte load:
// lane = 16 * row + col, col picks 8 dims. Each lane multiplies its 8 dims with
// the G query slices held in registers (bf16 pairs through v_dot2c_f32_bf16, or
// fp32 FMAs), and DPP sums over the 16 lanes of a row finish each inner product.
// The lanes then split the 4 tokens x G heads of a row among themselves to store
// the logits and keep a running (max, sum exp) per head; a second small kernel
// folds the per-unit pairs into (M_h, Z_h).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ts {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kUnroll = 4;        // pages in flight per wave

template <bool kBf16, int G> struct QRegs;
template <int G> struct QRegs<true, G> { uint32_t w[G][4]; };
template <int G> struct QRegs<false, G> { float w[G][8]; };

template <bool kBf16> struct PageRegs;
template <> struct PageRegs<true> { uint4 w[4]; };
template <> struct PageRegs<false> { float4 w[4][2]; };

// bf16: a token row is 256 B, lane col reads dims [8 col, 8 col + 8).
// fp32: a token row is 512 B, lane col reads dims [4 col, 4 col + 4) and
// [64 + 4 col, 64 + 4 col + 4), so each load instruction covers 256 contiguous bytes.
template <int G>
__device__ __forceinline__ void load_q(QRegs<true, G>& qr, const uint16_t* qb, int col) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 v = *reinterpret_cast<const uint4*>(qb + h * kHeadDim + 8 * col);
    qr.w[h][0] = v.x; qr.w[h][1] = v.y; qr.w[h][2] = v.z; qr.w[h][3] = v.w;
  }
}
template <int G>
__device__ __forceinline__ void load_q(QRegs<false, G>& qr, const float* qb, int col) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float4 a = *reinterpret_cast<const float4*>(qb + h * kHeadDim + 4 * col);
    const float4 c = *reinterpret_cast<const float4*>(qb + h * kHeadDim + 64 + 4 * col);
    qr.w[h][0] = a.x; qr.w[h][1] = a.y; qr.w[h][2] = a.z; qr.w[h][3] = a.w;
    qr.w[h][4] = c.x; qr.w[h][5] = c.y; qr.w[h][6] = c.z; qr.w[h][7] = c.w;
  }
}

__device__ __forceinline__ void load_page(PageRegs<true>& pr, const uint16_t* base, int row, int col) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    pr.w[j] = *reinterpret_cast<const uint4*>(base + (4 * j + row) * kHeadDim + 8 * col);
}
__device__ __forceinline__ void load_page(PageRegs<false>& pr, const float* base, int row, int col) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    pr.w[j][0] = *reinterpret_cast<const float4*>(base + (4 * j + row) * kHeadDim + 4 * col);
    pr.w[j][1] = *reinterpret_cast<const float4*>(base + (4 * j + row) * kHeadDim + 64 + 4 * col);
  }
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int G>
__device__ __forceinline__ void lane_dots(const PageRegs<true>& pr, const QRegs<true, G>& qr,
                                          float (&acc)[4][G]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = dot2(pr.w[j].x, qr.w[h][0], 0.f);
      a = dot2(pr.w[j].y, qr.w[h][1], a);
      a = dot2(pr.w[j].z, qr.w[h][2], a);
      acc[j][h] = dot2(pr.w[j].w, qr.w[h][3], a);
    }
  }
}
template <int G>
__device__ __forceinline__ void lane_dots(const PageRegs<false>& pr, const QRegs<false, G>& qr,
                                          float (&acc)[4][G]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = pr.w[j][0].x * qr.w[h][0];
      a = fmaf(pr.w[j][0].y, qr.w[h][1], a);
      a = fmaf(pr.w[j][0].z, qr.w[h][2], a);
      a = fmaf(pr.w[j][0].w, qr.w[h][3], a);
      a = fmaf(pr.w[j][1].x, qr.w[h][4], a);
      a = fmaf(pr.w[j][1].y, qr.w[h][5], a);
      a = fmaf(pr.w[j][1].z, qr.w[h][6], a);
      acc[j][h] = fmaf(pr.w[j][1].w, qr.w[h][7], a);
    }
  }
}

template <bool kBf16, int G>
__global__ __launch_bounds__(256) void score_kernel(ScoreParams p) {
  using T = typename std::conditional<kBf16, uint16_t, float>::type;
  constexpr int kSlots = (4 * G + 15) / 16;   // (token, head) values a lane owns per page
  __shared__ int64_t s_tok[kMaxBatch + 1];
  __shared__ int32_t s_chunk[kMaxBatch + 1];
  __shared__ float s_red[4][4 * G][4][2];

  const int b = p.b;
  const int chunk_tokens = p.chunk_pages * kPage;
  block_prefix(s_tok, b, [&](int r) -> int64_t { return p.seq_lens[r]; });
  block_prefix(s_chunk, b, [&](int r) -> int32_t {
    if (p.skip && p.skip[r]) return 0;
    return (p.seq_lens[r] + chunk_tokens - 1) / chunk_tokens;
  });

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane >> 4, col = lane & 15;
  const int H = p.H, Hkv = p.Hkv;
  const int total_units = s_chunk[b] * Hkv;
  const T* qall = static_cast<const T*>(p.q);
  const T* pool = static_cast<const T*>(p.k_pool);
  float(*red)[4][2] = s_red[wave];

  // Which (token j, head h) of its row this lane stores, per slot.
  int slot_j[kSlots], slot_h[kSlots];
  bool slot_on[kSlots];
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    const int idx = col + 16 * s;
    slot_on[s] = idx < 4 * G;
    slot_j[s] = idx / G;
    slot_h[s] = idx % G;
  }

  for (int u = blockIdx.x * 4 + wave; u < total_units; u += gridDim.x * 4) {
    const int cg = u / Hkv, g = u - cg * Hkv;
    const int r = find_segment(s_chunk, b, cg);
    const int c = cg - s_chunk[r];
    const int N = p.seq_lens[r];
    const int n_pages = (N + kPage - 1) / kPage;
    const int pg0 = c * p.chunk_pages;
    const int pg1 = min(n_pages, pg0 + p.chunk_pages);

    QRegs<kBf16, G> q;
    load_q(q, qall + ((int64_t)r * H + g * G) * kHeadDim, col);
    const int32_t* bt = p.block_table + (int64_t)r * p.stride;
    float* zrow = p.logits + s_tok[r] * H + (int64_t)(g * G) * N;

    float m[kSlots], s[kSlots];
#pragma unroll
    for (int k = 0; k < kSlots; ++k) { m[k] = kNegInf; s[k] = 0.f; }

    for (int pg = pg0; pg < pg1; pg += kUnroll) {
      PageRegs<kBf16> pr[kUnroll];
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) {
        if (pg + k < pg1) {
          const int64_t phys = bt[pg + k];
          load_page(pr[k], pool + (phys * Hkv + g) * (kPage * kHeadDim), row, col);
        }
      }
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) {
        if (pg + k >= pg1) break;
        float acc[4][G];
        lane_dots(pr[k], q, acc);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int h = 0; h < G; ++h) acc[j][h] = row_sum16(acc[j][h]);
        const int tok0 = (pg + k) * kPage + row;
#pragma unroll
        for (int sl = 0; sl < kSlots; ++sl) {
          float val = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int h = 0; h < G; ++h)
              val = (slot_j[sl] == j && slot_h[sl] == h) ? acc[j][h] : val;
          const int i = tok0 + 4 * slot_j[sl];
          if (slot_on[sl] && i < N) {
            const float z = val * p.score_scale;
            zrow[(int64_t)slot_h[sl] * N + i] = z;
            const float mn = fmaxf(m[sl], z);
            s[sl] = s[sl] * exp_via2(m[sl] - mn) + exp_via2(z - mn);
            m[sl] = mn;
          }
        }
      }
    }

    // Fold the per-lane pairs of each head: 4 tokens-in-row x 4 rows per head.
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      if (slot_on[sl]) {
        const int idx = slot_j[sl] * G + slot_h[sl];
        red[idx][row][0] = m[sl];
        red[idx][row][1] = s[sl];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < G) {
      float M = kNegInf, S = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) merge_ms(M, S, red[j * G + lane][rr][0], red[j * G + lane][rr][1]);
      float* dst = p.partials + ((int64_t)cg * H + g * G + lane) * 2;
      dst[0] = M;
      dst[1] = S;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// One workgroup per (request, head): fold the per-unit (max, sum exp) pairs.
__global__ __launch_bounds__(256) void stats_kernel(ScoreParams p) {
  __shared__ int32_t s_chunk[kMaxBatch + 1];
  __shared__ float s_m[4], s_s[4];
  const int b = p.b, H = p.H;
  const int r = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const int chunk_tokens = p.chunk_pages * kPage;
  block_prefix(s_chunk, b, [&](int rr) -> int32_t {
    if (p.skip && p.skip[rr]) return 0;
    return (p.seq_lens[rr] + chunk_tokens - 1) / chunk_tokens;
  });
  if (p.skip && p.skip[r]) return;
  const int c0 = s_chunk[r], c1 = s_chunk[r + 1];
  float M = kNegInf, S = 0.f;
  for (int c = c0 + threadIdx.x; c < c1; c += blockDim.x) {
    const float* src = p.partials + ((int64_t)c * H + h) * 2;
    merge_ms(M, S, src[0], src[1]);
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(M, o), s2 = __shfl_xor(S, o);
    merge_ms(M, S, m2, s2);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { s_m[wave] = M; s_s[wave] = S; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) merge_ms(M, S, s_m[w], s_s[w]);
    p.head_stats[((int64_t)r * H + h) * 2 + 0] = M;
    p.head_stats[((int64_t)r * H + h) * 2 + 1] = S;
  }
}

template <bool kBf16>
hipError_t launch_score_t(const ScoreParams& p, hipStream_t st) {
  const int G = p.H / p.Hkv;
  dim3 grid(p.grid), block(256);
  switch (G) {
    case 1: hipLaunchKernelGGL((score_kernel<kBf16, 1>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((score_kernel<kBf16, 2>), grid, block, 0, st, p); break;
    case 3: hipLaunchKernelGGL((score_kernel<kBf16, 3>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((score_kernel<kBf16, 4>), grid, block, 0, st, p); break;
    case 5: hipLaunchKernelGGL((score_kernel<kBf16, 5>), grid, block, 0, st, p); break;
    case 6: hipLaunchKernelGGL((score_kernel<kBf16, 6>), grid, block, 0, st, p); break;
    case 7: hipLaunchKernelGGL((score_kernel<kBf16, 7>), grid, block, 0, st, p); break;
    case 8: hipLaunchKernelGGL((score_kernel<kBf16, 8>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const ScoreParams& p, hipStream_t st) {
  hipError_t e = p.bf16 ? launch_score_t<true>(p, st) : launch_score_t<false>(p, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stats_kernel, dim3(p.b * p.H), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace ts
