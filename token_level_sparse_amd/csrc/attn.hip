// Step 5 of the decode step: scaled-dot-product attention over the selected set.
//
// Source: TokenSelect deepnotes page, selective sparse attention formalisation:
// each head's output is the softmax of its query against the selected keys plus
// the current one, scaled by 1/sqrt(d), applied to the matching values. The blog
// page (section 3, Fig. 4) hands only the selected indices to the attention
// kernel, with the paged KV left in place; section 4.2 adds a window of local
// tokens to the selected budget.
//
// gfx950 design. The selected set of request r is the TopK list (ascending)
// united with the window [N - L, N), L >= 1 (with a window size of 0 the window is
// the current token alone); TopK entries inside the window are skipped
// because the window covers them, so no sort or merge is needed. A workgroup
// covers 128 selected slots (4 waves of 32) of the TopK list or of the window, for
// one KV head and all G query heads of its group: each key and value row (256 B in
// bf16) is gathered once through the block table. Lane = 16 * row + col: the 4 rows
// of a wave take every 4th token and col picks 8 dims; the inner products run on
// bf16 pairs (v_dot2_f32_bf16) and DPP sums finish them, and each row keeps a
// (max, sum, o[8 dims]) online softmax in registers. The 16 rows of the workgroup
// leave their partials in LDS (G x 16 x 132 floats) and merge there in one pass
// into one partial per workgroup (no cross-row shuffles); a small kernel merges
// the partials of each (request, head) and rounds the output. (Merging in the last
// workgroup behind an atomic ticket was measured slower: the device-scope release
// each workgroup then needs writes back its XCD's whole L2.)
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "timeline.h"

TS_TIMELINE_DEFINE(attn)

namespace ts {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
constexpr int kTokPerRow = kAttnSplit / 4;   // 8 tokens per row of a wave

template <bool kBf16> struct Row8;            // 8 dims of one token row held by a lane
template <> struct Row8<true> { uint4 w; };
template <> struct Row8<false> { float4 a, b; };

__device__ __forceinline__ void load_row(Row8<true>& x, const uint16_t* rowp, int col) {
  x.w = *reinterpret_cast<const uint4*>(rowp + 8 * col);
}
__device__ __forceinline__ void load_row(Row8<false>& x, const float* rowp, int col) {
  x.a = *reinterpret_cast<const float4*>(rowp + 4 * col);
  x.b = *reinterpret_cast<const float4*>(rowp + 64 + 4 * col);
}
__device__ __forceinline__ void to_f32(const Row8<true>& x, float (&f)[8]) {
  f[0] = bf16_lo(x.w.x); f[1] = bf16_hi(x.w.x); f[2] = bf16_lo(x.w.y); f[3] = bf16_hi(x.w.y);
  f[4] = bf16_lo(x.w.z); f[5] = bf16_hi(x.w.z); f[6] = bf16_lo(x.w.w); f[7] = bf16_hi(x.w.w);
}
__device__ __forceinline__ void to_f32(const Row8<false>& x, float (&f)[8]) {
  f[0] = x.a.x; f[1] = x.a.y; f[2] = x.a.z; f[3] = x.a.w;
  f[4] = x.b.x; f[5] = x.b.y; f[6] = x.b.z; f[7] = x.b.w;
}
// LDS stride of a row partial per head: d dims, m, l, padded to a multiple of 4
// floats for 16-byte stores.
constexpr int kPartStride = kHeadDim + 4;

// A lane's 8 query dims of one head: bf16 pairs (dims 8 col .. 8 col + 7) or fp32.
template <bool kBf16> struct QSlice;
template <> struct QSlice<true> { uint4 w; };
template <> struct QSlice<false> { float f[8]; };
__device__ __forceinline__ void load_q(QSlice<true>& q, const uint16_t* rowp, int col) {
  q.w = *reinterpret_cast<const uint4*>(rowp + 8 * col);
}
__device__ __forceinline__ void load_q(QSlice<false>& q, const float* rowp, int col) {
  Row8<false> x;
  load_row(x, rowp, col);
  to_f32(x, q.f);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}
// This lane's part of <k, q> over its 8 dims (v_dot2_f32_bf16 on bf16 pairs, fp32 FMAs).
__device__ __forceinline__ float dot8(const Row8<true>& k, const QSlice<true>& q) {
  float a = dot2_bf16(k.w.x, q.w.x, 0.f);
  a = dot2_bf16(k.w.y, q.w.y, a);
  a = dot2_bf16(k.w.z, q.w.z, a);
  return dot2_bf16(k.w.w, q.w.w, a);
}
__device__ __forceinline__ float dot8(const Row8<false>& k, const QSlice<false>& q) {
  float kf[8];
  to_f32(k, kf);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = fmaf(kf[e], q.f[e], acc);
  return acc;
}

// A lane's 8 output dims of one head into its row partial (the dims of load_row).
template <bool kBf16>
__device__ __forceinline__ void store_o(float* dst, int col, const float (&o)[8]) {
  if (kBf16) {
    *reinterpret_cast<float4*>(dst + 8 * col) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(dst + 8 * col + 4) = make_float4(o[4], o[5], o[6], o[7]);
  } else {
    *reinterpret_cast<float4*>(dst + 4 * col) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(dst + 64 + 4 * col) = make_float4(o[4], o[5], o[6], o[7]);
  }
}

template <bool kBf16, int G>
__global__ __launch_bounds__(256) void attn_kernel(AttnParams p) {
  TS_TIMELINE_SCOPE(attn, kTlAttn);
  using T = typename std::conditional<kBf16, uint16_t, float>::type;
  constexpr int kTile = kAttnTile;
  constexpr int kAttnRows = 16;                      // 4 waves x 4 rows
  __shared__ __align__(16) float s_part[kAttnRows][G][kPartStride];
  __shared__ float s_w[G][kAttnRows];
  __shared__ float s_max[G];
  const int S = attn_splits(p.top_k, p.n_local);
  const int nT = (p.top_k + kTile - 1) / kTile;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane >> 4, col = lane & 15;
  const int s = blockIdx.x % S;
  const int rg = blockIdx.x / S;
  const int g = rg % p.Hkv;
  const int r = rg / p.Hkv;
  const int H = p.H;
  // The request's length, its TopK count and this lane's TopK entry are independent
  // loads, all issued before any of them is used (the entry is read within the row).
  const int e_sel = min(s * kTile + wave * kAttnSplit + (lane & (kAttnSplit - 1)), p.sel_stride - 1);
  const int cand = (s < nT) ? p.sel_idx[(int64_t)r * p.sel_stride + e_sel] : 0;
  const int N = p.seq_lens[r];
  const int cnt = (s < nT) ? min(p.sel_count[r], p.sel_stride) : 0;
  // p.n_local >= 1: the window always holds the current token N - 1
  const int lstart = max(0, N - p.n_local);
  float* part = p.partials + ((int64_t)r * H + g * G) * S * (kHeadDim + 2);
  if (N <= 0) {
    // An empty request reaches no page: its block-table row is not read at all
    // and the partial is the empty one (o = 0, m = -inf, l = 0).
    for (int e = threadIdx.x; e < G * (kHeadDim + 2); e += blockDim.x) {
      const int h = e / (kHeadDim + 2), c = e % (kHeadDim + 2);
      part[((int64_t)h * S + s) * (kHeadDim + 2) + c] = (c == kHeadDim) ? kNegInf : 0.f;
    }
    return;
  }

  // Token of this wave's slot e = lane (lanes 0..31), then broadcast by shuffle.
  // A slot that holds no selected token gathers the current token N - 1 (always a
  // reached page) and gets weight 0.
  int tok = N - 1;
  bool ok = false;
  if (lane < kAttnSplit) {
    if (s < nT) {
      const int e = s * kTile + wave * kAttnSplit + lane;
      if (e < cnt) {
        ok = cand >= 0 && cand < lstart;
        if (ok) tok = cand;
      }
    } else {
      const int t = lstart + (s - nT) * kTile + wave * kAttnSplit + lane;
      ok = t < N;
      if (ok) tok = t;
    }
  }
  const int32_t* bt = p.block_table + (int64_t)r * p.stride;
  int64_t rowoff = 0;
  if (lane < kAttnSplit) {
    const int64_t phys = bt[tok / kPage];
    rowoff = ((phys * p.Hkv + g) * kPage + (tok % kPage)) * kHeadDim;
  }

  const T* kp = static_cast<const T*>(p.k_pool);
  const T* vp = static_cast<const T*>(p.v_pool);
  Row8<kBf16> kr[kTokPerRow], vr[kTokPerRow];
  bool okr[kTokPerRow];
#pragma unroll
  for (int t = 0; t < kTokPerRow; ++t) {
    const int e = row + 4 * t;
    const int64_t off = __shfl(rowoff, e);
    okr[t] = __shfl((int)ok, e) != 0;
    load_row(kr[t], kp + off, col);
    load_row(vr[t], vp + off, col);
  }

  // query slices of the group's G heads (bf16: packed pairs for v_dot2_f32_bf16)
  const T* qb = static_cast<const T*>(p.q) + ((int64_t)r * H + g * G) * kHeadDim;
  QSlice<kBf16> qs[G];
#pragma unroll
  for (int h = 0; h < G; ++h) load_q(qs[h], qb + h * kHeadDim, col);

  float m[G], l[G], o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float a[kTokPerRow];
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < kTokPerRow; ++t) {
      const float acc = row_sum16(dot8(kr[t], qs[h])) * p.attn_scale;
      a[t] = okr[t] ? acc : kNegInf;
      mx = fmaxf(mx, a[t]);
    }
    m[h] = mx;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
    if (mx != kNegInf) {
#pragma unroll
      for (int t = 0; t < kTokPerRow; ++t) {
        const float pw = okr[t] ? exp_via2(a[t] - mx) : 0.f;
        l[h] += pw;
        float vf[8];
        to_f32(vr[t], vf);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = fmaf(pw, vf[e], o[h][e]);
      }
    }
  }

  // The rows' (m, l, o) go to LDS and merge there in one pass: per-row weights
  // exp(m_row - M) first, then each thread sums its output dims over the rows in
  // row order.
  const int prow = wave * 4 + row;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float* dst = &s_part[prow][h][0];
    store_o<kBf16>(dst, col, o[h]);
    if (col == 0) {
      dst[kHeadDim] = m[h];
      dst[kHeadDim + 1] = l[h];
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < G * kAttnRows) {
    const int h = threadIdx.x / kAttnRows, j = threadIdx.x % kAttnRows;
    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < kAttnRows; ++i) M = fmaxf(M, s_part[i][h][kHeadDim]);
    const float mj = s_part[j][h][kHeadDim];
    s_w[h][j] = (mj == kNegInf) ? 0.f : exp_via2(mj - M);
    if (j == 0) s_max[h] = M;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * kHeadDim; e += blockDim.x) {
    const int h = e / kHeadDim, dim = e % kHeadDim;
    float acc = 0.f, L = 0.f;
#pragma unroll
    for (int j = 0; j < kAttnRows; ++j) {
      const float w = s_w[h][j];
      acc = fmaf(w, s_part[j][h][dim], acc);
      L = fmaf(w, s_part[j][h][kHeadDim + 1], L);
    }
    float* dst = part + ((int64_t)h * S + s) * (kHeadDim + 2);
    dst[dim] = acc;
    if (dim == 0) {
      dst[kHeadDim] = s_max[h];
      dst[kHeadDim + 1] = L;
    }
  }
}

// One workgroup of d threads per (request, head) merges the workgroup partials and
// rounds the output. Above kAttnCombineSpan (256) partials (a selection of more
// than ~32K positions, such as the dense k = N reference) a first launch merges
// each run of 256 partials into one, so no workgroup loops over thousands of them.
// The per-partial weights exp(m_s - M) are computed once by spread threads and
// kept in LDS; each thread (one output dim) then sums its column with independent
// loads, the first kPre of them issued at the start together with the maxima (one
// memory round trip less for the usual 20 or 40 partials).
constexpr int kCombineChunk = 1024;

// Partials [j0, j0 + n) of (request, head) rh in `src` (rows of d + 2 floats:
// o[d], m, l). kFinal: write the rounded output of rh; else the merged partial
// (o, M, L) to row (rh, c) of p.partials2.
template <bool kBf16, int kPre, bool kFinal>
__global__ __launch_bounds__(kHeadDim) void combine_kernel(AttnParams p, const float* src, int S_src,
                                                           int n_chunks) {
  TS_TIMELINE_SCOPE(attn, kTlCombine);
  __shared__ float s_w[kCombineChunk];
  __shared__ float s_red[2];
  const int rh = kFinal ? blockIdx.x : blockIdx.x / n_chunks;
  const int c = kFinal ? 0 : blockIdx.x - rh * n_chunks;
  const int j0 = c * kAttnCombineSpan;
  const int S = kFinal ? S_src : min(kAttnCombineSpan, S_src - j0);
  const int tid = threadIdx.x;
  const float* base = src + ((int64_t)rh * S_src + j0) * (kHeadDim + 2);
  // this thread's column of the first kPre partials, loaded with the maxima
  float opre[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) opre[j] = base[min(j, S - 1) * (kHeadDim + 2) + tid];
  float M = kNegInf;
  for (int j = tid; j < S; j += kHeadDim) M = fmaxf(M, base[j * (kHeadDim + 2) + kHeadDim]);
  M = wave_max(M);
  if ((tid & 63) == 0) s_red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(s_red[0], s_red[1]);
  float acc = 0.f, L = 0.f;
  for (int c0 = 0; c0 < S; c0 += kCombineChunk) {
    const int n = min(kCombineChunk, S - c0);
    __syncthreads();
    for (int j = tid; j < n; j += kHeadDim) {
      const float* row = base + (c0 + j) * (kHeadDim + 2);
      const float mj = row[kHeadDim], lj = row[kHeadDim + 1];
      const float w = (mj == kNegInf || lj == 0.f) ? 0.f : exp_via2(mj - M);
      s_w[j] = w;
      L = fmaf(w, lj, L);
    }
    __syncthreads();
    int j = 0;
    if (c0 == 0) {
#pragma unroll
      for (int u = 0; u < kPre; ++u)
        if (u < n) acc = fmaf(s_w[u], opre[u], acc);
      j = min(n, kPre);
    }
#pragma unroll 4
    for (; j < n; ++j) acc = fmaf(s_w[j], base[(c0 + j) * (kHeadDim + 2) + tid], acc);
  }
  L = wave_sum(L);
  __syncthreads();
  if ((tid & 63) == 0) s_red[tid >> 6] = L;
  __syncthreads();
  L = s_red[0] + s_red[1];
  if (!kFinal) {
    float* dst = p.partials2 + ((int64_t)rh * n_chunks + c) * (kHeadDim + 2);
    dst[tid] = acc;
    if (tid == 0) {
      dst[kHeadDim] = M;
      dst[kHeadDim + 1] = L;
    }
    return;
  }
  const float res = (L > 0.f) ? acc / L : 0.f;   // an empty set (N_r = 0) gives zeros
  if (kBf16)
    static_cast<uint16_t*>(p.out)[(int64_t)rh * kHeadDim + tid] = f32_to_bf16(res);
  else
    static_cast<float*>(p.out)[(int64_t)rh * kHeadDim + tid] = res;
}

template <bool kBf16>
void launch_final_combine(const AttnParams& p, const float* src, int S, hipStream_t st) {
  const dim3 grid(p.b * p.H), block(kHeadDim);
  if (S <= 32)
    hipLaunchKernelGGL((combine_kernel<kBf16, 32, true>), grid, block, 0, st, p, src, S, 1);
  else
    hipLaunchKernelGGL((combine_kernel<kBf16, 64, true>), grid, block, 0, st, p, src, S, 1);
}

template <bool kBf16>
hipError_t launch_attn_t(const AttnParams& p, hipStream_t st) {
  const int G = p.H / p.Hkv;
  dim3 grid(p.b * p.Hkv * attn_splits(p.top_k, p.n_local)), block(256);
  switch (G) {
    case 1: hipLaunchKernelGGL((attn_kernel<kBf16, 1>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((attn_kernel<kBf16, 2>), grid, block, 0, st, p); break;
    case 3: hipLaunchKernelGGL((attn_kernel<kBf16, 3>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((attn_kernel<kBf16, 4>), grid, block, 0, st, p); break;
    case 5: hipLaunchKernelGGL((attn_kernel<kBf16, 5>), grid, block, 0, st, p); break;
    case 6: hipLaunchKernelGGL((attn_kernel<kBf16, 6>), grid, block, 0, st, p); break;
    case 7: hipLaunchKernelGGL((attn_kernel<kBf16, 7>), grid, block, 0, st, p); break;
    case 8: hipLaunchKernelGGL((attn_kernel<kBf16, 8>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  const int S = attn_splits(p.top_k, p.n_local);
  if (S <= kAttnCombineSpan) {
    launch_final_combine<kBf16>(p, p.partials, S, st);
  } else {
    const int chunks = attn_combine_chunks(S);
    hipLaunchKernelGGL((combine_kernel<kBf16, 64, false>), dim3(p.b * p.H * chunks), dim3(kHeadDim), 0, st, p,
                       p.partials, S, chunks);
    launch_final_combine<kBf16>(p, p.partials2, chunks, st);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnParams& p, hipStream_t st) {
  return p.bf16 ? launch_attn_t<true>(p, st) : launch_attn_t<false>(p, st);
}

}  // namespace ts
