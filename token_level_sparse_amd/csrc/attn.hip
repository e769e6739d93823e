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
// covers 128 selected slots (32 per wavefront) of the TopK list or of the window,
// for one KV head and all G query heads of its group: each key and value row
// (256 B in bf16) is gathered once through the block table. Lane = 16 * row +
// col: the 4 rows of a wave take every 4th token and col picks 8 dims, DPP sums
// finish the inner products, and each row keeps a (max, sum, o[8 dims]) online
// softmax in registers. Rows merge by cross-row shuffles and waves through LDS
// into one partial per workgroup; a small kernel merges the partials of each
// (request, head) and rounds the output. (Merging in the last workgroup behind an
// atomic ticket was measured slower: the device-scope release each workgroup then
// needs writes back its XCD's whole L2.)
#include <type_traits>

#include "common.h"
#include "kernels.h"

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
// Dim index of element e of a lane's 8 (matches load_row).
__device__ __forceinline__ int lane_dim(bool bf16, int col, int e) {
  return bf16 ? 8 * col + e : (e < 4 ? 4 * col + e : 64 + 4 * col + (e - 4));
}

template <bool kBf16, int G>
__global__ __launch_bounds__(256) void attn_kernel(AttnParams p) {
  using T = typename std::conditional<kBf16, uint16_t, float>::type;
  __shared__ float s_part[4][G][kHeadDim + 2];
  const int S = attn_splits(p.top_k, p.n_local);
  const int nT = (p.top_k + kAttnTile - 1) / kAttnTile;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane >> 4, col = lane & 15;
  const int s = blockIdx.x % S;
  const int rg = blockIdx.x / S;
  const int g = rg % p.Hkv;
  const int r = rg / p.Hkv;
  const int H = p.H;
  // The request's length, its TopK count and this lane's TopK entry are independent
  // loads, all issued before any of them is used (the entry is read within the row).
  const int e_sel = min(s * kAttnTile + wave * kAttnSplit + (lane & (kAttnSplit - 1)), p.sel_stride - 1);
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
      const int e = s * kAttnTile + wave * kAttnSplit + lane;
      if (e < cnt) {
        ok = cand >= 0 && cand < lstart;
        if (ok) tok = cand;
      }
    } else {
      const int t = lstart + (s - nT) * kAttnTile + wave * kAttnSplit + lane;
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

  // query slices of the group's G heads
  const T* qb = static_cast<const T*>(p.q) + ((int64_t)r * H + g * G) * kHeadDim;
  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    Row8<kBf16> x;
    load_row(x, qb + h * kHeadDim, col);
    to_f32(x, qf[h]);
  }

  float m[G], l[G], o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float a[kTokPerRow];
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < kTokPerRow; ++t) {
      float kf[8];
      to_f32(kr[t], kf);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(kf[e], qf[h][e], acc);
      acc = row_sum16(acc) * p.attn_scale;
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

  // merge the 4 rows of the wave (partners at lane ^ 16 and lane ^ 32)
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int x = 16; x <= 32; x <<= 1) {
      const float m2 = __shfl_xor(m[h], x);
      const float l2 = __shfl_xor(l[h], x);
      const float mn = fmaxf(m[h], m2);
      const float c1 = (m[h] == kNegInf) ? 0.f : exp_via2(m[h] - mn);
      const float c2 = (m2 == kNegInf) ? 0.f : exp_via2(m2 - mn);
      l[h] = l[h] * c1 + l2 * c2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float o2 = __shfl_xor(o[h][e], x);
        o[h][e] = o[h][e] * c1 + o2 * c2;
      }
      m[h] = mn;
    }
  }
  // the 4 waves of the workgroup merge through LDS into one partial per head
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_part[wave][h][lane_dim(kBf16, col, e)] = o[h][e];
      if (col == 0) {
        s_part[wave][h][kHeadDim] = m[h];
        s_part[wave][h][kHeadDim + 1] = l[h];
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * kHeadDim; e += blockDim.x) {
    const int h = e / kHeadDim, dim = e % kHeadDim;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_part[w][h][kHeadDim]);
    float acc = 0.f, L = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = s_part[w][h][kHeadDim];
        const float c = (mw == kNegInf) ? 0.f : exp_via2(mw - M);
        acc = fmaf(c, s_part[w][h][dim], acc);
        L = fmaf(c, s_part[w][h][kHeadDim + 1], L);
      }
    }
    float* dst = part + ((int64_t)h * S + s) * (kHeadDim + 2);
    dst[dim] = acc;
    if (dim == 0) {
      dst[kHeadDim] = M;
      dst[kHeadDim + 1] = L;
    }
  }
}

// One workgroup of d threads per (request, head): merge the workgroup partials.
// The per-partial weights exp(m_s - M) are computed once by spread threads and
// kept in LDS; each thread (one output dim) then sums its column with
// independent loads, the first 32 of them issued at the start together with the
// maxima (one memory round trip less for the usual 20 partials).
constexpr int kCombineChunk = 1024;

template <bool kBf16>
__global__ __launch_bounds__(kHeadDim) void combine_kernel(AttnParams p) {
  __shared__ float s_w[kCombineChunk];
  __shared__ float s_red[2];
  const int S = attn_splits(p.top_k, p.n_local);
  const int rh = blockIdx.x;
  const int tid = threadIdx.x;
  const float* base = p.partials + (int64_t)rh * S * (kHeadDim + 2);
  // this thread's column of the first kPre partials, loaded with the maxima
  constexpr int kPre = 32;
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
      const float* src = base + (c0 + j) * (kHeadDim + 2);
      const float mj = src[kHeadDim], lj = src[kHeadDim + 1];
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
  const float res = (L > 0.f) ? acc / L : 0.f;   // an empty set (N_r = 0) gives zeros
  if (kBf16)
    static_cast<uint16_t*>(p.out)[(int64_t)rh * kHeadDim + tid] = f32_to_bf16(res);
  else
    static_cast<float*>(p.out)[(int64_t)rh * kHeadDim + tid] = res;
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
  hipLaunchKernelGGL(combine_kernel<kBf16>, dim3(p.b * p.H), dim3(kHeadDim), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnParams& p, hipStream_t st) {
  return p.bf16 ? launch_attn_t<true>(p, st) : launch_attn_t<false>(p, st);
}

}  // namespace ts
