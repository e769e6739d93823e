// Selection-function ablations: scores other than the head soft vote, on which the
// same radix TopK runs (tokenselect_select_ablation).
//
// Source: TokenSelect deepnotes page, selection-function design (the naive TopK over
// Q.K_cache^T, and the head hard vote TopK(sum_h I(i in TopK(Q^h K^h^T))), which the
// page notes needs a scatter-add and several top-ks), and the token-level
// motivation (Fig. 2b: block-level selection recalls fewer critical tokens); blog
// review of the same paper, section 2.
//
// * Naive: a position's score is its largest raw logit over the H heads.
// * Hard vote: the logits are regrouped as one segment per (request, head), each
//   segment gets its own TopK from the radix select, and a scatter-add counts the
//   heads that picked each position; the TopK of the counts follows (ties to the
//   lower position).
// * Block: blocks of B positions score the sum of their tokens' votes, kept in the
//   log2 domain like the vote itself: log2 sum 2^lv = m + log2 sum 2^(lv - m) with
//   m the block's largest lv, summed by one thread in position order in fp64 and
//   rounded once to fp32 (deterministic, no underflow, exactly lv for B = 1); the
//   radix select picks max(1, k / B) blocks, expanded to positions.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace ts {
namespace {

constexpr int kT = 256;

__device__ __forceinline__ int64_t seg_prefix(int64_t* s_tok, const AblationParams& p) {
  block_prefix(s_tok, p.b, [&](int r) -> int64_t { return p.seq_lens[r]; });
  return s_tok[p.b];
}

__global__ __launch_bounds__(kT) void naive_kernel(AblationParams p) {
  __shared__ int64_t s_tok[kMaxBatch + 1];
  const int64_t total = seg_prefix(s_tok, p);
  const int G = p.H / p.Hkv;
  for (int64_t x = blockIdx.x * (int64_t)kT + threadIdx.x; x < total; x += (int64_t)gridDim.x * kT) {
    const int r = find_segment(s_tok, p.b, x);
    const int64_t i = x - s_tok[r];
    const int64_t N = p.seq_lens[r];
    const float* z = p.logits + s_tok[r] * p.H;
    float m = kNegInf;
    for (int g = 0; g < p.Hkv; ++g)
      for (int j = 0; j < G; ++j) m = fmaxf(m, z[(g * N + i) * G + j]);
    p.score[x] = m;
  }
}

// Regroup the logits as [b][H][N_r] (one TopK segment per head); zero the counts.
__global__ __launch_bounds__(kT) void head_scores_kernel(AblationParams p) {
  __shared__ int64_t s_tok[kMaxBatch + 1];
  const int64_t total = seg_prefix(s_tok, p);
  const int G = p.H / p.Hkv;
  for (int64_t x = blockIdx.x * (int64_t)kT + threadIdx.x; x < total; x += (int64_t)gridDim.x * kT) {
    const int r = find_segment(s_tok, p.b, x);
    const int64_t i = x - s_tok[r];
    const int64_t N = p.seq_lens[r];
    const float* z = p.logits + s_tok[r] * p.H;
    float* hs = p.head_scores + s_tok[r] * p.H;
    for (int g = 0; g < p.Hkv; ++g)
      for (int j = 0; j < G; ++j) hs[(g * G + j) * N + i] = z[(g * N + i) * G + j];
    p.score[x] = 0.f;
  }
  for (int s = blockIdx.x * kT + threadIdx.x; s < p.b * p.H; s += gridDim.x * kT)
    p.seg_lens[s] = p.seq_lens[s / p.H];
}

// counts[i] += 1 for every head whose TopK holds position i (exact: small integers).
__global__ __launch_bounds__(kT) void count_votes_kernel(AblationParams p) {
  __shared__ int64_t s_tok[kMaxBatch + 1];
  seg_prefix(s_tok, p);
  const int64_t entries = (int64_t)p.b * p.H * p.head_stride;
  for (int64_t x = blockIdx.x * (int64_t)kT + threadIdx.x; x < entries; x += (int64_t)gridDim.x * kT) {
    const int seg = (int)(x / p.head_stride), e = (int)(x - (int64_t)seg * p.head_stride);
    if (e >= p.head_cnt[seg]) continue;
    const int r = seg / p.H;
    const int pos = p.head_sel[x];
    if (pos >= 0 && pos < p.seq_lens[r]) atomicAdd(&p.score[s_tok[r] + pos], 1.f);
  }
}

__global__ __launch_bounds__(kT) void block_scores_kernel(AblationParams p) {
  __shared__ int64_t s_tok[kMaxBatch + 1];
  __shared__ int64_t s_blk[kMaxBatch + 1];
  seg_prefix(s_tok, p);
  const int B = p.block;
  block_prefix(s_blk, p.b, [&](int r) -> int64_t { return (p.seq_lens[r] + B - 1) / B; });
  for (int r = blockIdx.x * kT + threadIdx.x; r < p.b; r += gridDim.x * kT)
    p.seg_lens[r] = (p.seq_lens[r] + B - 1) / B;
  const int64_t nblk = s_blk[p.b];
  for (int64_t y = blockIdx.x * (int64_t)kT + threadIdx.x; y < nblk; y += (int64_t)gridDim.x * kT) {
    const int r = find_segment(s_blk, p.b, y);
    const int64_t j = y - s_blk[r];
    const int64_t N = p.seq_lens[r];
    const float* lv = p.vote + s_tok[r];
    const int64_t i0 = j * B, i1 = min(N, i0 + B);
    float m = kNegInf;
    for (int64_t i = i0; i < i1; ++i) m = fmaxf(m, lv[i]);
    double sum = 0.0;
    for (int64_t i = i0; i < i1; ++i) sum += exp2((double)lv[i] - (double)m);
    p.score[y] = (float)((double)m + log2(sum));
  }
}

// Selected blocks (ascending) -> positions (ascending); only the request's last
// block can be short, and it is the last one written.
__global__ __launch_bounds__(kT) void expand_blocks_kernel(AblationParams p) {
  const int r = blockIdx.x;
  const int B = p.block, N = p.seq_lens[r];
  const int m = p.head_cnt[r];
  const int32_t* blk = p.head_sel + (int64_t)r * p.head_stride;
  int32_t* out = p.sel_idx + (int64_t)r * p.top_k;
  for (int t = threadIdx.x; t < m * B; t += kT) {
    const int pos = blk[t / B] * B + t % B;
    if (pos < N) out[t] = pos;
  }
  if (threadIdx.x == 0) {
    int cnt = m * B;
    if (m > 0) cnt -= max(0, (blk[m - 1] + 1) * B - N);
    p.sel_count[r] = cnt;
  }
}

int grid_for(int64_t n) { return (int)std::min<int64_t>(2048, (n + kT - 1) / kT + 1); }

}  // namespace

hipError_t launch_naive_scores(const AblationParams& p, hipStream_t s) {
  hipLaunchKernelGGL(naive_kernel, dim3(2048), dim3(kT), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_head_scores(const AblationParams& p, hipStream_t s) {
  hipLaunchKernelGGL(head_scores_kernel, dim3(2048), dim3(kT), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_count_votes(const AblationParams& p, hipStream_t s) {
  hipLaunchKernelGGL(count_votes_kernel, dim3(grid_for((int64_t)p.b * p.H * p.head_stride)), dim3(kT), 0,
                     s, p);
  return hipGetLastError();
}
hipError_t launch_block_scores(const AblationParams& p, hipStream_t s) {
  hipLaunchKernelGGL(block_scores_kernel, dim3(2048), dim3(kT), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_expand_blocks(const AblationParams& p, hipStream_t s) {
  hipLaunchKernelGGL(expand_blocks_kernel, dim3(p.b), dim3(kT), 0, s, p);
  return hipGetLastError();
}

}  // namespace ts
