// Steps 3-4 of the decode step: head soft vote and TopK over all N positions.
//
// Source: TokenSelect deepnotes page, head soft vote equation: the TopK of the
// sum over the H query heads of each head's softmax-normalised inner products.
// Ties go to the lower position; the result is written in ascending position
// order.
//
// gfx950 design.
// * The vote is kept in the log2 domain: lv_i = log2 sum_h 2^(x_hi) with
//   x_hi = (z_hi - M_h) log2(e) - log2(Z_h), accumulated by an online
//   log-sum-exp over the heads. The TopK of lv equals the TopK of the vote (log
//   is monotone), and lv stays finite where the linear fp32 vote would underflow
//   to 0 (any token whose every head weight is below 2^-126), so tiny votes keep
//   their order instead of tying at zero.
// * The vote kernel streams the H x N logits (the largest read after the K
//   stream) in tiles of 1024 positions, 4 per thread, with coalesced dword loads
//   issued unconditionally (the last tile clamps its addresses), so every
//   thread keeps 32 loads in flight.
// * TopK is a radix select on the order-preserving 32-bit key of lv, most
//   significant digit first (11, 11, 10 bits). The vote kernel builds the first
//   digit's histogram (LDS, then global atomics); each later pass reads the
//   previous histogram, finds the digit holding the k-th largest key (every
//   workgroup redoes this scan instead of paying a launch), and histograms the
//   next digit of the keys sharing the prefix. The second pass also counts, per
//   tile, the keys above the 22-bit prefix it fixes and lists the keys on that
//   prefix with their positions (a handful near the k-th vote); the write pass
//   then knows, for any tile, how many keys of the earlier tiles sort before its
//   own without a counting pass of its own, and writes positions through a prefix
//   over tiles; equal keys are taken in position order until k is reached, so the
//   result is deterministic.
// * Dynamic top-p budget (RTPurbo team post: dynamic token selection and its
//   histogram-based top-p decode kernel; UniPrefill page: the minimal set holding
//   99% of the importance). Each vote also carries an integer mass
//   q = rint(v * 2^40), v = 2^lv, and every histogram pass accumulates per-bin masses
//   beside the counts (64-bit integer atomics: exact and order-independent, so the
//   budget is deterministic). At each digit the walk from the top stops at the
//   first bin where either k keys or the target mass ceil(p * sum q) is reached, so
//   one radix walk gives min(top-p budget, k); the keys equal to the final threshold
//   are taken in position order up to that count.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "timeline.h"

TS_TIMELINE_DEFINE(select)

namespace ts {
namespace {

constexpr int kThreads = 256;
#ifndef TS_VOTE_MAX_GRID
#define TS_VOTE_MAX_GRID 512
#endif
// Vote workgroups: each takes several tiles and flushes its histogram once.
constexpr int kVoteMaxGrid = TS_VOTE_MAX_GRID;
constexpr int kMaxFoldGrid = 2048;   // fold-mode vote workgroups (they loop over the tiles)
#ifndef TS_REFINE_MAX_GRID
#define TS_REFINE_MAX_GRID 2048
#endif
constexpr int kRefineMaxGrid = TS_REFINE_MAX_GRID;
constexpr int kPerThread = kVoteTile / kThreads;   // positions per thread
constexpr float kLog2eF = 1.4426950408889634f;

typedef unsigned long long u64;

// Order-preserving map of an fp32 value to uint32 (larger value, larger key).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
  return __uint_as_float(u);
}



struct Tables {
  int64_t tok[kMaxBatch + 1];
  int32_t tile[kMaxBatch + 1];
};

// Request 0's length and skip flag, read by every thread at the kernel's start with
// uniform addresses: scalar loads, which do not queue behind the vector loads issued
// after them. Both are unconditional (a null skip array reads seq_lens instead and
// is ignored), so nothing waits for them before they are used.
struct OneReq {
  int n, skip;
  bool has_skip;
};
__device__ __forceinline__ OneReq one_request(const VoteParams& p) {
  OneReq o;
  o.n = p.seq_lens[0];
  o.has_skip = p.skip != nullptr;
  o.skip = (o.has_skip ? p.skip : p.seq_lens)[0];
  return o;
}

__device__ void build_tables(Tables& t, const VoteParams& p, const OneReq& o) {
  if (p.b == 1) {
    if (threadIdx.x == 0) {
      t.tok[0] = 0;
      t.tok[1] = o.n;
      t.tile[0] = 0;
      t.tile[1] = (o.has_skip && o.skip) ? 0 : (o.n + kVoteTile - 1) / kVoteTile;
    }
    __syncthreads();
    return;
  }
  block_prefix(t.tok, p.b, [&](int r) -> int64_t { return p.seq_lens[r]; });
  block_prefix(t.tile, p.b, [&](int r) -> int32_t {
    if (p.skip && p.skip[r]) return 0;
    return (p.seq_lens[r] + kVoteTile - 1) / kVoteTile;
  });
}

// Exclusive prefix over the block's threads (thread order), 256 threads.
__device__ uint32_t block_excl_scan(uint32_t x, uint32_t* s_w) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = x;
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) s_w[wave] = inc;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += s_w[w];
  __syncthreads();
  return base + inc - x;
}

__device__ u64 block_excl_scan64(u64 x, u64* s_w) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u64 inc = x;
  for (int o = 1; o < 64; o <<= 1) {
    const u64 t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) s_w[wave] = inc;
  __syncthreads();
  u64 base = 0;
  for (int w = 0; w < wave; ++w) base += s_w[w];
  __syncthreads();
  return base + inc - x;
}

// Digit of the top-p walk: walking the bins from the top, the first bin where the
// cumulative count reaches kk or the cumulative mass reaches mm. s_out = {bin,
// kk - count above}, *s_mres = mm - mass above.
template <int kBins>
__device__ void find_digit_pk(const uint32_t* hist, const u64* mhist, int kk, u64 mm, int* s_out,
                              u64* s_mres, uint32_t* s_w, u64* s_w64, int* s_bin) {
  constexpr int kPer = kBins / kThreads;
  const int hi = kBins - kPer * threadIdx.x;
  uint32_t c[kPer];
  u64 m[kPer];
  uint32_t sc = 0;
  u64 sm = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    c[e] = hist[hi - 1 - e]; m[e] = mhist[hi - 1 - e];
    sc += c[e]; sm += m[e];
  }
  if (threadIdx.x == 0) { s_bin[0] = -1; s_bin[1] = -1; }
  const uint32_t ac = block_excl_scan(sc, s_w);
  const u64 am = block_excl_scan64(sm, s_w64);
  if (ac < (uint32_t)kk && (uint32_t)kk <= ac + sc) {
    uint32_t acc = ac;
    bool done = false;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if (!done && acc + c[e] >= (uint32_t)kk) { s_bin[0] = hi - 1 - e; done = true; }
      acc += c[e];
    }
  }
  if (am < mm && mm <= am + sm) {
    u64 acc = am;
    bool done = false;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if (!done && acc + m[e] >= mm) { s_bin[1] = hi - 1 - e; done = true; }
      acc += m[e];
    }
  }
  __syncthreads();
  const int bin = max(max(s_bin[0], s_bin[1]), 0);
  if ((int)threadIdx.x == (kBins - 1 - bin) / kPer) {
    uint32_t acc = ac;
    u64 accm = am;
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      if (hi - 1 - e > bin) { acc += c[e]; accm += m[e]; }
    s_out[0] = bin;
    s_out[1] = kk - (int)acc;
    *s_mres = mm - accm;
  }
  __syncthreads();
}

// Digit holding the kk-th largest key among the counts in hist[0..kBins) (bins in
// increasing key order): s_out = {bin, kk - count(keys in higher bins)}.
// 1 <= kk <= total count is required; exactly one thread finds the crossing.
// Thread t owns bins [kBins - kPer (t + 1), kBins - kPer t), highest first (thread 0
// owns the top bins); load_counts reads them, find_digit_c finds the digit.
template <int kBins>
__device__ __forceinline__ void load_counts(const uint32_t* hist, uint32_t (&c)[kBins / kThreads]) {
  constexpr int kPer = kBins / kThreads;
  const int hi = kBins - kPer * threadIdx.x;
#pragma unroll
  for (int e = 0; e < kPer; ++e) c[e] = hist[hi - 1 - e];
}
template <int kBins>
__device__ void find_digit_c(const uint32_t (&c)[kBins / kThreads], int kk, int* s_out, uint32_t* s_w) {
  constexpr int kPer = kBins / kThreads;            // 8 or 4 bins per thread
  const int hi = kBins - kPer * threadIdx.x;        // thread 0 owns the top bins
  uint32_t sum = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) sum += c[e];
  const uint32_t above = block_excl_scan(sum, s_w);
  if (above < (uint32_t)kk && (uint32_t)kk <= above + sum) {
    uint32_t acc = above;
    bool done = false;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if (!done && acc + c[e] >= (uint32_t)kk) {
        s_out[0] = hi - 1 - e;
        s_out[1] = kk - (int)acc;
        done = true;
      }
      acc += c[e];
    }
  }
  __syncthreads();
}
template <int kBins>
__device__ void find_digit(const uint32_t* hist, int kk, int* s_out, uint32_t* s_w) {
  uint32_t c[kBins / kThreads];
  load_counts<kBins>(hist, c);
  find_digit_c<kBins>(c, kk, s_out, s_w);
}

// Keys of this thread's positions i0 + e * kThreads (clamped addresses; positions
// past N get key 0, below every real key).
__device__ __forceinline__ void load_keys(const float* lv, int i0, int N, uint32_t (&key)[kPerThread]) {
  float x[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) x[e] = lv[min(i0 + e * kThreads, N - 1)];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) key[e] = (i0 + e * kThreads < N) ? order_key(x[e]) : 0u;
}

// ---------------------------------------------------------------- vote + digit-0 histogram
// Logits are [H_kv][N][G] per request: for each KV head a thread reads the G
// adjacent logits of each of its positions (16-byte loads when G is a multiple
// of 4).
template <int G>
__device__ __forceinline__ void load_group(const float* zg, int i, float (&x)[G]) {
  if constexpr (G % 4 == 0) {
#pragma unroll
    for (int j = 0; j < G; j += 4) {
      const float4 v = *reinterpret_cast<const float4*>(zg + (int64_t)i * G + j);
      x[j] = v.x; x[j + 1] = v.y; x[j + 2] = v.z; x[j + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < G; ++j) x[j] = zg[(int64_t)i * G + j];
  }
}

// KV heads whose logits a thread requests at once (about 128 values in registers).
template <int G> struct VoteBatch { static constexpr int kB = G == 1 ? 8 : 32 / G; };

// Logits of KV heads [g0, g0 + kB) at this thread's positions; heads past Hkv - 1
// reload the last one (unused), so every load is unconditional and the waits of
// whatever was requested before them stay exact. `head_stride` = N * G floats per KV head.
template <int G, int kB, int kP>
__device__ __forceinline__ void load_batch(float (&x)[kB][kP][G], const float* z, int64_t head_stride,
                                           const int (&idx)[kP], int g0, int Hkv) {
#pragma unroll
  for (int j = 0; j < kB; ++j) {
    const float* zg = z + (int64_t)min(g0 + j, Hkv - 1) * head_stride;
#pragma unroll
    for (int e = 0; e < kP; ++e) load_group<G>(zg, idx[e], x[j][e]);
  }
}

// Selection Cache miss of request r in fold mode (every score wave has read C_Q):
// C_Q <- Q, valid <- 1, by the calling workgroup.
__device__ __forceinline__ void apply_cache_miss(const VoteParams& p, int r) {
  const uint4* src = static_cast<const uint4*>(p.q) + (int64_t)r * p.q_chunks;
  uint4* dst = static_cast<uint4*>(p.cached_q) + (int64_t)r * p.q_chunks;
  for (int i = threadIdx.x; i < p.q_chunks; i += blockDim.x) dst[i] = src[i];
  if (threadIdx.x == 0) p.valid[r] = 1;
}

// Fold mode: (M_h, log2 Z_h) of every head of request r from the score kernel's
// per-unit pairs [h][c0, c1) (rows of pair_stride units), by a workgroup of
// kFoldThreads: 16 lanes per head, 32 heads per pass; a lane takes every 16th unit,
// kFoldIn at a time in registers: their maximum, then one independent exp per pair
// for the sum, merged into the lane's running pair; a butterfly over the 16 lanes
// ends it. The first round of the first 32 heads is requested by fold_issue, ahead
// of the logits.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
constexpr int kFoldThreads = 512;          // fold-mode vote workgroup
constexpr int kFoldTile = kFoldThreads;    // its positions, one per thread
constexpr int kFoldLanes = 16, kFoldIn = 16;
constexpr int kFoldHeads = kFoldThreads / kFoldLanes;
struct FoldPairs {
  f32x2_t v[kFoldIn];
};

// First round of head threadIdx.x / 16: units c0 + l + 16 k, addresses clamped below
// c_end (>= 1); fold_finish drops the units at or past the request's end and the
// lanes past the last head, so the loads need no mask and nothing waits for them here.
__device__ __forceinline__ void fold_issue(const VoteParams& p, int c0, int c_end, FoldPairs& f) {
  const int l = threadIdx.x % kFoldLanes, h = threadIdx.x / kFoldLanes;
  const f32x2_t* src = reinterpret_cast<const f32x2_t*>(p.partials) + (int64_t)min(h, p.H - 1) * p.pair_stride;
#pragma unroll
  for (int k = 0; k < kFoldIn; ++k) f.v[k] = src[min(c0 + l + k * kFoldLanes, c_end - 1)];
}

// Max and sum of exp of one round of kFoldIn pairs (units at or past c1 dropped).
__device__ __forceinline__ void fold_round(const f32x2_t (&v)[kFoldIn], int c, int c1, float& M, float& S) {
  float mr = kNegInf;
#pragma unroll
  for (int k = 0; k < kFoldIn; ++k) mr = fmaxf(mr, c + k * kFoldLanes < c1 ? v[k].x : kNegInf);
  float sr = 0.f;
  if (mr != kNegInf) {
#pragma unroll
    for (int k = 0; k < kFoldIn; ++k)
      if (c + k * kFoldLanes < c1) sr += v[k].y * exp_via2(v[k].x - mr);
  }
  merge_ms(M, S, mr, sr);
}

// Every thread of the kFoldThreads workgroup must call it; `f` holds the first round
// from fold_issue (requested with any upper bound: units at or past c1 are dropped
// here). The first round is folded in straight-line code, so it waits only for its
// own loads and not for the logits requested after them.
__device__ void fold_finish(const VoteParams& p, int c0, int c1, const FoldPairs& f, float* s_m, float* s_l) {
  const int l = threadIdx.x % kFoldLanes;
  float M = kNegInf, S = 0.f;
  fold_round(f.v, c0 + l, c1, M, S);
  for (int h0 = 0; h0 < p.H; h0 += kFoldHeads) {
    const int h = h0 + (int)threadIdx.x / kFoldLanes;
    if (h0 > 0) { M = kNegInf; S = 0.f; }
    if (h < p.H) {
      const f32x2_t* src = reinterpret_cast<const f32x2_t*>(p.partials) + (int64_t)h * p.pair_stride;
      for (int c = c0 + l + (h0 == 0 ? kFoldIn * kFoldLanes : 0); c < c1; c += kFoldIn * kFoldLanes) {
        f32x2_t v[kFoldIn];
#pragma unroll
        for (int k = 0; k < kFoldIn; ++k) v[k] = src[min(c + k * kFoldLanes, c1 - 1)];
        fold_round(v, c, c1, M, S);
      }
    } else {
      M = kNegInf; S = 0.f;
    }
#pragma unroll
    for (int x = 1; x < kFoldLanes; x <<= 1) merge_ms(M, S, __shfl_xor(M, x), __shfl_xor(S, x));
    if (l == 0 && h < p.H) {
      s_m[h] = M;
      s_l[h] = __builtin_amdgcn_logf(S);
    }
  }
}

// One KV-head group g of a thread's positions: online log-sum-exp in base 2 over the
// group's G terms at once (one rescale of the running sum per group, then one exp
// per term); x_hi = (z_hi - M_h) log2e - log2 Z_h, where z - M is exact near the
// head maximum.
template <int G, int kP>
__device__ __forceinline__ void vote_group(const float (&x)[kP][G], const float* s_m, const float* s_l,
                                           int g, float (&m)[kP], float (&s)[kP]) {
  float mh[G], lh[G];
#pragma unroll
  for (int j = 0; j < G; ++j) { mh[j] = s_m[g * G + j]; lh[j] = s_l[g * G + j]; }
#pragma unroll
  for (int e = 0; e < kP; ++e) {
    float xv[G];
    float gm = m[e];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      xv[j] = fmaf(x[e][j] - mh[j], kLog2eF, -lh[j]);
      gm = fmaxf(gm, xv[j]);
    }
    float acc = s[e] * fast_exp2(m[e] - gm);   // 0 while m is -inf (gm is finite)
#pragma unroll
    for (int j = 0; j < G; ++j) acc += fast_exp2(xv[j] - gm);
    s[e] = acc;
    m[e] = gm;
  }
}

// Votes of 1024-position tiles (4 per thread) from the head statistics of the
// stats kernel; the logits are read one KV head group at a time.
template <int G, bool kTopP>
__global__ __launch_bounds__(kThreads) void vote_kernel(VoteParams p) {
  TS_TIMELINE_SCOPE(select, kTlVote);
  __shared__ Tables tb;
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ u64 s_mass[kTopP ? kHistBins : 1];
  __shared__ float s_m[256], s_l[256];
  const int H = p.H, Hkv = H / G;
  float x[1][kPerThread][G];
  build_tables(tb, p, one_request(p));
  TS_TIMELINE_MARK_HERE();                       // mark 0: request tables ready
  const int total = tb.tile[p.b];
  // The LDS histogram accumulates every tile this workgroup takes of one request
  // and is flushed to the global histogram (atomics) when the request changes
  // and at the end: fewer global atomics on the hot bins.
  int cur_r = -1;
  auto flush = [&](int r) {
    __syncthreads();
    uint32_t* gh = p.hist + (int64_t)r * 3 * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kThreads)
      if (s_hist[i]) atomicAdd(&gh[i], s_hist[i]);
    if (kTopP) {
      u64* gm = p.mass + (int64_t)r * 3 * kHistBins;
      for (int i = threadIdx.x; i < kHistBins; i += kThreads)
        if (s_mass[i]) atomicAdd(&gm[i], s_mass[i]);
    }
  };
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int r = find_segment(tb.tile, p.b, tile);
    const int t = tile - tb.tile[r];
    const int N = (int)(tb.tok[r + 1] - tb.tok[r]);
    const int i0 = t * kVoteTile + threadIdx.x;
    const float* z = p.logits + tb.tok[r] * H;
    const int64_t hs = (int64_t)N * G;
    int idx[kPerThread];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) idx[e] = min(i0 + e * kThreads, N - 1);
    float m[kPerThread], s[kPerThread];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) { m[e] = kNegInf; s[e] = 0.f; }
    if (r != cur_r) {
      // a new request: flush the last one's histogram, stage this one's head statistics
      if (cur_r >= 0) flush(cur_r);
      __syncthreads();
      for (int i = threadIdx.x; i < kHistBins; i += kThreads) s_hist[i] = 0;
      if (kTopP)
        for (int i = threadIdx.x; i < kHistBins; i += kThreads) s_mass[i] = 0;
      for (int h = threadIdx.x; h < H; h += kThreads) {
        s_m[h] = p.head_stats[((int64_t)r * H + h) * 2 + 0];
        s_l[h] = __builtin_amdgcn_logf(p.head_stats[((int64_t)r * H + h) * 2 + 1]);
      }
      __syncthreads();
      cur_r = r;
      TS_TIMELINE_MARK_HERE();                     // mark 1: head statistics staged
    }
#pragma unroll 2
    for (int g = 0; g < Hkv; ++g) {
      load_batch(x, z + (int64_t)g * hs, 0, idx, 0, 1);
      vote_group<G>(x[0], s_m, s_l, g, m, s);
    }
    TS_TIMELINE_MARK_HERE();                       // mark 2: votes of the tile computed
    float* vout = p.vote + tb.tok[r];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int i = i0 + e * kThreads;
      if (i < N) {
        const float lv = m[e] + __builtin_amdgcn_logf(s[e]);
        vout[i] = lv;
        const uint32_t bin = order_key(lv) >> (32 - kDigitBits0);
        atomicAdd(&s_hist[bin], 1u);
        if (kTopP) atomicAdd(&s_mass[bin], vote_mass(lv));
      }
    }
    TS_TIMELINE_MARK_HERE();                       // mark 3: stored, LDS histogram updated
  }
  if (cur_r >= 0) flush(cur_r);
}

// Fold mode (decode step, selections of at most kFoldMaxPairs (head, unit) pairs): the
// head statistics come from folding the score kernel's pairs here instead of a stats
// kernel, and Selection Cache misses are applied here. Workgroups of 512 threads
// take 512-position tiles, one position per thread, so at 128K tokens the launch fills
// every CU with two waves per SIMD and each workgroup's fold (a fixed cost: all
// pairs of the request) is spread over 512 threads. A new request's pairs are
// requested first, then the logits of its first KV heads, so the fold waits only for
// the pairs; with one request, the first tile's pairs go out before the request table
// is built.
template <int G, bool kTopP>
__global__ __launch_bounds__(kFoldThreads) void vote_fold_kernel(VoteParams p) {
  TS_TIMELINE_SCOPE(select, kTlVote);
  __shared__ int64_t s_tok[kMaxBatch + 1];
  __shared__ int32_t s_sub[kMaxBatch + 1];       // prefix of the requests' 512-position tiles
  __shared__ int32_t s_chunk[kMaxBatch + 1];     // prefix of the requests' score units
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ u64 s_mass[kTopP ? kHistBins : 1];
  __shared__ float s_m[256], s_l[256];
  const int H = p.H, Hkv = H / G;
  constexpr int kB = VoteBatch<G>::kB;           // KV heads per register set (about 32 logits)
  float x[kB][1][G], x2[kB][1][G];
  FoldPairs fp;
  const OneReq one = one_request(p);
  __builtin_amdgcn_sched_barrier(0);
  const bool pre = p.b == 1;
  if (pre) fold_issue(p, 0, p.pair_stride, fp);
  auto units = [&](int n) { return max(1, (n + p.chunk_tokens - 1) / p.chunk_tokens); };
  auto subs = [&](int n, bool skip) { return skip ? 0 : (n + kFoldTile - 1) / kFoldTile; };
  if (p.b == 1) {
    if (threadIdx.x == 0) {
      s_tok[0] = 0; s_tok[1] = one.n;
      s_sub[0] = 0; s_sub[1] = subs(one.n, one.has_skip && one.skip);
      s_chunk[0] = 0; s_chunk[1] = units(one.n);
    }
    __syncthreads();
  } else {
    block_prefix(s_tok, p.b, [&](int r) -> int64_t { return p.seq_lens[r]; });
    block_prefix(s_sub, p.b, [&](int r) -> int32_t { return subs(p.seq_lens[r], p.skip && p.skip[r]); });
    block_prefix(s_chunk, p.b, [&](int r) -> int32_t { return units(p.seq_lens[r]); });
  }
  if (p.cached_q) {
    // a request without positions has no vote tile: its Selection Cache miss is
    // applied here, by workgroup r mod grid
    for (int r = blockIdx.x; r < p.b; r += gridDim.x) {
      if (s_tok[r + 1] != s_tok[r] || (p.skip && p.skip[r])) continue;
      apply_cache_miss(p, r);
    }
  }
  TS_TIMELINE_MARK_HERE();                       // mark 0: request tables ready
  const int total = s_sub[p.b];
  int cur_r = -1;
  auto flush = [&](int r) {
    __syncthreads();
    uint32_t* gh = p.hist + (int64_t)r * 3 * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kFoldThreads)
      if (s_hist[i]) atomicAdd(&gh[i], s_hist[i]);
    if (kTopP) {
      u64* gm = p.mass + (int64_t)r * 3 * kHistBins;
      for (int i = threadIdx.x; i < kHistBins; i += kFoldThreads)
        if (s_mass[i]) atomicAdd(&gm[i], s_mass[i]);
    }
  };
  for (int st = blockIdx.x; st < total; st += gridDim.x) {
    const int r = find_segment(s_sub, p.b, st);
    const int t = st - s_sub[r];
    const int N = (int)(s_tok[r + 1] - s_tok[r]);
    const int i = t * kFoldTile + threadIdx.x;
    const int idx[1] = {min(i, N - 1)};
    const float* z = p.logits + s_tok[r] * H;
    const int64_t hs = (int64_t)N * G;
    float m[1] = {kNegInf}, s[1] = {0.f};
    if (r != cur_r && !(pre && st == (int)blockIdx.x)) fold_issue(p, s_chunk[r], s_chunk[r + 1], fp);
    __builtin_amdgcn_sched_barrier(0);           // the pairs before the logits (loads return in order)
    load_batch(x, z, hs, idx, 0, Hkv);
    if (r != cur_r) {
      // a new request: flush the last one's histogram, fold this one's head statistics
      if (cur_r >= 0) flush(cur_r);
      __syncthreads();
      for (int j = threadIdx.x; j < kHistBins; j += kFoldThreads) s_hist[j] = 0;
      if (kTopP)
        for (int j = threadIdx.x; j < kHistBins; j += kFoldThreads) s_mass[j] = 0;
      fold_finish(p, s_chunk[r], s_chunk[r + 1], fp, s_m, s_l);
      if (p.cached_q && t == 0) apply_cache_miss(p, r);
      __syncthreads();
      cur_r = r;
      TS_TIMELINE_MARK_HERE();                     // mark 1: head statistics folded
    }
    for (int g0 = 0; g0 < Hkv; g0 += 2 * kB) {
      if (g0 > 0) load_batch(x, z, hs, idx, g0, Hkv);
      if (g0 + kB < Hkv) load_batch(x2, z, hs, idx, g0 + kB, Hkv);
#pragma unroll
      for (int j = 0; j < kB; ++j)
        if (g0 + j < Hkv) vote_group<G>(x[j], s_m, s_l, g0 + j, m, s);
#pragma unroll
      for (int j = 0; j < kB; ++j)
        if (g0 + kB + j < Hkv) vote_group<G>(x2[j], s_m, s_l, g0 + kB + j, m, s);
    }
    TS_TIMELINE_MARK_HERE();                       // mark 2: votes of the tile computed
    if (i < N) {
      const float lv = m[0] + __builtin_amdgcn_logf(s[0]);
      p.vote[s_tok[r] + i] = lv;
      const uint32_t bin = order_key(lv) >> (32 - kDigitBits0);
      atomicAdd(&s_hist[bin], 1u);
      if (kTopP) atomicAdd(&s_mass[bin], vote_mass(lv));
    }
    TS_TIMELINE_MARK_HERE();                       // mark 3: stored, LDS histogram updated
  }
  if (cur_r >= 0) flush(cur_r);
}

// ---------------------------------------------------------------- TopK phases
// Three kernels (refine digit 1, refine digit 2, write); every workgroup loops over
// its share of the tiles.
// (A single cooperative kernel with grid barriers between the phases was measured
// on MI355X at 321 us per 1M-token step against 26 us for the four launches.)
template <bool kTopP>
struct SelectShared {
  Tables tb;
  uint32_t hist[kHistBins];
  u64 mass[kTopP ? kHistBins : 1];
  uint32_t w[4];
  u64 w64[4];
  u64 mres;
  int dig[2];
  int bin[2];
  int cnt[2][4];
};

// One request without top-p: a select kernel's loads for its first tile need no
// request table, so they go out before it is built, together with the table's own
// loads. Addresses are clamped to the max_tokens positions the vote buffer holds;
// positions at or past N are masked once N is known, as on the other path.
struct SelPre {
  float lv[kPerThread];             // log2 votes of the first tile (refine: strided; write: consecutive)
  uint32_t c[kHistBins / kThreads]; // refine: counts of the digit's histogram; write: digit 2's (first 4)
  int4 st[2];                       // request 0's select state
  int2 cnd0;                        // write: candidate threadIdx.x (the list is usually short)
  int tcv[4];                       // write: keys above the prefix of tiles t + 256 u (used below the first tile)
};
constexpr int kPreTiles = 4 * kThreads;   // earlier tiles whose counts are preloaded
static_assert(kPreTiles / kThreads == 4, "SelPre::tcv holds four counts per thread");

template <int kPhase>
__device__ __forceinline__ void sel_preload(const VoteParams& p, SelPre& q) {
  const int tile = blockIdx.x;
  const int4* st = reinterpret_cast<const int4*>(p.state);
  if (kPhase == 2 || kPhase == 4) { q.st[0] = st[0]; q.st[1] = st[1]; }
  if (kPhase == 1 || kPhase == 2) {
    const int i0 = tile * kVoteTile + threadIdx.x;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) q.lv[e] = p.vote[min(i0 + e * kThreads, p.max_tokens - 1)];
    load_counts<kHistBins>(p.hist + (kPhase - 1) * kHistBins, q.c);
  } else {
    const int i0 = tile * kVoteTile + threadIdx.x * kPerThread;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) q.lv[e] = p.vote[min(i0 + e, p.max_tokens - 1)];
    uint32_t c2[(1 << kDigitBits2) / kThreads];
    load_counts<1 << kDigitBits2>(p.hist + 2 * kHistBins, c2);
#pragma unroll
    for (int e = 0; e < (1 << kDigitBits2) / kThreads; ++e) q.c[e] = c2[e];
    q.cnd0 = p.cand[threadIdx.x];
    // tiles up to the first one exist in tile_counts (the grid has at most max_tiles
    // workgroups); entries at or past it are dropped at use
#pragma unroll
    for (int u = 0; u < kPreTiles / kThreads; ++u)
      q.tcv[u] = p.tile_counts[2 * min((int)threadIdx.x + u * kThreads, tile)];
  }
}

// kPass 1: find digit 0 from hist[0], histogram digit 1 of matching keys into hist[1].
// kPass 2: read digit 0 from state, find digit 1 from hist[1], histogram digit 2 into hist[2].
// A workgroup finds a request's digit once, accumulates its LDS histogram over all
// its tiles of that request and flushes it once. With kTopP the masses go along and
// each digit comes from the count-or-mass walk.
template <int kPass, bool kTopP>
__device__ void refine_phase(const VoteParams& p, SelectShared<kTopP>& sh, const SelPre& pq, bool pre TS_TIMELINE_PARAM) {
  const int total = sh.tb.tile[p.b];
  constexpr int kShift = (kPass == 1) ? (32 - kDigitBits0) : (32 - kDigitBits0 - kDigitBits1);
  constexpr int kNextBits = (kPass == 1) ? kDigitBits1 : kDigitBits2;
  constexpr int kNextShift = kShift - kNextBits;
  int cur_r = -1;
  uint32_t prefix = 0;
  auto flush = [&](int r) {
    __syncthreads();
    uint32_t* gn = p.hist + ((int64_t)r * 3 + kPass) * kHistBins;
    for (int i = threadIdx.x; i < (1 << kNextBits); i += kThreads)
      if (sh.hist[i]) atomicAdd(&gn[i], sh.hist[i]);
    if (kTopP) {
      u64* gm = p.mass + ((int64_t)r * 3 + kPass) * kHistBins;
      for (int i = threadIdx.x; i < (1 << kNextBits); i += kThreads)
        if (sh.mass[i]) atomicAdd(&gm[i], sh.mass[i]);
    }
  };
  auto record = [&](int r) {
    int32_t* st = p.state + r * 8;
    if (kPass == 1) { st[0] = sh.dig[0]; st[1] = sh.dig[1]; st[7] = 0; }
    else { st[2] = sh.dig[0]; st[3] = sh.dig[1]; }
    if (kTopP) p.mstate[r * 4 + kPass] = sh.mres;
  };
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int r = find_segment(sh.tb.tile, p.b, tile);
    const int t = tile - sh.tb.tile[r];
    const int N = (int)(sh.tb.tok[r + 1] - sh.tb.tok[r]);
    if (!kTopP && p.top_k >= N) continue;             // whole request selected: no radix work
    const int i0 = t * kVoteTile + threadIdx.x;
    const bool have = pre && tile == (int)blockIdx.x;   // the first tile was preloaded
    uint32_t key[kPerThread];
    if (have) {
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) key[e] = (i0 + e * kThreads < N) ? order_key(pq.lv[e]) : 0u;
    } else {
      load_keys(p.vote + sh.tb.tok[r], i0, N, key);
    }
    if (r != cur_r) {
      if (cur_r >= 0) flush(cur_r);
      __syncthreads();
      int32_t* st = p.state + r * 8;
      const uint32_t* gh = p.hist + (int64_t)r * 3 * kHistBins;
      const u64* gm = p.mass + (int64_t)r * 3 * kHistBins;
      if (have) {
        if (kPass == 1) {
          find_digit_c<1 << kDigitBits0>(pq.c, p.top_k, sh.dig, sh.w);
          prefix = (uint32_t)sh.dig[0];
        } else {
          find_digit_c<1 << kDigitBits1>(pq.c, pq.st[0].y, sh.dig, sh.w);
          prefix = ((uint32_t)pq.st[0].x << kDigitBits1) | (uint32_t)sh.dig[0];
        }
      } else if (kPass == 1) {
        if (kTopP) {
          // target mass: ceil(p * total mass of the request)
          u64 part = 0;
#pragma unroll
          for (int e = 0; e < kHistBins / kThreads; ++e) part += gm[threadIdx.x + e * kThreads];
          const u64 Q = block_excl_scan64(part, sh.w64) + part;    // inclusive: thread 255 holds the total
          if (threadIdx.x == kThreads - 1) sh.mres = Q;
          __syncthreads();
          const u64 total_mass = sh.mres;
          __syncthreads();
          u64 target = (u64)ceil(p.top_p * (double)total_mass);
          if (target < 1) target = 1;
          if (t == 0 && threadIdx.x == 0) p.mstate[r * 4 + 0] = target;
          find_digit_pk<1 << kDigitBits0>(gh, gm, min(p.top_k, N), target, sh.dig, &sh.mres, sh.w,
                                          sh.w64, sh.bin);
        } else {
          find_digit<1 << kDigitBits0>(gh, p.top_k, sh.dig, sh.w);
        }
        prefix = (uint32_t)sh.dig[0];
      } else {
        const int d0 = st[0], k0 = st[1];
        if (kTopP)
          find_digit_pk<1 << kDigitBits1>(gh + kHistBins, gm + kHistBins, k0, p.mstate[r * 4 + 1],
                                          sh.dig, &sh.mres, sh.w, sh.w64, sh.bin);
        else
          find_digit<1 << kDigitBits1>(gh + kHistBins, k0, sh.dig, sh.w);
        prefix = ((uint32_t)d0 << kDigitBits1) | (uint32_t)sh.dig[0];
      }
      if (t == 0 && threadIdx.x == 0) record(r);
      for (int i = threadIdx.x; i < (1 << kNextBits); i += kThreads) sh.hist[i] = 0;
      if (kTopP)
        for (int i = threadIdx.x; i < (1 << kNextBits); i += kThreads) sh.mass[i] = 0;
      __syncthreads();
      cur_r = r;
      TS_TIMELINE_MARK_HERE();                     // mark 1: digit found
    } else if (t == 0 && threadIdx.x == 0) {
      record(r);
    }
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (i0 + e * kThreads < N && (key[e] >> kShift) == prefix) {
        const uint32_t bin = (key[e] >> kNextShift) & ((1u << kNextBits) - 1);
        atomicAdd(&sh.hist[bin], 1u);
        if (kTopP) atomicAdd(&sh.mass[bin], vote_mass(key_value(key[e])));
      }
    }
    TS_TIMELINE_MARK_HERE();                       // mark 2: LDS histogram of the tile
    if (kPass == 2) {
      // The threshold key shares the 22-bit prefix found here. For the write pass:
      // how many of this tile's keys lie above the prefix (all selected) and on it,
      // and the keys on it with their positions, appended to the request's list
      // (one atomic per wavefront and slot group; entries past kCandCap are counted,
      // not stored).
      const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
      int above = 0, on = 0;
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) {
        const int i = i0 + e * kThreads;
        const bool in = i < N;
        const uint32_t top = key[e] >> kShift;
        above += (in && top > prefix) ? 1 : 0;
        const bool m = in && top == prefix;
        on += m ? 1 : 0;
        const unsigned long long mask = __ballot(m);
        if (mask) {
          const int leader = __ffsll((long long)mask) - 1;
          int base = 0;
          if (lane == leader) base = atomicAdd(&p.state[r * 8 + 7], __popcll(mask));
          base = __shfl(base, leader);
          if (m) {
            const int slot = base + __popcll(mask & ((1ull << lane) - 1ull));
            if (slot < kCandCap) p.cand[(int64_t)r * kCandCap + slot] = make_int2((int)key[e], i);
          }
        }
      }
      above = wave_sum_i(above);
      on = wave_sum_i(on);
      if (lane == 0) { sh.cnt[0][wave] = above; sh.cnt[1][wave] = on; }
      __syncthreads();
      if (threadIdx.x == 0) {
        p.tile_counts[(int64_t)tile * 2 + 0] = sh.cnt[0][0] + sh.cnt[0][1] + sh.cnt[0][2] + sh.cnt[0][3];
        p.tile_counts[(int64_t)tile * 2 + 1] = sh.cnt[1][0] + sh.cnt[1][1] + sh.cnt[1][2] + sh.cnt[1][3];
      }
      __syncthreads();
    }
  }
  if (cur_r >= 0) flush(cur_r);
}

// Exact threshold key of request r, how many keys equal to it are taken, and the
// size of the selection (top_k, or the top-p budget capped at min(top_k, N)).
template <bool kTopP>
__device__ void threshold(const VoteParams& p, int r, int N, uint32_t& key_t, int& take_eq, int& m_sel,
                          SelectShared<kTopP>& sh, bool record, const SelPre& pq, bool pre) {
  int32_t* st = p.state + r * 8;
  const int d0 = pre ? pq.st[0].x : st[0], d1 = pre ? pq.st[0].z : st[2], k1 = pre ? pq.st[0].w : st[3];
  const uint32_t* h2 = p.hist + ((int64_t)r * 3 + 2) * kHistBins;
  if (pre) {
    uint32_t c2[(1 << kDigitBits2) / kThreads];
#pragma unroll
    for (int e = 0; e < (1 << kDigitBits2) / kThreads; ++e) c2[e] = pq.c[e];
    find_digit_c<1 << kDigitBits2>(c2, k1, sh.dig, sh.w);
  } else if (kTopP) {
    find_digit_pk<1 << kDigitBits2>(h2, p.mass + ((int64_t)r * 3 + 2) * kHistBins, k1,
                                    p.mstate[r * 4 + 2], sh.dig, &sh.mres, sh.w, sh.w64, sh.bin);
  } else {
    find_digit<1 << kDigitBits2>(h2, k1, sh.dig, sh.w);
  }
  key_t = ((uint32_t)d0 << (kDigitBits1 + kDigitBits2)) | ((uint32_t)d1 << kDigitBits2) |
          (uint32_t)sh.dig[0];
  const int kres = sh.dig[1];
  if (kTopP) {
    // keys equal to key_t all carry the same mass q; take just enough of them
    const u64 q = vote_mass(key_value(key_t));
    const u64 mres = sh.mres;
    const u64 need = q ? (mres + q - 1) / q : (u64)kres;
    take_eq = (int)min((u64)kres, need);
    m_sel = min(p.top_k, N) - kres + take_eq;
  } else {
    take_eq = kres;
    m_sel = p.top_k;
  }
  if (record && threadIdx.x == 0) { st[4] = sh.dig[0]; st[5] = take_eq; st[6] = m_sel; }
}

// Ascending positions through a prefix over the request's tiles.
template <bool kTopP>
__device__ void write_phase(const VoteParams& p, SelectShared<kTopP>& sh, const SelPre& pq, bool pre TS_TIMELINE_PARAM) {
  const int total = sh.tb.tile[p.b];
  // a request with no positions (a first prefill chunk) has no tile to do it
  if (blockIdx.x == 0)
    for (int r = threadIdx.x; r < p.b; r += kThreads)
      if (p.seq_lens[r] == 0 && !(p.skip && p.skip[r])) p.sel_count[r] = 0;
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int r = find_segment(sh.tb.tile, p.b, tile);
    const int t = tile - sh.tb.tile[r];
    const int N = (int)(sh.tb.tok[r + 1] - sh.tb.tok[r]);
    const int k = p.top_k;
    int32_t* out = p.sel_idx + (int64_t)r * k;
    // this thread owns kPerThread consecutive positions
    const int i0 = t * kVoteTile + threadIdx.x * kPerThread;
    if (!kTopP) {
      if (t == 0 && threadIdx.x == 0) p.sel_count[r] = min(k, N);
      if (k >= N) {
        for (int e = 0; e < kPerThread; ++e)
          if (i0 + e < N) out[i0 + e] = i0 + e;
        continue;
      }
    }
    const float* lv = p.vote + sh.tb.tok[r];
    const bool have = pre && tile == (int)blockIdx.x;   // the first tile was preloaded
    float x[kPerThread];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) x[e] = have ? pq.lv[e] : lv[min(i0 + e, N - 1)];
    // Keys of the request's earlier tiles that sort before this tile's: every key
    // above the threshold's 22-bit prefix (counted per tile by the previous pass;
    // 8-byte loads, four in flight per thread before they are added), plus the keys
    // on the prefix that are greater than or equal to the exact threshold (from the
    // request's list of prefix keys, or, when the list overflowed, by reading the
    // earlier tiles that hold prefix keys again).
    const int n_cand = have ? pq.st[1].w : p.state[r * 8 + 7];
    const int tile_lo = t * kVoteTile;
    int gtb = 0, eqb = 0;
    if (have) {
#pragma unroll
      for (int u = 0; u < kPreTiles / kThreads; ++u) gtb += ((int)threadIdx.x + u * kThreads < t) ? pq.tcv[u] : 0;
    }
    typedef int32_t i32x2_t __attribute__((ext_vector_type(2)));
    const i32x2_t* tc = reinterpret_cast<const i32x2_t*>(p.tile_counts) + sh.tb.tile[r];
    int tt = threadIdx.x + (have ? kPreTiles : 0);
    for (; tt + 3 * kThreads < t; tt += 4 * kThreads) {
      i32x2_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = tc[tt + u * kThreads];
#pragma unroll
      for (int u = 0; u < 4; ++u) gtb += v[u].x;
    }
    for (; tt < t; tt += kThreads) gtb += tc[tt].x;
    int2 cnd[kCandCap / kThreads];
    if (n_cand <= kCandCap) {
#pragma unroll
      for (int u = 0; u < kCandCap / kThreads; ++u) {
        const int j = threadIdx.x + u * kThreads;
        cnd[u] = (j >= n_cand) ? make_int2(0, 0x7fffffff) : (have && u == 0) ? pq.cnd0 : p.cand[(int64_t)r * kCandCap + j];
      }
    }
    __syncthreads();
    uint32_t key_t;
    int take_eq, m_sel;
    threshold<kTopP>(p, r, N, key_t, take_eq, m_sel, sh, false, pq, have);
    TS_TIMELINE_MARK_HERE();                       // mark 1: threshold found
    if (kTopP && t == 0 && threadIdx.x == 0) p.sel_count[r] = m_sel;
    if (n_cand <= kCandCap) {
#pragma unroll
      for (int u = 0; u < kCandCap / kThreads; ++u) {
        if (cnd[u].y < tile_lo) {
          gtb += ((uint32_t)cnd[u].x > key_t) ? 1 : 0;
          eqb += ((uint32_t)cnd[u].x == key_t) ? 1 : 0;
        }
      }
    } else {
      // overflow (many keys within 2^-13 of the threshold, e.g. exact ties): read
      // the earlier tiles that hold prefix keys again, four tiles a round
      const uint32_t pre22 = key_t >> kDigitBits2;
      for (int t0 = 0; t0 < t; t0 += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int t1 = t0 + u;
          if (t1 < t && tc[t1].y > 0) {
            uint32_t k2[kPerThread];
            load_keys(lv, t1 * kVoteTile + threadIdx.x, N, k2);
#pragma unroll
            for (int e = 0; e < kPerThread; ++e) {
              const bool on = (t1 * kVoteTile + threadIdx.x + e * kThreads < N) && (k2[e] >> kDigitBits2) == pre22;
              gtb += (on && k2[e] > key_t) ? 1 : 0;
              eqb += (on && k2[e] == key_t) ? 1 : 0;
            }
          }
        }
      }
    }
    gtb = wave_sum_i(gtb);
    eqb = wave_sum_i(eqb);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { sh.cnt[0][wave] = gtb; sh.cnt[1][wave] = eqb; }
    __syncthreads();
    gtb = sh.cnt[0][0] + sh.cnt[0][1] + sh.cnt[0][2] + sh.cnt[0][3];
    eqb = sh.cnt[1][0] + sh.cnt[1][1] + sh.cnt[1][2] + sh.cnt[1][3];
    TS_TIMELINE_MARK_HERE();                       // mark 2: keys before the tile counted
    uint32_t keys[kPerThread];
    uint32_t packed = 0;                              // (equal << 16) | greater
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const bool in = i0 + e < N;
      keys[e] = in ? order_key(x[e]) : 0u;
      if (in) packed += (keys[e] > key_t) ? 1u : ((keys[e] == key_t) ? (1u << 16) : 0u);
    }
    const uint32_t pre = block_excl_scan(packed, sh.w);
    int g_run = gtb + (int)(pre & 0xffffu);
    int e_run = eqb + (int)(pre >> 16);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int i = i0 + e;
      const bool in = i < N;
      const bool greater = in && keys[e] > key_t;
      const bool equal = in && keys[e] == key_t;
      const int pos = g_run + min(e_run, take_eq);
      if ((greater || (equal && e_run < take_eq)) && pos < k) out[pos] = i;
      g_run += greater;
      e_run += equal;
    }
  }
}

template <int kPhase, bool kTopP>
__global__ __launch_bounds__(kThreads) void select_phase_kernel(VoteParams p) {
  TS_TIMELINE_SCOPE(select, kTlVote + kPhase);
  __shared__ SelectShared<kTopP> sh;
  SelPre q;
  const OneReq one = one_request(p);
  __builtin_amdgcn_sched_barrier(0);               // the length goes out before the preloads
  const bool pre = !kTopP && p.b == 1 && p.max_tokens > 0;
  if (pre) sel_preload<kPhase>(p, q);
  build_tables(sh.tb, p, one);
  TS_TIMELINE_MARK_HERE();                         // mark 0: request tables ready
  if (kPhase == 1) refine_phase<1, kTopP>(p, sh, q, pre TS_TIMELINE_ARG);
  if (kPhase == 2) refine_phase<2, kTopP>(p, sh, q, pre TS_TIMELINE_ARG);
  if (kPhase == 4) write_phase<kTopP>(p, sh, q, pre TS_TIMELINE_ARG);
}

// Digit-0 histogram of any score array (the selection-function ablations run the
// TopK phases on scores other than the soft vote): same tiles as the vote kernel.
__global__ __launch_bounds__(kThreads) void hist0_kernel(VoteParams p) {
  __shared__ Tables tb;
  __shared__ uint32_t s_hist[kHistBins];
  build_tables(tb, p, one_request(p));
  const int total = tb.tile[p.b];
  int cur_r = -1;
  auto flush = [&](int r) {
    __syncthreads();
    uint32_t* gh = p.hist + (int64_t)r * 3 * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kThreads)
      if (s_hist[i]) atomicAdd(&gh[i], s_hist[i]);
  };
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int r = find_segment(tb.tile, p.b, tile);
    const int t = tile - tb.tile[r];
    const int N = (int)(tb.tok[r + 1] - tb.tok[r]);
    if (r != cur_r) {
      if (cur_r >= 0) flush(cur_r);
      __syncthreads();
      for (int i = threadIdx.x; i < kHistBins; i += kThreads) s_hist[i] = 0;
      __syncthreads();
      cur_r = r;
    }
    const int i0 = t * kVoteTile + threadIdx.x;
    uint32_t key[kPerThread];
    load_keys(p.vote + tb.tok[r], i0, N, key);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      if (i0 + e * kThreads < N) atomicAdd(&s_hist[key[e] >> (32 - kDigitBits0)], 1u);
  }
  if (cur_r >= 0) flush(cur_r);
}

__global__ void zero_u32(uint32_t* x, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    x[i] = 0u;
}

template <bool kTopP, bool kFold>
hipError_t launch_vote_kernel(const VoteParams& p, hipStream_t s) {
  if (kFold) {
    const dim3 fgrid(std::max(1, std::min(p.fold_grid, kMaxFoldGrid))), fblock(kFoldThreads);
    switch (p.G) {
      case 1: hipLaunchKernelGGL((vote_fold_kernel<1, kTopP>), fgrid, fblock, 0, s, p); break;
      case 2: hipLaunchKernelGGL((vote_fold_kernel<2, kTopP>), fgrid, fblock, 0, s, p); break;
      case 3: hipLaunchKernelGGL((vote_fold_kernel<3, kTopP>), fgrid, fblock, 0, s, p); break;
      case 4: hipLaunchKernelGGL((vote_fold_kernel<4, kTopP>), fgrid, fblock, 0, s, p); break;
      case 5: hipLaunchKernelGGL((vote_fold_kernel<5, kTopP>), fgrid, fblock, 0, s, p); break;
      case 6: hipLaunchKernelGGL((vote_fold_kernel<6, kTopP>), fgrid, fblock, 0, s, p); break;
      case 7: hipLaunchKernelGGL((vote_fold_kernel<7, kTopP>), fgrid, fblock, 0, s, p); break;
      case 8: hipLaunchKernelGGL((vote_fold_kernel<8, kTopP>), fgrid, fblock, 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
    return hipSuccess;
  }
  const dim3 vgrid(std::min(p.grid, kVoteMaxGrid)), block(kThreads);
  switch (p.G) {
    case 1: hipLaunchKernelGGL((vote_kernel<1, kTopP>), vgrid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((vote_kernel<2, kTopP>), vgrid, block, 0, s, p); break;
    case 3: hipLaunchKernelGGL((vote_kernel<3, kTopP>), vgrid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((vote_kernel<4, kTopP>), vgrid, block, 0, s, p); break;
    case 5: hipLaunchKernelGGL((vote_kernel<5, kTopP>), vgrid, block, 0, s, p); break;
    case 6: hipLaunchKernelGGL((vote_kernel<6, kTopP>), vgrid, block, 0, s, p); break;
    case 7: hipLaunchKernelGGL((vote_kernel<7, kTopP>), vgrid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL((vote_kernel<8, kTopP>), vgrid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}

template <bool kTopP>
hipError_t launch_vote_topk_t(const VoteParams& p, hipStream_t s, bool zero_hist) {
  if (zero_hist) {
    const int64_t n = (int64_t)p.b * 3 * kHistBins;
    hipLaunchKernelGGL(zero_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p.hist, n);
    if (kTopP)
      hipLaunchKernelGGL(zero_u32, dim3((unsigned)((2 * n + 255) / 256)), dim3(256), 0, s,
                         reinterpret_cast<uint32_t*>(p.mass), 2 * n);
  }
  const dim3 grid(p.grid), block(kThreads);
  const hipError_t e = p.fold ? launch_vote_kernel<kTopP, true>(p, s) : launch_vote_kernel<kTopP, false>(p, s);
  if (e != hipSuccess) return e;
  const dim3 rgrid(std::min(p.grid, kRefineMaxGrid));
  hipLaunchKernelGGL((select_phase_kernel<1, kTopP>), rgrid, block, 0, s, p);
  hipLaunchKernelGGL((select_phase_kernel<2, kTopP>), grid, block, 0, s, p);
  hipLaunchKernelGGL((select_phase_kernel<4, kTopP>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_vote_topk(const VoteParams& p, hipStream_t s, bool zero_hist) {
  return p.topp ? launch_vote_topk_t<true>(p, s, zero_hist) : launch_vote_topk_t<false>(p, s, zero_hist);
}

hipError_t launch_vote_only(const VoteParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.b * 3 * kHistBins;
  hipLaunchKernelGGL(zero_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p.hist, n);
  const hipError_t e = launch_vote_kernel<false, false>(p, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_score_select(const VoteParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.b * 3 * kHistBins;
  hipLaunchKernelGGL(zero_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p.hist, n);
  const dim3 grid(p.grid), block(kThreads);
  hipLaunchKernelGGL(hist0_kernel, dim3(std::min(p.grid, kVoteMaxGrid)), block, 0, s, p);
  hipLaunchKernelGGL((select_phase_kernel<1, false>), dim3(std::min(p.grid, kRefineMaxGrid)), block, 0, s, p);
  hipLaunchKernelGGL((select_phase_kernel<2, false>), grid, block, 0, s, p);
  hipLaunchKernelGGL((select_phase_kernel<4, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace ts
