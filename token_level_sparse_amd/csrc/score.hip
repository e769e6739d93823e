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
// folds the per-unit pairs into (M_h, Z_h). Logits are laid out [H_kv][N][G], so
// a page's 16 tokens x G heads land as one contiguous 64 G-byte block.
#include <type_traits>

#include "cache.h"
#include "common.h"
#include "kernels.h"
#include "timeline.h"

TS_TIMELINE_DEFINE(score)

namespace ts {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

#ifndef TS_SCORE_UNROLL
#define TS_SCORE_UNROLL 4
#endif
constexpr int kUnroll = TS_SCORE_UNROLL;   // pages in flight per wave

// Query head slots. A lane holds kSlots query slices; slot s of lane col is head
//   h(col, s) = (sA ^ b3) + 2 (sB ^ b2 ^ b3) + 4 sC,  s = sA + 2 sB + 4 sC,
// with b2, b3 bits 2 and 3 of col (heads >= G are zero). This per-lane order makes
// the first two butterfly steps of the row reduction below pair equal heads with
// a plain DPP add, without selects.
template <int G> struct Slots { static constexpr int kN = (G <= 4) ? 4 : 8; };

__device__ __forceinline__ int slot_head(int col, int s) {
  const int b2 = (col >> 2) & 1, b3 = (col >> 3) & 1;
  return ((s & 1) ^ b3) + 2 * (((s >> 1) & 1) ^ b2 ^ b3) + 4 * (s >> 2);
}

template <bool kBf16, int S> struct QRegs;
template <int S> struct QRegs<true, S> { uint32_t w[S][4]; };
template <int S> struct QRegs<false, S> { float w[S][8]; };
// fp32 query against bf16 keys (the mean query of a prefill chunk): dims
// [8 col, 8 col + 8) as floats.
template <int S> struct QRegsMixed { float w[S][8]; };

template <bool kBf16, bool kQ32, int S> struct QSel {
  using type = QRegs<kBf16, S>;
  using elem = typename std::conditional<kBf16, uint16_t, float>::type;
};
template <int S> struct QSel<true, true, S> {
  using type = QRegsMixed<S>;
  using elem = float;
};

template <bool kBf16> struct PageRegs;
template <> struct PageRegs<true> { uint4 w[4]; };
template <> struct PageRegs<false> { float4 w[4][2]; };

#ifndef TS_SCORE_NT
#define TS_SCORE_NT 1
#endif
// The K stream is read once per step: its loads are marked nontemporal.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
#if TS_SCORE_NT
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *p;
#endif
}
__device__ __forceinline__ float4 stream_load(const float4* p) {
#if TS_SCORE_NT
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
#else
  return *p;
#endif
}

#ifndef TS_SCORE_NT_STORE
#define TS_SCORE_NT_STORE 0
#endif
__device__ __forceinline__ void stream_store(float* p, float v) {
#if TS_SCORE_NT_STORE
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// bf16: a token row is 256 B, lane col reads dims [8 col, 8 col + 8).
// fp32: a token row is 512 B, lane col reads dims [4 col, 4 col + 4) and
// [64 + 4 col, 64 + 4 col + 4), so each load instruction covers 256 contiguous bytes.
template <int G, int S>
__device__ __forceinline__ void load_q(QRegs<true, S>& qr, const uint16_t* qb, int col) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int h = slot_head(col, s);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (h < G) v = *reinterpret_cast<const uint4*>(qb + h * kHeadDim + 8 * col);
    qr.w[s][0] = v.x; qr.w[s][1] = v.y; qr.w[s][2] = v.z; qr.w[s][3] = v.w;
  }
}
template <int G, int S>
__device__ __forceinline__ void load_q(QRegs<false, S>& qr, const float* qb, int col) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int h = slot_head(col, s);
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), c = a;
    if (h < G) {
      a = *reinterpret_cast<const float4*>(qb + h * kHeadDim + 4 * col);
      c = *reinterpret_cast<const float4*>(qb + h * kHeadDim + 64 + 4 * col);
    }
    qr.w[s][0] = a.x; qr.w[s][1] = a.y; qr.w[s][2] = a.z; qr.w[s][3] = a.w;
    qr.w[s][4] = c.x; qr.w[s][5] = c.y; qr.w[s][6] = c.z; qr.w[s][7] = c.w;
  }
}

template <int G, int S>
__device__ __forceinline__ void load_q(QRegsMixed<S>& qr, const float* qb, int col) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int h = slot_head(col, s);
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), c = a;
    if (h < G) {
      a = *reinterpret_cast<const float4*>(qb + h * kHeadDim + 8 * col);
      c = *reinterpret_cast<const float4*>(qb + h * kHeadDim + 8 * col + 4);
    }
    qr.w[s][0] = a.x; qr.w[s][1] = a.y; qr.w[s][2] = a.z; qr.w[s][3] = a.w;
    qr.w[s][4] = c.x; qr.w[s][5] = c.y; qr.w[s][6] = c.z; qr.w[s][7] = c.w;
  }
}

__device__ __forceinline__ void load_page(PageRegs<true>& pr, const uint16_t* base, int row, int col) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    pr.w[j] = stream_load(reinterpret_cast<const uint4*>(base + (4 * j + row) * kHeadDim + 8 * col));
}
__device__ __forceinline__ void load_page(PageRegs<false>& pr, const float* base, int row, int col) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    pr.w[j][0] = stream_load(reinterpret_cast<const float4*>(base + (4 * j + row) * kHeadDim + 4 * col));
    pr.w[j][1] = stream_load(reinterpret_cast<const float4*>(base + (4 * j + row) * kHeadDim + 64 + 4 * col));
  }
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Partial inner products of the lane's 8 dims: acc[j][s] for token 4 j + row, slot s.
template <int S>
__device__ __forceinline__ void lane_dots(const PageRegs<true>& pr, const QRegs<true, S>& qr,
                                          float (&acc)[4][S]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      float a = dot2(pr.w[j].x, qr.w[s][0], 0.f);
      a = dot2(pr.w[j].y, qr.w[s][1], a);
      a = dot2(pr.w[j].z, qr.w[s][2], a);
      acc[j][s] = dot2(pr.w[j].w, qr.w[s][3], a);
    }
  }
}
template <int S>
__device__ __forceinline__ void lane_dots(const PageRegs<false>& pr, const QRegs<false, S>& qr,
                                          float (&acc)[4][S]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      float a = pr.w[j][0].x * qr.w[s][0];
      a = fmaf(pr.w[j][0].y, qr.w[s][1], a);
      a = fmaf(pr.w[j][0].z, qr.w[s][2], a);
      a = fmaf(pr.w[j][0].w, qr.w[s][3], a);
      a = fmaf(pr.w[j][1].x, qr.w[s][4], a);
      a = fmaf(pr.w[j][1].y, qr.w[s][5], a);
      a = fmaf(pr.w[j][1].z, qr.w[s][6], a);
      acc[j][s] = fmaf(pr.w[j][1].w, qr.w[s][7], a);
    }
  }
}

// bf16 keys widened to fp32 (exact), then fp32 FMAs with the fp32 query.
template <int S>
__device__ __forceinline__ void lane_dots(const PageRegs<true>& pr, const QRegsMixed<S>& qr,
                                          float (&acc)[4][S]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w[4] = {pr.w[j].x, pr.w[j].y, pr.w[j].z, pr.w[j].w};
    float k[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      k[2 * t] = __uint_as_float(w[t] << 16);
      k[2 * t + 1] = __uint_as_float(w[t] & 0xffff0000u);
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      float a = k[0] * qr.w[s][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) a = fmaf(k[e], qr.w[s][e], a);
      acc[j][s] = a;
    }
  }
}

constexpr int kDppXor3 = 0x1B;        // quad_perm [3,2,1,0]

// Reduce-scatter over the 16 lanes of a row: 4 tokens x S slots in, S/4 values
// out. Partners lane ^ 15, ^ 7, ^ 3, ^ 1 span the row. Steps 1-2 pair slots of
// equal head (see slot_head); steps 3-4 split the tokens by lane bits 1 and 0.
// Lane col ends with token j = col & 3 of its row and heads b3 + 2 (b2 ^ b3) + 4 c.
template <int S>
__device__ __forceinline__ void row_reduce_scatter(const float (&acc)[4][S], int col,
                                                   float (&out)[S / 4]) {
  float r1[4][S / 2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int t = 0; t < S / 2; ++t) r1[j][t] = acc[j][2 * t] + dpp_f<kDppMirror>(acc[j][2 * t + 1]);
  float r2[4][S / 4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int c = 0; c < S / 4; ++c) r2[j][c] = r1[j][2 * c] + dpp_f<kDppHalfMirror>(r1[j][2 * c + 1]);
  const bool b1 = (col >> 1) & 1, b0 = col & 1;
#pragma unroll
  for (int c = 0; c < S / 4; ++c) {
    float r3[2];
#pragma unroll
    for (int j0 = 0; j0 < 2; ++j0) {
      const float lo = r2[j0][c], hi = r2[j0 + 2][c];
      r3[j0] = (b1 ? hi : lo) + dpp_f<kDppXor3>(b1 ? lo : hi);
    }
    out[c] = (b0 ? r3[1] : r3[0]) + dpp_f<kDppXor1>(b0 ? r3[0] : r3[1]);
  }
}

// Work chunks of request r. With the Selection Cache every request has at least one
// (an empty request's units only take the cache decision), so the score kernel
// writes hit[r] for all of them; a skipped request has none.
__device__ __forceinline__ int32_t score_chunks(const ScoreParams& p, int r, int chunk_tokens) {
  const int32_t c = (p.seq_lens[r] + chunk_tokens - 1) / chunk_tokens;
  if (p.cache) return c > 1 ? c : 1;
  return (p.skip && p.skip[r]) ? 0 : c;
}

template <bool kBf16, bool kQ32, int G>
__global__ __launch_bounds__(256) void score_kernel(ScoreParams p) {
  TS_TIMELINE_SCOPE(score, kTlScore);
  using T = typename std::conditional<kBf16, uint16_t, float>::type;
  constexpr int S = Slots<G>::kN;
  using QR = typename QSel<kBf16, kQ32, S>::type;
  using TQ = typename QSel<kBf16, kQ32, S>::elem;
  constexpr int C = S / 4;                     // values a lane owns per page
  __shared__ int64_t s_tok[kMaxBatch + 1];
  __shared__ int32_t s_chunk[kMaxBatch + 1];

  const int b = p.b;
  const int chunk_tokens = p.chunk_pages * kPage;
  __shared__ double s_red[3][4];
  // One request: its length is a scalar load at the start (no wait behind vector
  // loads), and the Selection Cache test needs no request table, so its query chunks
  // go out at once and the request is decided once, before the units.
  // (Unconditional scalar loads: a null skip or valid array reads seq_lens instead.)
  const int n0 = p.seq_lens[0];
  const int skip0 = (p.skip ? p.skip : p.seq_lens)[0];
  const int valid0 = (p.valid ? p.valid : p.seq_lens)[0];
  const bool decide_first = p.cache && b == 1;
  CachePre cpre;
  if (decide_first && p.theta <= kCacheNeverHit) cache_preload<kBf16>(p.q, p.cached_q, 0, p.H * kHeadDim, cpre);
  if (p.fold) {
    // fold mode runs no stats kernel: the workgroups clear the radix histograms (and
    // top-p masses) of the TopK that follows, every request's (a cache hit's are
    // not read)
    uint4* hg = reinterpret_cast<uint4*>(p.hist);
    const int64_t nh = (int64_t)b * 3 * kHistBins / 4, nm = p.mass ? 2 * nh : 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nh + nm; i += (int64_t)gridDim.x * 256) {
      uint4* dst = (i < nh) ? hg + i : reinterpret_cast<uint4*>(p.mass) + (i - nh);
      *dst = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  if (b == 1) {
    if (threadIdx.x == 0) {
      s_tok[0] = 0;
      s_tok[1] = n0;
      const int32_t c = (n0 + chunk_tokens - 1) / chunk_tokens;
      s_chunk[0] = 0;
      s_chunk[1] = p.cache ? (c > 1 ? c : 1) : ((p.skip && skip0) ? 0 : c);
    }
    __syncthreads();
  } else {
    block_prefix(s_tok, b, [&](int r) -> int64_t { return p.seq_lens[r]; });
    block_prefix(s_chunk, b, [&](int r) -> int32_t { return score_chunks(p, r, chunk_tokens); });
  }
  TS_TIMELINE_MARK_HERE();                     // mark 0: request tables ready (after a barrier)

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int dec_lo = -1, dec_hi = -1;                // requests of the last decided block (uniform)
  int hit_v = 0;                               // the cache decision of this wave's request
  if (decide_first) {
    hit_v = cache_hit_wg<kBf16>(p.q, p.cached_q, 0, p.H * kHeadDim, valid0, p.theta, s_red, &cpre);
    if (threadIdx.x == 0) p.hit[0] = hit_v;
    dec_lo = dec_hi = 0;
    TS_TIMELINE_MARK_HERE();                   // mark 1: Selection Cache decided
  }
  const int row = lane >> 4, col = lane & 15;
  const int H = p.H, Hkv = p.Hkv;
  const int total_units = s_chunk[b] * Hkv;
  const TQ* qall = static_cast<const TQ*>(p.q);
  const T* pool = static_cast<const T*>(p.k_pool);
  // this lane's outputs: token 4 (col & 3) + row of each page, heads hd[c]
  const int tok_in_page = 4 * (col & 3) + row;
  int hd[C];
#pragma unroll
  for (int c = 0; c < C; ++c) hd[c] = slot_head(col, 4 * c);

  // XCD-aware order: workgroup i runs on XCD i % 8, so each XCD takes one
  // contiguous range of unit blocks (4 units = 4 waves), and all KV heads of a
  // chunk (adjacent blocks in the pool) are read through the same L2 and TLB.
  const int n_xcd = (gridDim.x % kXcds == 0) ? kXcds : 1;
  const int xcd = blockIdx.x % n_xcd, rank = blockIdx.x / n_xcd;
  const int per_xcd_wg = gridDim.x / n_xcd;
  const int blocks = (total_units + 3) / 4;
  const int blk_lo = (int)((int64_t)blocks * xcd / n_xcd);
  const int blk_hi = (int)((int64_t)blocks * (xcd + 1) / n_xcd);
  for (int blk = blk_lo + rank; blk < blk_hi; blk += per_xcd_wg) {
    const int u = blk * 4 + wave;
    // Wave-uniform unit coordinates (readfirstlane lets the block-table reads
    // below be scalar loads, which do not wait on the in-flight page loads).
    const int cg = __builtin_amdgcn_readfirstlane(min(u, total_units - 1) / Hkv);
    const int g = __builtin_amdgcn_readfirstlane(u - cg * Hkv);
    const int r = __builtin_amdgcn_readfirstlane(find_segment(s_chunk, b, cg));
    if (p.cache) {
      // Selection Cache (step 0): the workgroup decides each request its block
      // touches, the same way in every workgroup; a hit skips the request's scoring.
      // The block's first and last requests are uniform over the workgroup, so are
      // the barriers inside the decision.
      const int r_lo = find_segment(s_chunk, b, (blk * 4) / Hkv);
      const int r_hi = find_segment(s_chunk, b, min(blk * 4 + 3, total_units - 1) / Hkv);
      if (r_lo != dec_lo || r_hi != dec_hi) {
        for (int rr = r_lo; rr <= r_hi; ++rr) {
          const int h = cache_hit_wg<kBf16>(p.q, p.cached_q, rr, H * kHeadDim, p.valid[rr],
                                            p.theta, s_red);
          if (rr == r) hit_v = h;
          if (threadIdx.x == 0) p.hit[rr] = h;
        }
        dec_lo = r_lo;
        dec_hi = r_hi;
        TS_TIMELINE_MARK_HERE();                 // mark 1: Selection Cache decided
      }
    }
    if (u >= total_units) break;                 // only in the workgroup's last block
    if (p.cache && hit_v) continue;
    const int c0 = cg - __builtin_amdgcn_readfirstlane(s_chunk[r]);
    const int N = (int)(s_tok[r + 1] - s_tok[r]);
    const int n_pages = (N + kPage - 1) / kPage;
    const int pg0 = c0 * p.chunk_pages;
    const int pg1 = min(n_pages, pg0 + p.chunk_pages);

    QR q;
    load_q<G>(q, qall + ((int64_t)r * H + g * G) * kHeadDim, col);
    const int32_t* bt = p.block_table + (int64_t)r * p.stride;
    // logits of KV head g: [N][G] (token-major, the group's heads adjacent)
    float* zrow = p.logits + (int64_t)__builtin_amdgcn_readfirstlane((int)s_tok[r]) * H +
                  (int64_t)(g * G) * N;

    float m[C], s[C];
#pragma unroll
    for (int c = 0; c < C; ++c) { m[c] = kNegInf; s[c] = 0.f; }

    // Logits of a group are stored after the next group's loads are issued, so
    // the in-order memory counter never makes a page load wait on a store.
    float zq[kUnroll][C];
    int iq[kUnroll];
    bool pending = false;
    auto flush = [&]() {
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) {
        if (iq[k] < N) {
#pragma unroll
          for (int c = 0; c < C; ++c)
            if (hd[c] < G) stream_store(&zrow[(int64_t)iq[k] * G + hd[c]], zq[k][c]);
        }
      }
    };

    for (int pg = pg0; pg < pg1; pg += kUnroll) {
      PageRegs<kBf16> pr[kUnroll];
      int64_t phys[kUnroll];
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) phys[k] = bt[min(pg + k, pg1 - 1)];
      // pages past the unit's end reload its last page (in bounds); they are not used
#pragma unroll
      for (int k = 0; k < kUnroll; ++k)
        load_page(pr[k], pool + (phys[k] * Hkv + g) * (kPage * kHeadDim), row, col);
      if (pending) flush();
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) {
        const int i = (pg + k) * kPage + tok_in_page;
        iq[k] = (pg + k < pg1) ? i : N;
        float acc[4][S];
        lane_dots(pr[k], q, acc);
        float v[C];
        row_reduce_scatter(acc, col, v);
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const float z = v[c] * p.score_scale;
          zq[k][c] = z;
          if (iq[k] < N && hd[c] < G) {
            // online (max, sum exp) with one exp per element
            const float d = z - m[c];
            const float w = exp_via2(-fabsf(d));
            s[c] = (d > 0.f) ? fmaf(s[c], w, 1.f) : s[c] + w;
            m[c] = fmaxf(m[c], z);
          }
        }
      }
      pending = true;
    }
    if (pending) flush();

    // fold the 16 lanes that own each head: col bits 0-1 (DPP) and the 4 rows
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float mm = m[c], ss = s[c];
      merge_ms(mm, ss, dpp_f<kDppXor1>(mm), dpp_f<kDppXor1>(ss));
      merge_ms(mm, ss, dpp_f<kDppXor2>(mm), dpp_f<kDppXor2>(ss));
#pragma unroll
      for (int x = 16; x <= 32; x <<= 1) merge_ms(mm, ss, __shfl_xor(mm, x), __shfl_xor(ss, x));
      if (row == 0 && (col & 3) == 0 && hd[c] < G) {
        float* dst = p.partials + ((int64_t)(g * G + hd[c]) * p.pair_stride + cg) * 2;
        dst[0] = mm;
        dst[1] = ss;
      }
    }
  }
}

// One workgroup per (request, head): fold the per-unit (max, sum exp) pairs.
__global__ __launch_bounds__(256) void stats_kernel(ScoreParams p) {
  TS_TIMELINE_SCOPE(score, kTlStats);
  __shared__ int32_t s_chunk[kMaxBatch + 1];
  __shared__ float s_m[4], s_s[4];
  const int b = p.b, H = p.H;
  const int r = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const int chunk_tokens = p.chunk_pages * kPage;
  block_prefix(s_chunk, b, [&](int rr) -> int32_t { return score_chunks(p, rr, chunk_tokens); });
  if (p.cache) {
    // every score wave has read C_Q: apply request r's decision (hit[r] was written by
    // the score kernel). A miss stores the query and clears the radix histograms;
    // the H workgroups of the request split the work.
    if (p.hit[r]) return;
    const int hd = kHeadDim * (p.bf16 ? 2 : 4) / 16;          // 16-byte chunks per head
    const uint4* src = static_cast<const uint4*>(p.q) + ((int64_t)r * H + h) * hd;
    uint4* dst = static_cast<uint4*>(p.cached_q) + ((int64_t)r * H + h) * hd;
    for (int i = threadIdx.x; i < hd; i += blockDim.x) dst[i] = src[i];
    if (h == 0 && threadIdx.x == 0) p.valid[r] = 1;
  } else if (p.skip && p.skip[r]) {
    return;
  }
  if (p.hist) {
    // the radix histograms of the TopK that follows start from zero; the H
    // workgroups of the request split them
    const int per = (3 * kHistBins + H - 1) / H;
    const int i0 = h * per, i1 = min(3 * kHistBins, i0 + per);
    uint32_t* hg = p.hist + (int64_t)r * 3 * kHistBins;
    for (int i = i0 + threadIdx.x; i < i1; i += blockDim.x) hg[i] = 0u;
    if (p.mass) {
      unsigned long long* mg = p.mass + (int64_t)r * 3 * kHistBins;
      for (int i = i0 + threadIdx.x; i < i1; i += blockDim.x) mg[i] = 0ull;
    }
  }
  const int c0 = s_chunk[r], c1 = s_chunk[r + 1];
  float M = kNegInf, S = 0.f;
  // [H][chunks] pairs: coalesced 8-byte loads, 8 per thread in flight before they are
  // merged in chunk order
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t* src = reinterpret_cast<const f32x2_t*>(p.partials) + (int64_t)h * p.pair_stride;
  const int step = blockDim.x;
  int c = c0 + threadIdx.x;
  for (; c + 7 * step < c1; c += 8 * step) {
    f32x2_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = src[c + k * step];
#pragma unroll
    for (int k = 0; k < 8; ++k) merge_ms(M, S, v[k].x, v[k].y);
  }
  for (; c < c1; c += step) {
    const f32x2_t v = src[c];
    merge_ms(M, S, v.x, v.y);
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

template <bool kBf16, bool kQ32>
hipError_t launch_score_t(const ScoreParams& p, hipStream_t st) {
  const int G = p.H / p.Hkv;
  dim3 grid(p.grid), block(256);
  switch (G) {
    case 1: hipLaunchKernelGGL((score_kernel<kBf16, kQ32, 1>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((score_kernel<kBf16, kQ32, 2>), grid, block, 0, st, p); break;
    case 3: hipLaunchKernelGGL((score_kernel<kBf16, kQ32, 3>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((score_kernel<kBf16, kQ32, 4>), grid, block, 0, st, p); break;
    case 5: hipLaunchKernelGGL((score_kernel<kBf16, kQ32, 5>), grid, block, 0, st, p); break;
    case 6: hipLaunchKernelGGL((score_kernel<kBf16, kQ32, 6>), grid, block, 0, st, p); break;
    case 7: hipLaunchKernelGGL((score_kernel<kBf16, kQ32, 7>), grid, block, 0, st, p); break;
    case 8: hipLaunchKernelGGL((score_kernel<kBf16, kQ32, 8>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const ScoreParams& p, hipStream_t st) {
  hipError_t e = !p.bf16  ? launch_score_t<false, false>(p, st)
                 : p.q_f32 ? launch_score_t<true, true>(p, st)
                           : launch_score_t<true, false>(p, st);
  if (e != hipSuccess) return e;
  // no statistics wanted (tokenselect_score with head_stats NULL), or folded by the vote kernel
  if (!p.fold && p.head_stats) hipLaunchKernelGGL(stats_kernel, dim3(p.b * p.H), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace ts
