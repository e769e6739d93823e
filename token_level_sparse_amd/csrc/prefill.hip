// Chunk-wise prefill: the mean query of a chunk, and the attention of every chunk
// query over the chunk's shared selection plus the causal part of the chunk.
//
// Source: TokenSelect deepnotes page, selection frequency of the prefill stage (the
// c queries of a chunk are averaged into one query that goes through the selection
// function, and the chunk shares the result), and the selective sparse attention
// formalisation; blog review of the same paper, section 3.2 (chunk-wise selection
// in prefill) and section 3.3 (Fig. 5: the chunk-prefill step with chunk 512).
//
// Selection reuses the decode kernels: the mean query (fp64 sum of the chunk's
// queries, one division, rounded to fp32) is scored against the past positions
// [0, P) with the fp32-query score mode, then voted and TopK'd as in decode.
//
// Attention. Chunk query j of request r sees the gathered key list
//   x < n_sel:  the TopK positions below the window start w0 = max(0, P - L),
//   x >= n_sel: positions w0 + (x - n_sel), i.e. the window and the chunk,
// truncated at x <= base + j with base = n_sel + P - w0 (causal inside the chunk).
// That is a causal attention with a key offset over an index-mapped paged pool, a
// dense contraction of c*G rows by ~k+L+c keys, so it runs on the matrix cores.
//
// gfx950 design. A workgroup owns 256 (query, head) rows of one (request, KV head)
// (64 for fp32): row = j * G + head-in-group, so one staged key block serves all G
// heads of the group. Each of the 8 waves (4 for fp32) owns 32 rows (16 for fp32), so
// every K and V fragment a wave reads from LDS feeds 32 rows, and each block staged
// in LDS serves 256 rows. Per block of keys:
//   * bf16: K and V rows go from global memory straight into LDS as [key][d]
//     (global_load_lds_dwordx4, one 1 KiB window per wave and load) into three
//     buffers each, two blocks ahead (K at the top of an iteration, V after its
//     scores), so each block has more than one iteration to land; fp32: staged
//     through registers, K and V as [key][d];
//   * S^T = K Q^T on MFMA (A = 32 keys x 16 dims from LDS, B = the wave's queries
//     held in registers), so a lane ends with 16 keys of one row: row = lane % 32;
//   * online softmax in base 2 per row (row max across the 2 lane halves); in bf16
//     the exp2 of block n runs between the MFMAs of block n + 1's scores and the
//     maximum of block n + 1 between the MFMAs of block n's P V;
//   * O^T += V^T P^T on MFMA: the lane's probabilities are already the B operand
//     (row = lane % 32, 8 keys per step); in bf16 the A operand (V^T) is read from the
//     [key][d] rows with LDS transpose reads (ds_read_b64_tr_b16) in the key order of
//     the probabilities, so P never leaves registers.
// The fp32 staging registers are clang vector types: with HIP's struct vector types
// the compiler kept them in scratch memory, and each block waited for its prefetch.
// bf16 uses v_mfma_f32_32x32x16_bf16 on 64-key blocks (accumulators in VGPRs, two
// waves per SIMD); fp32 uses v_mfma_f32_16x16x4_f32 on 32-key blocks with 16-row
// waves and the same index and mask logic.
// Key splits of kChunkSplitKeys list entries give more workgroups; a combine kernel
// merges the per-split (o, m, l) rows.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "timeline.h"

TS_TIMELINE_DEFINE(prefill)

namespace ts {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kRescaleSlack = 8.f;
constexpr int kPartStride = kChunkPartStride;   // o[128], m, l, 2 pad: 16-byte aligned rows
static_assert(kChunkPartStride == kHeadDim + 4, "partial row layout");

// Geometry of request r's chunk. Out-of-contract lengths are clamped so that no
// access leaves the request's pages (results are then unspecified).
struct ChunkGeom {
  int c, P, w0, N;
};

// Number of entries of the ascending a[0, n) below x, found by one wave (every lane
// returns it): each round probes the 64 entries lo + step (l + 1) - 1 of the run
// [lo, hi) the answer lies in; the probes below x form a prefix of k lanes, so the
// answer is in [lo + k step, min(hi, lo + (k + 1) step - 1)]. A round shrinks the run
// 64-fold; with step 1 the probes cover it and the answer is exact.
__device__ int count_below(const int32_t* a, int n, int x) {
  const int lane = threadIdx.x & (kWave - 1);
  int lo = 0, hi = n;
  while (lo < hi) {
    const int step = (hi - lo + kWave - 1) / kWave;
    const int pos = lo + step * (lane + 1) - 1;
    const bool below = pos < hi && a[pos] < x;
    const int k = __popcll(__ballot(below));
    const int nlo = lo + step * k;
    hi = min(hi, nlo + step - 1);
    lo = nlo;
    if (step == 1) hi = lo;
  }
  return lo;
}

__device__ ChunkGeom chunk_geom(const ChunkParams& p, int r) {
  ChunkGeom gm;
  gm.N = max(0, p.seq_lens[r]);
  gm.c = min(max(p.chunk_lens[r], 0), min(p.max_chunk, gm.N));
  gm.P = gm.N - gm.c;
  gm.w0 = max(0, gm.P - p.n_local);
  return gm;
}

// ---------------------------------------------------------------- mean query
// One workgroup of 1024 threads per (request, head): qbar = (sum_j q_j) / c with the
// sum in fp64 (exact for bf16 queries of ordinary range), rounded once to fp32.
// Thread t owns dims 8 (t % 16) + [0, 8) of rows j = t / 16 (mod 64): 16-byte loads,
// 64 rows in flight per pass; then the 64 row groups are added in LDS in two levels
// (8 slices of 8 groups, then the 8 slices), so no thread adds 64 values in a chain.
constexpr int kMeanThreads = 1024;
constexpr int kMeanGroups = kMeanThreads / 16;
constexpr int kMeanSlices = kMeanThreads / kHeadDim;
static_assert(kMeanGroups % kMeanSlices == 0, "row groups split evenly over the slices");
template <bool kBf16>
__global__ __launch_bounds__(kMeanThreads) void chunk_mean_kernel(ChunkParams p) {
  __shared__ double s_acc[kMeanGroups][kHeadDim];
  __shared__ double s_part[kMeanSlices][kHeadDim];
  const int r = blockIdx.x / p.H, h = blockIdx.x - (blockIdx.x / p.H) * p.H;
  const ChunkGeom gm = chunk_geom(p, r);
  const int dc = threadIdx.x & 15, rg = threadIdx.x >> 4;
  double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  const int64_t row_stride = (int64_t)p.H * kHeadDim;
  const int64_t base = ((int64_t)r * p.max_chunk * p.H + h) * kHeadDim + 8 * dc;
#pragma unroll 2
  for (int j = rg; j < gm.c; j += kMeanGroups) {
    if (kBf16) {
      const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + base + j * row_stride);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += (double)bf16_lo(ws[e]);
        acc[2 * e + 1] += (double)bf16_hi(ws[e]);
      }
    } else {
      const float* src = static_cast<const float*>(p.q) + base + j * row_stride;
      const float4 x0 = *reinterpret_cast<const float4*>(src);
      const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
      acc[0] += (double)x0.x; acc[1] += (double)x0.y; acc[2] += (double)x0.z; acc[3] += (double)x0.w;
      acc[4] += (double)x1.x; acc[5] += (double)x1.y; acc[6] += (double)x1.z; acc[7] += (double)x1.w;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_acc[rg][8 * dc + e] = acc[e];
  __syncthreads();
  {
    const int d = threadIdx.x % kHeadDim, sl = threadIdx.x / kHeadDim;
    constexpr int kPer = kMeanGroups / kMeanSlices;
    double t = 0.0;
#pragma unroll
    for (int g = 0; g < kPer; ++g) t += s_acc[kPer * sl + g][d];
    s_part[sl][d] = t;
  }
  __syncthreads();
  if (threadIdx.x < kHeadDim) {
    double t = 0.0;
#pragma unroll
    for (int sl = 0; sl < kMeanSlices; ++sl) t += s_part[sl][threadIdx.x];
    p.qbar[((int64_t)r * p.H + h) * kHeadDim + threadIdx.x] = (float)(t / (double)max(gm.c, 1));
  }
  if (h == 0 && threadIdx.x == 0) p.past_lens[r] = gm.P;
}

// ---------------------------------------------------------------- attention
template <bool kBf16> struct Tile;
template <> struct Tile<true> {
  static constexpr int kKeys = 64;                 // keys per staged block
  static constexpr int kRow = kHeadDim * 2;        // bytes per K or V row in LDS (no padding)
};
template <> struct Tile<false> {
  static constexpr int kKeys = 32;
  static constexpr int kStride = kHeadDim + 4;     // floats per K / V row in LDS
  static constexpr int kLds = 2 * kKeys * kStride * 4;
  f32x4_t k[4], v[4];                              // staging registers: 1 key x 16 dims
};

struct KeyMap {
  const int64_t* off;      // LDS: element offset of the split's key-list entries (this KV head)
  int x_begin, x_end;
  __device__ int64_t row(int x) const { return off[min(x, x_end - 1) - x_begin]; }
};

// bf16 blocks are staged straight from global memory into LDS (global_load_lds_dwordx4:
// lane i of a wave's load writes bytes 16 i .. 16 i + 15 of a 1 KiB LDS window, i.e.
// 4 rows of 256 bytes). Rows keep no padding; instead the 16-byte chunks are permuted
// per row so the operand reads are conflict-free: chunk c of K row x sits at position
// c ^ (x mod 16), chunk c of V row x at position c ^ 2 (x mod 4). A lane therefore
// fetches the global chunk that belongs at its LDS position.
__device__ __forceinline__ int k_pos(int x, int c) { return c ^ (x & 15); }
__device__ __forceinline__ int v_pos(int x, int c) { return c ^ ((x & 3) << 1); }

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void global_cvoid;

// One 1 KiB LDS window per wave (global_load_lds_dwordx4, LDS address in M0): lane i's
// 16 bytes at gptr land at window bytes 16 i. Written as inline assembly: the compiler's
// own wait-count model treats this load as a flat access that may also touch LDS, and
// while one is in flight it makes every LDS read wait for all outstanding LDS operations
// (lgkmcnt(0)) instead of only the ones it needs. The compiler does not see these loads,
// so every caller waits for them itself (vmcnt) before the barrier that publishes the
// window; the M0 write is followed by the one wait state the load needs.
__device__ __forceinline__ void dma16(const void* gptr, const char* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(gptr), "{m0}"(m0) : "memory");
}

// Wave w stages rows 8 w .. 8 w + 7 of the block (K into kl and/or V into vl) starting
// at list entry x0.
__device__ __forceinline__ void stage_direct(char* kl, char* vl, const uint16_t* kp, const uint16_t* vp,
                                             const KeyMap& km, int x0, bool do_k, bool do_v) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 8 * wave + 4 * j + (lane >> 4), pos = lane & 15;
    const int64_t off = km.row(x0 + row);
    const int at = (8 * wave + 4 * j) * Tile<true>::kRow;
    if (do_k)
      dma16(kp + off + 8 * k_pos(row, pos), kl + at);
    if (do_v)
      dma16(vp + off + 8 * v_pos(row, pos), vl + at);
  }
}
// The staging split in two: the key-list offsets of the wave's 4-row windows (LDS reads
// of the split's key table, issued one iteration ahead) and the loads themselves, one
// dma16 per window, so a staged block costs kStageWindows vector-memory operations per
// wave (the explicit waits count them).
constexpr int kStageWindows = 2;
// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector-memory operations
// of the wave are outstanding; the export and LDS/scalar counters are left unconstrained.
constexpr int vmcnt_at_most(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
struct StageOff { int64_t off[kStageWindows]; };
__device__ __forceinline__ StageOff stage_offsets(const KeyMap& km, int x0) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  StageOff so;
#pragma unroll
  for (int j = 0; j < kStageWindows; ++j) so.off[j] = km.row(x0 + 4 * kStageWindows * wave + 4 * j + (lane >> 4));
  return so;
}
template <bool kIsK>
__device__ __forceinline__ void stage_issue(char* buf, const uint16_t* pool, const StageOff& so) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < kStageWindows; ++j) {
    const int row0 = 4 * kStageWindows * wave + 4 * j, row = row0 + (lane >> 4), pos = lane & 15;
    dma16(pool + so.off[j] + 8 * (kIsK ? k_pos(row, pos) : v_pos(row, pos)), buf + row0 * Tile<true>::kRow);
  }
}
// Every staged write of this thread has landed in LDS (the barrier that follows makes
// them visible to the other waves).
__device__ __forceinline__ void stage_wait() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ void stage_load(Tile<false>& t, const float* kp, const float* vp,
                                           const KeyMap& km, int x0) {
  const int key = threadIdx.x >> 3, dq = threadIdx.x & 7;
  const int64_t off = km.row(x0 + key) + 16 * dq;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    t.k[m] = *reinterpret_cast<const f32x4_t*>(kp + off + 4 * m);
    t.v[m] = *reinterpret_cast<const f32x4_t*>(vp + off + 4 * m);
  }
}
__device__ __forceinline__ void stage_store(const Tile<false>& t, char* lds) {
  float* Ks = reinterpret_cast<float*>(lds);
  float* Vs = Ks + Tile<false>::kKeys * Tile<false>::kStride;
  const int key = threadIdx.x >> 3, dq = threadIdx.x & 7;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    *reinterpret_cast<f32x4_t*>(Ks + key * Tile<false>::kStride + 16 * dq + 4 * m) = t.k[m];
    *reinterpret_cast<f32x4_t*>(Vs + key * Tile<false>::kStride + 16 * dq + 4 * m) = t.v[m];
  }
}

// Query operand (B of S^T = K Q^T). fp32 (16x16x4): the lane holds dims 4 ks + a of
// its row. bf16 (32x32x16): the lane holds dims 16 ks + 8 lg + [0, 8).
struct QOpF32 { float v[32]; };
struct QOp32 { bf16x8_t v[8]; };

__device__ __forceinline__ void load_qop32(QOp32& q, const uint16_t* qrow, bool ok, int lg) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (ok) w = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * lg);
    q.v[ks] = __builtin_bit_cast(bf16x8_t, u32x4_t{w.x, w.y, w.z, w.w});
  }
}

// bf16 S^T tiles of one staged block on v_mfma_f32_32x32x16_bf16: s[t][j] =
// <q_row, k_{32 t + 8 (j / 4) + 4 lg + j % 4}> for the lane's row l32.
__device__ __forceinline__ void qk_block32(const char* lds, const QOp32& q, int l32, int lg,
                                           f32x16_t (&s)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x16_t acc = {};
    const int x = 32 * t + l32;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8_t ak = *reinterpret_cast<const bf16x8_t*>(lds + x * Tile<true>::kRow + 16 * k_pos(x, 2 * ks + lg));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, q.v[ks], acc, 0, 0, 0);
    }
    s[t] = acc;
  }
}

// bf16 O^T += V^T P^T: o[dt][j] = O[row][32 dt + 8 (j / 4) + 4 lg + j % 4]. The B operand
// of the 16-key step (t, hh) is the lane's pv[t][8 hh .. 8 hh + 8) (keys 32 t + 16 hh +
// 4 lg + [0, 4) and + 8), so the A operand (dim 32 dt + l32 of those 8 keys) is read in
// that order from the [key][d] V rows with ds_read_b64_tr_b16: in each 16-lane group,
// element k of lane i is element i % 4 of the 8 bytes that lane 4 k + i / 4 addresses, so
// lane s of the group addresses key (first key + s / 4), dims (group's first dim + 4 (s % 4)).
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
__device__ __forceinline__ bf16x8_t v_frag(const char* Vs, int i, int lg, int s, int half) {
  const int t = i >> 3, hh = (i >> 2) & 1, dt = i & 3;
  const int x = 32 * t + 16 * hh + 4 * lg + (s >> 2);
  const int c = 4 * dt + 2 * half + ((s & 3) >> 1), b = 8 * (s & 1);
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(Vs + x * Tile<true>::kRow + 16 * v_pos(x, c) + b));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(Vs + (x + 8) * Tile<true>::kRow + 16 * v_pos(x + 8, c) + b));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
template <typename Hook>
__device__ __forceinline__ void pv_block32(const char* lds, const f32x16_t (&pv)[2], int l32, int lg,
                                           f32x16_t (&o)[4], Hook hook) {
  const char* Vs = lds;
  const int s = threadIdx.x & 15, half = l32 >> 4;
  bf16x8_t av = v_frag(Vs, 0, lg, s, half);
  bf16x8_t pb;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = i >> 3, hh = (i >> 2) & 1, dt = i & 3;
    if (dt == 0) {
      const int b8 = 8 * hh;
      pb = bf16x8_t{(__bf16)pv[t][b8], (__bf16)pv[t][b8 + 1], (__bf16)pv[t][b8 + 2],
                    (__bf16)pv[t][b8 + 3], (__bf16)pv[t][b8 + 4], (__bf16)pv[t][b8 + 5],
                    (__bf16)pv[t][b8 + 6], (__bf16)pv[t][b8 + 7]};
    }
    bf16x8_t an = av;
    if (i + 1 < 16) an = v_frag(Vs, i + 1, lg, s, half);
    __builtin_amdgcn_sched_barrier(0);
    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, o[dt], 0, 0, 0);
    hook(i);
    av = an;
  }
}

__device__ __forceinline__ void load_qop(QOpF32& q, const float* qrow, bool ok, int a) {
#pragma unroll
  for (int ks = 0; ks < 32; ++ks) q.v[ks] = ok ? qrow[4 * ks + a] : 0.f;
}

// fp32: S^T tiles of one staged block: s[t][i] = <q_row, k_{16 t + 4 a + i}>.
__device__ __forceinline__ void qk_block(const char* lds, const QOpF32& q, int l16, int a,
                                         f32x4_t (&s)[2]) {
  const float* Ks = reinterpret_cast<const float*>(lds);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 32; ++ks)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Ks[(16 * t + l16) * Tile<false>::kStride + 4 * ks + a],
                                                 q.v[ks], acc, 0, 0, 0);
    s[t] = acc;
  }
}

// fp32: O^T += V^T P^T over one staged block. o[dt][i] = O[row][16 dt + 4 a + i].
__device__ __forceinline__ void pv_block(const char* lds, const float (&pv)[2][4], int l16, int a,
                                         f32x4_t (&o)[8]) {
  const float* Vs = reinterpret_cast<const float*>(lds) + Tile<false>::kKeys * Tile<false>::kStride;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
            Vs[(16 * t + 4 * a + i) * Tile<false>::kStride + 16 * dt + l16], pv[t][i], o[dt], 0, 0, 0);
}

// Work of one attention workgroup: a unit (request, KV head, split) and a tile of
// rows_per_wg (query, head) rows. The split's key-list entries are expanded into
// element offsets of this KV head in LDS. Returns false (the same for every thread)
// when the workgroup has nothing to do.
struct UnitWork {
  int r, g, split, G, rows, row0, base, x_begin, x_end;
  KeyMap km;
};

__device__ bool chunk_unit(const ChunkParams& p, int rows_per_wg, int* s_geom, int64_t* s_keys,
                           UnitWork& w) {
  const int H = p.H, Hkv = p.Hkv;
  w.G = H / Hkv;
  const int rt = (p.max_chunk * w.G + rows_per_wg - 1) / rows_per_wg;
  // XCD-aware order: workgroup i runs on XCD i % 8. All row tiles of one unit
  // (request, KV head, split) go to the same XCD, one after another, so the unit's
  // staged K/V rows come from that XCD's L2 after the first tile.
  const int units = p.b * Hkv * p.splits;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int u = (slot / rt) * kXcds + xcd;
  if (u >= units) return false;
  const int tile = slot % rt;
  w.split = u % p.splits;
  w.g = (u / p.splits) % Hkv;
  w.r = u / (p.splits * Hkv);
  // The request's geometry (uniform scalar loads in every thread); the number of
  // TopK entries below the window start w0 is found by every wave with a 64-way
  // search of the ascending TopK: each round probes 64 evenly spaced entries at once
  // and keeps the run between the last probe below w0 and the first one not below
  // (two rounds for a few thousand entries, instead of a binary search of dependent
  // loads).
  const ChunkGeom g0 = chunk_geom(p, w.r);
  const int cnt = min(max(p.sel_count[w.r], 0), min(p.sel_stride, g0.P));
  const int32_t* sel_r = p.sel_idx + (int64_t)w.r * p.sel_stride;
  const int n_sel = count_below(sel_r, cnt, g0.w0);
  const int gbase = n_sel + g0.P - g0.w0;
  // for the combine kernel (every workgroup of the request writes the same value)
  if (w.split == 0 && tile == 0 && threadIdx.x == 0) p.key_base[w.r] = gbase;
  const int c = g0.c;
  w.base = gbase;
  w.rows = c * w.G;
  w.row0 = tile * rows_per_wg;
  if (w.row0 >= w.rows) return false;
  const int jmax = (min(w.row0 + rows_per_wg, w.rows) - 1) / w.G;
  const int n_vis = w.base + jmax + 1;                        // entries the last query sees
  w.x_begin = w.split * p.split_keys;
  if (w.x_begin >= n_vis) return false;
  w.x_end = min(w.x_begin + p.split_keys, n_vis);
  // key-list entry x: the x-th selected position below the window (the TopK is
  // ascending), then the window and the chunk [w0, P + c); its row of this KV head
  const int w0 = g0.w0, N = g0.N;
  const int32_t* bt = p.block_table + (int64_t)w.r * p.stride;
  for (int x = w.x_begin + (int)threadIdx.x; x < w.x_end; x += blockDim.x) {
    int pos = x < n_sel ? sel_r[x] : w0 + (x - n_sel);
    pos = min(max(pos, 0), max(N - 1, 0));
    const int64_t page = bt[pos >> 4];
    s_keys[x - w.x_begin] = ((page * Hkv + w.g) * kPage + (pos & (kPage - 1))) * kHeadDim;
  }
  __syncthreads();
  w.km.off = s_keys; w.km.x_begin = w.x_begin; w.km.x_end = w.x_end;
  return true;
}

// Online softmax step shared by both kernels. Rescale only when some row's block
// maximum exceeds its running maximum by more than kRescaleSlack (base 2): o and l stay
// relative to the same m_run, so the result is unchanged, and probabilities stay below
// 2^kRescaleSlack. pv holds scaled scores (-inf where masked) and returns probabilities.
template <int kN, typename Rescale>
__device__ __forceinline__ void softmax_step(float (&pv)[kN], float mloc, float& m_run, float& l_run,
                                             Rescale rescale) {
  if (__builtin_amdgcn_ballot_w64(mloc > m_run + kRescaleSlack)) {
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
    l_run *= alpha;
    m_run = m_new;
    rescale(alpha);
  }
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < kN; ++i) {
    pv[i] = (pv[i] == kNegInf) ? 0.f : fast_exp2(pv[i] - m_run);
    psum += pv[i];
  }
  l_run += psum;
}

// bf16: 8 waves x 32 rows, v_mfma_f32_32x32x16_bf16. Lane l holds row l % 32 (lg = l / 32
// picks which keys and dims of that row it carries).
constexpr int kRows32 = kChunkRowsBf16;
constexpr int kThreads32 = 512;
static_assert(kThreads32 / 64 * 32 == kRows32, "32 rows per wave");
static_assert(kThreads32 / 64 * 4 * kStageWindows == Tile<true>::kKeys, "each wave stages 4 rows per window of a block");
__global__ __launch_bounds__(kThreads32) __attribute__((amdgpu_waves_per_eu(2, 2)))
void chunk_attn_bf16_kernel(ChunkParams p) {
  TS_TIMELINE_SCOPE(prefill, kTlChunkAttn);
  constexpr int KB = Tile<true>::kKeys;
  constexpr int kBuf = Tile<true>::kKeys * Tile<true>::kRow;
  __shared__ __align__(16) char s_kb[3 * kBuf];
  __shared__ __align__(16) char s_vb[3 * kBuf];
  __shared__ int64_t s_keys[kChunkSplitKeys];
  __shared__ int s_geom[5];
  UnitWork w;
  if (!chunk_unit(p, kRows32, s_geom, s_keys, w)) return;
  TS_TIMELINE_MARK();                            // mark 0: key list of the split in LDS
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l32 = lane & 31, lg = lane >> 5;
  const int rho = w.row0 + 32 * wave + l32;
  const bool row_ok = rho < w.rows;
  const int j = row_ok ? rho / w.G : 0;
  const int h = w.g * w.G + (row_ok ? rho - (rho / w.G) * w.G : 0);
  const int lim = row_ok ? w.base + j : -1;                   // last visible key-list entry
  const int wave_lim = w.base + min(w.row0 + 32 * wave, w.rows - 1) / w.G;

  const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                         (((int64_t)w.r * p.max_chunk + j) * p.H + h) * kHeadDim;
  QOp32 q;
  load_qop32(q, qrow, row_ok, lg);
  const uint16_t* kp = static_cast<const uint16_t*>(p.k_pool);
  const uint16_t* vp = static_cast<const uint16_t*>(p.v_pool);
  const float sl2 = p.attn_scale * kLog2e;
  float m_run = kNegInf, l_run = 0.f;
  f32x16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16_t{};

  // Online softmax of one block, first half: the block maximum (max_part, two scores per
  // call, folded in between the products of the previous block; max_done joins the lane's
  // two key halves) and the rescale of the running state (rescale). In a block every key
  // of which is visible to every row of the wave (wave-uniform, block_full) the scores
  // stay raw (the maximum is taken on them: scaling by sl2 > 0 commutes with the rounded
  // max); otherwise they are scaled, with -inf where masked.
  auto block_full = [&](int x0) { return x0 + KB <= w.x_end && x0 + KB - 1 <= wave_lim; };
  auto max_part = [&](auto full_c, f32x16_t (&s)[2], int x0, int i, float& mloc) {
    constexpr bool kFull = decltype(full_c)::value;
#pragma unroll
    for (int e = 2 * i; e < 2 * i + 2; ++e) {
      const int t = e >> 4, ii = e & 15;
      if (kFull) {
        mloc = fmaxf(mloc, s[t][ii]);
      } else {
        // key x0 + c + 4 lg is visible iff c <= bnd (c is a constant of the element)
        const int bnd = min(w.x_end - 1, lim) - x0 - 4 * lg;
        const int c = 32 * t + 8 * (ii >> 2) + (ii & 3);
        s[t][ii] = (c <= bnd) ? s[t][ii] * sl2 : kNegInf;
        mloc = fmaxf(mloc, s[t][ii]);
      }
    }
  };
  auto max_done = [&](bool full, float mloc) {
    if (full) mloc *= sl2;
    return fmaxf(mloc, __shfl_xor(mloc, 32));
  };
  auto rescale = [&](float mloc) {
    if (__builtin_amdgcn_ballot_w64(mloc > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    }
  };

  // Second half, fused with the scores of the next block: the probabilities of block n
  // (in place in cur) are computed between the MFMAs of S_{n+1} = K_{n+1} Q^T (into nxt,
  // from the K buffer kb), so the matrix cores and the VALU work at the same time. In a
  // fully visible block every probability is one exp2 of an fma and the running
  // maximum is finite, so no -inf guard is needed.
  auto exp_qk = [&](auto full_c, f32x16_t (&cur)[2], f32x16_t (&nxt)[2], const char* kb) {
    constexpr bool kFull = decltype(full_c)::value;
    const float nm = -m_run;
    f32x16_t a0 = {}, a1 = {};
    float psum = 0.f;
    auto kread = [&](int row, int ks) {
      return *reinterpret_cast<const bf16x8_t*>(kb + row * Tile<true>::kRow + 16 * k_pos(row, 2 * ks + lg));
    };
    bf16x8_t k0 = kread(l32, 0), k1 = kread(32 + l32, 0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bf16x8_t n0 = k0, n1 = k1;
      if (ks + 1 < 8) { n0 = kread(l32, ks + 1); n1 = kread(32 + l32, ks + 1); }
      __builtin_amdgcn_sched_barrier(0);
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, q.v[ks], a0, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float x = cur[ks >> 2][4 * (ks & 3) + e];
        const float pr = kFull ? fast_exp2(fmaf(x, sl2, nm)) : ((x == kNegInf) ? 0.f : fast_exp2(x - m_run));
        cur[ks >> 2][4 * (ks & 3) + e] = pr;
        psum += pr;
      }
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, q.v[ks], a1, 0, 0, 0);
#pragma unroll
      for (int e = 2; e < 4; ++e) {
        const float x = cur[ks >> 2][4 * (ks & 3) + e];
        const float pr = kFull ? fast_exp2(fmaf(x, sl2, nm)) : ((x == kNegInf) ? 0.f : fast_exp2(x - m_run));
        cur[ks >> 2][4 * (ks & 3) + e] = pr;
        psum += pr;
      }
      k0 = n0; k1 = n1;
      __builtin_amdgcn_sched_barrier(0);
    }
    nxt[0] = a0;
    nxt[1] = a1;
    l_run += psum;
  };

  // Software pipeline, one barrier per block, three LDS buffers each for K and V (block m
  // in buffer m % 3). Entering iteration n, S_n and its maximum are in registers and
  // K_{n+1}, V_n are in LDS. Iteration n starts the staging of K_{n+3} over K_n (read in
  // iteration n - 1), computes P_n with S_{n+1} = K_{n+1} Q^T, starts the staging of
  // V_{n+2} over V_{n-1} (read in iteration n - 1), and accumulates P_n V_n with the
  // maximum of S_{n+1} folded in between the products. Before its barrier it waits only
  // for the staging started one iteration earlier (K_{n+2}, V_{n+1}), so each staged block
  // has more than one iteration to land.
  const int nb = (w.x_end - w.x_begin + KB - 1) / KB;
  auto kbuf = [&](int m) { return s_kb + (m % 3) * kBuf; };
  auto vbuf = [&](int m) { return s_vb + (m % 3) * kBuf; };
  for (int m = 0; m < 3 && m < nb; ++m) stage_direct(kbuf(m), vbuf(m), kp, vp, w.km, w.x_begin + m * KB, true, m < 2);
  stage_wait();
  __syncthreads();
  f32x16_t sa[2], sb[2];
  qk_block32(s_kb, q, l32, lg, sa);
  bool full_n = block_full(w.x_begin);
  float mloc_n = kNegInf;
  if (full_n) {
#pragma unroll
    for (int i = 0; i < 16; ++i) max_part(std::true_type{}, sa, w.x_begin, i, mloc_n);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) max_part(std::false_type{}, sa, w.x_begin, i, mloc_n);
  }
  mloc_n = max_done(full_n, mloc_n);
  __syncthreads();
  TS_TIMELINE_MARK();                            // mark 1: first blocks staged, S_0 computed
  StageOff off_k = stage_offsets(w.km, w.x_begin + 3 * KB), off_v = stage_offsets(w.km, w.x_begin + 2 * KB);
  // timeline builds: marks 2-5 split iteration kTlBlock into its parts (scores of the
  // next block with this block's exp2; P V with the next maximum; the wait for the
  // staging and the barrier, up to the start of the next iteration)
  constexpr int kTlBlock = 8;
  auto step = [&](int n, f32x16_t (&cur)[2], f32x16_t (&nxt)[2]) {
    const int x0 = w.x_begin + n * KB;
    const bool sk = n + 3 < nb, sv = n + 2 < nb;
    if (n == kTlBlock || n == kTlBlock + 1) { TS_TIMELINE_MARK_HERE(); }
    rescale(mloc_n);
    if (sk) {
      stage_issue<true>(kbuf(n + 3), kp, off_k);                                          // K_{n+3}
      off_k = stage_offsets(w.km, x0 + 4 * KB);
    }
    // S_{n+1} is computed even past the last block (from stale, in-bounds LDS) and unused
    if (full_n) exp_qk(std::true_type{}, cur, nxt, kbuf(n + 1));
    else exp_qk(std::false_type{}, cur, nxt, kbuf(n + 1));
    if (n == kTlBlock) { TS_TIMELINE_MARK_HERE(); }
    if (sv) {
      stage_issue<false>(vbuf(n + 2), vp, off_v);                                         // V_{n+2}
      off_v = stage_offsets(w.km, x0 + 3 * KB);
    }
    const int x1 = x0 + KB;
    const bool full1 = block_full(x1);
    float m1 = kNegInf;
    if (full1) pv_block32(vbuf(n), cur, l32, lg, o, [&](int i) { max_part(std::true_type{}, nxt, x1, i, m1); });
    else pv_block32(vbuf(n), cur, l32, lg, o, [&](int i) { max_part(std::false_type{}, nxt, x1, i, m1); });
    mloc_n = max_done(full1, m1);
    full_n = full1;
    if (n == kTlBlock) { TS_TIMELINE_MARK_HERE(); }
    // this iteration's staging may still be in flight
    if (sk && sv) __builtin_amdgcn_s_waitcnt(vmcnt_at_most(2 * kStageWindows));
    else if (sk || sv) __builtin_amdgcn_s_waitcnt(vmcnt_at_most(kStageWindows));
    else __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
    __syncthreads();
  };
  for (int n = 0; n < nb; n += 2) {
    step(n, sa, sb);
    if (n + 1 < nb) step(n + 1, sb, sa);
  }

  const float lt = l_run + __shfl_xor(l_run, 32);
  if (row_ok) {
    float* dst = p.partials +
                 ((((int64_t)w.r * p.max_chunk + j) * p.H + h) * p.splits + w.split) * kPartStride;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<float4*>(dst + 32 * dt + 8 * qd + 4 * lg) =
            make_float4(o[dt][4 * qd], o[dt][4 * qd + 1], o[dt][4 * qd + 2], o[dt][4 * qd + 3]);
    if (lg == 0) { dst[kHeadDim] = m_run; dst[kHeadDim + 1] = lt; }
  }
}

// fp32: 4 waves x 16 rows, v_mfma_f32_16x16x4_f32, 32-key blocks. Lane l holds row
// l % 16 (a = l / 16 picks which keys and dims of that row it carries).
constexpr int kRows16 = kChunkRows;
__global__ __launch_bounds__(256) void chunk_attn_f32_kernel(ChunkParams p) {
  constexpr int KB = Tile<false>::kKeys;
  constexpr int NT = KB / 16;
  __shared__ __align__(16) char s_lds[Tile<false>::kLds];
  __shared__ int64_t s_keys[kChunkSplitKeys];
  __shared__ int s_geom[5];
  UnitWork w;
  if (!chunk_unit(p, kRows16, s_geom, s_keys, w)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, a = lane >> 4;
  const int rho = w.row0 + 16 * wave + l16;
  const bool row_ok = rho < w.rows;
  const int j = row_ok ? rho / w.G : 0;
  const int h = w.g * w.G + (row_ok ? rho - (rho / w.G) * w.G : 0);
  const int lim = row_ok ? w.base + j : -1;
  const int wave_lim = w.base + min(w.row0 + 16 * wave, w.rows - 1) / w.G;

  const float* qrow = static_cast<const float*>(p.q) + (((int64_t)w.r * p.max_chunk + j) * p.H + h) * kHeadDim;
  QOpF32 q;
  load_qop(q, qrow, row_ok, a);
  const float* kp = static_cast<const float*>(p.k_pool);
  const float* vp = static_cast<const float*>(p.v_pool);
  const float sl2 = p.attn_scale * kLog2e;
  float m_run = kNegInf, l_run = 0.f;
  f32x4_t o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  Tile<false> st;
  stage_load(st, kp, vp, w.km, w.x_begin);
  for (int x0 = w.x_begin; x0 < w.x_end; x0 += KB) {
    __syncthreads();
    stage_store(st, s_lds);
    __syncthreads();
    if (x0 + KB < w.x_end) stage_load(st, kp, vp, w.km, x0 + KB);

    f32x4_t s[NT];
    qk_block(s_lds, q, l16, a, s);
    float pv[NT][4];
    float mloc = kNegInf;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int x = x0 + 16 * t + 4 * a + i;
        const bool vis = (x0 + KB <= w.x_end && x0 + KB - 1 <= wave_lim) || (x < w.x_end && x <= lim);
        pv[t][i] = vis ? s[t][i] * sl2 : kNegInf;
        mloc = fmaxf(mloc, pv[t][i]);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    softmax_step(reinterpret_cast<float(&)[NT * 4]>(pv), mloc, m_run, l_run, [&](float alpha) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    });
    pv_block(s_lds, pv, l16, a, o);
  }

  float lt = l_run + __shfl_xor(l_run, 16);
  lt += __shfl_xor(lt, 32);
  if (row_ok) {
    float* dst = p.partials +
                 ((((int64_t)w.r * p.max_chunk + j) * p.H + h) * p.splits + w.split) * kPartStride;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<float4*>(dst + 16 * dt + 4 * a) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (a == 0) { dst[kHeadDim] = m_run; dst[kHeadDim + 1] = lt; }
  }
}

// Merge the splits of each (request, chunk query, head) row: 32 threads per row,
// 4 dims each, 8 rows per workgroup.
template <bool kBf16>
__global__ __launch_bounds__(256) void chunk_combine_kernel(ChunkParams p) {
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  const int64_t rows = (int64_t)p.b * p.max_chunk * p.H;
  if (row >= rows) return;
  const int j = (int)((row / p.H) % p.max_chunk);
  const int r = (int)(row / ((int64_t)p.H * p.max_chunk));
  const ChunkGeom gm = chunk_geom(p, r);
  if (j >= gm.c) return;
  // splits that hold entries visible to chunk query j (the attention kernel stored the
  // request's key-list base, so no search of the TopK list here)
  const int S = min(p.splits, (p.key_base[r] + j + p.split_keys) / p.split_keys);
  const int d4 = 4 * (threadIdx.x & 31);
  const float* src = p.partials + row * p.splits * kPartStride;
  // one pass: the splits' loads are independent, the merge keeps a running maximum
  float M = kNegInf, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int s = 0; s < S; ++s) {
    const float ms = src[s * kPartStride + kHeadDim];
    const float ls = src[s * kPartStride + kHeadDim + 1];
    const float4 o = *reinterpret_cast<const float4*>(src + s * kPartStride + d4);
    const float Mn = fmaxf(M, ms);
    const float a = (M == kNegInf) ? 0.f : fast_exp2(M - Mn);     // rescale of the running sums
    const float w = (ms == kNegInf) ? 0.f : fast_exp2(ms - Mn);
    L = fmaf(w, ls, L * a);
    acc.x = fmaf(w, o.x, acc.x * a); acc.y = fmaf(w, o.y, acc.y * a);
    acc.z = fmaf(w, o.z, acc.z * a); acc.w = fmaf(w, o.w, acc.w * a);
    M = Mn;
  }
  const float inv = 1.f / L;
  const int64_t oi = row * kHeadDim + d4;
  if (kBf16) {
    uint2 v;
    v.x = (uint32_t)f32_to_bf16(acc.x * inv) | ((uint32_t)f32_to_bf16(acc.y * inv) << 16);
    v.y = (uint32_t)f32_to_bf16(acc.z * inv) | ((uint32_t)f32_to_bf16(acc.w * inv) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + oi) = v;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(p.out) + oi) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
}

}  // namespace

hipError_t launch_chunk_mean(const ChunkParams& p, hipStream_t s) {
  const dim3 grid(p.b * p.H), block(kMeanThreads);
  if (p.bf16) hipLaunchKernelGGL(chunk_mean_kernel<true>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(chunk_mean_kernel<false>, grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_chunk_attn(const ChunkParams& p, hipStream_t s) {
  const int G = p.H / p.Hkv;
  const int rows_per_wg = p.bf16 ? kRows32 : kRows16;
  const int rt = (p.max_chunk * G + rows_per_wg - 1) / rows_per_wg;
  const dim3 block(256);
  const int units = p.b * p.Hkv * p.splits;
  const dim3 grid(kXcds * rt * ((units + kXcds - 1) / kXcds));
  if (p.bf16) hipLaunchKernelGGL(chunk_attn_bf16_kernel, grid, dim3(kThreads32), 0, s, p);
  else hipLaunchKernelGGL(chunk_attn_f32_kernel, grid, block, 0, s, p);
  const dim3 cgrid((unsigned)(((int64_t)p.b * p.max_chunk * p.H + 7) / 8));
  if (p.bf16) hipLaunchKernelGGL(chunk_combine_kernel<true>, cgrid, block, 0, s, p);
  else hipLaunchKernelGGL(chunk_combine_kernel<false>, cgrid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace ts
