// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ts {

// Tokens per vote / top-k tile (one workgroup of 256 threads, 4 tokens each).
constexpr int kVoteTile = 1024;
// Radix digits of the top-k select over the 32-bit vote keys, most significant first.
constexpr int kDigitBits0 = 11, kDigitBits1 = 11, kDigitBits2 = 10;
constexpr int kHistBins = 1 << 11;
// Keys that share the top 22 bits of the TopK threshold key are listed per request
// (key, position) up to this many; past it, the write pass counts them in the tiles.
constexpr int kCandCap = 2048;
// Selected tokens per attention wavefront and per attention workgroup (4 waves).
#ifndef TS_ATTN_SPLIT
#define TS_ATTN_SPLIT 32
#endif
constexpr int kAttnSplit = TS_ATTN_SPLIT;
constexpr int kAttnTile = 4 * kAttnSplit;

struct ScoreParams {
  const void* q;              // [b][H][d]
  const void* k_pool;         // [pages][H_kv][16][d]
  const int32_t* block_table; // [b][stride]
  const int32_t* seq_lens;    // [b]
  const int32_t* skip;        // [b] nonzero: request skipped (cache hit); may be null
  // Selection Cache (decode step): the score kernel decides each request's hit itself
  // and writes hit[r] (= skip); the stats kernel applies a miss (C_Q <- Q, valid <- 1).
  // cache == 0: no cache.
  int cache;
  void* cached_q;             // [b][H * d]
  int32_t* valid;             // [b]
  int32_t* hit;               // [b]
  // Radix histograms of the TopK launched next, or null: the stats kernel zeroes
  // them for every request it folds (not for cache hits or skipped requests).
  uint32_t* hist;             // [b][3][kHistBins]
  unsigned long long* mass;   // [b][3][kHistBins] or null
  double theta;
  float* logits;              // ragged [H][N_r] per request
  float* partials;            // [H][pair_stride][2] per-unit (max, sum exp), units of all requests
  int pair_stride;            // units per head row of partials (at least the launch's units)
  float* head_stats;          // [b][H][2]
  int H, Hkv, b, stride;
  int chunk_pages;            // pages per work unit
  float score_scale;
  int bf16;                   // element type of the pool (and of q unless q_f32)
  int q_f32;                  // q is fp32 whatever the pool type (the chunk mean query)
  int grid;                   // workgroups of the score kernel
  // Decode step with the pairs folded by the vote kernel (vote_folds_pairs): no stats
  // kernel runs; the score kernel clears the radix histograms of each request it scores.
  int fold;
};

struct VoteParams {
  const float* logits;
  const float* head_stats;    // [b][H][2]
  const int32_t* seq_lens;
  const int32_t* skip;
  float* vote;                // ragged [N_r]
  uint32_t* hist;             // [b][3][kHistBins]
  unsigned long long* mass;   // [b][3][kHistBins] integer vote mass per bin (top-p)
  unsigned long long* mstate; // [b][4] top-p state (target, mass left after digits 0, 1)
  int32_t* state;             // [b][8] select state (digits found, counts left, candidates)
  int32_t* tile_counts;       // [tiles][2] keys above the 22-bit threshold prefix, keys on it
  int2* cand;                 // [b][kCandCap] (key, position) of the keys on the prefix
  int32_t* sel_idx;           // [b][top_k]
  int32_t* sel_count;         // [b]
  int max_tokens;             // positions the vote buffer holds (first-tile loads before the tables)
  int H, G, b, top_k;
  int topp;                   // nonzero: dynamic top-p budget with fraction top_p, capped at top_k
  double top_p;
  int grid;                   // workgroups of the tile kernels
  // Decode step, fold mode: each vote workgroup folds the score kernel's per-unit
  // pairs of its request itself (head_stats unused) and the workgroup of a request's
  // first tile applies its Selection Cache miss (C_Q <- Q, valid <- 1).
  int fold;
  const float* partials;      // [H][pair_stride][2] per-unit (max, sum exp), units of all requests
  int pair_stride;
  int chunk_tokens;           // positions per score unit
  int fold_grid;              // workgroups of the fold-mode vote kernel (512-position tiles)
  const void* q;              // [b][H * d]
  void* cached_q;             // [b][H * d]
  int32_t* valid;             // [b]
  int q_chunks;               // 16-byte chunks of one request's query
};

// The vote kernel folds the pairs itself when a request has at most this many
// (heads x score units): every vote workgroup of the request reads them, and at this
// size the fold hides under its first logit loads.
constexpr int kFoldMaxPairs = 16384;

// Integer vote mass of the top-p budget: rint(v * 2^kMassBits) with v = 2^lv. Votes
// are at most H <= 256, so a request's total stays below 2^48 + N; integer sums are
// exact and independent of the order of the atomics.
constexpr int kMassBits = 40;
__device__ __forceinline__ unsigned long long vote_mass(float lv) {
  return (unsigned long long)rint(exp2((double)lv + (double)kMassBits));
}

struct AttnParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* sel_idx;     // [b][top_k] ascending
  const int32_t* sel_count;   // [b]
  float* partials;            // [b][H][splits][d + 2]
  float* partials2;           // [b][H][attn_combine_chunks(splits)][d + 2] (splits > 256 only)
  void* out;                  // [b][H][d]
  int H, Hkv, b, stride;
  int sel_stride;             // int32 entries per sel_idx row (the caller's top_k)
  int top_k, n_local;         // min(top_k, max tokens), max(1, min(n_local, max tokens)): work items
  float attn_scale;
  int bf16;
};


// Chunk-wise prefill. A request's chunk of c_r queries sits at positions
// [P_r, P_r + c_r) of its cache, P_r = N_r - c_r. The attention of chunk query j
// runs over a gathered key list: the TopK positions below the window start
// w0 = max(0, P_r - L) (n_sel of them), then the contiguous range
// [w0, P_r + c_r); query j sees the first base + j + 1 entries, base = n_sel + P_r - w0.
constexpr int kChunkRows = 64;        // (query, head) rows per fp32 attention workgroup (the fewest)
constexpr int kChunkRowsBf16 = 256;   // (query, head) rows per bf16 attention workgroup
#ifndef TS_CHUNK_SPLIT_KEYS
#define TS_CHUNK_SPLIT_KEYS 1024
#endif
constexpr int kChunkSplitKeys = TS_CHUNK_SPLIT_KEYS;  // most key-list entries per attention split
constexpr int kChunkPartStride = 128 + 4;  // floats per split partial: o[128], m, l, pad

struct ChunkParams {
  const void* q;              // [b][max_chunk][H][d]
  const int32_t* chunk_lens;  // [b]
  const int32_t* seq_lens;    // [b] N_r, chunk included
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* sel_idx;     // [b][sel_stride] TopK over the past, ascending
  const int32_t* sel_count;   // [b]
  float* qbar;                // [b][H][d] fp32 mean query (output of the mean kernel)
  int32_t* past_lens;         // [b] P_r (output of the mean kernel)
  int32_t* key_base;          // [b] entries before the chunk's own keys (written by the attention kernel)
  float* partials;            // [b][max_chunk][H][splits][kChunkPartStride]
  void* out;                  // [b][max_chunk][H][d]
  int H, Hkv, b, stride, max_chunk, sel_stride, n_local, splits;
  int split_keys;             // key-list entries per split (<= kChunkSplitKeys)
  float attn_scale;
  int bf16;
};

// Upper bound of a chunk's key-list length: TopK below the window, window, chunk.
__host__ __device__ inline long long chunk_max_keys(int top_k, int n_local, int max_chunk) {
  return (long long)top_k + n_local + max_chunk;
}
// Key-list entries per attention split: kChunkSplitKeys, or fewer (a multiple of 64;
// at most ceil(keys / 256) splits) when the workgroups of one split (`wgs_per_split`,
// from the largest chunk) would not fill the machine's compute units once.
__host__ __device__ inline int chunk_split_keys(int top_k, int n_local, int max_chunk, long long wgs_per_split,
                                                int num_cus) {
  const long long keys = chunk_max_keys(top_k, n_local, max_chunk);
  long long splits = (keys + kChunkSplitKeys - 1) / kChunkSplitKeys;
  if (wgs_per_split * splits < num_cus) {
    const long long want = (num_cus + wgs_per_split - 1) / wgs_per_split;
    const long long most = (keys + 255) / 256;
    splits = want < most ? want : most;
    if (splits < 1) splits = 1;
  }
  const long long per = (keys + splits - 1) / splits;
  const long long rounded = (per + 63) / 64 * 64;
  return (int)(rounded < kChunkSplitKeys ? rounded : kChunkSplitKeys);
}
__host__ __device__ inline int chunk_splits(int top_k, int n_local, int max_chunk, int split_keys) {
  return (int)((chunk_max_keys(top_k, n_local, max_chunk) + split_keys - 1) / split_keys);
}

__host__ __device__ inline int attn_splits(int top_k, int n_local) {
  return (int)(((long long)top_k + kAttnTile - 1) / kAttnTile + ((long long)n_local + kAttnTile - 1) / kAttnTile);
}
// Partials one workgroup of the first merge launch takes when a selection has more
// than this many; the partials that launch leaves (0 when the final merge reads the
// splits directly).
constexpr int kAttnCombineSpan = 256;
__host__ __device__ inline int attn_combine_chunks(int splits) {
  return splits > kAttnCombineSpan ? (splits + kAttnCombineSpan - 1) / kAttnCombineSpan : 0;
}

hipError_t launch_score(const ScoreParams& p, hipStream_t s);
hipError_t launch_vote_topk(const VoteParams& p, hipStream_t s, bool zero_hist);
hipError_t launch_attn(const AttnParams& p, hipStream_t s);
// Soft vote only (log2 votes into p.vote and the digit-0 histogram).
hipError_t launch_vote_only(const VoteParams& p, hipStream_t s);
// Radix TopK over any fp32 score array p.vote (segments p.seq_lens): histogram + phases.
hipError_t launch_score_select(const VoteParams& p, hipStream_t s);

// Selection-function ablations over the decode logits.
enum AblationFn { kAblSoftVote = 0, kAblNaive = 1, kAblHardVote = 2, kAblBlock = 3 };
struct AblationParams {
  const float* logits;        // decode layout [H_kv][N_r][G] per request
  const int32_t* seq_lens;    // [b]
  int32_t* seg_lens;          // [b * H] (hard vote) or [b] (block) segment lengths
  float* score;               // the per-position (or per-block) score the final TopK runs on
  float* head_scores;         // hard vote: [b][H][N_r] logits, one segment per (request, head)
  int32_t* head_sel;          // hard vote: [b * H][top_k] per-head TopK; block: [b][top_k] blocks
  int32_t* head_cnt;          // [b * H]
  int head_stride;            // int32 entries per head_sel row
  const float* vote;          // block: log2 votes [sum N_r]
  int32_t* sel_idx;           // [b][top_k]
  int32_t* sel_count;         // [b]
  int H, Hkv, b, top_k, block;
};
hipError_t launch_naive_scores(const AblationParams& p, hipStream_t s);
hipError_t launch_head_scores(const AblationParams& p, hipStream_t s);
hipError_t launch_count_votes(const AblationParams& p, hipStream_t s);
hipError_t launch_block_scores(const AblationParams& p, hipStream_t s);
hipError_t launch_expand_blocks(const AblationParams& p, hipStream_t s);

// Input checks (tokenselect_validate).
struct ValidateParams {
  const int32_t* block_table;
  const int32_t* seq_lens;
  int b, stride;
  int64_t pool_pages;
  unsigned long long* report;   // [4]
};
hipError_t launch_validate(const ValidateParams& p, hipStream_t s);

// Selection checks (tokenselect_validate_selection).
struct SelValidateParams {
  const int32_t* seq_lens;
  const int32_t* sel_idx;     // [b][top_k]
  const int32_t* sel_count;   // [b]
  int b, top_k;
  unsigned long long* report; // [4]
};
hipError_t launch_validate_selection(const SelValidateParams& p, hipStream_t s);

hipError_t launch_chunk_mean(const ChunkParams& p, hipStream_t s);
hipError_t launch_chunk_attn(const ChunkParams& p, hipStream_t s);

}  // namespace ts
