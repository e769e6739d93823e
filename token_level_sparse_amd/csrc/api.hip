// C ABI of the decode-step path: argument validation, workspace layout, launches.
// The entry points and their contracts are declared and documented in
// include/tokenselect.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "common.h"
#include "kernels.h"
#include "tokenselect.h"

namespace {

thread_local std::string g_err;

ts_status fail(ts_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ts_status fail(ts_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ts_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return TS_OK;
  return fail(TS_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Score work units: runs of chunk_pages pages of one KV head, sized so a launch
// has about kScoreUnitsTarget units; the grid is capped at kScoreMaxGrid
// workgroups of 4 waves that loop over the units.
#ifndef TS_SCORE_UNITS_TARGET
#define TS_SCORE_UNITS_TARGET 2048
#endif
#ifndef TS_SCORE_MAX_GRID
#define TS_SCORE_MAX_GRID 2048
#endif
#ifndef TS_SCORE_MAX_CHUNK_PAGES
#define TS_SCORE_MAX_CHUNK_PAGES 32
#endif
constexpr int kMinChunkPages = 4;     // smallest score work unit (pages)
constexpr int kMaxChunkPages = TS_SCORE_MAX_CHUNK_PAGES;
constexpr int kScoreUnitsTarget = TS_SCORE_UNITS_TARGET;
constexpr int kScoreMaxGrid = TS_SCORE_MAX_GRID;
constexpr int kMaxGrid = 2048;

// Byte offsets of the workspace regions.
struct Layout {
  size_t logits, partials, stats, vote, hist, mass, mstate, state, tiles, cand, attn, attn2, total;
};

int64_t max_chunks(const ts_shape& s) {
  return cdiv(s.max_total_tokens, (int64_t)kMinChunkPages * ts::kPage) + s.batch;
}
// Most vote tiles a batch can have: sum_r ceil(N_r / V) <= floor((T + b (V - 1)) / V).
int64_t max_tiles(const ts_shape& s) {
  return cdiv(s.max_total_tokens + (int64_t)(s.batch - 1) * (ts::kVoteTile - 1), ts::kVoteTile);
}

// Attention work items per (request, KV head): TopK list plus window, capped by
// the largest possible N.
int eff_top_k(const ts_shape& s, const ts_select& sel) {
  return (int)std::min<int64_t>(sel.top_k, s.max_total_tokens);
}
int eff_local(const ts_shape& s, const ts_select& sel) {
  return (int)std::min<int64_t>(sel.n_local, s.max_total_tokens);
}
// Window of the decode attention: the n_local newest positions, and never fewer
// than one, so the current token is always attended.
int decode_window(const ts_shape& s, const ts_select& sel) {
  return std::max(1, eff_local(s, sel));
}

Layout layout(const ts_shape& s, const ts_select& sel) {
  Layout L;
  size_t off = 0;
  const int64_t T = s.max_total_tokens;
  const int H = s.num_q_heads;
  L.logits = off;   off += align_up(sizeof(float) * (size_t)H * T);
  L.partials = off; off += align_up(sizeof(float) * 2 * (size_t)H * max_chunks(s));
  L.stats = off;    off += align_up(sizeof(float) * 2 * (size_t)H * s.batch);
  L.vote = off;     off += align_up(sizeof(float) * (size_t)T);
  L.hist = off;     off += align_up(sizeof(uint32_t) * 3 * ts::kHistBins * (size_t)s.batch);
  L.mass = off;     off += align_up(sizeof(uint64_t) * 3 * ts::kHistBins * (size_t)s.batch);
  L.mstate = off;   off += align_up(sizeof(uint64_t) * 4 * (size_t)s.batch);
  L.state = off;    off += align_up(sizeof(int32_t) * 8 * (size_t)s.batch);
  L.tiles = off;    off += align_up(sizeof(int32_t) * 2 * (size_t)max_tiles(s));
  L.cand = off;     off += align_up(sizeof(int2) * ts::kCandCap * (size_t)s.batch);
  const int S = ts::attn_splits(eff_top_k(s, sel), decode_window(s, sel));
  L.attn = off;     off += align_up(sizeof(float) * (ts::kHeadDim + 2) * (size_t)s.batch * H * S);
  L.attn2 = off;    off += align_up(sizeof(float) * (ts::kHeadDim + 2) * (size_t)s.batch * H *
                                    ts::attn_combine_chunks(S));
  L.total = off;
  return L;
}

ts_status check_shape(const ts_shape* s, const ts_select* sel) {
  if (!s || !sel) return fail(TS_ERR_INVALID_ARG, "shape and select must not be NULL");
  if (s->num_q_heads < 1 || s->num_kv_heads < 1)
    return fail(TS_ERR_INVALID_ARG, "num_q_heads (%d) and num_kv_heads (%d) must be >= 1",
                s->num_q_heads, s->num_kv_heads);
  if (s->num_q_heads % s->num_kv_heads != 0)
    return fail(TS_ERR_INVALID_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                s->num_q_heads, s->num_kv_heads);
  if (s->num_q_heads / s->num_kv_heads > ts::kMaxGroup)
    return fail(TS_ERR_UNSUPPORTED, "GQA group %d > %d", s->num_q_heads / s->num_kv_heads, ts::kMaxGroup);
  if (s->num_q_heads > 256) return fail(TS_ERR_UNSUPPORTED, "num_q_heads %d > 256", s->num_q_heads);
  if (s->head_dim != ts::kHeadDim) return fail(TS_ERR_UNSUPPORTED, "head_dim %d != 128", s->head_dim);
  if (s->page_size != ts::kPage) return fail(TS_ERR_UNSUPPORTED, "page_size %d != 16", s->page_size);
  if (s->batch < 1 || s->batch > ts::kMaxBatch)
    return fail(TS_ERR_INVALID_ARG, "batch %d outside [1, %d]", s->batch, ts::kMaxBatch);
  if (s->block_table_stride < 1)
    return fail(TS_ERR_INVALID_ARG, "block_table_stride %d < 1", s->block_table_stride);
  if (s->max_total_tokens < s->batch || s->max_total_tokens > (int64_t)1 << 31)
    return fail(TS_ERR_INVALID_ARG, "max_total_tokens %lld outside [batch, 2^31]",
                (long long)s->max_total_tokens);
  if (s->dtype != TS_F32 && s->dtype != TS_BF16)
    return fail(TS_ERR_UNSUPPORTED, "dtype %d is neither TS_F32 nor TS_BF16", s->dtype);
  if (sel->top_k < 1) return fail(TS_ERR_INVALID_ARG, "top_k %d < 1", sel->top_k);
  if (sel->n_local < 0) return fail(TS_ERR_INVALID_ARG, "n_local %d < 0", sel->n_local);
  if (!(sel->top_p >= 0.0 && sel->top_p <= 1.0))
    return fail(TS_ERR_INVALID_ARG, "top_p %g outside [0, 1] (0 turns the top-p budget off)", sel->top_p);
  // the attention grid has one workgroup per (request, KV head, slice of 128 selected
  // or window positions)
  const int64_t slices = (int64_t)ts::attn_splits(eff_top_k(*s, *sel), decode_window(*s, *sel));
  if ((int64_t)s->batch * s->num_kv_heads * slices > INT32_MAX)
    return fail(TS_ERR_UNSUPPORTED, "batch x num_kv_heads x attention slices of (top_k + n_local) too "
                "large for the attention grid");
  return TS_OK;
}

ts_status check_ws(const ts_shape& s, const ts_select& sel, const void* ws, size_t ws_bytes) {
  const size_t need = layout(s, sel).total;
  if (!ws) return fail(TS_ERR_INVALID_ARG, "workspace is NULL");
  if (ws_bytes < need)
    return fail(TS_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign)
    return fail(TS_ERR_INVALID_ARG, "workspace must be %zu-byte aligned", kAlign);
  return TS_OK;
}

#define TS_REQUIRE(ptr) \
  do { if (!(ptr)) return fail(TS_ERR_INVALID_ARG, "%s must not be NULL", #ptr); } while (0)

// The kernels read q, the pools and the cached query with 16-byte loads.
#define TS_REQUIRE16(ptr)                                                                 \
  do {                                                                                    \
    if (!(ptr)) return fail(TS_ERR_INVALID_ARG, "%s must not be NULL", #ptr);             \
    if (reinterpret_cast<uintptr_t>(ptr) % 16)                                            \
      return fail(TS_ERR_INVALID_ARG, "%s must be 16-byte aligned", #ptr);               \
  } while (0)

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

int score_chunk_pages(const ts_shape& s) {
  const int64_t pages = cdiv(s.max_total_tokens, ts::kPage) + s.batch;
  int64_t cp = pages * s.num_kv_heads / kScoreUnitsTarget;
  int c = kMinChunkPages;
  while (c * 2 <= cp && c * 2 <= kMaxChunkPages) c *= 2;
  return c;
}

ts::ScoreParams score_params(const ts_shape& s, const ts_select& sel, const void* q,
                             const void* k_pool, const int32_t* bt, const int32_t* seq,
                             const int32_t* skip, float* logits, float* stats, void* ws) {
  const Layout L = layout(s, sel);
  ts::ScoreParams p{};
  p.q = q; p.k_pool = k_pool; p.block_table = bt; p.seq_lens = seq; p.skip = skip;
  p.logits = logits; p.head_stats = stats; p.partials = at<float>(ws, L.partials);
  p.pair_stride = (int)max_chunks(s);
  p.H = s.num_q_heads; p.Hkv = s.num_kv_heads; p.b = s.batch; p.stride = s.block_table_stride;
  p.chunk_pages = score_chunk_pages(s);
  p.score_scale = sel.score_scale;
  p.bf16 = s.dtype == TS_BF16;
  const int64_t units = (cdiv(cdiv(s.max_total_tokens, ts::kPage) + s.batch, p.chunk_pages) + s.batch) *
                        s.num_kv_heads;
  p.grid = (int)std::max<int64_t>(1, std::min<int64_t>(kScoreMaxGrid, cdiv(units, 4)));
  if (p.grid >= 8 * ts::kXcds) p.grid -= p.grid % ts::kXcds;   // whole rounds over the XCDs
  return p;
}

// Decode step: the vote kernel folds the score kernel's per-unit pairs itself (no stats
// kernel launch) when no request can have more than kFoldMaxPairs of them.
bool vote_folds_pairs(const ts_shape& s, const ts::ScoreParams& sp) {
  const int64_t units = std::max<int64_t>(1, cdiv(s.max_total_tokens, (int64_t)sp.chunk_pages * ts::kPage));
  return units * s.num_q_heads <= ts::kFoldMaxPairs;
}

ts::VoteParams vote_params(const ts_shape& s, const ts_select& sel, const float* logits,
                           const float* stats, const int32_t* seq, const int32_t* skip,
                           float* vote, int32_t* sel_idx, int32_t* sel_count, void* ws) {
  const Layout L = layout(s, sel);
  ts::VoteParams p{};
  p.logits = logits; p.head_stats = stats; p.seq_lens = seq; p.skip = skip;
  p.vote = vote ? vote : at<float>(ws, L.vote);
  p.hist = at<uint32_t>(ws, L.hist);
  p.mass = at<unsigned long long>(ws, L.mass);
  p.mstate = at<unsigned long long>(ws, L.mstate);
  p.topp = sel.top_p > 0.0;
  p.top_p = sel.top_p;
  p.state = at<int32_t>(ws, L.state);
  p.tile_counts = at<int32_t>(ws, L.tiles);
  p.cand = at<int2>(ws, L.cand);
  p.sel_idx = sel_idx; p.sel_count = sel_count;
  // the select kernels may read the workspace vote buffer (max_total_tokens floats) up to
  // its end before they know N; a caller's buffer is read only below N
  p.max_tokens = vote ? 0 : (int)std::min<int64_t>(s.max_total_tokens, INT32_MAX);
  p.H = s.num_q_heads; p.G = s.num_q_heads / s.num_kv_heads; p.b = s.batch; p.top_k = sel.top_k;
  p.grid = (int)std::max<int64_t>(1, std::min<int64_t>(kMaxGrid, max_tiles(s)));
  return p;
}

ts::AttnParams attn_params(const ts_shape& s, const ts_select& sel, const void* q,
                           const void* k_pool, const void* v_pool, const int32_t* bt,
                           const int32_t* seq, const int32_t* sel_idx, const int32_t* sel_count,
                           void* out, void* ws) {
  const Layout L = layout(s, sel);
  ts::AttnParams p{};
  p.q = q; p.k_pool = k_pool; p.v_pool = v_pool; p.block_table = bt; p.seq_lens = seq;
  p.sel_idx = sel_idx; p.sel_count = sel_count; p.out = out;
  p.partials = at<float>(ws, L.attn);
  p.partials2 = at<float>(ws, L.attn2);
  p.H = s.num_q_heads; p.Hkv = s.num_kv_heads; p.b = s.batch; p.stride = s.block_table_stride;
  p.sel_stride = sel.top_k;
  p.top_k = eff_top_k(s, sel);
  p.n_local = decode_window(s, sel);
  p.attn_scale = sel.attn_scale;
  p.bf16 = s.dtype == TS_BF16;
  return p;
}

// ---------------------------------------------------------------- prefill
struct PrefillLayout {
  Layout dec;                  // the decode regions, used by the selection over the past
  size_t qbar, past, kbase, cpart, total;
};

// Compute units a chunk-attention launch should fill at least once.
constexpr int kComputeUnits = 256;

int chunk_split_keys_for(const ts_shape& s, const ts_select& sel, int max_chunk) {
  const int G = s.num_q_heads / s.num_kv_heads;
  const int rows = s.dtype == TS_BF16 ? ts::kChunkRowsBf16 : ts::kChunkRows;
  const int64_t wgs = cdiv((int64_t)max_chunk * G, rows) * s.num_kv_heads * s.batch;
  return ts::chunk_split_keys(eff_top_k(s, sel), eff_local(s, sel), max_chunk, wgs, kComputeUnits);
}

int chunk_splits_for(const ts_shape& s, const ts_select& sel, int max_chunk) {
  return ts::chunk_splits(eff_top_k(s, sel), eff_local(s, sel), max_chunk, chunk_split_keys_for(s, sel, max_chunk));
}

int64_t chunk_max_keys_for(const ts_shape& s, const ts_select& sel, int max_chunk) {
  return ts::chunk_max_keys(eff_top_k(s, sel), eff_local(s, sel), max_chunk);
}

PrefillLayout prefill_layout(const ts_shape& s, const ts_select& sel, int max_chunk) {
  PrefillLayout L;
  L.dec = layout(s, sel);
  size_t off = L.dec.total;
  const size_t bH = (size_t)s.batch * s.num_q_heads;
  L.qbar = off;  off += align_up(sizeof(float) * bH * ts::kHeadDim);
  L.past = off;  off += align_up(sizeof(int32_t) * (size_t)s.batch);
  L.kbase = off; off += align_up(sizeof(int32_t) * (size_t)s.batch);
  L.cpart = off; off += align_up(sizeof(float) * bH * (size_t)max_chunk *
                                 chunk_splits_for(s, sel, max_chunk) * ts::kChunkPartStride);
  L.total = off;
  return L;
}

ts_status check_chunk(const ts_shape& s, const ts_select& sel, int max_chunk) {
  if (max_chunk < 1) return fail(TS_ERR_INVALID_ARG, "max_chunk %d < 1", max_chunk);
  if ((int64_t)max_chunk > s.max_total_tokens)
    return fail(TS_ERR_INVALID_ARG, "max_chunk %d > max_total_tokens %lld", max_chunk,
                (long long)s.max_total_tokens);
  const int G = s.num_q_heads / s.num_kv_heads;
  const int64_t tiles = cdiv((int64_t)max_chunk * G, ts::kChunkRows) * s.num_kv_heads * s.batch;
  if (tiles * (chunk_splits_for(s, sel, max_chunk) + ts::kXcds) > INT32_MAX ||
      (int64_t)s.batch * max_chunk * s.num_q_heads / 8 > INT32_MAX)
    return fail(TS_ERR_UNSUPPORTED, "batch x max_chunk %lld too large", (long long)s.batch * max_chunk);
  if (chunk_max_keys_for(s, sel, max_chunk) > INT32_MAX / 2 ||
      (int64_t)s.batch * chunk_max_keys_for(s, sel, max_chunk) > INT32_MAX)
    return fail(TS_ERR_UNSUPPORTED, "top_k + n_local + max_chunk too large");
  if (chunk_splits_for(s, sel, max_chunk) > 65535)
    return fail(TS_ERR_UNSUPPORTED, "top_k + n_local + max_chunk too large for the split grid");
  return TS_OK;
}

ts_status check_prefill_ws(const ts_shape& s, const ts_select& sel, int max_chunk, const void* ws,
                           size_t ws_bytes) {
  const size_t need = prefill_layout(s, sel, max_chunk).total;
  if (!ws) return fail(TS_ERR_INVALID_ARG, "workspace is NULL");
  if (ws_bytes < need)
    return fail(TS_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign)
    return fail(TS_ERR_INVALID_ARG, "workspace must be %zu-byte aligned", kAlign);
  return TS_OK;
}

ts::ChunkParams chunk_params(const ts_shape& s, const ts_select& sel, int max_chunk, const void* q,
                             const int32_t* chunk_lens, const int32_t* seq, const void* k_pool,
                             const void* v_pool, const int32_t* bt, const int32_t* sel_idx,
                             const int32_t* sel_count, void* out, void* ws) {
  const PrefillLayout L = prefill_layout(s, sel, max_chunk);
  ts::ChunkParams p{};
  p.q = q; p.chunk_lens = chunk_lens; p.seq_lens = seq; p.k_pool = k_pool; p.v_pool = v_pool;
  p.block_table = bt; p.sel_idx = sel_idx; p.sel_count = sel_count;
  p.qbar = at<float>(ws, L.qbar); p.past_lens = at<int32_t>(ws, L.past);
  p.key_base = at<int32_t>(ws, L.kbase);
  p.partials = at<float>(ws, L.cpart); p.out = out;
  p.H = s.num_q_heads; p.Hkv = s.num_kv_heads; p.b = s.batch; p.stride = s.block_table_stride;
  p.max_chunk = max_chunk; p.sel_stride = sel.top_k; p.n_local = sel.n_local;
  p.splits = chunk_splits_for(s, sel, max_chunk);
  p.split_keys = chunk_split_keys_for(s, sel, max_chunk);
  p.attn_scale = sel.attn_scale;
  p.bf16 = s.dtype == TS_BF16;
  return p;
}

// Mean query, then the decode selection over the past positions.
ts_status prefill_select_launch(const ts_shape& s, const ts_select& sel, int max_chunk,
                                const void* q_chunk, const int32_t* chunk_lens,
                                const void* k_pool, const int32_t* bt, const int32_t* seq,
                                float* logits, float* stats, float* vote, int32_t* sel_idx,
                                int32_t* sel_count, void* ws, hipStream_t stream) {
  const PrefillLayout L = prefill_layout(s, sel, max_chunk);
  const ts::ChunkParams cp = chunk_params(s, sel, max_chunk, q_chunk, chunk_lens, seq, k_pool,
                                          nullptr, bt, nullptr, nullptr, nullptr, ws);
  ts_status st = device_status(ts::launch_chunk_mean(cp, stream), "chunk mean launch");
  if (st != TS_OK) return st;
  const int32_t* past = cp.past_lens;
  if (!logits) logits = at<float>(ws, L.dec.logits);
  if (!stats) stats = at<float>(ws, L.dec.stats);
  ts::ScoreParams sp = score_params(s, sel, cp.qbar, k_pool, bt, past, nullptr, logits, stats, ws);
  sp.q_f32 = 1;
  const ts::VoteParams vp = vote_params(s, sel, logits, stats, past, nullptr, vote, sel_idx,
                                        sel_count, ws);
  // the stats kernel clears the radix histograms (no separate clearing launch)
  sp.hist = vp.hist;
  sp.mass = vp.topp ? vp.mass : nullptr;
  if ((st = device_status(ts::launch_score(sp, stream), "score launch")) != TS_OK) return st;
  return device_status(ts::launch_vote_topk(vp, stream, false), "vote/top-k launch");
}

// ---------------------------------------------------------------- ablations
struct AblLayout {
  size_t vote, score, head_scores, head_sel, head_cnt, seg_lens, hist, mstate, state, tiles, cand, total;
  int segs, stride;
  int64_t positions;           // positions the radix select may see in one call
};

AblLayout abl_layout(const ts_shape& s, const ts_select& sel, int fn, int block) {
  AblLayout L;
  const int64_t T = s.max_total_tokens;
  const int H = s.num_q_heads;
  const bool hard = fn == ts::kAblHardVote, blk = fn == ts::kAblBlock;
  L.segs = hard ? s.batch * H : s.batch;
  L.stride = blk ? std::max(1, sel.top_k / block) : sel.top_k;
  L.positions = hard ? (int64_t)H * T : T;
  size_t off = 0;
  L.vote = off;        off += align_up(sizeof(float) * (size_t)T);
  L.score = off;       off += align_up(sizeof(float) * (size_t)(T + s.batch));
  L.head_scores = off; off += hard ? align_up(sizeof(float) * (size_t)H * T) : 0;
  L.head_sel = off;    off += align_up(sizeof(int32_t) * (size_t)L.segs * L.stride);
  L.head_cnt = off;    off += align_up(sizeof(int32_t) * (size_t)L.segs);
  L.seg_lens = off;    off += align_up(sizeof(int32_t) * (size_t)L.segs);
  L.hist = off;        off += align_up(sizeof(uint32_t) * 3 * ts::kHistBins * (size_t)L.segs);
  L.mstate = off;      off += align_up(sizeof(uint64_t) * 4 * (size_t)L.segs);
  L.state = off;       off += align_up(sizeof(int32_t) * 8 * (size_t)L.segs);
  L.tiles = off;       off += align_up(sizeof(int32_t) * 2 * (size_t)(cdiv(L.positions, ts::kVoteTile) + L.segs));
  L.cand = off;        off += align_up(sizeof(int2) * ts::kCandCap * (size_t)L.segs);
  L.total = off;
  return L;
}

ts_status check_ablation(const ts_shape& s, const ts_select& sel, int fn, int block) {
  if (fn < ts::kAblSoftVote || fn > ts::kAblBlock)
    return fail(TS_ERR_INVALID_ARG, "selection function %d is not a ts_select_fn", fn);
  if (fn == ts::kAblBlock && (block < 1 || block > 4096))
    return fail(TS_ERR_INVALID_ARG, "block %d outside [1, 4096]", block);
  if (fn == ts::kAblHardVote && (int64_t)s.batch * s.num_q_heads > ts::kMaxBatch)
    return fail(TS_ERR_UNSUPPORTED, "hard vote needs batch x num_q_heads <= %d (one TopK segment per head)",
                ts::kMaxBatch);
  if (fn == ts::kAblHardVote && (int64_t)s.num_q_heads * s.max_total_tokens > INT32_MAX)
    return fail(TS_ERR_UNSUPPORTED, "hard vote needs num_q_heads x max_total_tokens < 2^31");
  if (sel.top_p != 0.0) return fail(TS_ERR_UNSUPPORTED, "the ablations use a fixed top_k (top_p must be 0)");
  return TS_OK;
}

ts::VoteParams abl_vote_params(const AblLayout& L, void* ws, const float* score, const int32_t* lens,
                               int segs, int top_k, int32_t* sel_idx, int32_t* sel_count) {
  ts::VoteParams p{};
  p.vote = const_cast<float*>(score);
  p.seq_lens = lens;
  p.hist = at<uint32_t>(ws, L.hist);
  p.mstate = at<unsigned long long>(ws, L.mstate);
  p.state = at<int32_t>(ws, L.state);
  p.tile_counts = at<int32_t>(ws, L.tiles);
  p.cand = at<int2>(ws, L.cand);
  p.sel_idx = sel_idx; p.sel_count = sel_count;
  p.b = segs; p.top_k = top_k;
  p.grid = (int)std::max<int64_t>(1, std::min<int64_t>(kMaxGrid, cdiv(L.positions, ts::kVoteTile) + segs));
  return p;
}

}  // namespace

extern "C" {

size_t tokenselect_ablation_workspace_size(const ts_shape* shape, const ts_select* sel, int32_t fn,
                                           int32_t block) {
  if (check_shape(shape, sel) != TS_OK || check_ablation(*shape, *sel, fn, block) != TS_OK) return 0;
  return abl_layout(*shape, *sel, fn, block).total;
}

ts_status tokenselect_select_ablation(const ts_shape* shape, const ts_select* sel, int32_t fn,
                                      int32_t block, const float* logits, const float* head_stats,
                                      const int32_t* seq_lens, float* score, int32_t* sel_idx,
                                      int32_t* sel_count, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
  ts_status st = check_shape(shape, sel);
  if (st != TS_OK) return st;
  if ((st = check_ablation(*shape, *sel, fn, block)) != TS_OK) return st;
  TS_REQUIRE(logits); TS_REQUIRE(seq_lens); TS_REQUIRE(sel_idx); TS_REQUIRE(sel_count);
  if (fn == ts::kAblSoftVote || fn == ts::kAblBlock) TS_REQUIRE(head_stats);
  const AblLayout L = abl_layout(*shape, *sel, fn, block);
  if (!ws) return fail(TS_ERR_INVALID_ARG, "workspace is NULL");
  if (ws_bytes < L.total) return fail(TS_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", ws_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(TS_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const int b = shape->batch, H = shape->num_q_heads, k = sel->top_k;
  float* sc = score ? score : at<float>(ws, L.score);
  ts::AblationParams ap{};
  ap.logits = logits; ap.seq_lens = seq_lens; ap.seg_lens = at<int32_t>(ws, L.seg_lens);
  ap.score = sc; ap.head_scores = at<float>(ws, L.head_scores);
  ap.head_sel = at<int32_t>(ws, L.head_sel); ap.head_cnt = at<int32_t>(ws, L.head_cnt);
  ap.head_stride = L.stride; ap.vote = at<float>(ws, L.vote);
  ap.sel_idx = sel_idx; ap.sel_count = sel_count;
  ap.H = H; ap.Hkv = shape->num_kv_heads; ap.b = b; ap.top_k = k; ap.block = block;
  auto soft_votes = [&](float* dst) {
    ts::VoteParams vp = abl_vote_params(L, ws, dst, seq_lens, b, k, sel_idx, sel_count);
    vp.logits = logits; vp.head_stats = head_stats; vp.H = H; vp.G = H / shape->num_kv_heads;
    return vp;
  };
  switch (fn) {
    case ts::kAblSoftVote:
      return device_status(ts::launch_vote_topk(soft_votes(sc), stream, true), "vote/top-k launch");
    case ts::kAblNaive: {
      if ((st = device_status(ts::launch_naive_scores(ap, stream), "naive score launch")) != TS_OK) return st;
      return device_status(ts::launch_score_select(abl_vote_params(L, ws, sc, seq_lens, b, k, sel_idx, sel_count),
                                                   stream), "top-k launch");
    }
    case ts::kAblHardVote: {
      if ((st = device_status(ts::launch_head_scores(ap, stream), "head score launch")) != TS_OK) return st;
      const ts::VoteParams hp = abl_vote_params(L, ws, ap.head_scores, ap.seg_lens, b * H, k, ap.head_sel,
                                                ap.head_cnt);
      if ((st = device_status(ts::launch_score_select(hp, stream), "per-head top-k launch")) != TS_OK) return st;
      if ((st = device_status(ts::launch_count_votes(ap, stream), "vote count launch")) != TS_OK) return st;
      return device_status(ts::launch_score_select(abl_vote_params(L, ws, sc, seq_lens, b, k, sel_idx, sel_count),
                                                   stream), "top-k launch");
    }
    default: {  // block
      ts::VoteParams vp = soft_votes(at<float>(ws, L.vote));
      if ((st = device_status(ts::launch_vote_only(vp, stream), "vote launch")) != TS_OK) return st;
      if ((st = device_status(ts::launch_block_scores(ap, stream), "block score launch")) != TS_OK) return st;
      const ts::VoteParams bp = abl_vote_params(L, ws, sc, ap.seg_lens, b, L.stride, ap.head_sel, ap.head_cnt);
      if ((st = device_status(ts::launch_score_select(bp, stream), "block top-k launch")) != TS_OK) return st;
      return device_status(ts::launch_expand_blocks(ap, stream), "block expand launch");
    }
  }
}

size_t tokenselect_prefill_workspace_size(const ts_shape* shape, const ts_select* sel,
                                          int32_t max_chunk) {
  if (check_shape(shape, sel) != TS_OK) return 0;
  if (check_chunk(*shape, *sel, max_chunk) != TS_OK) return 0;
  return prefill_layout(*shape, *sel, max_chunk).total;
}

ts_status tokenselect_prefill_select(const ts_shape* shape, const ts_select* sel, int32_t max_chunk,
                                     const void* q_chunk, const int32_t* chunk_lens,
                                     const void* k_pool, const int32_t* block_table,
                                     const int32_t* seq_lens, float* logits, float* head_stats,
                                     float* vote, int32_t* sel_idx, int32_t* sel_count, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  ts_status st = check_shape(shape, sel);
  if (st != TS_OK) return st;
  if ((st = check_chunk(*shape, *sel, max_chunk)) != TS_OK) return st;
  TS_REQUIRE16(q_chunk); TS_REQUIRE(chunk_lens); TS_REQUIRE16(k_pool); TS_REQUIRE(block_table);
  TS_REQUIRE(seq_lens); TS_REQUIRE(sel_idx); TS_REQUIRE(sel_count);
  if ((st = check_prefill_ws(*shape, *sel, max_chunk, ws, ws_bytes)) != TS_OK) return st;
  return prefill_select_launch(*shape, *sel, max_chunk, q_chunk, chunk_lens, k_pool, block_table,
                               seq_lens, logits, head_stats, vote, sel_idx, sel_count, ws, stream);
}

ts_status tokenselect_chunk_attn(const ts_shape* shape, const ts_select* sel, int32_t max_chunk,
                                 const void* q_chunk, const int32_t* chunk_lens,
                                 const void* k_pool, const void* v_pool,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const int32_t* sel_idx, const int32_t* sel_count, void* out,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  ts_status st = check_shape(shape, sel);
  if (st != TS_OK) return st;
  if ((st = check_chunk(*shape, *sel, max_chunk)) != TS_OK) return st;
  TS_REQUIRE16(q_chunk); TS_REQUIRE(chunk_lens); TS_REQUIRE16(k_pool); TS_REQUIRE16(v_pool);
  TS_REQUIRE(block_table); TS_REQUIRE(seq_lens); TS_REQUIRE(sel_idx); TS_REQUIRE(sel_count);
  TS_REQUIRE(out);
  if ((st = check_prefill_ws(*shape, *sel, max_chunk, ws, ws_bytes)) != TS_OK) return st;
  const ts::ChunkParams cp = chunk_params(*shape, *sel, max_chunk, q_chunk, chunk_lens, seq_lens,
                                          k_pool, v_pool, block_table, sel_idx, sel_count, out, ws);
  return device_status(ts::launch_chunk_attn(cp, stream), "chunk attention launch");
}

ts_status tokenselect_prefill_chunk(const ts_shape* shape, const ts_select* sel, int32_t max_chunk,
                                    const void* q_chunk, const int32_t* chunk_lens,
                                    const void* k_pool, const void* v_pool,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    int32_t* sel_idx, int32_t* sel_count, void* out, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
  ts_status st = check_shape(shape, sel);
  if (st != TS_OK) return st;
  if ((st = check_chunk(*shape, *sel, max_chunk)) != TS_OK) return st;
  TS_REQUIRE16(q_chunk); TS_REQUIRE(chunk_lens); TS_REQUIRE16(k_pool); TS_REQUIRE16(v_pool);
  TS_REQUIRE(block_table); TS_REQUIRE(seq_lens); TS_REQUIRE(sel_idx); TS_REQUIRE(sel_count);
  TS_REQUIRE(out);
  if ((st = check_prefill_ws(*shape, *sel, max_chunk, ws, ws_bytes)) != TS_OK) return st;
  st = prefill_select_launch(*shape, *sel, max_chunk, q_chunk, chunk_lens, k_pool, block_table,
                             seq_lens, nullptr, nullptr, nullptr, sel_idx, sel_count, ws, stream);
  if (st != TS_OK) return st;
  const ts::ChunkParams cp = chunk_params(*shape, *sel, max_chunk, q_chunk, chunk_lens, seq_lens,
                                          k_pool, v_pool, block_table, sel_idx, sel_count, out, ws);
  return device_status(ts::launch_chunk_attn(cp, stream), "chunk attention launch");
}

}  // extern "C"

extern "C" {

size_t tokenselect_workspace_size(const ts_shape* shape, const ts_select* sel) {
  if (check_shape(shape, sel) != TS_OK) return 0;
  return layout(*shape, *sel).total;
}

ts_status tokenselect_score(const ts_shape* shape, const ts_select* sel, const void* q,
                            const void* k_pool, const int32_t* block_table,
                            const int32_t* seq_lens, float* logits, float* head_stats,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  ts_status st = check_shape(shape, sel);
  if (st != TS_OK) return st;
  TS_REQUIRE16(q); TS_REQUIRE16(k_pool); TS_REQUIRE(block_table); TS_REQUIRE(seq_lens);
  TS_REQUIRE(logits);   // head_stats may be NULL: the statistics are then not computed
  if ((st = check_ws(*shape, *sel, ws, ws_bytes)) != TS_OK) return st;
  const ts::ScoreParams p = score_params(*shape, *sel, q, k_pool, block_table, seq_lens, nullptr,
                                         logits, head_stats, ws);
  return device_status(ts::launch_score(p, stream), "score launch");
}

ts_status tokenselect_vote_topk(const ts_shape* shape, const ts_select* sel, const float* logits,
                                const float* head_stats, const int32_t* seq_lens, float* vote,
                                int32_t* sel_idx, int32_t* sel_count, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  ts_status st = check_shape(shape, sel);
  if (st != TS_OK) return st;
  TS_REQUIRE(logits); TS_REQUIRE(head_stats); TS_REQUIRE(seq_lens);
  TS_REQUIRE(sel_idx); TS_REQUIRE(sel_count);
  if ((st = check_ws(*shape, *sel, ws, ws_bytes)) != TS_OK) return st;
  const ts::VoteParams p = vote_params(*shape, *sel, logits, head_stats, seq_lens, nullptr, vote,
                                       sel_idx, sel_count, ws);
  return device_status(ts::launch_vote_topk(p, stream, true), "vote/top-k launch");
}

ts_status tokenselect_sparse_attn(const ts_shape* shape, const ts_select* sel, const void* q,
                                  const void* k_pool, const void* v_pool,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  const int32_t* sel_idx, const int32_t* sel_count, void* out,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
  ts_status st = check_shape(shape, sel);
  if (st != TS_OK) return st;
  TS_REQUIRE16(q); TS_REQUIRE16(k_pool); TS_REQUIRE16(v_pool); TS_REQUIRE(block_table);
  TS_REQUIRE(seq_lens); TS_REQUIRE(sel_idx); TS_REQUIRE(sel_count); TS_REQUIRE(out);
  if ((st = check_ws(*shape, *sel, ws, ws_bytes)) != TS_OK) return st;
  const ts::AttnParams p = attn_params(*shape, *sel, q, k_pool, v_pool, block_table, seq_lens,
                                       sel_idx, sel_count, out, ws);
  return device_status(ts::launch_attn(p, stream), "sparse attention launch");
}

}  // extern "C"

namespace {

ts_status check_decode_args(const ts_shape* shape, const ts_select* sel, const void* q,
                            const void* k_pool, const void* v_pool, const int32_t* block_table,
                            const int32_t* seq_lens, const ts_cache* cache, const int32_t* hit,
                            const void* out) {
  ts_status st = check_shape(shape, sel);
  if (st != TS_OK) return st;
  TS_REQUIRE16(q); TS_REQUIRE16(k_pool); TS_REQUIRE16(v_pool); TS_REQUIRE(block_table);
  TS_REQUIRE(seq_lens); TS_REQUIRE(cache); TS_REQUIRE(hit); TS_REQUIRE(out);
  TS_REQUIRE16(cache->cached_q); TS_REQUIRE(cache->cached_idx); TS_REQUIRE(cache->cached_count);
  TS_REQUIRE(cache->valid);
  return TS_OK;
}

// Launches of one decode step on a checked workspace.
ts_status decode_step_launch(const ts_shape* shape, const ts_select* sel, const void* q,
                             const void* k_pool, const void* v_pool,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const ts_cache* cache, int32_t* hit, void* out, void* ws,
                             hipStream_t stream) {
  ts_status st;
  const Layout L = layout(*shape, *sel);
  float* logits = at<float>(ws, L.logits);
  float* stats = at<float>(ws, L.stats);

  // Step 0 runs inside the score kernel: it decides hit[r] and skips the hits. Each
  // miss (C_Q <- Q, valid <- 1, cleared radix histograms) is applied after every read
  // of C_Q: by the stats kernel, or in fold mode by the score kernel (histograms) and
  // the vote kernel (C_Q, valid), which then also folds the per-unit pairs itself.
  ts::ScoreParams sp = score_params(*shape, *sel, q, k_pool, block_table, seq_lens, nullptr,
                                    logits, stats, ws);
  sp.cache = 1;
  sp.cached_q = cache->cached_q; sp.valid = cache->valid; sp.hit = hit;
  sp.hist = at<uint32_t>(ws, L.hist);
  sp.mass = sel->top_p > 0.0 ? at<unsigned long long>(ws, L.mass) : nullptr;
  sp.theta = sel->cos_threshold;
  ts::VoteParams vp = vote_params(*shape, *sel, logits, stats, seq_lens, hit, nullptr,
                                  cache->cached_idx, cache->cached_count, ws);
  if (vote_folds_pairs(*shape, sp)) {
    sp.fold = 1;
    vp.fold = 1;
    vp.partials = sp.partials;
    vp.pair_stride = sp.pair_stride;
    // most 512-position tiles a batch can have: sum_r ceil(N_r / 512)
    vp.fold_grid = (int)std::min<int64_t>(
        2048, cdiv(shape->max_total_tokens + (int64_t)(shape->batch - 1) * 511, 512));
    vp.chunk_tokens = sp.chunk_pages * ts::kPage;
    vp.q = q;
    vp.cached_q = cache->cached_q;
    vp.valid = cache->valid;
    vp.q_chunks = shape->num_q_heads * ts::kHeadDim * (shape->dtype == TS_BF16 ? 2 : 4) / 16;
  }
  if ((st = device_status(ts::launch_score(sp, stream), "score launch")) != TS_OK) return st;

  if ((st = device_status(ts::launch_vote_topk(vp, stream, false), "vote/top-k launch")) != TS_OK)
    return st;

  const ts::AttnParams ap = attn_params(*shape, *sel, q, k_pool, v_pool, block_table, seq_lens,
                                        cache->cached_idx, cache->cached_count, out, ws);
  return device_status(ts::launch_attn(ap, stream), "sparse attention launch");
}

// Static scratch of tokenselect_decode_step_noalloc. In host code `scratch` is only
// a stand-in for the symbol: its device address on the current device comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kScratchBytes = TS_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

ts_status scratch_for_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(TS_ERR_UNSUPPORTED, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_status(e, "hipGetSymbolAddress(scratch)");
    if (!p || reinterpret_cast<uintptr_t>(p) % kAlign)
      return fail(TS_ERR_DEVICE, "static scratch address %p is not %zu-byte aligned", p, kAlign);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return TS_OK;
}

}  // namespace

extern "C" {

ts_status tokenselect_decode_step(const ts_shape* shape, const ts_select* sel, const void* q,
                                  const void* k_pool, const void* v_pool,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  const ts_cache* cache, int32_t* hit, void* out, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  ts_status st = check_decode_args(shape, sel, q, k_pool, v_pool, block_table, seq_lens, cache, hit,
                                   out);
  if (st != TS_OK) return st;
  if ((st = check_ws(*shape, *sel, ws, ws_bytes)) != TS_OK) return st;
  return decode_step_launch(shape, sel, q, k_pool, v_pool, block_table, seq_lens, cache, hit, out,
                            ws, stream);
}

ts_status tokenselect_decode_step_noalloc(const ts_shape* shape, const ts_select* sel,
                                          const void* q, const void* k_pool, const void* v_pool,
                                          const int32_t* block_table, const int32_t* seq_lens,
                                          const ts_cache* cache, int32_t* hit, void* out,
                                          hipStream_t stream) {
  ts_status st = check_decode_args(shape, sel, q, k_pool, v_pool, block_table, seq_lens, cache, hit,
                                   out);
  if (st != TS_OK) return st;
  const size_t need = layout(*shape, *sel).total;
  if (need > kScratchBytes)
    return fail(TS_ERR_WORKSPACE,
                "this shape needs %zu bytes of scratch, above the %zu-byte static scratch of "
                "tokenselect_decode_step_noalloc (lower max_total_tokens, or call "
                "tokenselect_decode_step with a caller workspace)", need, kScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != TS_OK) return st;
  return decode_step_launch(shape, sel, q, k_pool, v_pool, block_table, seq_lens, cache, hit, out,
                            ws, stream);
}

ts_status tokenselect_validate(const ts_shape* shape, const int32_t* block_table,
                               const int32_t* seq_lens, int64_t num_pool_pages, uint64_t* report,
                               hipStream_t stream) {
  if (!shape) return fail(TS_ERR_INVALID_ARG, "shape must not be NULL");
  TS_REQUIRE(block_table); TS_REQUIRE(seq_lens); TS_REQUIRE(report);
  if (shape->batch < 1 || shape->batch > ts::kMaxBatch)
    return fail(TS_ERR_INVALID_ARG, "batch %d outside [1, %d]", shape->batch, ts::kMaxBatch);
  if (shape->block_table_stride < 1)
    return fail(TS_ERR_INVALID_ARG, "block_table_stride %d < 1", shape->block_table_stride);
  if (shape->page_size != ts::kPage)
    return fail(TS_ERR_UNSUPPORTED, "page_size %d != 16", shape->page_size);
  if (num_pool_pages < 1) return fail(TS_ERR_INVALID_ARG, "num_pool_pages %lld < 1", (long long)num_pool_pages);
  if (reinterpret_cast<uintptr_t>(report) % 8) return fail(TS_ERR_INVALID_ARG, "report must be 8-byte aligned");
  ts::ValidateParams p{};
  p.block_table = block_table; p.seq_lens = seq_lens; p.b = shape->batch;
  p.stride = shape->block_table_stride; p.pool_pages = num_pool_pages;
  p.report = reinterpret_cast<unsigned long long*>(report);
  return device_status(ts::launch_validate(p, stream), "validate launch");
}

ts_status tokenselect_validate_selection(const ts_shape* shape, const ts_select* sel,
                                         const int32_t* seq_lens, const int32_t* sel_idx,
                                         const int32_t* sel_count, uint64_t* report,
                                         hipStream_t stream) {
  if (!shape || !sel) return fail(TS_ERR_INVALID_ARG, "shape and select must not be NULL");
  TS_REQUIRE(seq_lens); TS_REQUIRE(sel_idx); TS_REQUIRE(sel_count); TS_REQUIRE(report);
  if (shape->batch < 1 || shape->batch > ts::kMaxBatch)
    return fail(TS_ERR_INVALID_ARG, "batch %d outside [1, %d]", shape->batch, ts::kMaxBatch);
  if (sel->top_k < 1) return fail(TS_ERR_INVALID_ARG, "top_k %d < 1", sel->top_k);
  if (reinterpret_cast<uintptr_t>(report) % 8) return fail(TS_ERR_INVALID_ARG, "report must be 8-byte aligned");
  ts::SelValidateParams p{};
  p.seq_lens = seq_lens; p.sel_idx = sel_idx; p.sel_count = sel_count;
  p.b = shape->batch; p.top_k = sel->top_k;
  p.report = reinterpret_cast<unsigned long long*>(report);
  return device_status(ts::launch_validate_selection(p, stream), "validate_selection launch");
}

const char* tokenselect_status_string(ts_status s) {
  switch (s) {
    case TS_OK: return "ok";
    case TS_ERR_INVALID_ARG: return "invalid argument";
    case TS_ERR_UNSUPPORTED: return "unsupported configuration";
    case TS_ERR_WORKSPACE: return "workspace too small";
    case TS_ERR_DEVICE: return "device launch failed";
  }
  return "unknown status";
}

const char* tokenselect_last_error(void) { return g_err.c_str(); }

}  // extern "C"
