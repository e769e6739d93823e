/* Host-side exercise of the C ABI, built with AddressSanitizer and UndefinedBehavior-
 * Sanitizer on the host code (tests/test_host_sanitizers.py builds and runs it on a
 * machine without a GPU). Every call below fails validation before any launch, so no
 * device is touched: the sanitizers watch the size arithmetic, the argument checks
 * and the error-message formatting of every entry point, over ordinary and extreme
 * shapes. Prints one line per failed expectation and exits with their count. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tokenselect.h"

static int failures = 0;

#define EXPECT(cond, ...)                                  \
  do {                                                     \
    if (!(cond)) {                                         \
      ++failures;                                          \
      printf("FAIL line %d: ", __LINE__);                  \
      printf(__VA_ARGS__);                                 \
      printf("\n");                                        \
    }                                                      \
  } while (0)

static void* const F = (void*)(uintptr_t)4096;       /* non-null, 256-byte aligned, never read */
static void* const MIS = (void*)(uintptr_t)4100;     /* misaligned */

static ts_shape shape(int H, int Hkv, int b, int stride, int64_t total, int dtype) {
  ts_shape s;
  memset(&s, 0, sizeof s);
  s.num_q_heads = H; s.num_kv_heads = Hkv; s.head_dim = 128; s.page_size = 16;
  s.batch = b; s.block_table_stride = stride; s.max_total_tokens = total; s.dtype = dtype;
  return s;
}

static ts_select sel(int k, int L, double top_p) {
  ts_select x;
  memset(&x, 0, sizeof x);
  x.top_k = k; x.n_local = L; x.score_scale = 1.0f; x.attn_scale = 0.088f;
  x.cos_threshold = 0.9; x.top_p = top_p;
  return x;
}

static void check_error_text(ts_status st, ts_status want, const char* what) {
  EXPECT(st == want, "%s: status %d, want %d (%s)", what, (int)st, (int)want, tokenselect_last_error());
  EXPECT(strlen(tokenselect_last_error()) > 0, "%s: empty error text", what);
  EXPECT(strlen(tokenselect_status_string(st)) > 0, "%s: empty status string", what);
}

int main(void) {
  /* workspace sizes over ordinary and extreme shapes: either 0 (invalid) or a
     256-byte multiple that holds at least the H x max_total_tokens fp32 logits */
  const int heads[][2] = {{1, 1}, {8, 2}, {32, 8}, {28, 4}, {64, 8}, {256, 32}, {72, 8}, {30, 8}};
  const int batches[] = {1, 16, 1024, 1025, 0};
  const int64_t totals[] = {1, 8192, 131072, (int64_t)1 << 20, (int64_t)1 << 31, ((int64_t)1 << 31) + 1};
  const int ks[] = {1, 2048, 1 << 20, 0x7fffffff, 0};
  const int ls[] = {0, 512, 0x7fffffff, -1};
  for (unsigned a = 0; a < sizeof heads / sizeof heads[0]; ++a)
    for (unsigned bi = 0; bi < sizeof batches / sizeof batches[0]; ++bi)
      for (unsigned t = 0; t < sizeof totals / sizeof totals[0]; ++t)
        for (unsigned ki = 0; ki < sizeof ks / sizeof ks[0]; ++ki)
          for (unsigned li = 0; li < sizeof ls / sizeof ls[0]; ++li)
            for (int dt = 0; dt < 3; ++dt) {
              const int b = batches[bi];
              if ((int64_t)b > totals[t]) continue;
              ts_shape s = shape(heads[a][0], heads[a][1], b, 65536, totals[t], dt);
              ts_select x = sel(ks[ki], ls[li], 0.0);
              const size_t ws = tokenselect_workspace_size(&s, &x);
              if (ws) {
                EXPECT(ws % 256 == 0, "workspace %zu not 256-aligned", ws);
                EXPECT(ws >= (size_t)heads[a][0] * (size_t)totals[t] * 4u, "workspace %zu below the logits", ws);
                const size_t pw = tokenselect_prefill_workspace_size(&s, &x, 512);
                EXPECT(pw == 0 || pw >= ws, "prefill workspace %zu below decode %zu", pw, ws);
                for (int fn = 0; fn < 4; ++fn)
                  (void)tokenselect_ablation_workspace_size(&s, &x, fn, fn == 3 ? 16 : 1);
              }
            }

  ts_shape s = shape(32, 8, 4, 8192, 131072, TS_BF16);
  ts_select x = sel(2048, 512, 0.0);
  const size_t need = tokenselect_workspace_size(&s, &x);
  EXPECT(need > 0, "workspace of the 128K shape is 0");
  EXPECT(tokenselect_workspace_size(NULL, &x) == 0, "NULL shape accepted");
  EXPECT(tokenselect_workspace_size(&s, NULL) == 0, "NULL select accepted");

  /* every entry point rejects a NULL argument, a misaligned buffer or a small
     workspace before any launch */
  check_error_text(tokenselect_score(&s, &x, NULL, F, F, F, F, F, F, need, NULL), TS_ERR_INVALID_ARG, "score q");
  check_error_text(tokenselect_score(&s, &x, MIS, F, F, F, F, F, F, need, NULL), TS_ERR_INVALID_ARG, "score q align");
  check_error_text(tokenselect_score(&s, &x, F, F, F, F, F, F, F, need - 1, NULL), TS_ERR_WORKSPACE, "score ws");
  check_error_text(tokenselect_score(&s, &x, F, F, F, F, F, F, MIS, need, NULL), TS_ERR_INVALID_ARG, "score ws align");
  check_error_text(tokenselect_vote_topk(&s, &x, F, F, F, NULL, NULL, F, F, need, NULL), TS_ERR_INVALID_ARG,
                   "vote sel_idx");
  check_error_text(tokenselect_sparse_attn(&s, &x, F, F, F, F, F, F, NULL, F, F, need, NULL), TS_ERR_INVALID_ARG,
                   "attn sel_count");
  ts_cache c;
  c.cached_q = F; c.cached_idx = (int32_t*)F; c.cached_count = NULL; c.valid = (int32_t*)F;
  check_error_text(tokenselect_decode_step(&s, &x, F, F, F, F, F, &c, (int32_t*)F, F, F, need, NULL),
                   TS_ERR_INVALID_ARG, "decode cached_count");
  check_error_text(tokenselect_decode_step(&s, &x, F, F, F, F, F, NULL, (int32_t*)F, F, F, need, NULL),
                   TS_ERR_INVALID_ARG, "decode cache");
  c.cached_count = (int32_t*)F;
  check_error_text(tokenselect_decode_step_noalloc(&s, &x, F, F, F, F, F, &c, NULL, F, NULL), TS_ERR_INVALID_ARG,
                   "noalloc hit");
  ts_shape big = shape(32, 8, 1, 65536, (int64_t)1 << 20, TS_BF16);
  check_error_text(tokenselect_decode_step_noalloc(&big, &x, F, F, F, F, F, &c, (int32_t*)F, F, NULL),
                   TS_ERR_WORKSPACE, "noalloc scratch");
  const size_t pneed = tokenselect_prefill_workspace_size(&s, &x, 512);
  EXPECT(pneed > need, "prefill workspace %zu not above decode %zu", pneed, need);
  check_error_text(tokenselect_prefill_select(&s, &x, 512, F, NULL, F, F, F, NULL, NULL, NULL, F, F, F, pneed, NULL),
                   TS_ERR_INVALID_ARG, "prefill chunk_lens");
  check_error_text(tokenselect_prefill_select(&s, &x, 0, F, F, F, F, F, NULL, NULL, NULL, F, F, F, pneed, NULL),
                   TS_ERR_INVALID_ARG, "prefill max_chunk");
  check_error_text(tokenselect_chunk_attn(&s, &x, 512, F, F, F, F, F, F, F, F, F, F, pneed - 1, NULL),
                   TS_ERR_WORKSPACE, "chunk attn ws");
  check_error_text(tokenselect_prefill_chunk(&s, &x, 512, F, F, F, F, F, F, F, F, NULL, F, pneed, NULL),
                   TS_ERR_INVALID_ARG, "prefill chunk out");
  check_error_text(tokenselect_select_ablation(&s, &x, 7, 1, F, F, F, NULL, F, F, F, need, NULL),
                   TS_ERR_INVALID_ARG, "ablation fn");
  check_error_text(tokenselect_select_ablation(&s, &x, 3, 0, F, F, F, NULL, F, F, F, need, NULL),
                   TS_ERR_INVALID_ARG, "ablation block");
  ts_select xp = sel(2048, 512, 0.5);
  check_error_text(tokenselect_select_ablation(&s, &xp, 1, 1, F, F, F, NULL, F, F, F, need, NULL),
                   TS_ERR_UNSUPPORTED, "ablation top_p");
  ts_select bad_p = sel(2048, 512, 1.5);
  check_error_text(tokenselect_score(&s, &bad_p, F, F, F, F, F, F, F, need, NULL), TS_ERR_INVALID_ARG, "top_p");
  ts_shape g9 = shape(72, 8, 1, 64, 1024, TS_BF16);
  check_error_text(tokenselect_score(&g9, &x, F, F, F, F, F, F, F, need, NULL), TS_ERR_UNSUPPORTED, "group 9");
  ts_shape huge = shape(256, 256, 1024, 1, (int64_t)1 << 31, TS_BF16);
  ts_select hk = sel(0x7fffffff, 0, 0.0);
  check_error_text(tokenselect_sparse_attn(&huge, &hk, F, F, F, F, F, F, F, F, F, (size_t)1 << 40, NULL),
                   TS_ERR_UNSUPPORTED, "attention grid");
  check_error_text(tokenselect_validate(&s, NULL, F, 100, (uint64_t*)F, NULL), TS_ERR_INVALID_ARG, "validate bt");
  check_error_text(tokenselect_validate(&s, F, F, 100, (uint64_t*)MIS, NULL), TS_ERR_INVALID_ARG,
                   "validate report align");
  check_error_text(tokenselect_validate_selection(&s, &x, F, NULL, F, (uint64_t*)F, NULL), TS_ERR_INVALID_ARG,
                   "validate_selection sel_idx");
  for (int st = 0; st < 6; ++st) EXPECT(tokenselect_status_string((ts_status)st) != NULL, "status %d", st);

  printf("%d failures\n", failures);
  return failures;
}
