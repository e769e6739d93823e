"""GPU parity of the HIP path against the fp64 oracle (through the C ABI).

Sizes: the tiny fp32 workload in full; Llama-3-8B-shaped bf16 cases that span
several vote tiles and end on a partial page; the 128K workload in full; the
ragged 16-request batch at reduced and full lengths; the 1M workload (one layer)
in full; and the edge cases (k >= N, N <= L, N = 1, n_local = 0, exact ties).
"""
import numpy as np
import pytest
import torch

import token_level_sparse_amd as ts
from tests import gpu_helpers as gh
from synth import workloads as wl
from oracle import tokenselect_oracle as ora

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _check_all(batch, geo, **kw):
    po = gh.run_path(batch, geo, **{k: v for k, v in kw.items() if k in ("top_k", "n_local", "score_scale")})
    stats = []
    for r, req in enumerate(batch.requests):
        stats.append(gh.check_request(po, r, req, geo, **kw))
    return po, stats


def test_tiny_f32_full():
    geo = wl.workload("tiny-f32-8k")
    gh.log(f"[tiny-f32-8k] N={geo.seq_len} H={geo.num_q_heads}/{geo.num_kv_heads} fp32")
    batch = wl.make_batch(geo, device=DEV)
    po, st = _check_all(batch, geo)
    gh.log(f"  {st}")


def test_tiny_f32_paging_invariance_bit_identical():
    geo = wl.workload("tiny-f32-8k")
    gh.log("[tiny-f32-8k] shuffled vs identity block table")
    a = gh.run_path(wl.make_batch(geo, device=DEV), geo)
    b = gh.run_path(wl.make_batch(geo, device=DEV, permute=False), geo)
    for x, y in zip(a.logits + a.vote + a.T, b.logits + b.vote + b.T):
        assert np.array_equal(x, y)
    assert np.array_equal(a.stats, b.stats)
    assert np.array_equal(a.out, b.out)


def test_repeat_runs_bit_identical():
    geo = wl.workload("llama3-8b-128k", seq_len=20000)
    gh.log("[llama3 N=20000] two runs")
    batch = wl.make_batch(geo, device=DEV)
    a = gh.run_path(batch, geo)
    b = gh.run_path(batch, geo)
    for x, y in zip(a.logits + a.vote + a.T, b.logits + b.vote + b.T):
        assert np.array_equal(x, y)
    assert np.array_equal(a.out, b.out)


@pytest.mark.parametrize("n", [5000, 4099, 12345])
def test_llama3_shape_ragged_tail(n):
    geo = wl.workload("llama3-8b-128k", seq_len=n, top_k=256, n_local=64, n_planted=16)
    gh.log(f"[llama3 N={n} k=256 L=64]")
    po, st = _check_all(wl.make_batch(geo, device=DEV), geo)
    gh.log(f"  {st}")


def test_qwen2_shape_group7():
    geo = wl.workload("qwen2-7b-cache256", seq_len=9000, top_k=300, n_local=100)
    gh.log("[qwen2 G=7 N=9000]")
    po, st = _check_all(wl.make_batch(geo, device=DEV), geo)
    gh.log(f"  {st}")


def test_score_scale_parameter():
    geo = wl.workload("llama3-8b-128k", seq_len=3000, top_k=128, n_local=32, n_planted=8)
    gh.log("[llama3 N=3000 score_scale=1/sqrt(d)]")
    _check_all(wl.make_batch(geo, device=DEV), geo, score_scale=geo.attn_scale)


def test_llama3_128k_full():
    geo = wl.workload("llama3-8b-128k")
    gh.log(f"[llama3-8b-128k] N={geo.seq_len} full oracle")
    po, st = _check_all(wl.make_batch(geo, device=DEV), geo)
    gh.log(f"  {st}")


def test_ragged_batch_reduced():
    geo = wl.workload("llama3-8b-ragged16", min_len=1500, max_len=20000, top_k=512, n_local=128,
                      n_planted=16)
    gh.log("[ragged16 reduced lengths]")
    batch = wl.make_batch(geo, device=DEV)
    gh.log(f"  lens={batch.seq_lens.tolist()}")
    po, st = _check_all(batch, geo)
    gh.log(f"  {st}")


def _decode_step_matches(batch, geo, po):
    """The benchmark's configuration: one tokenselect_decode_step with theta = 2 (every
    request reselects) gives the oracle-checked TopK and outputs of the separate entry
    points bit for bit; then theta = -1 makes every request a hit that reuses them."""
    b = batch.q.shape[0]
    H, d = geo.num_q_heads, geo.head_dim
    shape = ts.make_shape(H, geo.num_kv_heads, b, batch.block_table.shape[1], batch.total_tokens,
                          geo.torch_dtype)
    cache = ts.CacheState.allocate(b, H, d, geo.top_k, geo.torch_dtype, DEV)
    hit = torch.full((b,), -1, dtype=torch.int32, device=DEV)
    out = torch.empty(b, H, d, dtype=geo.torch_dtype, device=DEV)
    for theta, want_hit in ((2.0, 0), (-1.0, 1)):
        sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, theta)
        ws = ts.alloc_workspace(shape, sel, DEV)
        ts.decode_step(shape, sel, batch.q, batch.k_pool, batch.v_pool, batch.block_table, batch.seq_lens,
                       cache, hit, out, ws)
        torch.cuda.synchronize()
        assert hit.cpu().tolist() == [want_hit] * b
        counts = cache.cached_count.cpu().tolist()
        idx = cache.cached_idx.cpu().numpy()
        for r in range(b):
            assert np.array_equal(idx[r, :counts[r]].astype(np.int64), po.T[r]), (theta, r)
        assert np.array_equal(gh.np32(out), po.out)
        del ws


def test_ragged_batch_full():
    geo = wl.workload("llama3-8b-ragged16")
    gh.log("[llama3-8b-ragged16] full lengths")
    batch = wl.make_batch(geo, device=DEV)
    gh.log(f"  lens={batch.seq_lens.tolist()} total={batch.total_tokens}")
    po, st = _check_all(batch, geo)
    gh.log(f"  {st}")
    _decode_step_matches(batch, geo, po)


def test_llama3_1m_one_layer_full():
    geo = wl.workload("llama3-8b-1m")
    gh.log(f"[llama3-8b-1m] layer 0, N={geo.seq_len}")
    batch = wl.make_batch(geo, device=DEV)
    po, st = _check_all(batch, geo)
    gh.log(f"  {st}")
    # planted recall (the vote bound): any position with vote > H/k is selected
    big = np.nonzero(np.exp2(po.vote[0].astype(np.float64)) > geo.num_q_heads / geo.top_k)[0]
    assert np.all(np.isin(big, po.T[0]))
    _decode_step_matches(batch, geo, po)


def test_planted_recall_without_scale_spread():
    geo = wl.workload("llama3-8b-128k", seq_len=32768)
    gh.log("[llama3 N=32768, s=1] planted recall")
    batch = wl.make_batch(geo, device=DEV, scale_spread=False)
    po, st = _check_all(batch, geo)
    gh.log(f"  {st}")
    planted = np.unique(batch.requests[0].planted_pos.cpu().numpy())
    assert np.all(np.isin(planted, po.T[0]))
    # without the per-head key scales the logits stay small and fp32 meets the strict
    # relative 1e-4 of band (a) on every vote
    assert st[0]["n_loose"] == 0, st


# ------------------------------------------------------------------ edge cases
@pytest.mark.parametrize("n,k,L", [
    (100, 256, 64),      # k >= N: everything selected
    (50, 10, 64),        # window covers everything
    (1, 1, 1),           # single token
    (17, 4, 0),          # no window, partial second page
    (2048, 2047, 3),     # exactly one vote tile
    (2049, 2048, 1),     # one position left out, two tiles
])
def test_edge_sizes(n, k, L):
    geo = wl.workload("llama3-8b-128k", seq_len=n, top_k=k, n_local=L, n_planted=min(4, n))
    gh.log(f"[edge N={n} k={k} L={L}]")
    _check_all(wl.make_batch(geo, device=DEV), geo)


def test_mixed_batch_k_above_and_below_n():
    geo = wl.workload("tiny-f32-8k", top_k=300, n_local=16, batch=1)
    gh.log("[mixed batch fp32] lens 100, 5000, 300, 7")
    gen = torch.Generator(device=DEV).manual_seed(77)
    reqs = [wl.make_request(gen, geo, n, DEV) for n in (100, 5000, 300, 7)]
    batch = wl.page_requests(reqs, geo, gen, DEV, spare_pages=5)
    po, st = _check_all(batch, geo)


def test_exact_ties_take_lowest_positions():
    # identical keys make every vote exactly H/N in fp32: TopK must be [0, k)
    geo = wl.workload("llama3-8b-128k", seq_len=5000, top_k=700, n_local=10, n_planted=1)
    gh.log("[ties] identical keys")
    gen = torch.Generator(device=DEV).manual_seed(5)
    req = wl.make_request(gen, geo, 5000, DEV)
    req.k[:] = req.k[:, :1, :]
    batch = wl.page_requests([req], geo, gen, DEV)
    po = gh.run_path(batch, geo)
    assert np.all(po.vote[0] == po.vote[0][0])
    assert np.array_equal(po.T[0], np.arange(700))


def test_attention_given_oracle_selection():
    # step 5 alone on the oracle's own TopK, so its check does not depend on step 4
    geo = wl.workload("llama3-8b-128k", seq_len=6000, top_k=512, n_local=128, n_planted=16)
    gh.log("[attn on oracle TopK]")
    batch = wl.make_batch(geo, device=DEV)
    r = batch.requests[0]
    q, K, V = gh.np32(r.q), gh.np32(r.k), gh.np32(r.v)
    T = ora.select(q, K, geo.top_k)["T"]
    sel_idx = torch.tensor(T, dtype=torch.int32, device=DEV)[None]
    sel_count = torch.tensor([len(T)], dtype=torch.int32, device=DEV)
    po = gh.run_path(batch, geo, sel_override=(sel_idx, sel_count))
    ref = ora.sparse_attention(q, K, V, ora.union_local(T, 6000, geo.n_local), geo.attn_scale)
    assert np.max(np.abs(po.out[0] - ref)) <= 2e-2


@pytest.mark.parametrize("dtype,H,Hkv", [("bf16", 32, 8), ("f32", 32, 8), ("bf16", 28, 4)])
def test_attention_over_every_position(dtype, H, Hkv):
    # k = N selects everything: step 5 is then dense attention over the whole cache
    # (the dense reference the benchmark times at 1M), here at 40000 positions: 313
    # selection slices of 128 and the window overlapping the selection, so the
    # partials go through both merge launches
    n = 40000
    geo = wl.workload("llama3-8b-128k", seq_len=n, top_k=n, n_local=512, n_planted=4, dtype=dtype,
                      num_q_heads=H, num_kv_heads=Hkv)
    gh.log(f"[attn over all {n} positions, {dtype}, G = {H // Hkv}]")
    batch = wl.make_batch(geo, device=DEV)
    r = batch.requests[0]
    q, K, V = gh.np32(r.q), gh.np32(r.k), gh.np32(r.v)
    sel_idx = torch.arange(n, dtype=torch.int32, device=DEV)[None]
    sel_count = torch.tensor([n], dtype=torch.int32, device=DEV)
    po = gh.run_path(batch, geo, sel_override=(sel_idx, sel_count))
    gh.check_attention(po.out[0], q, K, V, np.arange(n), n, geo.n_local, geo.attn_scale, dtype == "f32")


# ------------------------------------------------------------------ head groupings and batch limits
@pytest.mark.parametrize("H,Hkv,dtype", [(8, 8, "bf16"), (16, 8, "f32"), (12, 4, "bf16"), (40, 8, "bf16"),
                                         (48, 8, "f32"), (64, 8, "bf16")])
def test_every_group_size(H, Hkv, dtype):
    # G = 1, 2, 3, 5, 6, 8 (4 and 7 are covered above): every score, vote and
    # attention instantiation
    geo = wl.workload("llama3-8b-128k", num_q_heads=H, num_kv_heads=Hkv, dtype=dtype, seq_len=3000,
                      top_k=96, n_local=40, n_planted=8, seed=7100 + H)
    gh.log(f"[group {H // Hkv}] H={H} H_kv={Hkv} {dtype}")
    _check_all(wl.make_batch(geo, device=DEV), geo)


def test_max_batch_of_1024_requests():
    # the LDS prefix tables of every kernel hold up to 1024 requests
    geo = wl.workload("llama3-8b-ragged16", batch=1024, min_len=40, max_len=400, top_k=24, n_local=8,
                      n_planted=4, seed=7300)
    gh.log("[batch 1024] N_r in [40, 400]")
    batch = wl.make_batch(geo, device=DEV)
    po = gh.run_path(batch, geo)
    rng = np.random.default_rng(0)
    for r in sorted(set(rng.integers(0, 1024, 12).tolist()) | {0, 1023}):
        gh.check_request(po, r, batch.requests[r], geo)


def test_score_without_statistics_gives_the_same_logits():
    """tokenselect_score with head_stats NULL runs only the scoring kernel: the logits
    equal, bit for bit, those of the full launch (which also folds the statistics)."""
    geo = wl.workload("llama3-8b-128k", seq_len=20000)
    gh.log("[score] head_stats NULL vs full launch, N=20000")
    batch = wl.make_batch(geo, device=DEV)
    H, total = geo.num_q_heads, batch.total_tokens
    shape = ts.make_shape(H, geo.num_kv_heads, 1, batch.block_table.shape[1], total, geo.torch_dtype)
    sel = gh.select_params(geo)
    ws = ts.alloc_workspace(shape, sel, DEV)
    a = torch.full((H * total,), float("nan"), dtype=torch.float32, device=DEV)
    b = torch.full((H * total,), float("nan"), dtype=torch.float32, device=DEV)
    stats = torch.full((H * 2,), float("nan"), dtype=torch.float32, device=DEV)
    ts.score(shape, sel, batch.q, batch.k_pool, batch.block_table, batch.seq_lens, a, stats, ws)
    ts.score(shape, sel, batch.q, batch.k_pool, batch.block_table, batch.seq_lens, b, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.isfinite(stats).all()
