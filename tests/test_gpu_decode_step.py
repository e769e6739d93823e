"""GPU parity of tokenselect_decode_step (Selection Cache + steps 1-5) against the oracle."""
import numpy as np
import pytest
import torch

import token_level_sparse_amd as ts
from tests import gpu_helpers as gh
from synth import workloads as wl
from oracle import tokenselect_oracle as ora

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_sequence(geo, N0, steps, theta, qs=None, reset_at=()):
    """Decode `steps` consecutive steps; token N0 + t - 1 is the newest at step t."""
    gen = torch.Generator(device=DEV).manual_seed(geo.seed)
    req = wl.make_request(gen, geo, N0, DEV, extra_tokens=steps - 1)
    batch = wl.page_requests([req], geo, gen, DEV)
    if qs is None:
        qs, _ = wl.ar1_queries(geo, req.q_master, steps, seed=geo.seed + 1, device=DEV)
    H, d = geo.num_q_heads, geo.head_dim
    shape = ts.make_shape(H, geo.num_kv_heads, 1, batch.block_table.shape[1], N0 + steps - 1,
                          geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, theta)
    ws = ts.alloc_workspace(shape, sel, DEV)
    cache = ts.CacheState.allocate(1, H, d, geo.top_k, geo.torch_dtype, DEV)
    hit = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.empty(1, H, d, dtype=geo.torch_dtype, device=DEV)
    lens = torch.arange(N0, N0 + steps, dtype=torch.int32, device=DEV)
    hits, Ts, outs = [], [], []
    for t in range(steps):
        if t in reset_at:
            cache.valid.zero_()
        ts.decode_step(shape, sel, qs[t:t + 1].contiguous(), batch.k_pool, batch.v_pool,
                       batch.block_table, lens[t:t + 1], cache, hit, out, ws)
        hits.append(hit.clone())
        Ts.append(cache.cached_idx[0, :].clone())
        outs.append(out.clone())
        Ts[-1] = (Ts[-1], cache.cached_count.clone())
    torch.cuda.synchronize()
    hits = np.array([int(h.item()) for h in hits], dtype=bool)
    T = [ti[: int(c.item())].cpu().numpy().astype(np.int64) for ti, c in Ts]
    outs = np.stack([gh.np32(o[0]) for o in outs])
    return req, qs, lens.cpu().numpy(), hits, T, outs


def compare(geo, req, qs, lens, hits, T, outs, theta, band_steps=24):
    q_all = gh.np32(qs)
    K, V = gh.np32(req.k), gh.np32(req.v)
    ref = ora.decode_sequence(q_all, K, V, lens, geo.top_k, geo.n_local, theta, want_outputs=False)
    c = ref["cos"]
    margin = np.abs(c[~np.isnan(c)] - theta)
    gh.log(f"  hits gpu={hits.sum()}/{len(hits)} min|cos-theta|={margin.min() if len(margin) else float('nan'):.3e}")
    assert margin.size == 0 or margin.min() > 1e-9
    assert np.array_equal(hits, ref["hit"]), f"hit vectors differ at {np.nonzero(hits != ref['hit'])[0][:10]}"
    checked = 0
    last_miss_T = None
    for t in range(len(hits)):
        N = int(lens[t])
        if not hits[t]:
            last_miss_T = T[t]
            if checked < band_steps:
                sel = ora.select(q_all[t], K[:, :N], geo.top_k)
                rel = gh.tol.vote_rel_budget(q_all[t], K[:, :N], sel["z"], sel["p"], sel["M"],
                                             sel["vote"])
                amb = gh.tol.ambiguous_positions_log(sel["vote"], rel, geo.top_k)
                diff = np.setxor1d(T[t], sel["T"])
                assert np.all(amb[diff]), (t, diff[~amb[diff]][:10])
                checked += 1
        else:
            assert np.array_equal(T[t], last_miss_T), f"step {t}: a hit must reuse the last miss's TopK"
        gh.check_attention(outs[t], q_all[t], K[:, :N], V[:, :N], T[t], N, geo.n_local,
                           geo.attn_scale, geo.dtype == "f32")


def test_decode_sequence_reduced():
    geo = wl.workload("qwen2-7b-cache256", top_k=256, n_local=64, n_planted=16)
    gh.log("[qwen2 decode N0=4096 48 steps k=256]")
    res = run_sequence(geo, 4096, 48, 0.9)
    compare(geo, *res, theta=0.9)


def test_decode_sequence_full_256_steps():
    geo = wl.workload("qwen2-7b-cache256")
    gh.log(f"[qwen2-7b-cache256] N0={geo.seq_len} {geo.steps} steps")
    res = run_sequence(geo, geo.seq_len, geo.steps, geo.cos_threshold)
    compare(geo, *res, theta=geo.cos_threshold)


def test_cache_identical_queries_and_thresholds():
    geo = wl.workload("llama3-8b-128k", seq_len=3000, top_k=128, n_local=16, n_planted=4)
    gh.log("[cache] identical queries / theta extremes / reset")
    gen = torch.Generator(device=DEV).manual_seed(3)
    q0 = torch.randn(1, geo.num_q_heads, geo.head_dim, generator=gen, device=DEV).to(torch.bfloat16)
    same = q0.repeat(6, 1, 1)
    _, _, _, hits, T, _ = run_sequence(geo, 3000, 6, 0.9, qs=same)
    assert hits.tolist() == [False] + [True] * 5
    _, _, _, hits, _, _ = run_sequence(geo, 3000, 6, 1.5, qs=same)
    assert hits.tolist() == [False] * 6
    other = torch.randn(6, geo.num_q_heads, geo.head_dim, generator=gen, device=DEV).to(torch.bfloat16)
    _, _, _, hits, T, _ = run_sequence(geo, 3000, 6, -1.0, qs=other)
    assert hits.tolist() == [False] + [True] * 5
    assert all(np.array_equal(T[i], T[0]) for i in range(6))
    _, _, _, hits, _, _ = run_sequence(geo, 3000, 6, 0.9, qs=same, reset_at=(3,))
    assert hits.tolist() == [False, True, True, False, True, True]


def test_zero_query_misses():
    geo = wl.workload("llama3-8b-128k", seq_len=500, top_k=64, n_local=8, n_planted=4)
    gh.log("[cache] zero query")
    q = torch.zeros(3, geo.num_q_heads, geo.head_dim, dtype=torch.bfloat16, device=DEV)
    _, _, _, hits, _, _ = run_sequence(geo, 500, 3, -1.0, qs=q)
    assert hits.tolist() == [False, False, False]


def test_ragged_batch_mixed_hits():
    """Four requests of different lengths decoded together: requests 0 and 2 repeat
    their query (hits after the first step), 1 and 3 draw a new one every step
    (misses), so every kernel sees skipped and active requests in one launch."""
    geo = wl.workload("llama3-8b-128k", top_k=300, n_local=40, n_planted=8)
    gh.log("[decode ragged b=4 mixed hits]")
    steps, lens0 = 5, [3000, 5000, 2000, 7001]
    gen = torch.Generator(device=DEV).manual_seed(11)
    reqs = [wl.make_request(gen, geo, n, DEV, extra_tokens=steps - 1) for n in lens0]
    batch = wl.page_requests(reqs, geo, gen, DEV)
    H, d, b = geo.num_q_heads, geo.head_dim, len(reqs)
    qs = torch.randn(steps, b, H, d, generator=gen, device=DEV).to(torch.bfloat16)
    qs[:, 0] = qs[0, 0]
    qs[:, 2] = qs[0, 2]
    shape = ts.make_shape(H, geo.num_kv_heads, b, batch.block_table.shape[1],
                          sum(lens0) + b * (steps - 1), geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, 0.9)
    ws = ts.alloc_workspace(shape, sel, DEV)
    cache = ts.CacheState.allocate(b, H, d, geo.top_k, geo.torch_dtype, DEV)
    hit = torch.zeros(b, dtype=torch.int32, device=DEV)
    out = torch.empty(b, H, d, dtype=geo.torch_dtype, device=DEV)
    hits, Ts, outs = [], [], []
    for t in range(steps):
        lens = torch.tensor([n + t for n in lens0], dtype=torch.int32, device=DEV)
        ts.decode_step(shape, sel, qs[t].contiguous(), batch.k_pool, batch.v_pool,
                       batch.block_table, lens, cache, hit, out, ws)
        torch.cuda.synchronize()
        hits.append(hit.cpu().numpy().astype(bool))
        cnt = cache.cached_count.cpu().numpy()
        idx = cache.cached_idx.cpu().numpy()
        Ts.append([idx[r, :cnt[r]].astype(np.int64) for r in range(b)])
        outs.append(gh.np32(out))
    hits = np.array(hits)                              # [steps][b]
    assert hits[:, 0].tolist() == [False] + [True] * (steps - 1)
    assert hits[:, 2].tolist() == [False] + [True] * (steps - 1)
    assert not hits[:, 1].any() and not hits[:, 3].any()
    for r in range(b):
        q_all = gh.np32(qs[:, r])
        K, V = gh.np32(reqs[r].k), gh.np32(reqs[r].v)
        lens_r = np.array([lens0[r] + t for t in range(steps)])
        ref = ora.decode_sequence(q_all, K, V, lens_r, geo.top_k, geo.n_local, 0.9, want_outputs=False)
        assert np.array_equal(hits[:, r], ref["hit"])
        for t in range(steps):
            N = int(lens_r[t])
            if not hits[t, r]:
                s = ora.select(q_all[t], K[:, :N], geo.top_k)
                rel = gh.tol.vote_rel_budget(q_all[t], K[:, :N], s["z"], s["p"], s["M"], s["vote"])
                amb = gh.tol.ambiguous_positions_log(s["vote"], rel, geo.top_k)
                diff = np.setxor1d(Ts[t][r], s["T"])
                assert np.all(amb[diff]), (r, t)
            else:
                assert np.array_equal(Ts[t][r], Ts[t - 1][r])
            gh.check_attention(outs[t][r], q_all[t], K[:, :N], V[:, :N], Ts[t][r], N, geo.n_local,
                               geo.attn_scale, False)


def test_requests_sharing_score_blocks_and_an_empty_request():
    """H_kv = 3 with one-chunk requests: the score kernel's 4-unit blocks straddle
    requests, so a workgroup decides several requests' cache tests in one block.
    Request 1 has N = 0 (no tokens): it still gets a decision, an empty TopK and a
    zero output. Requests 0, 1 and 4 repeat their query (hits after step 0); the
    others draw a new one every step."""
    geo = wl.workload("llama3-8b-128k", num_q_heads=6, num_kv_heads=3, top_k=40, n_local=8,
                      n_planted=2)
    gh.log("[decode H_kv=3 shared score blocks, empty request]")
    steps, lens0 = 4, [100, 50, 37, 2000, 16, 1, 700]
    gen = torch.Generator(device=DEV).manual_seed(12)
    reqs = [wl.make_request(gen, geo, n, DEV, extra_tokens=steps - 1) for n in lens0]
    batch = wl.page_requests(reqs, geo, gen, DEV)
    H, d, b = geo.num_q_heads, geo.head_dim, len(reqs)
    qs = torch.randn(steps, b, H, d, generator=gen, device=DEV).to(torch.bfloat16)
    for r in (0, 1, 4):
        qs[:, r] = qs[0, r]
    lens_all = np.array([[0 if r == 1 else lens0[r] + t for r in range(b)] for t in range(steps)])
    shape = ts.make_shape(H, geo.num_kv_heads, b, batch.block_table.shape[1],
                          sum(lens0) + b * (steps - 1), geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, 0.9)
    ws = ts.alloc_workspace(shape, sel, DEV)
    cache = ts.CacheState.allocate(b, H, d, geo.top_k, geo.torch_dtype, DEV)
    hit = torch.full((b,), -7, dtype=torch.int32, device=DEV)
    out = torch.full((b, H, d), float("nan"), dtype=geo.torch_dtype, device=DEV)
    hits, Ts, outs = [], [], []
    for t in range(steps):
        lens = torch.from_numpy(lens_all[t].astype(np.int32)).to(DEV)
        ts.decode_step(shape, sel, qs[t].contiguous(), batch.k_pool, batch.v_pool,
                       batch.block_table, lens, cache, hit, out, ws)
        torch.cuda.synchronize()
        hits.append(hit.cpu().numpy().copy())
        cnt = cache.cached_count.cpu().numpy()
        idx = cache.cached_idx.cpu().numpy()
        Ts.append([idx[r, :cnt[r]].astype(np.int64) for r in range(b)])
        outs.append(gh.np32(out))
    hits = np.array(hits)                              # [steps][b]
    assert set(np.unique(hits)) <= {0, 1}
    hits = hits.astype(bool)
    for r in (0, 1, 4):
        assert hits[:, r].tolist() == [False] + [True] * (steps - 1), (r, hits[:, r])
    for r in (2, 3, 5, 6):
        assert not hits[:, r].any(), (r, hits[:, r])
    for t in range(steps):
        assert Ts[t][1].size == 0
        assert np.all(outs[t][1] == 0.0)
    for r in (0, 2, 3, 4, 5, 6):
        q_all = gh.np32(qs[:, r])
        K, V = gh.np32(reqs[r].k), gh.np32(reqs[r].v)
        ref = ora.decode_sequence(q_all, K, V, lens_all[:, r], geo.top_k, geo.n_local, 0.9,
                                  want_outputs=False)
        assert np.array_equal(hits[:, r], ref["hit"])
        for t in range(steps):
            N = int(lens_all[t, r])
            if not hits[t, r]:
                s = ora.select(q_all[t], K[:, :N], geo.top_k)
                rel = gh.tol.vote_rel_budget(q_all[t], K[:, :N], s["z"], s["p"], s["M"], s["vote"])
                amb = gh.tol.ambiguous_positions_log(s["vote"], rel, geo.top_k)
                diff = np.setxor1d(Ts[t][r], s["T"])
                assert np.all(amb[diff]), (r, t)
            else:
                assert np.array_equal(Ts[t][r], Ts[t - 1][r])
            gh.check_attention(outs[t][r], q_all[t], K[:, :N], V[:, :N], Ts[t][r], N, geo.n_local,
                               geo.attn_scale, False)


def test_empty_request_with_invalid_block_table_row():
    """A request with N_r = 0 reaches no page, so its block-table row may hold
    anything: here every entry is -1 and its TopK row holds stale, negative and
    out-of-range positions. Its output is zero, and the other requests' outputs are
    bit-identical to a run where the empty request's row holds valid pages."""
    geo = wl.workload("llama3-8b-128k", top_k=64, n_local=16, n_planted=2)
    gh.log("[empty request, block-table row of -1]")
    gen = torch.Generator(device=DEV).manual_seed(31)
    lens0 = [300, 40, 1000]
    reqs = [wl.make_request(gen, geo, n, DEV) for n in lens0]
    batch = wl.page_requests(reqs, geo, gen, DEV)
    H, d, b = geo.num_q_heads, geo.head_dim, len(reqs)
    lens = torch.tensor([300, 0, 1000], dtype=torch.int32, device=DEV)
    shape = ts.make_shape(H, geo.num_kv_heads, b, batch.block_table.shape[1], sum(lens0),
                          geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, 0.9)
    ws = ts.alloc_workspace(shape, sel, DEV)
    outs = {}
    for name in ("valid_row", "row_of_minus_one"):
        bt = batch.block_table.clone()
        if name == "row_of_minus_one":
            bt[1] = -1
        report = ts.validate(shape, bt, lens, batch.k_pool.shape[0])
        torch.cuda.synchronize()
        assert report.cpu().tolist()[0] == 0, (name, report.cpu().tolist())
        cache = ts.CacheState.allocate(b, H, d, geo.top_k, geo.torch_dtype, DEV)
        cache.cached_idx[1] = torch.tensor([5, -3, 10 ** 6] * 21 + [7], dtype=torch.int32, device=DEV)
        hit = torch.zeros(b, dtype=torch.int32, device=DEV)
        res = []
        for step in range(2):                   # a miss, then a hit with the same query
            out = torch.full((b, H, d), float("nan"), dtype=geo.torch_dtype, device=DEV)
            ts.decode_step(shape, sel, batch.q, batch.k_pool, batch.v_pool, bt, lens, cache, hit,
                           out, ws)
            torch.cuda.synchronize()
            assert hit.cpu().tolist() == [step, step, step], (name, step, hit.cpu().tolist())
            assert int(cache.cached_count[1]) == 0
            res.append(gh.np32(out))
        # step 5 alone with a stale TopK row and count for the empty request
        sel_idx = cache.cached_idx.clone()
        sel_idx[1] = torch.tensor([5, -3, 10 ** 6] * 21 + [7], dtype=torch.int32, device=DEV)
        sel_count = cache.cached_count.clone()
        sel_count[1] = geo.top_k
        out = torch.full((b, H, d), float("nan"), dtype=geo.torch_dtype, device=DEV)
        ts.sparse_attn(shape, sel, batch.q, batch.k_pool, batch.v_pool, bt, lens, sel_idx, sel_count,
                       out, ws)
        torch.cuda.synchronize()
        res.append(gh.np32(out))
        for o in res:
            assert np.all(o[1] == 0.0), name
        outs[name] = res
    for a, c in zip(outs["valid_row"], outs["row_of_minus_one"]):
        assert np.array_equal(a[[0, 2]], c[[0, 2]])
    # the non-empty requests against the oracle (window and TopK of the miss step)
    for r in (0, 2):
        N = int(lens[r])
        q, K, V = gh.np32(reqs[r].q), gh.np32(reqs[r].k)[:, :N], gh.np32(reqs[r].v)[:, :N]
        T = ora.select(q, K, geo.top_k)["T"]
        ref = ora.sparse_attention(q, K, V, ora.union_local(T, N, geo.n_local), geo.attn_scale)
        assert np.max(np.abs(outs["valid_row"][0][r] - ref)) <= 2e-2
