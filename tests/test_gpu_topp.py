"""GPU parity of the dynamic top-p budget (ts_select.top_p) against the oracle.

The budget is an integer decision taken from float votes, so it is checked twice:
  * in the GPU's own precision: with q_i = rint(2^(lv_i + 40)) from the GPU's log2
    votes and target = ceil(p * sum q), sel_count must be the smallest m whose m
    largest votes (ties to the lower position) reach the target, capped at
    min(k, N) (each q_i allowed +-1 for the last bit of exp2), and the set must be
    exactly the top m of the GPU's votes;
  * against the fp64 oracle: the set must hold at least p of the oracle's vote mass
    and lose that property when its smallest member is dropped, both up to a
    relative 1e-4 (far above the vote band of the fp32 path at these sizes).
"""
import numpy as np
import pytest
import torch

import token_level_sparse_amd as ts
from oracle import tokenselect_oracle as ora
from synth import workloads as wl
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ts.load_library()


def _run(batch, geo, top_p, top_k=None):
    b = batch.q.shape[0]
    H = geo.num_q_heads
    k = geo.top_k if top_k is None else top_k
    total = batch.total_tokens
    shape = ts.make_shape(H, geo.num_kv_heads, b, batch.block_table.shape[1], total, geo.torch_dtype)
    sel = ts.make_select(k, geo.n_local, 1.0, geo.attn_scale, geo.cos_threshold, top_p)
    ws = ts.alloc_workspace(shape, sel, DEV)
    logits = torch.empty(H * total, dtype=torch.float32, device=DEV)
    stats = torch.empty(b * H * 2, dtype=torch.float32, device=DEV)
    vote = torch.empty(total, dtype=torch.float32, device=DEV)
    si = torch.full((b, k), -7, dtype=torch.int32, device=DEV)
    sc = torch.full((b,), -7, dtype=torch.int32, device=DEV)
    ts.score(shape, sel, batch.q, batch.k_pool, batch.block_table, batch.seq_lens, logits, stats, ws)
    ts.vote_topk(shape, sel, logits, stats, batch.seq_lens, vote, si, sc, ws)
    torch.cuda.synchronize()
    return vote.cpu().numpy(), si.cpu().numpy(), sc.cpu().numpy()


def _check_request(lv, T, m, p, k, v_ora=None):
    N = len(lv)
    cap = min(k, N)
    assert 1 <= m <= cap
    assert np.all(np.diff(T) > 0)
    # exactly the top m of the GPU's own votes
    assert np.array_equal(T, ora.topk_indices(lv.astype(np.float64), m))
    # the integer budget recomputed from the GPU votes
    q = np.rint(np.exp2(lv.astype(np.float64) + 40.0))
    order = np.lexsort((np.arange(N), -lv.astype(np.float64)))
    qs = q[order]
    lo, hi = np.cumsum(np.maximum(qs - 1, 0)), np.cumsum(qs + 1)
    tgt_lo = np.ceil(p * lo[-1])
    tgt_hi = np.ceil(p * hi[-1])
    if m < cap:
        assert hi[m - 1] >= tgt_lo, "budget too small for the GPU votes"
    if m > 1:
        assert lo[m - 2] < tgt_hi, "budget larger than needed for the GPU votes"
    if v_ora is not None:
        tot = v_ora.sum()
        mass = v_ora[T].sum()
        if m < cap:
            assert mass >= p * tot * (1 - REL), (mass / tot, p)
        if m > 1:
            smallest = v_ora[T].min()
            assert mass - smallest < p * tot * (1 + REL), ((mass - smallest) / tot, p)
        m_ora = ora.topp_count(v_ora, p, k)
        return m_ora
    return None


@pytest.mark.parametrize("p", [0.5, 0.9, 0.99])
def test_topp_reduced_llama3(p):
    geo = wl.workload("llama3-8b-128k", seq_len=32768)
    gh.log(f"[top-p p={p}] N=32768 k=2048")
    batch = wl.make_batch(geo, device=DEV)
    lv, si, sc = _run(batch, geo, p)
    r = batch.requests[0]
    sel = ora.select(gh.np32(r.q), gh.np32(r.k), geo.top_k)
    m = int(sc[0])
    m_ora = _check_request(lv, si[0, :m].astype(np.int64), m, p, geo.top_k, sel["vote"])
    gh.log(f"  budget {m} (oracle {m_ora})")


def test_topp_peaked_votes_need_few_tokens():
    # no scale spread: every head's softmax mass sits on its planted keys
    geo = wl.workload("llama3-8b-128k", seq_len=32768, n_planted=16)
    gh.log("[top-p peaked] N=32768, 16 planted per KV head, p=0.9")
    batch = wl.make_batch(geo, device=DEV, scale_spread=False)
    lv, si, sc = _run(batch, geo, 0.9)
    m = int(sc[0])
    r = batch.requests[0]
    sel = ora.select(gh.np32(r.q), gh.np32(r.k), geo.top_k)
    _check_request(lv, si[0, :m].astype(np.int64), m, 0.9, geo.top_k, sel["vote"])
    planted = np.unique(r.planted_pos.cpu().numpy())
    gh.log(f"  budget {m} for {len(planted)} planted tokens")
    assert m <= 2 * len(planted)


def test_topp_tiny_f32_and_full_mass():
    geo = wl.workload("tiny-f32-8k")
    batch = wl.make_batch(geo, device=DEV)
    r = batch.requests[0]
    sel = ora.select(gh.np32(r.q), gh.np32(r.k), geo.top_k)
    for p in (0.3, 0.95, 1.0):
        lv, si, sc = _run(batch, geo, p, top_k=4096)
        m = int(sc[0])
        _check_request(lv, si[0, :m].astype(np.int64), m, p, 4096, sel["vote"])
        gh.log(f"[top-p tiny f32 p={p}] budget {m}")


def test_topp_ragged_batch_and_small_requests():
    # requests with N <= k still take the top-p budget (it can stop before N)
    geo = wl.workload("llama3-8b-ragged16", batch=5, min_len=600, max_len=40000, seed=3100)
    gh.log("[top-p ragged] 5 requests")
    batch = wl.make_batch(geo, device=DEV)
    lv, si, sc = _run(batch, geo, 0.8)
    offs = batch.token_offsets.cpu().tolist()
    for r in range(5):
        N = int(batch.seq_lens[r])
        m = int(sc[r])
        req = batch.requests[r]
        sel = ora.select(gh.np32(req.q), gh.np32(req.k), geo.top_k)
        _check_request(lv[offs[r]: offs[r] + N], si[r, :m].astype(np.int64), m, 0.8, geo.top_k,
                       sel["vote"])
        gh.log(f"  request {r}: N={N} budget {m}")


def test_topp_is_deterministic():
    geo = wl.workload("llama3-8b-128k", seq_len=65536)
    batch = wl.make_batch(geo, device=DEV)
    a = _run(batch, geo, 0.9)
    b = _run(batch, geo, 0.9)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])


def test_topp_decode_step_with_cache():
    # the decode step carries the budget into the cache: a hit reuses C_T and its count
    geo = wl.workload("qwen2-7b-cache256", seq_len=16384, steps=24)
    gh.log("[top-p decode sequence] 24 steps, p=0.9")
    gen = torch.Generator(device=DEV).manual_seed(geo.seed)
    req = wl.make_request(gen, geo, geo.seq_len, DEV, extra_tokens=geo.steps - 1)
    batch = wl.page_requests([req], geo, gen, DEV)
    qs, _ = wl.ar1_queries(geo, req.q_master, geo.steps, seed=geo.seed + 1, device=DEV)
    H, d = geo.num_q_heads, geo.head_dim
    shape = ts.make_shape(H, geo.num_kv_heads, 1, batch.block_table.shape[1], geo.seq_len + geo.steps,
                          geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, geo.cos_threshold, 0.9)
    ws = ts.alloc_workspace(shape, sel, DEV)
    cache = ts.CacheState.allocate(1, H, d, geo.top_k, geo.torch_dtype, DEV)
    hit = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.empty(1, H, d, dtype=geo.torch_dtype, device=DEV)
    last_T = None
    for t in range(geo.steps):
        N = geo.seq_len + t
        lens = torch.tensor([N], dtype=torch.int32, device=DEV)
        q = qs[t:t + 1].contiguous()
        ts.decode_step(shape, sel, q, batch.k_pool, batch.v_pool, batch.block_table, lens, cache, hit, out, ws)
        torch.cuda.synchronize()
        m = int(cache.cached_count[0])
        T = cache.cached_idx[0, :m].cpu().numpy().astype(np.int64)
        if int(hit[0]):
            assert np.array_equal(T, last_T)
        else:
            # a miss reselects with the top-p budget over the current N
            Kt = gh.np32(req.k[:, :N])
            s = ora.select(gh.np32(q[0]), Kt, geo.top_k)
            assert 1 <= m <= geo.top_k
            tot = s["vote"].sum()
            assert s["vote"][T].sum() >= 0.9 * tot * (1 - REL)
        last_T = T
        # attention over the cached selection and the window
        S = ora.union_local(T, N, geo.n_local)
        ref = ora.sparse_attention(gh.np32(q[0]), gh.np32(req.k[:, :N]), gh.np32(req.v[:, :N]), S,
                                   geo.attn_scale)
        assert np.abs(gh.np32(out[0]) - ref).max() <= 2e-2
