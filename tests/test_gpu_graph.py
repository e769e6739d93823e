"""The decode step under HIP graph capture: tokenselect_decode_step makes no host
synchronisation and allocates nothing, so a step can be captured once and replayed.
The graph is replayed over a query sequence (each replay after a host copy of the
next query into the captured input buffer, with eager work and synchronisation in
between), and every replay must equal, bit for bit, the same step run eagerly:
hit flag, cached TopK and count, and the attention output. The Selection Cache
state lives in device buffers, so it evolves across replays as it does eagerly.
"""
import numpy as np
import pytest
import torch

import token_level_sparse_amd as ts
from synth import workloads as wl
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ts.load_library()


def _state(cache, hit, out):
    return (hit.clone(), cache.cached_idx.clone(), cache.cached_count.clone(), cache.valid.clone(),
            out.clone())


def test_decode_step_graph_replay_matches_eager():
    geo = wl.workload("qwen2-7b-cache256", seq_len=20000, steps=8)
    gh.log("[graph] qwen2 shapes, N = 20000, 8 steps, theta = 0.9")
    gen = torch.Generator(device=DEV).manual_seed(geo.seed)
    req = wl.make_request(gen, geo, geo.seq_len, DEV)
    batch = wl.page_requests([req], geo, gen, DEV)
    qs, _ = wl.ar1_queries(geo, req.q_master, geo.steps, seed=geo.seed + 1, device=DEV)
    H, d = geo.num_q_heads, geo.head_dim
    shape = ts.make_shape(H, geo.num_kv_heads, 1, batch.block_table.shape[1], geo.seq_len, geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, geo.cos_threshold)
    lens = torch.tensor([geo.seq_len], dtype=torch.int32, device=DEV)

    def buffers():
        ws = ts.alloc_workspace(shape, sel, DEV)
        cache = ts.CacheState.allocate(1, H, d, geo.top_k, geo.torch_dtype, DEV)
        hit = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        out = torch.zeros(1, H, d, dtype=geo.torch_dtype, device=DEV)
        q = torch.empty(1, H, d, dtype=geo.torch_dtype, device=DEV)
        return ws, cache, hit, out, q

    # eager reference
    ws, cache, hit, out, q = buffers()
    eager = []
    for t in range(geo.steps):
        q.copy_(qs[t:t + 1])
        ts.decode_step(shape, sel, q, batch.k_pool, batch.v_pool, batch.block_table, lens, cache, hit, out, ws)
        torch.cuda.synchronize()
        eager.append(_state(cache, hit, out))
    hits = [int(e[0][0]) for e in eager]
    gh.log(f"  eager hits {hits}")
    assert hits[0] == 0 and 1 in hits, "the sequence should start with a miss and reuse the cache"

    # capture one step on fresh buffers, then replay it step by step
    ws, cache, hit, out, q = buffers()
    q.copy_(qs[0:1])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ts.decode_step(shape, sel, q, batch.k_pool, batch.v_pool, batch.block_table, lens, cache, hit, out, ws)
    torch.cuda.synchronize()
    # capture does not execute: the state is still the fresh one
    assert int(cache.valid[0]) == 0
    scratch = torch.empty(1 << 20, device=DEV)
    for t in range(geo.steps):
        q.copy_(qs[t:t + 1])
        g.replay()
        torch.cuda.synchronize()
        got = _state(cache, hit, out)
        for a, b, name in zip(got, eager[t], ("hit", "cached_idx", "cached_count", "valid", "out")):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), (t, name)
        # unrelated eager work between replays
        scratch.normal_()
        float(scratch.sum())
