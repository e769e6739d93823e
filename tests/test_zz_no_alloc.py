"""tokenselect_decode_step_noalloc against tokenselect_decode_step (same kernels, the
library's static scratch instead of a caller workspace).

Two calls in a row on the static scratch, the second with a smaller input, each
compared bit for bit with the workspace entry point on the same inputs (hit flags,
cached TopK and count, attention output), plus the Selection Cache's second step
(a hit) on the same scratch; a shape beyond the scratch is rejected before any
launch.
"""
import numpy as np
import pytest
import torch

import token_level_sparse_amd as ts
from synth import workloads as wl
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(geo, lens, seed, noalloc, steps=2):
    gen = torch.Generator(device=DEV).manual_seed(seed)
    reqs = [wl.make_request(gen, geo, n, DEV) for n in lens]
    batch = wl.page_requests(reqs, geo, gen, DEV)
    H, d, b = geo.num_q_heads, geo.head_dim, len(reqs)
    shape = ts.make_shape(H, geo.num_kv_heads, b, batch.block_table.shape[1], sum(lens),
                          geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, 0.9)
    cache = ts.CacheState.allocate(b, H, d, geo.top_k, geo.torch_dtype, DEV)
    hit = torch.full((b,), -7, dtype=torch.int32, device=DEV)
    ws = None if noalloc else ts.alloc_workspace(shape, sel, DEV)
    if noalloc:
        assert ts.workspace_size(shape, sel) <= ts.NOALLOC_SCRATCH_BYTES
    res = []
    for _ in range(steps):           # a miss, then a hit with the same query
        out = torch.full((b, H, d), float("nan"), dtype=geo.torch_dtype, device=DEV)
        if noalloc:
            ts.decode_step_noalloc(shape, sel, batch.q, batch.k_pool, batch.v_pool, batch.block_table,
                                   batch.seq_lens, cache, hit, out)
        else:
            ts.decode_step(shape, sel, batch.q, batch.k_pool, batch.v_pool, batch.block_table,
                           batch.seq_lens, cache, hit, out, ws)
        torch.cuda.synchronize()
        res.append((hit.cpu().numpy().copy(), cache.cached_idx.cpu().numpy().copy(),
                    cache.cached_count.cpu().numpy().copy(), gh.np32(out)))
    return res


def _same(a, b):
    for (h1, i1, c1, o1), (h2, i2, c2, o2) in zip(a, b):
        assert np.array_equal(h1, h2)
        assert np.array_equal(c1, c2)
        for r in range(len(c1)):
            assert np.array_equal(i1[r, : c1[r]], i2[r, : c2[r]])
        assert np.array_equal(o1, o2)


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    geo = wl.workload("llama3-8b-128k", top_k=2048, n_local=512, n_planted=16)
    gh.log("[noalloc] 128K request, then a smaller ragged batch")
    big = _run(geo, [131072], 901, noalloc=True)
    _same(big, _run(geo, [131072], 901, noalloc=False))
    assert big[0][0].tolist() == [0] and big[1][0].tolist() == [1]
    small = _run(geo, [5000, 300, 9000], 902, noalloc=True)
    _same(small, _run(geo, [5000, 300, 9000], 902, noalloc=False))
    assert small[0][0].tolist() == [0, 0, 0] and small[1][0].tolist() == [1, 1, 1]


def test_noalloc_rejects_shapes_beyond_the_scratch():
    geo = wl.workload("llama3-8b-1m")
    shape = ts.make_shape(geo.num_q_heads, geo.num_kv_heads, 1, 65536, 1 << 20, geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, 0.9)
    assert ts.workspace_size(shape, sel) > ts.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(16, dtype=torch.int32, device=DEV)
    cache = ts.CacheState.allocate(1, geo.num_q_heads, geo.head_dim, geo.top_k, geo.torch_dtype, DEV)
    with pytest.raises(ts.TokenSelectError) as e:
        ts.decode_step_noalloc(shape, sel, t, t, t, t, t, cache, t, t)
    assert e.value.status == ts.TS_ERR_WORKSPACE
    assert "static scratch" in str(e.value)
