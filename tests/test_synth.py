"""Generator checks: reproducibility, planted structure, scale range, paging layout."""
import math

import numpy as np
import torch

from synth import workloads as wl


def test_same_seed_same_tensors():
    geo = wl.workload("tiny-f32-8k", seq_len=1000)
    a = wl.make_batch(geo)
    b = wl.make_batch(geo)
    for x, y in ((a.q, b.q), (a.k_pool, b.k_pool), (a.v_pool, b.v_pool),
                 (a.block_table, b.block_table)):
        assert torch.equal(torch.nan_to_num(x.float(), 7.0), torch.nan_to_num(y.float(), 7.0))
    c = wl.make_batch(geo, layer=1)
    assert not torch.equal(a.q, c.q)


def test_planted_positions_distinct_and_targets_follow_groups():
    geo = wl.workload("llama3-8b-128k", seq_len=4096)
    r = wl.make_batch(geo).requests[0]
    G = geo.group
    for g in range(geo.num_kv_heads):
        pos = r.planted_pos[g]
        assert len(torch.unique(pos)) == geo.n_planted
        assert int(pos.min()) >= 0 and int(pos.max()) < 4096
        heads = r.planted_head[g].tolist()
        assert heads == [g * G + j % G for j in range(geo.n_planted)]


def test_planted_keys_point_at_their_query_heads():
    geo = wl.workload("tiny-f32-8k", seq_len=2048)
    r = wl.make_batch(geo).requests[0]
    q = r.q.double()
    for g in range(geo.num_kv_heads):
        for j in range(4):
            i = int(r.planted_pos[g, j])
            h = int(r.planted_head[g, j])
            key = r.k[g, i].double() / float(r.scales[g])
            cos = float(key @ q[h] / (key.norm() * q[h].norm()))
            assert cos > 0.97          # |8 q_hat| = 8 against noise of norm ~0.1*sqrt(128)
            assert abs(float(key.norm()) - 8.0) < 0.5


def test_scales_in_range_and_whole_head_scaled():
    geo = wl.workload("llama3-8b-128k", seq_len=2048)
    for layer in range(4):
        r = wl.make_batch(geo, layer=layer).requests[0]
        s = r.scales
        assert float(s.min()) >= 1.0 and float(s.max()) < 1000.0
        rms = r.k.float().pow(2).mean(dim=(1, 2)).sqrt()
        assert torch.allclose(rms, s, rtol=0.1)
    r1 = wl.make_batch(geo, scale_spread=False).requests[0]
    assert torch.all(r1.scales == 1.0)


def test_bf16_rounding_is_round_to_nearest_even():
    x = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], dtype=torch.float32)
    y = x.to(torch.bfloat16).float().tolist()
    assert y == [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7]


def test_paged_pool_holds_logical_tokens():
    geo = wl.workload("tiny-f32-8k", seq_len=1000)        # last page partial (1000 = 62*16 + 8)
    b = wl.make_batch(geo)
    r = b.requests[0]
    P = geo.page_size
    bt = b.block_table[0]
    for i in (0, 1, 15, 16, 517, 999):
        page = int(bt[i // P])
        assert torch.equal(b.k_pool[page, :, i % P], r.k[:, i])
        assert torch.equal(b.v_pool[page, :, i % P], r.v[:, i])
    last = int(bt[999 // P])
    assert torch.isnan(b.k_pool[last, :, 8:]).all()
    assert sorted(bt[:63].tolist()) == list(range(63))
    assert bt[:63].tolist() != list(range(63))             # shuffled
    ident = wl.make_batch(geo, permute=False)
    assert ident.block_table[0, :63].tolist() == list(range(63))


def test_ragged_lengths_and_offsets():
    geo = wl.workload("llama3-8b-ragged16")
    gen = torch.Generator().manual_seed(geo.seed)
    lens = wl.request_lengths(gen, geo, "cpu")
    assert len(lens) == 16
    assert all(32768 <= n < 262144 for n in lens)
    assert len(set(lens)) == 16


def test_ar1_queries_follow_the_recursion():
    geo = wl.workload("qwen2-7b-cache256")
    q0 = torch.randn(geo.num_q_heads, geo.head_dim, dtype=torch.float64,
                     generator=torch.Generator().manual_seed(1))
    qs, rho = wl.ar1_queries(geo, q0, 64, seed=7)
    assert qs.shape == (64, geo.num_q_heads, geo.head_dim)
    assert torch.equal(qs[0], q0.to(torch.bfloat16))
    r = rho[1:].numpy()
    assert set(np.unique(r).tolist()) <= {0.97, 0.5}
    frac = float(np.mean(r == 0.97))
    assert 0.6 < frac < 0.95
    # consecutive cosine tracks rho (H*d = 3584 elements)
    for t in range(1, 64):
        a, b = qs[t - 1].double().flatten(), qs[t].double().flatten()
        c = float(a @ b / (a.norm() * b.norm()))
        assert abs(c - rho[t]) < 0.05


def test_chunk_batch_layout_and_seed():
    geo = wl.workload("prefill-tiny-f32", seq_len=700, chunk=40, batch=2, min_len=300, max_len=900)
    a = wl.make_chunk_batch(geo, "cpu", chunk_lens=[40, 7])
    b = wl.make_chunk_batch(geo, "cpu", chunk_lens=[40, 7])
    assert torch.equal(a.q_chunk, b.q_chunk) and torch.equal(a.paged.k_pool.nan_to_num(), b.paged.k_pool.nan_to_num())
    assert a.q_chunk.shape == (2, 40, 8, 128)
    for r in range(2):
        req = a.paged.requests[r]
        P = a.past_lens[r]
        assert int(a.seq_lens[r]) == P + int(a.chunk_lens[r])
        assert req.k.shape[1] == P + 40
        assert int(req.planted_pos.max()) < P          # critical tokens in the past only
