"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself: a
hand-worked closed form, brute force on tiny inputs, a textbook routine, an
invariant the definition implies, or a theorem (Lemma 1, the vote bound).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import tokenselect_oracle as ora
from synth import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _np(t):
    return t.to(torch.float32).cpu().numpy()


# ------------------------------------------------------------------ hand-worked example
def test_soft_vote_hand_example():
    gx = _load("soft_vote_hand.json")
    q = np.array(gx["q"])
    K = np.array(gx["K"])
    V = np.array(gx["V"])
    sel = ora.select(q, K, 1, gx["score_scale"])
    np.testing.assert_array_equal(sel["z"], np.array(gx["logits"]))
    np.testing.assert_allclose(sel["vote"], gx["vote"], rtol=1e-14)
    assert abs(sel["vote"].sum() - gx["vote_sum"]) < 1e-14
    for k, T in gx["topk"].items():
        assert ora.topk_indices(sel["vote"], int(k)).tolist() == T
    assert ora.naive_topk(q, K, 1).tolist() == gx["naive_topk_1"]
    w = gx["window"]
    T = ora.topk_indices(sel["vote"], w["k"])
    S = ora.union_local(T, K.shape[1], w["n_local"])
    assert S.tolist() == w["S"]
    out = ora.sparse_attention(q, K, V, S, gx["attn_scale"])
    np.testing.assert_allclose(out, gx["attention_on_S_1_2"], rtol=1e-14)


def _unit(deg):
    r = math.radians(deg)
    return [math.cos(r), math.sin(r)]


def test_selection_cache_hand_sequence():
    gx = _load("selection_cache_hand.json")
    qs = []
    for x in gx["queries"]:
        qs.append(_unit(float(x[4:])) if isinstance(x, str) else x)
    qs = np.array(qs)[:, None, :]                      # [steps][H=1][d=2]
    rng = np.random.default_rng(5)
    K = rng.standard_normal((1, 6, 2))
    V = rng.standard_normal((1, 6, 2))
    res = ora.decode_sequence(qs, K, V, [6] * len(qs), k=2, n_local=1, theta=gx["theta"])
    assert res["hit"].tolist() == gx["hit"]
    # a hit reuses the TopK chosen at the last miss
    last = None
    for t, hit in enumerate(res["hit"]):
        if hit:
            assert np.array_equal(res["T"][t], last)
        last = res["T"][t]


# ------------------------------------------------------------------ step 1: logits
def test_logits_integer_brute_force_with_gqa_and_scale():
    rng = np.random.default_rng(1)
    H, Hkv, d, N = 6, 2, 5, 7
    q = rng.integers(-9, 10, size=(H, d))
    K = rng.integers(-9, 10, size=(Hkv, N, d))
    z = ora.score_logits(q, K, score_scale=0.5)
    G = H // Hkv
    for h in range(H):
        for i in range(N):
            exact = sum(int(q[h, j]) * int(K[h // G, i, j]) for j in range(d))
            assert z[h, i] == 0.5 * exact


def test_logits_basis_queries_read_key_columns():
    # q_h = e_j picks column j of its own KV head: catches a transposed operand or
    # a query head mapped to the wrong KV head (h % H_kv instead of h // G).
    rng = np.random.default_rng(2)
    H, Hkv, d, N = 4, 2, 3, 5
    K = rng.standard_normal((Hkv, N, d))
    q = np.zeros((H, d))
    cols = [0, 2, 1, 0]
    for h, c in enumerate(cols):
        q[h, c] = 1.0
    z = ora.score_logits(q, K)
    for h, c in enumerate(cols):
        np.testing.assert_array_equal(z[h], K[h // 2, :, c])


# ------------------------------------------------------------------ steps 2-3: softmax, vote
def _rand_case(seed, H=8, Hkv=2, d=16, N=300, spread=30.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, d))
    K = rng.standard_normal((Hkv, N, d)) * np.exp(rng.uniform(0, np.log(spread), Hkv))[:, None, None]
    return q, K


def test_softmax_rows_sum_to_one_and_vote_sums_to_H():
    q, K = _rand_case(3)
    sel = ora.select(q, K, 10)
    np.testing.assert_allclose(sel["p"].sum(axis=1), 1.0, rtol=0, atol=1e-13)
    assert abs(sel["vote"].sum() - q.shape[0]) < 1e-12
    assert np.all(sel["p"] >= 0)


def test_vote_invariant_to_key_shift_per_kv_head():
    # Adding one vector u to every key of KV head g shifts each of its query heads'
    # logits by the constant <q_h, u>, which the per-head softmax removes.
    q, K = _rand_case(4)
    u = np.random.default_rng(9).standard_normal(K.shape[2]) * 3.0
    K2 = K.copy()
    K2[1] += u
    v1 = ora.select(q, K, 10)["vote"]
    v2 = ora.select(q, K2, 10)["vote"]
    np.testing.assert_allclose(v2, v1, rtol=1e-9, atol=1e-15)


def test_vote_invariant_to_head_order_within_group_only():
    q, K = _rand_case(6)
    v = ora.select(q, K, 10)["vote"]
    perm_in = [2, 0, 3, 1, 5, 7, 4, 6]               # stays inside each group of 4
    np.testing.assert_allclose(ora.select(q[perm_in], K, 10)["vote"], v, rtol=1e-13, atol=1e-16)
    perm_across = [4, 1, 2, 3, 0, 5, 6, 7]           # swaps heads between groups
    v3 = ora.select(q[perm_across], K, 10)["vote"]
    assert np.max(np.abs(v3 - v)) > 1e-3


def test_each_head_has_one_unit_of_say():
    # Scaling one KV head's keys changes how peaked its heads are, but each query
    # head still contributes exactly 1 to the total vote.
    q, K = _rand_case(7)
    K2 = K.copy()
    K2[0] *= 50.0
    p = ora.select(q, K2, 10)["p"]
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-13)


# ------------------------------------------------------------------ step 4: top-k
def test_single_head_topk_equals_argsort_of_raw_logits():
    # With H = 1 the softmax is monotone, so TopK of the vote is TopK of the logits.
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 12))
    K = rng.standard_normal((1, 500, 12))
    K[0, 100] = K[0, 200]                             # an exact tie
    K[0, 300] = K[0, 200]
    z = ora.score_logits(q, K)[0]
    for k in (1, 7, 101, 499, 500, 800):
        ref = np.sort(np.argsort(-z, kind="stable")[:k])
        assert np.array_equal(ora.topk_indices(ora.select(q, K, k)["vote"], k), ref)


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(1, 11))
    v = np.round(rng.uniform(0, 1, N), 1)              # many exact ties
    for k in range(1, N + 2):
        T = ora.topk_indices(v, k)
        if k >= N:
            assert T.tolist() == list(range(N))
            continue
        valid = []
        for comb in itertools.combinations(range(N), k):
            inside = set(comb)
            ok = all(v[i] > v[j] or (v[i] == v[j] and i < j)
                     for i in inside for j in range(N) if j not in inside)
            if ok:
                valid.append(list(comb))
        assert len(valid) == 1
        assert T.tolist() == valid[0]


def test_window_union():
    assert ora.union_local([0, 8], 10, 3).tolist() == [0, 7, 8, 9]
    assert ora.union_local([1], 2, 5).tolist() == [0, 1]
    assert ora.union_local([3, 4], 5, 0).tolist() == [3, 4]
    # the current token (position N - 1) is attended whatever the window size:
    # the deepnotes formalisation attends [K_select, K_current]
    assert ora.union_local([0, 2], 10, 0).tolist() == [0, 2, 9]
    assert ora.union_local([], 1, 0).tolist() == [0]
    assert ora.union_local([], 0, 0).tolist() == []


def test_decode_step_without_window_attends_current_token():
    # H = 1, d = 1, q = 1, keys 3, 1, 0: the TopK (k = 1) is position 0, the
    # current token is position 2. S = {0, 2}; with attn_scale 1 the weights are
    # e^3 / (e^3 + 1) and 1 / (e^3 + 1), so o = (10 e^3 + 30) / (e^3 + 1).
    q = np.array([[1.0]])
    K = np.array([[[3.0], [1.0], [0.0]]])
    V = np.array([[[10.0], [20.0], [30.0]]])
    res = ora.decode_step(q, K, V, k=1, n_local=0, attn_scale=1.0)
    assert res["T"].tolist() == [0]
    assert res["S"].tolist() == [0, 2]
    e3 = math.exp(3.0)
    assert abs(res["out"][0, 0] - (10.0 * e3 + 30.0) / (e3 + 1.0)) < 1e-12


def test_lemma1_topk_invariant_within_angle():
    # Lemma 1 (TokenSelect deepnotes appendix): write q2_hat = q1_hat cos t + p_hat sin t
    # with p_hat orthogonal to q1. For i in T(q1), j not in T(q1):
    # q2_hat.(k_i - k_j) >= cos t * g - sin t * D with g = min q1_hat.(k_i - k_j) and
    # D = max |k_i - k_j|, so T(q2) = T(q1) whenever tan t < g / D.
    rng = np.random.default_rng(11)
    d, N, k = 8, 40, 5
    for trial in range(30):
        K = rng.standard_normal((1, N, d))
        q1 = rng.standard_normal(d)
        q1h = q1 / np.linalg.norm(q1)
        T = ora.topk_indices(ora.select(q1[None], K, k)["vote"], k)
        out = np.setdiff1d(np.arange(N), T)
        diffs = K[0][T][:, None, :] - K[0][out][None, :, :]
        g = np.min(diffs @ q1h)
        D = np.max(np.linalg.norm(diffs, axis=2))
        assert g > 0
        tmax = math.atan(g / D)
        for _ in range(5):
            p = rng.standard_normal(d)
            p -= (p @ q1h) * q1h
            p /= np.linalg.norm(p)
            t = rng.uniform(0, 0.999) * tmax
            q2 = (math.cos(t) * q1h + math.sin(t) * p) * rng.uniform(0.1, 10)
            T2 = ora.topk_indices(ora.select(q2[None], K, k)["vote"], k)
            assert np.array_equal(T2, T)


# ------------------------------------------------------------------ step 5: attention
def test_full_budget_equals_dense_sdpa_textbook():
    # k >= N: every position is selected, and the result is plain SDPA, checked
    # against torch's scaled_dot_product_attention in fp64 with KV heads repeated.
    rng = np.random.default_rng(12)
    H, Hkv, d, N = 8, 2, 16, 97
    q = rng.standard_normal((H, d))
    K = rng.standard_normal((Hkv, N, d)) * 3
    V = rng.standard_normal((Hkv, N, d))
    res = ora.decode_step(q, K, V, k=N + 5, n_local=4)
    assert res["S"].tolist() == list(range(N))
    G = H // Hkv
    Kt = torch.from_numpy(K).repeat_interleave(G, dim=0)
    Vt = torch.from_numpy(V).repeat_interleave(G, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :], Kt, Vt)[:, 0, :].numpy()
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-13)


def test_single_selected_token_returns_its_value_row():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((4, 8))
    K = rng.standard_normal((2, 20, 8))
    V = rng.standard_normal((2, 20, 8))
    out = ora.sparse_attention(q, K, V, [11], 0.3)
    for h in range(4):
        np.testing.assert_array_equal(out[h], V[h // 2, 11])


def test_attention_invariant_to_order_of_selected_set():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((4, 8))
    K = rng.standard_normal((2, 50, 8))
    V = rng.standard_normal((2, 50, 8))
    S = np.array([3, 9, 10, 17, 33, 49])
    a = ora.sparse_attention(q, K, V, S, 0.35)
    b = ora.sparse_attention(q, K, V, S[::-1].copy(), 0.35)
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-15)


# ------------------------------------------------------------------ step 0: Selection Cache
def _cache_seq(qs, theta):
    K = np.random.default_rng(15).standard_normal((1, 8, qs.shape[-1]))
    return ora.decode_sequence(qs, K, K, [8] * len(qs), k=2, n_local=1, theta=theta,
                               want_outputs=False)["hit"].tolist()


def test_cache_identical_queries_hit_and_extreme_thresholds():
    rng = np.random.default_rng(16)
    q = rng.standard_normal((1, 2, 6))
    qs = np.repeat(q, 5, axis=0)
    assert _cache_seq(qs, 0.9) == [False] + [True] * 4
    qs2 = rng.standard_normal((6, 2, 6))
    assert _cache_seq(qs2, 1.0000001) == [False] * 6        # theta > 1: never hit
    assert _cache_seq(qs2, -1.0) == [False] + [True] * 5     # theta <= -1: hit after first


def test_cache_orthogonal_query_misses():
    a = np.zeros((1, 4)); a[0, 0] = 1
    b = np.zeros((1, 4)); b[0, 1] = 1
    assert _cache_seq(np.stack([a, b, b]), 0.0) == [False, True, True]   # cos 0 >= 0
    assert _cache_seq(np.stack([a, b, b]), 0.5) == [False, False, True]


# ------------------------------------------------------------------ planted recall
def test_vote_above_H_over_k_is_always_selected():
    # Theorem: the votes sum to H, so fewer than k positions can exceed H/k;
    # every such position is therefore in TopK.
    geo = wl.workload("tiny-f32-8k")
    b = wl.make_batch(geo)
    r = b.requests[0]
    sel = ora.select(_np(r.q), _np(r.k), geo.top_k)
    big = np.nonzero(sel["vote"] > geo.num_q_heads / geo.top_k)[0]
    assert len(big) > 0
    assert np.all(np.isin(big, sel["T"]))


def _planted_top_per_head(sel, r, H):
    """For each query head, the planted position it targets with the largest p."""
    pos = r.planted_pos.cpu().numpy()
    heads = r.planted_head.cpu().numpy()
    best = []
    for h in range(H):
        cand = pos[heads == h]
        best.append(int(cand[np.argmax(sel["p"][h][cand])]))
    return np.array(best)


def test_planted_tokens_all_recalled_without_scale_spread():
    geo = wl.workload("tiny-f32-8k")
    b = wl.make_batch(geo, scale_spread=False)
    r = b.requests[0]
    sel = ora.select(_np(r.q), _np(r.k), geo.top_k)
    planted = np.unique(r.planted_pos.cpu().numpy())
    assert np.all(np.isin(planted, sel["T"]))


def test_soft_vote_recalls_every_heads_top_planted_token_naive_does_not():
    geo = wl.workload("tiny-f32-8k")
    b = wl.make_batch(geo)
    r = b.requests[0]
    q, K = _np(r.q), _np(r.k)
    sel = ora.select(q, K, geo.top_k)
    best = _planted_top_per_head(sel, r, geo.num_q_heads)
    assert np.all(np.isin(best, sel["T"]))
    naive = ora.naive_topk(q, K, geo.top_k)
    # the naive TopK over raw logits is dominated by the large-scale KV head
    assert not np.all(np.isin(best, naive))


# ------------------------------------------------------------------ dynamic top-p budget
def test_topp_hand_cases():
    gx = _load("topp_hand.json")
    for cs in gx["cases"]:
        m = ora.topp_count(cs["v"], cs["p"], cs["k_max"])
        assert m == cs["m"], cs
        assert ora.topp_indices(cs["v"], cs["p"], cs["k_max"]).tolist() == cs["T"], cs


def test_topp_brute_force_small():
    rng = np.random.default_rng(11)
    for _ in range(200):
        N = int(rng.integers(1, 7))
        v = rng.integers(0, 5, N).astype(np.float64)   # integer masses: ties and exact sums
        if v.sum() == 0:
            v[0] = 1.0
        p = float(rng.choice([0.2, 0.5, 0.75, 0.9, 1.0]))
        kmax = int(rng.integers(1, N + 2))
        # brute force: the smallest m whose best m-subset (by mass) reaches p of the total
        best = None
        for m in range(1, N + 1):
            top = max(sum(v[list(c)]) for c in itertools.combinations(range(N), m))
            if top >= p * v.sum():
                best = m
                break
        assert ora.topp_count(v, p, kmax) == min(best, kmax, N), (v, p, kmax)
        T = ora.topp_indices(v, p, kmax)
        # the chosen positions are the largest votes, lower positions first among equals
        m = len(T)
        key = sorted(range(N), key=lambda i: (-v[i], i))[:m]
        assert sorted(key) == T.tolist()


def test_topp_full_mass_and_cap_reduce_to_topk():
    rng = np.random.default_rng(12)
    v = rng.random(500)
    assert np.array_equal(ora.topp_indices(v, 1.0, 40), ora.topk_indices(v, 40))
    # a tiny p keeps the single largest vote
    assert ora.topp_indices(v, 1e-9, 40).tolist() == [int(np.argmax(v))]


def test_topp_peaked_vote_selects_few_planted_tokens():
    # a needle-like distribution: most vote mass on the planted tokens (no scale
    # spread, so every head's softmax concentrates on its planted keys)
    geo = wl.workload("llama3-8b-128k", seq_len=4096, n_planted=16)
    b = wl.make_batch(geo, scale_spread=False)
    r = b.requests[0]
    sel = ora.select(_np(r.q), _np(r.k), 256)
    T = ora.topp_indices(sel["vote"], 0.9, 4096)
    planted = np.unique(r.planted_pos.numpy())
    assert len(T) <= 2 * len(planted)
    assert np.isin(T, planted).mean() > 0.5


# ------------------------------------------------------------------ selection-function ablations
def test_ablation_hand_cases():
    gx = _load("ablation_hand.json")
    hv = gx["hard_vote"]
    z = np.array(hv["z"])
    assert ora.hard_vote_topk(z, hv["k"]).tolist() == hv["T"]
    assert ora.topk_indices(z.max(axis=0), hv["k"]).tolist() == hv["naive_T"]
    bl = gx["block"]
    v = np.array(bl["v"])
    assert ora.topk_indices(v, bl["k"]).tolist() == bl["token_T"]
    for cs in bl["cases"]:
        if "sums" in cs:
            np.testing.assert_allclose(ora.block_scores(v, cs["block"]), cs["sums"], rtol=1e-15)
        T = ora.block_topk(v, bl["k"], cs["block"])
        assert T.tolist() == cs["T"]
        assert ora.recall(T, bl["token_T"]) == cs["recall"]


def test_hard_vote_single_head_is_per_head_topk():
    rng = np.random.default_rng(13)
    z = rng.standard_normal((1, 300))
    for k in (1, 7, 64):
        assert np.array_equal(ora.hard_vote_topk(z, k), np.sort(np.argsort(-z[0], kind="stable")[:k]))


def test_hard_vote_brute_force_counts():
    rng = np.random.default_rng(14)
    for _ in range(50):
        H, N, k = int(rng.integers(1, 5)), int(rng.integers(2, 9)), int(rng.integers(1, 5))
        z = rng.integers(-3, 4, (H, N)).astype(np.float64)
        counts = np.zeros(N)
        for h in range(H):
            # this head's k best positions, lower position first among equal logits
            best = sorted(range(N), key=lambda i: (-z[h, i], i))[:k]
            counts[best] += 1
        exp = sorted(sorted(range(N), key=lambda i: (-counts[i], i))[:k])
        assert ora.hard_vote_topk(z, k).tolist() == exp


def test_block_selection_reduces_to_token_level_and_covers_blocks():
    rng = np.random.default_rng(15)
    v = rng.random(1000) ** 8
    assert np.array_equal(ora.block_topk(v, 64, 1), ora.topk_indices(v, 64))
    for B in (2, 8, 32, 128):
        T = ora.block_topk(v, 256, B)
        assert len(T) == (256 // B) * B
        blocks = np.unique(T // B)
        assert len(blocks) == 256 // B and np.all(np.isin(blocks * B, T))
        # brute force: no unselected block has a larger sum than a selected one
        sums = ora.block_scores(v, B)
        rest = np.setdiff1d(np.arange(len(sums)), blocks)
        assert sums[blocks].min() >= sums[rest].max()


def test_block_recall_falls_with_granularity_on_scattered_tokens():
    # scattered critical tokens (planted at uniform positions): token-level selection
    # recalls all of the token-level TopK, block-level selection loses more of it as
    # blocks grow (the deepnotes page's Fig. 2b trend, on synthetic data)
    geo = wl.workload("llama3-8b-128k", seq_len=16384, n_planted=32, top_k=512)
    b = wl.make_batch(geo, scale_spread=False)
    r = b.requests[0]
    v = ora.select(_np(r.q), _np(r.k), geo.top_k)["vote"]
    ref = ora.topk_indices(v, geo.top_k)
    rec = [ora.recall(ora.block_topk(v, geo.top_k, B), ref) for B in (1, 4, 16, 64, 128)]
    assert rec[0] == 1.0
    assert all(x >= y for x, y in zip(rec, rec[1:]))
    assert rec[-1] < 0.6


def test_block_budget_rounds_down_and_recall_is_over_the_reference():
    v = np.array([0.1, 0.9, 0.0, 0.0, 0.3, 0.3, 0.3, 0.0, 0.05, 0.05])
    # budget 5 with blocks of 2: two whole blocks (4 tokens), never more than k
    T = ora.block_topk(v, 5, 2)
    assert T.tolist() == [0, 1, 4, 5]
    # recall is the covered fraction of the reference set
    assert ora.recall([1, 2, 3], [1]) == 1.0
    assert ora.recall([1], [1, 2, 3, 4]) == 0.25
