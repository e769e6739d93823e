"""Pins of the chunk-wise prefill oracle against what the pages and the mathematics fix.

Each check compares the oracle with something other than itself: hand-worked
closed forms (tests/golden/prefill_chunk_hand.json), torch's fp64 scaled
dot-product attention with an explicit mask (a library routine) in the cases
where the sparse chunk attention must reduce to dense causal attention, the
already pinned decode selection in the case of identical queries, and
invariants the definitions imply (causality, unattended positions).
"""
import json
import math
import os

import numpy as np
import torch

from oracle import prefill_oracle as pre
from oracle import tokenselect_oracle as ora

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLDEN, "prefill_chunk_hand.json")) as f:
        return json.load(f)


def _rand(seed, c, H, Hkv, P, d=16, kscale=3.0):
    rng = np.random.default_rng(seed)
    Qc = rng.standard_normal((c, H, d))
    K = kscale * rng.standard_normal((Hkv, P + c, d))
    V = rng.standard_normal((Hkv, P + c, d))
    return Qc, K, V


def _sdpa_masked(Qc, K, V, allowed, scale):
    """torch fp64 SDPA of Qc [c][H][d] over K, V [Hkv][N][d] with a boolean mask [c][N]."""
    c, H, d = Qc.shape
    G = H // K.shape[0]
    q = torch.from_numpy(Qc).permute(1, 0, 2)                       # [H][c][d]
    k = torch.from_numpy(np.repeat(K, G, axis=0))                     # [H][N][d]
    v = torch.from_numpy(np.repeat(V, G, axis=0))
    m = torch.from_numpy(allowed)[None].expand(H, -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)
    return o.permute(1, 0, 2).numpy()                                 # [c][H][d]


def test_hand_case_a_selection_and_attention():
    g = _gold()["case_a"]
    Qc, K, V = np.array(g["Qc"]), np.array(g["K"]), np.array(g["V"])
    res = pre.prefill_chunk(Qc, K, V, g["P"], g["k"], g["n_local"], g["score_scale"], g["attn_scale"])
    np.testing.assert_array_equal(res["qbar"], np.array(g["qbar"]))
    np.testing.assert_array_equal(res["z"], np.array(g["logits"]))
    assert res["T"].tolist() == g["T"]
    sets = pre.chunk_sets(res["T"], g["P"], g["c"], g["n_local"])
    assert [s.tolist() for s in sets] == g["sets"]
    np.testing.assert_allclose(res["out"], np.array(g["out"]), rtol=1e-13)


def test_hand_case_b_mean_not_sum():
    g = _gold()["case_b"]
    Qc, K = np.array(g["Qc"]), np.array(g["K"])
    sel = pre.prefill_select(Qc, K, g["P"], g["k"], g["score_scale"])
    np.testing.assert_allclose(sel["vote"], g["vote"], rtol=1e-14)
    assert sel["T"].tolist() == g["T"]
    assert g["T_if_summed"] != g["T"]


def test_identical_queries_reduce_to_decode_selection():
    Qc, K, _ = _rand(1, 1, 8, 2, 300)
    Qc = np.repeat(Qc, 6, axis=0)                  # six copies of one query
    P = 300
    sel = pre.prefill_select(Qc, np.concatenate([K, K[:, :5]], axis=1), P, 17)
    ref = ora.select(Qc[0], K[:, :P], 17)
    np.testing.assert_allclose(sel["vote"], ref["vote"], rtol=1e-13)
    assert np.array_equal(sel["T"], ref["T"])


def test_full_budget_equals_dense_causal_sdpa():
    # k >= P and L >= P: every past position and the causal chunk part are attended
    c, H, Hkv, P = 7, 6, 2, 40
    Qc, K, V = _rand(2, c, H, Hkv, P)
    scale = 1 / math.sqrt(Qc.shape[-1])
    out = pre.prefill_chunk(Qc, K, V, P, k=P + 5, n_local=P, attn_scale=scale)["out"]
    N = P + c
    allowed = np.arange(N)[None, :] <= (P + np.arange(c))[:, None]
    np.testing.assert_allclose(out, _sdpa_masked(Qc, K, V, allowed, scale), rtol=1e-12, atol=1e-13)


def test_first_chunk_is_causal_self_attention():
    c, H, Hkv = 9, 4, 4
    Qc, K, V = _rand(3, c, H, Hkv, 0)
    scale = 0.3
    res = pre.prefill_chunk(Qc, K, V, 0, k=8, n_local=4, attn_scale=scale)
    assert res["T"].size == 0
    allowed = np.tril(np.ones((c, c), dtype=bool))
    np.testing.assert_allclose(res["out"], _sdpa_masked(Qc, K, V, allowed, scale), rtol=1e-12, atol=1e-13)


def test_sparse_chunk_equals_masked_sdpa():
    # the attended sets written as an explicit mask for the library routine
    c, H, Hkv, P, k, L = 5, 8, 2, 200, 12, 6
    Qc, K, V = _rand(4, c, H, Hkv, P)
    scale = 1 / math.sqrt(Qc.shape[-1])
    res = pre.prefill_chunk(Qc, K, V, P, k, L, attn_scale=scale)
    T = res["T"]
    assert len(T) == k and T.max() < P
    allowed = np.zeros((c, P + c), dtype=bool)
    allowed[:, T] = True
    for j in range(c):
        allowed[j, P - L: P + j + 1] = True
    np.testing.assert_allclose(res["out"], _sdpa_masked(Qc, K, V, allowed, scale), rtol=1e-12, atol=1e-13)


def test_causality_and_unattended_positions():
    c, H, Hkv, P, k, L = 6, 4, 1, 120, 10, 8
    Qc, K, V = _rand(5, c, H, Hkv, P)
    res = pre.prefill_chunk(Qc, K, V, P, k, L)
    T = res["T"]
    # chunk keys do not enter the selection
    K2 = K.copy()
    K2[:, P:] *= 50.0
    assert np.array_equal(pre.prefill_select(Qc, K2, P, k)["T"], T)
    # later chunk tokens do not change earlier outputs
    for j in range(c - 1):
        K3, V3 = K.copy(), V.copy()
        K3[:, P + j + 1:] += 7.0
        V3[:, P + j + 1:] -= 3.0
        out3 = pre.chunk_attention(Qc, K3, V3, T, P, L, 1 / math.sqrt(Qc.shape[-1]))
        np.testing.assert_array_equal(out3[: j + 1], res["out"][: j + 1])
    # past positions outside TopK and the window are never read
    skipped = np.setdiff1d(np.arange(P - L), T)
    V4 = V.copy()
    V4[:, skipped] = 1e6
    out4 = pre.chunk_attention(Qc, K, V4, T, P, L, 1 / math.sqrt(Qc.shape[-1]))
    np.testing.assert_array_equal(out4, res["out"])


def test_mean_query_of_integer_rows():
    Qc = np.array([[[1.0, -2.0]], [[3.0, 4.0]], [[5.0, 1.0]], [[-1.0, 5.0]]])
    np.testing.assert_array_equal(pre.chunk_mean_query(Qc), np.array([[2.0, 2.0]]))
