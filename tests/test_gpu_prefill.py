"""GPU parity of chunk-wise prefill (mean-query selection + chunk attention) against
the fp64 oracle, through the C ABI. Bands are those of the decode path (see
gpu_helpers); the chunk attention is compared row by row with the oracle's
attention over T united with [max(0, P - L), P + j]."""
import numpy as np
import pytest
import torch

import token_level_sparse_amd as ts
from oracle import prefill_oracle as pre
from synth import workloads as wl
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ts.load_library()


def _run_all(cb, geo, **kw):
    po = gh.run_prefill(cb, geo, top_k=kw.get("top_k"), n_local=kw.get("n_local"))
    b = cb.q_chunk.shape[0]
    for r in range(b):
        s = gh.check_prefill_selection(po, r, cb, geo, top_k=kw.get("top_k"))
        w = gh.check_chunk_attention(po, r, cb, geo, po.T[r], n_local=kw.get("n_local"),
                                     rows=kw.get("rows"))
        gh.log(f"  request {r}: N={int(cb.seq_lens[r])} c={int(cb.chunk_lens[r])} "
               f"topk diff {s['n_diff']} attn max-abs {w:.2e}")
    return po


def test_prefill_tiny_f32_full():
    geo = wl.workload("prefill-tiny-f32")
    gh.log(f"[prefill tiny f32] N={geo.seq_len} c={geo.chunk}")
    cb = wl.make_chunk_batch(geo, DEV)
    _run_all(cb, geo)


def test_prefill_first_chunk_has_no_past():
    geo = wl.workload("prefill-tiny-f32", seq_len=100, chunk=100)
    gh.log("[prefill first chunk] P = 0")
    cb = wl.make_chunk_batch(geo, DEV)
    po = _run_all(cb, geo)
    assert po.T[0].size == 0


def test_prefill_ragged_batch_f32():
    # requests with P > k, P < k, P < L, and chunk lengths 64 (full), 17 and 1
    geo = wl.workload("prefill-tiny-f32", batch=3, min_len=150, max_len=6000, chunk=64, seed=5100)
    gh.log("[prefill ragged f32] 3 requests, chunk lengths 64 / 17 / 1")
    cb = wl.make_chunk_batch(geo, DEV, chunk_lens=[64, 17, 1])
    _run_all(cb, geo)


@pytest.mark.parametrize("P,c,k,L", [(40, 5, 16, 4), (300, 33, 8, 0), (1000, 70, 1, 3), (17, 16, 64, 64)])
def test_prefill_edge_sizes_f32(P, c, k, L):
    geo = wl.workload("prefill-tiny-f32", seq_len=P + c, chunk=c, top_k=k, n_local=L, seed=5200 + P)
    gh.log(f"[prefill edge f32] P={P} c={c} k={k} L={L}")
    cb = wl.make_chunk_batch(geo, DEV)
    _run_all(cb, geo)


def test_prefill_group7_bf16_small_budget():
    # G = 7 (rows not a multiple of the 64-row tile); a small set makes every key's
    # weight visible above the bf16 tolerance
    geo = wl.workload("prefill-tiny-f32", dtype="bf16", num_q_heads=28, num_kv_heads=4,
                      seq_len=2000, chunk=23, top_k=9, n_local=5, seed=5300)
    gh.log("[prefill G=7 bf16] N=2000 c=23 k=9 L=5")
    cb = wl.make_chunk_batch(geo, DEV)
    _run_all(cb, geo)


def test_prefill_attention_on_oracle_topk():
    geo = wl.workload("prefill-tiny-f32", seq_len=5000, chunk=48, seed=5400)
    gh.log("[prefill attention on oracle TopK] f32")
    cb = wl.make_chunk_batch(geo, DEV)
    c = geo.chunk
    P = geo.seq_len - c
    Qc = gh.np32(cb.q_chunk[0])
    K = gh.np32(cb.paged.requests[0].k[:, :P])
    T = pre.prefill_select(Qc, K, P, geo.top_k)["T"]
    si = torch.full((1, geo.top_k), -1, dtype=torch.int32, device=DEV)
    si[0, : len(T)] = torch.from_numpy(T.astype(np.int32)).to(DEV)
    sc = torch.tensor([len(T)], dtype=torch.int32, device=DEV)
    po = gh.run_prefill(cb, geo, sel_override=(si, sc))
    gh.check_chunk_attention(po, 0, cb, geo, T)


def test_prefill_llama3_128k_full_selection():
    geo = wl.workload("prefill-llama3-128k")
    gh.log(f"[prefill llama3 128k] N={geo.seq_len} c={geo.chunk} k={geo.top_k}")
    cb = wl.make_chunk_batch(geo, DEV)
    rows = [0, 1, 2, 63, 64, 255, 256, 300, 447, 510, 511]
    po = _run_all(cb, geo, rows=rows)
    # the vote bound: any past position with vote > H/k is selected
    big = np.nonzero(np.exp2(po.vote[0].astype(np.float64)) > geo.num_q_heads / geo.top_k)[0]
    assert np.all(np.isin(big, po.T[0]))


def test_prefill_planted_recall_without_scale_spread():
    geo = wl.workload("prefill-llama3-128k", seq_len=32768)
    gh.log("[prefill llama3 N=32768, s=1] planted recall of the mean query")
    cb = wl.make_chunk_batch(geo, DEV, scale_spread=False)
    po = gh.run_prefill(cb, geo)
    planted = np.unique(cb.paged.requests[0].planted_pos.cpu().numpy())
    assert np.all(np.isin(planted, po.T[0]))


def test_prefill_llama3_1m_sampled():
    geo = wl.workload("prefill-llama3-1m")
    gh.log(f"[prefill llama3 1m] N={geo.seq_len} c={geo.chunk} k={geo.top_k}")
    cb = wl.make_chunk_batch(geo, DEV)
    _run_all(cb, geo, rows=[0, 17, 200, 511])
