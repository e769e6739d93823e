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


@pytest.mark.parametrize("k", [8, 40, 100, 160, 260, 420, 700])
def test_prefill_bf16_key_blocks_per_split(k):
    # bf16 chunk attention stages 64-key blocks into three K and three V buffers, two
    # blocks ahead; key lists of 72 ... 764 entries give one to three splits of 2, 3 or
    # 4 blocks, most with a ragged last block, so the staging's prologue (fewer blocks
    # than buffers) and its tail (no K, then no V left to stage) are taken; the G = 7
    # test above has a single block, the 128K and 1024-query tests 8 to 16. All rows
    # are checked against the oracle.
    geo = wl.workload("prefill-tiny-f32", dtype="bf16", num_q_heads=16, num_kv_heads=4,
                      seq_len=3040, chunk=40, top_k=k, n_local=24, seed=5900 + k)
    gh.log(f"[prefill bf16 key blocks] P=3000 c=40 k={k} L=24 ({k + 64} list entries)")
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


def test_prefill_chunk1024_group8_ragged_bf16():
    # a chunk of 1024 queries with G = 8 (32 row tiles of 256 per KV head, 4 splits)
    # next to a chunk of 300: rows across row tiles, splits and the causal edge
    geo = wl.workload("prefill-llama3-128k", num_q_heads=32, num_kv_heads=4, batch=2, min_len=20000,
                      max_len=40000, chunk=1024, top_k=2048, n_local=512, seed=5700)
    cb = wl.make_chunk_batch(geo, DEV, chunk_lens=[1024, 300])
    gh.log(f"[prefill chunk 1024, G=8, bf16] N={[int(x) for x in cb.seq_lens.cpu()]} chunk lengths 1024 / 300")
    po = gh.run_prefill(cb, geo)
    rows = [0, 1, 31, 32, 255, 256, 299, 511, 512, 767, 1000, 1023]
    for r in range(2):
        c = int(cb.chunk_lens[r])
        s = gh.check_prefill_selection(po, r, cb, geo)
        w = gh.check_chunk_attention(po, r, cb, geo, po.T[r], rows=[j for j in rows if j < c])
        gh.log(f"  request {r}: c={c} topk diff {s['n_diff']} attn max-abs {w:.2e}")


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


@pytest.mark.parametrize("p", [0.5, 0.9])
def test_prefill_top_p_budget_and_workspace_reuse(p):
    # The dynamic top-p budget through the prefill selection (mean query over the
    # past): the set is exactly the top m of the GPU's own votes with m the budget
    # those votes imply, and it holds >= p of the oracle's vote mass. The score launch
    # clears the radix histograms and masses of the TopK that follows, so a second
    # call on the same workspace must give the same selection bit for bit.
    from tests.test_gpu_topp import _check_request
    geo = wl.workload("prefill-llama3-128k", batch=3, min_len=2000, max_len=30000, seed=5600)
    cb = wl.make_chunk_batch(geo, DEV, chunk_lens=[512, 100, 1])
    b, H, k = 3, geo.num_q_heads, geo.top_k
    mc = cb.q_chunk.shape[1]
    lens = [int(x) for x in cb.seq_lens.cpu()]
    clens = [int(x) for x in cb.chunk_lens.cpu()]
    past = [n - c for n, c in zip(lens, clens)]
    gh.log(f"[prefill top-p p={p}] past {past} chunk lengths {clens}")
    max_total = sum(lens)
    shape = ts.make_shape(H, geo.num_kv_heads, b, cb.paged.block_table.shape[1], max_total, geo.torch_dtype)
    sel = ts.make_select(k, geo.n_local, 1.0, geo.attn_scale, geo.cos_threshold, p)
    ws = ts.alloc_prefill_workspace(shape, sel, mc, DEV)
    runs = []
    for _ in range(2):
        vote = torch.full((max_total,), float("nan"), dtype=torch.float32, device=DEV)
        si = torch.full((b, k), -7, dtype=torch.int32, device=DEV)
        sc = torch.full((b,), -7, dtype=torch.int32, device=DEV)
        ts.prefill_select(shape, sel, mc, cb.q_chunk, cb.chunk_lens, cb.paged.k_pool, cb.paged.block_table,
                          cb.seq_lens, None, None, vote, si, sc, ws)
        torch.cuda.synchronize()
        runs.append((vote.cpu().numpy(), si.cpu().numpy(), sc.cpu().numpy()))
    assert np.array_equal(runs[0][2], runs[1][2])
    assert np.array_equal(runs[0][1], runs[1][1])
    lv, si, sc = runs[0]
    off = 0
    for r in range(b):
        P, m = past[r], int(sc[r])
        Qc = gh.np32(cb.q_chunk[r, :clens[r]])
        K = gh.np32(cb.paged.requests[r].k[:, :P])
        ref = pre.prefill_select(Qc, K, P, k)
        _check_request(lv[off: off + P], si[r, :m].astype(np.int64), m, p, k, ref["vote"])
        gh.log(f"  request {r}: P={P} budget {m}")
        off += P
