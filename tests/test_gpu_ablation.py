"""GPU parity of the selection-function ablations (tokenselect_select_ablation).

Each variant is an integer decision on float scores, so it is checked the way the
decode TopK is: the GPU result must equal the pinned oracle function applied to the
GPU's own fp32 logits / log2 votes (the decision in the GPU's precision), and the
GPU logits themselves are checked against the fp64 oracle by the decode parity
tests. The recall-vs-granularity study on the 128K workload is logged.
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


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ts.load_library()


def _logits(batch, geo):
    b = batch.q.shape[0]
    H = geo.num_q_heads
    total = batch.total_tokens
    shape = ts.make_shape(H, geo.num_kv_heads, b, batch.block_table.shape[1], total, geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale)
    ws = ts.alloc_workspace(shape, sel, DEV)
    logits = torch.empty(H * total, dtype=torch.float32, device=DEV)
    stats = torch.empty(b * H * 2, dtype=torch.float32, device=DEV)
    ts.score(shape, sel, batch.q, batch.k_pool, batch.block_table, batch.seq_lens, logits, stats, ws)
    return shape, sel, logits, stats


def _ablate(shape, sel, fn, block, logits, stats, batch, n_score):
    b = batch.q.shape[0]
    ws = ts.alloc_ablation_workspace(shape, sel, fn, block, DEV)
    score = torch.full((n_score,), float("nan"), dtype=torch.float32, device=DEV)
    si = torch.full((b, sel.top_k), -7, dtype=torch.int32, device=DEV)
    sc = torch.full((b,), -7, dtype=torch.int32, device=DEV)
    ts.select_ablation(shape, sel, fn, block, logits, stats, batch.seq_lens, score, si, sc, ws)
    torch.cuda.synchronize()
    return score.cpu().numpy(), si.cpu().numpy(), sc.cpu().numpy()


def _per_request_logits(lg, batch, geo):
    H, G = geo.num_q_heads, geo.group
    offs = batch.token_offsets.cpu().tolist()
    out = []
    for r in range(batch.q.shape[0]):
        n = int(batch.seq_lens[r])
        blk = lg[offs[r] * H: offs[r] * H + H * n].reshape(geo.num_kv_heads, n, G)
        out.append(np.ascontiguousarray(blk.transpose(0, 2, 1)).reshape(H, n).astype(np.float64))
    return out


def _check_all(batch, geo, blocks=(1, 4, 16, 128)):
    shape, sel, logits, stats = _logits(batch, geo)
    k = geo.top_k
    total = batch.total_tokens
    offs = batch.token_offsets.cpu().tolist()
    Z = _per_request_logits(logits.cpu().numpy(), batch, geo)
    b = batch.q.shape[0]
    # soft vote: the ablation entry reproduces tokenselect_vote_topk
    lv, T_soft, c_soft = _ablate(shape, sel, ts.SELECT_SOFT_VOTE, 1, logits, stats, batch, total)
    ws = ts.alloc_workspace(shape, sel, DEV)
    si = torch.empty(b, k, dtype=torch.int32, device=DEV)
    sc = torch.empty(b, dtype=torch.int32, device=DEV)
    ts.vote_topk(shape, sel, logits, stats, batch.seq_lens, None, si, sc, ws)
    torch.cuda.synchronize()
    for r in range(b):
        n = int(sc[r])
        assert int(c_soft[r]) == n and np.array_equal(T_soft[r, :n], si[r, :n].cpu().numpy())
    # naive
    s_naive, T_naive, c_naive = _ablate(shape, sel, ts.SELECT_NAIVE_TOPK, 1, logits, stats, batch, total)
    for r in range(b):
        n = int(batch.seq_lens[r])
        mx = Z[r].max(axis=0)
        assert np.array_equal(s_naive[offs[r]: offs[r] + n].astype(np.float64), mx)
        assert np.array_equal(T_naive[r, : c_naive[r]], ora.naive_topk_from_logits(Z[r], k))
    # hard vote
    s_hard, T_hard, c_hard = _ablate(shape, sel, ts.SELECT_HARD_VOTE, 1, logits, stats, batch, total)
    for r in range(b):
        n = int(batch.seq_lens[r])
        counts = np.zeros(n)
        for h in range(geo.num_q_heads):
            counts[ora.topk_indices(Z[r][h], k)] += 1
        assert np.array_equal(s_hard[offs[r]: offs[r] + n].astype(np.float64), counts)
        assert np.array_equal(T_hard[r, : c_hard[r]], ora.hard_vote_topk(Z[r], k))
    # block selection on the GPU's own log2 votes
    recalls = {}
    for B in blocks:
        nblk = sum(-(-int(batch.seq_lens[r]) // B) for r in range(b))
        s_blk, T_blk, c_blk = _ablate(shape, sel, ts.SELECT_BLOCK, B, logits, stats, batch, nblk)
        boff = 0
        for r in range(b):
            n = int(batch.seq_lens[r])
            nb = -(-n // B)
            v_gpu = lv[offs[r]: offs[r] + n].astype(np.float64)
            pad = np.full(nb * B, -np.inf)
            pad[:n] = v_gpu
            blk = pad.reshape(nb, B)
            m = blk.max(axis=1)
            sums = (m + np.log2(np.exp2(blk - m[:, None]).sum(axis=1))).astype(np.float32)
            got = s_blk[boff: boff + nb]
            # log2 of the block's vote sum, rounded once to fp32 (equal up to the last
            # bit of fp64 exp2 / log2)
            assert np.allclose(got, sums, rtol=1e-6, atol=1e-6), (B, np.abs(got - sums).max())
            if B == 1:
                assert np.array_equal(got, lv[offs[r]: offs[r] + n])
            # the selection is the block TopK of the GPU's block scores, expanded
            blocks_sel = ora.topk_indices(got.astype(np.float64), max(1, k // B))
            pos = (blocks_sel[:, None] * B + np.arange(B)[None, :]).reshape(-1)
            pos = pos[pos < n]
            assert np.array_equal(T_blk[r, : c_blk[r]], pos)
            ref = T_soft[r, : c_soft[r]]
            recalls.setdefault(B, []).append(ora.recall(pos, ref))
            boff += nb
    return {B: float(np.mean(v)) for B, v in recalls.items()}


def test_ablations_tiny_f32():
    geo = wl.workload("tiny-f32-8k")
    gh.log("[ablations tiny f32]")
    rec = _check_all(wl.make_batch(geo, device=DEV), geo)
    gh.log(f"  recall by block size {rec}")
    assert rec[1] == 1.0


def test_ablations_ragged_batch():
    geo = wl.workload("llama3-8b-ragged16", batch=4, min_len=3000, max_len=20000, seed=3200)
    gh.log("[ablations ragged] 4 requests")
    rec = _check_all(wl.make_batch(geo, device=DEV), geo, blocks=(1, 8, 64))
    assert rec[1] == 1.0


def test_recall_vs_granularity_128k():
    # the token-level motivation (Fig. 2b) on synthetic scattered critical tokens:
    # recall of the token-level soft-vote TopK by block-level selection
    geo = wl.workload("llama3-8b-128k")
    gh.log("[ablations llama3 128k] recall vs block size")
    rec = _check_all(wl.make_batch(geo, device=DEV), geo, blocks=(1, 2, 4, 8, 16, 32, 64, 128))
    gh.log("  " + ", ".join(f"B={B}: {r:.3f}" for B, r in rec.items()))
    assert rec[1] == 1.0
    assert rec[128] < rec[1]
