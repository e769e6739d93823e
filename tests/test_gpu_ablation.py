"""GPU parity of the selection-function ablations (tokenselect_select_ablation).

Each variant is an integer decision on float scores, and is checked twice:
- against the pinned oracle function applied to the GPU's own fp32 logits / log2
  votes (the decision taken in the GPU's precision must match exactly; block
  scores are the oracle's block sums of 2^lv);
- end to end against the fp64 oracle on the stored q and K (ora.naive_topk,
  ora.hard_vote_topk on the oracle's logits, ora.block_topk on the oracle's soft
  vote): the selected sets may differ only at positions whose oracle score lies
  within the fp32 error band of the k-th score (band (b) of the decode TopK,
  restated for each score).
The recall-vs-granularity study on the 128K workload is logged.
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


def _check_all(batch, geo, blocks=(1, 4, 16, 128), oracle=True):
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
            got = s_blk[boff: boff + nb]
            # log2 of the oracle's block sums of the GPU's votes 2^lv, rounded once to
            # fp32 (equal up to the last bits of fp64 exp2 / log2) wherever the fp64 sum
            # is a normal number; below 2^-1000 fp64 itself carries few bits (subnormal
            # from 2^-1022, zero below 2^-1074), and the GPU's log-domain sum must then
            # lie below -999
            with np.errstate(divide="ignore"):
                sums = np.log2(ora.block_scores(np.exp2(v_gpu), B))
            nrm = sums > -1000.0
            assert np.allclose(got[nrm], sums[nrm], rtol=1e-6, atol=1e-6), (B, np.abs(got[nrm] - sums[nrm]).max())
            assert np.all(got[~nrm] < -999.0), B
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
    if oracle:
        _check_against_oracle(batch, geo, blocks, Z, T_naive, c_naive, s_hard, T_hard, c_hard,
                              shape, sel, logits, stats)
    return {B: float(np.mean(v)) for B, v in recalls.items()}


def _band_diff_ok(T_gpu, T_ora, ambiguous):
    """Positions selected on one side only must all be ambiguous."""
    diff = np.setxor1d(np.asarray(T_gpu, dtype=np.int64), np.asarray(T_ora, dtype=np.int64))
    return diff, bool(np.all(ambiguous[diff]))


def _check_against_oracle(batch, geo, blocks, Z, T_naive, c_naive, s_hard, T_hard, c_hard,
                          shape, sel, logits, stats):
    k = geo.top_k
    offs = batch.token_offsets.cpu().tolist()
    U = gh.U32
    for r in range(batch.q.shape[0]):
        n = int(batch.seq_lens[r])
        req = batch.requests[r]
        q, K = gh.np32(req.q), gh.np32(req.k)[:, :n]
        so = ora.select(q, K, k)
        z = so["z"]
        A = gh.tol.abs_dot(q, K)                        # [H][N] sum_d |q_d k_d|
        eb = 16.0 * U * A                               # fp32 logit band (decode logits check)
        # GPU logits within their band of the fp64 logits (the inputs of every selector)
        assert np.all(np.abs(Z[r] - z) <= eb + 1e-30), r
        # naive TopK: score = largest logit over the heads
        s_ora = z.max(axis=0)
        e_n = eb.max(axis=0)
        T_ora = ora.naive_topk(q, K, k)
        if k < n:
            order = np.lexsort((np.arange(n), -s_ora))
            kth = order[k - 1]
            amb = np.abs(s_ora - s_ora[kth]) <= 1e-4 * abs(s_ora[kth]) + e_n + e_n[kth]
        else:
            amb = np.zeros(n, dtype=bool)
        diff, ok = _band_diff_ok(T_naive[r, : c_naive[r]], T_ora, amb)
        assert ok, ("naive", r, diff[:10])
        gh.log(f"  naive r={r}: {len(diff)} positions differ from the fp64 oracle (all in band)")
        # head hard vote: per head, positions robustly inside / ambiguous at the head's cut
        H = z.shape[0]
        lo = np.zeros(n)
        amb_cnt = np.zeros(n)
        for h in range(H):
            if k >= n:
                lo += 1.0
                continue
            order = np.lexsort((np.arange(n), -z[h]))
            kth = order[k - 1]
            near = np.abs(z[h] - z[h, kth]) <= eb[h] + eb[h, kth]
            inside = np.zeros(n, dtype=bool)
            inside[order[:k]] = True
            lo += inside & ~near
            amb_cnt += near
        hi = lo + amb_cnt
        counts_gpu = s_hard[offs[r]: offs[r] + n].astype(np.float64)
        assert np.all((counts_gpu >= lo) & (counts_gpu <= hi)), ("hard vote counts", r)
        T_ora = ora.hard_vote_topk(z, k)
        if k < n:
            t_lo, t_hi = np.sort(lo)[::-1][k - 1], np.sort(hi)[::-1][k - 1]
            amb = (hi >= t_lo) & (lo <= t_hi)
        else:
            amb = np.zeros(n, dtype=bool)
        diff, ok = _band_diff_ok(T_hard[r, : c_hard[r]], T_ora, amb)
        assert ok, ("hard vote", r, diff[:10])
        gh.log(f"  hard vote r={r}: {len(diff)} positions differ from the fp64 oracle (all in band)")
        # block selection on the oracle's soft vote
        v = so["vote"]
        rel = gh.tol.vote_rel_budget(q, K, z, so["p"], so["M"], v)
        relf = np.where(np.isfinite(rel), rel, 0.0)
        for B in blocks:
            nb = -(-n // B)
            S_ora = ora.block_scores(v, B)
            # relative budget of a block sum: the vote-weighted mean of its tokens' budgets
            R = ora.block_scores(v * relf, B) / np.where(S_ora > 0, S_ora, 1.0)
            n_sel = max(1, k // B)
            T_ora = ora.block_topk(v, k, B)
            T_gpu = _block_select(shape, sel, B, logits, stats, batch, r)
            amb_blk = gh.tol.ambiguous_positions_log(S_ora, R, n_sel) if n_sel < nb else np.zeros(nb, bool)
            amb = np.repeat(amb_blk, B)[:n]
            diff, ok = _band_diff_ok(T_gpu, T_ora, amb)
            assert ok, ("block", B, r, diff[:10])
            gh.log(f"  block B={B} r={r}: {len(diff)} positions differ from the fp64 oracle (all in band)")


_BLOCK_RUNS = {}


def _block_select(shape, sel, B, logits, stats, batch, r):
    key = (id(logits), B)
    if key not in _BLOCK_RUNS:
        _BLOCK_RUNS.clear()
        nblk = sum(-(-int(batch.seq_lens[i]) // B) for i in range(batch.q.shape[0]))
        _BLOCK_RUNS[key] = _ablate(shape, sel, ts.SELECT_BLOCK, B, logits, stats, batch, nblk)
    _, T_blk, c_blk = _BLOCK_RUNS[key]
    return T_blk[r, : c_blk[r]]


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
