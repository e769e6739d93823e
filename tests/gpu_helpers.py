"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle, compare.

Comparison bands (fp32 arithmetic on the GPU against the fp64 oracle):
  logits   |z_gpu - z_ora| <= 16 u * score_scale * sum_d |q_d k_d| + 1e-30
  (a) vote the GPU returns lv = log2(v) in fp32; |lv ln2 - ln v_ora| <= 1e-4 + r_i +
      4u |lv ln2|, r_i = e_i / v_i the oracle's first-order relative fp32 budget
  (b) TopK the GPU set differs from the oracle set only at positions whose oracle
      vote is within that relative tolerance of the k-th vote; and, with the
      decision taken in the GPU's own precision, it is exactly the TopK of the
      GPU's fp32 log2 votes (ties to the lower position)
  (c) out  max-abs <= 1e-4 (fp32; plus the attention budget) or 2e-2 (bf16)
      against the oracle's attention over the GPU's own selected set
"""
from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

import token_level_sparse_amd as ts
from oracle import tokenselect_oracle as ora
from oracle import tolerance as tol
from synth import workloads as wl

U32 = 2.0 ** -24


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def np32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


@dataclass
class PathOut:
    logits: List[np.ndarray]      # per request [H][N_r]
    stats: np.ndarray             # [b][H][2]
    vote: List[np.ndarray]        # per request [N_r]
    T: List[np.ndarray]           # per request ascending TopK
    out: np.ndarray               # [b][H][d] (as fp32)
    raw: dict


def select_params(geo: wl.Geometry, top_k=None, n_local=None, score_scale=1.0, theta=None):
    return ts.make_select(geo.top_k if top_k is None else top_k,
                          geo.n_local if n_local is None else n_local,
                          score_scale, geo.attn_scale,
                          geo.cos_threshold if theta is None else theta)


def run_path(batch: wl.PagedBatch, geo: wl.Geometry, top_k=None, n_local=None,
             score_scale=1.0, max_total: Optional[int] = None, sel_override=None) -> PathOut:
    """Run score -> vote_topk -> sparse_attn through the C ABI on the batch."""
    b = batch.q.shape[0]
    total = batch.total_tokens
    max_total = max_total or total
    shape = ts.make_shape(geo.num_q_heads, geo.num_kv_heads, b, batch.block_table.shape[1],
                          max_total, geo.torch_dtype)
    sel = select_params(geo, top_k, n_local, score_scale)
    k = sel.top_k
    dev = batch.q.device
    ws = ts.alloc_workspace(shape, sel, dev)
    H = geo.num_q_heads
    logits = torch.full((H * max_total,), float("nan"), dtype=torch.float32, device=dev)
    stats = torch.full((b * H * 2,), float("nan"), dtype=torch.float32, device=dev)
    vote = torch.full((max_total,), float("nan"), dtype=torch.float32, device=dev)
    sel_idx = torch.full((b, k), -7, dtype=torch.int32, device=dev)
    sel_count = torch.full((b,), -7, dtype=torch.int32, device=dev)
    out = torch.full((b, H, geo.head_dim), float("nan"), dtype=geo.torch_dtype, device=dev)
    ts.score(shape, sel, batch.q, batch.k_pool, batch.block_table, batch.seq_lens, logits, stats, ws)
    ts.vote_topk(shape, sel, logits, stats, batch.seq_lens, vote, sel_idx, sel_count, ws)
    if sel_override is not None:
        sel_idx, sel_count = sel_override
    ts.sparse_attn(shape, sel, batch.q, batch.k_pool, batch.v_pool, batch.block_table,
                   batch.seq_lens, sel_idx, sel_count, out, ws)
    torch.cuda.synchronize()
    offs = batch.token_offsets.cpu().tolist()
    lens = batch.seq_lens.cpu().tolist()
    lg = logits.cpu().numpy()
    vt = vote.cpu().numpy()
    si = sel_idx.cpu().numpy()
    sc = sel_count.cpu().numpy()
    L, V, T = [], [], []
    for r in range(b):
        n = lens[r]
        G = H // geo.num_kv_heads
        blk = lg[offs[r] * H: offs[r] * H + H * n].reshape(geo.num_kv_heads, n, G)
        L.append(np.ascontiguousarray(blk.transpose(0, 2, 1)).reshape(H, n))
        V.append(vt[offs[r]: offs[r] + n])
        assert sc[r] == min(k, n), (r, sc[r], k, n)
        T.append(si[r, : sc[r]].astype(np.int64))
    return PathOut(L, stats.cpu().numpy().reshape(b, H, 2), V, T, np32(out),
                   dict(logits=logits, vote=vote, sel_idx=sel_idx, sel_count=sel_count, out=out))


def check_logits(z_gpu, q, K, ref, score_scale=1.0, factor=16.0):
    A = tol.abs_dot(q, K)
    lim = factor * U32 * abs(score_scale) * A + 1e-30
    err = np.abs(z_gpu.astype(np.float64) - ref)
    bad = err > lim
    assert not bad.any(), f"logits: {bad.sum()} outside, worst excess {np.max(err - lim):.3e}"


def check_stats(stats_gpu, sel_ora, q, K, score_scale=1.0):
    """M_h within the logit band; Z_h within a relative 1e-4 plus the fp32 budget."""
    A = tol.abs_dot(q, K)
    for h in range(q.shape[0]):
        M, Z = stats_gpu[h]
        i = int(np.argmax(sel_ora["z"][h]))
        assert abs(M - sel_ora["M"][h]) <= 16 * U32 * score_scale * A[h, i] + 1e-30, (h, M, sel_ora["M"][h])
        bz = 4 * U32 * np.sum(sel_ora["p"][h] * (np.abs(sel_ora["z"][h]) + abs(sel_ora["M"][h])
                                                  + score_scale * A[h]))
        assert abs(Z - sel_ora["Z"][h]) <= 1e-4 * sel_ora["Z"][h] + bz * sel_ora["Z"][h], (h, Z, sel_ora["Z"][h])


def check_vote(lv_gpu, sel_ora, q, K, score_scale=1.0):
    rel = tol.vote_rel_budget(q, K, sel_ora["z"], sel_ora["p"], sel_ora["M"], sel_ora["vote"],
                              score_scale)
    ok, excess = tol.log_vote_within(lv_gpu, sel_ora["vote"], rel)
    assert ok.all(), f"vote: {(~ok).sum()} outside band (a), worst excess {excess.max():.3e}"
    v = sel_ora["vote"]
    strict = np.abs(np.exp2(lv_gpu.astype(np.float64)) - v) <= 1e-4 * v
    return rel, int((~strict).sum())


def check_topk(T_gpu, lv_gpu, sel_ora, rel, k):
    N = len(lv_gpu)
    assert np.all(np.diff(T_gpu) > 0), "TopK not strictly ascending"
    assert len(T_gpu) == min(k, N)
    assert T_gpu.min() >= 0 and T_gpu.max() < N
    # the decision in the GPU's own precision: exact TopK of its fp32 log2 votes
    exact = ora.topk_indices(lv_gpu.astype(np.float64), k)
    assert np.array_equal(T_gpu, exact), "TopK differs from the exact TopK of the GPU votes"
    amb = tol.ambiguous_positions_log(sel_ora["vote"], rel, k)
    diff = np.setxor1d(T_gpu, sel_ora["T"])
    assert np.all(amb[diff]), f"TopK differs from the oracle outside band (b) at {diff[~amb[diff]][:10]}"
    return len(diff)


def check_attention(out_gpu, q, K, V, T_gpu, N, n_local, attn_scale, fp32: bool):
    S = ora.union_local(T_gpu, N, n_local)
    ref = ora.sparse_attention(q, K, V, S, attn_scale)
    err = np.abs(out_gpu.astype(np.float64) - ref)
    if fp32:
        lim = 1e-4 + tol.attn_budget(q, K, V, S, attn_scale, ref)
    else:
        lim = 2e-2
    assert np.all(err <= lim), f"attention max-abs {err.max():.3e} (limit {np.max(lim):.3e})"
    return float(err.max())


def check_request(po: PathOut, r: int, req: wl.Request, geo: wl.Geometry, top_k=None,
                  n_local=None, score_scale=1.0):
    k = geo.top_k if top_k is None else top_k
    L = geo.n_local if n_local is None else n_local
    q, K, V = np32(req.q), np32(req.k), np32(req.v)
    sel = ora.select(q, K, k, score_scale)
    check_logits(po.logits[r], q, K, sel["z"], score_scale)
    check_stats(po.stats[r], sel, q, K, score_scale)
    rel, n_loose = check_vote(po.vote[r], sel, q, K, score_scale)
    n_diff = check_topk(po.T[r], po.vote[r], sel, rel, k)
    err = check_attention(po.out[r], q, K, V, po.T[r], K.shape[1], L, geo.attn_scale,
                          geo.dtype == "f32")
    # n_loose: votes outside a strict relative 1e-4 (inside band (a) through the fp32
    # budget r_i); max_r: the largest finite r_i of the request; n_under: positions whose
    # fp64 vote underflows to 0 (their r_i is unbounded: only the log-domain band applies)
    fin = np.isfinite(rel)
    return dict(n_loose=n_loose, max_r=float(np.max(rel[fin])) if fin.any() else 0.0,
                n_under=int((~fin).sum()), n_diff=n_diff, attn_err=err)


# ---------------------------------------------------------------- chunk-wise prefill
@dataclass
class PrefillOut:
    logits: List[np.ndarray]      # per request [H][P_r]
    stats: np.ndarray             # [b][H][2]
    vote: List[np.ndarray]        # per request [P_r]
    T: List[np.ndarray]           # per request ascending TopK over the past
    out: np.ndarray               # [b][max_chunk][H][d] (fp32 copy)
    raw: dict


def run_prefill(cb: wl.ChunkBatch, geo: wl.Geometry, top_k=None, n_local=None, score_scale=1.0,
                sel_override=None) -> PrefillOut:
    """prefill_select then chunk_attn through the C ABI; also runs prefill_chunk and
    checks that the one-call path gives bit-identical TopK and outputs."""
    pb = cb.paged
    b = pb.q.shape[0]
    H, d = geo.num_q_heads, geo.head_dim
    mc = cb.q_chunk.shape[1]
    lens = cb.seq_lens.cpu().tolist()
    past = [n - c for n, c in zip(lens, cb.chunk_lens.cpu().tolist())]
    # a capacity: at least the chunk capacity, which the ABI requires (max_chunk <= max_total_tokens)
    max_total = max(sum(lens), b, mc)
    shape = ts.make_shape(H, geo.num_kv_heads, b, pb.block_table.shape[1], max_total, geo.torch_dtype)
    sel = select_params(geo, top_k, n_local, score_scale)
    k = sel.top_k
    dev = pb.q.device
    ws = ts.alloc_prefill_workspace(shape, sel, mc, dev)
    logits = torch.full((H * max_total,), float("nan"), dtype=torch.float32, device=dev)
    stats = torch.full((b * H * 2,), float("nan"), dtype=torch.float32, device=dev)
    vote = torch.full((max_total,), float("nan"), dtype=torch.float32, device=dev)
    sel_idx = torch.full((b, k), -7, dtype=torch.int32, device=dev)
    sel_count = torch.full((b,), -7, dtype=torch.int32, device=dev)
    out = torch.full((b, mc, H, d), float("nan"), dtype=geo.torch_dtype, device=dev)
    ts.prefill_select(shape, sel, mc, cb.q_chunk, cb.chunk_lens, pb.k_pool, pb.block_table, cb.seq_lens,
                      logits, stats, vote, sel_idx, sel_count, ws)
    si, sc = (sel_idx, sel_count) if sel_override is None else sel_override
    ts.chunk_attn(shape, sel, mc, cb.q_chunk, cb.chunk_lens, pb.k_pool, pb.v_pool, pb.block_table,
                  cb.seq_lens, si, sc, out, ws)
    # one-call path on a fresh workspace
    ws2 = ts.alloc_prefill_workspace(shape, sel, mc, dev)
    sel_idx2 = torch.full((b, k), -9, dtype=torch.int32, device=dev)
    sel_count2 = torch.full((b,), -9, dtype=torch.int32, device=dev)
    out2 = torch.full((b, mc, H, d), float("nan"), dtype=geo.torch_dtype, device=dev)
    ts.prefill_chunk(shape, sel, mc, cb.q_chunk, cb.chunk_lens, pb.k_pool, pb.v_pool, pb.block_table,
                     cb.seq_lens, sel_idx2, sel_count2, out2, ws2)
    torch.cuda.synchronize()
    assert torch.equal(sel_count, sel_count2)
    for r in range(b):
        n = int(sel_count[r])
        assert torch.equal(sel_idx[r, :n], sel_idx2[r, :n])
    if sel_override is None:
        assert torch.equal(out.view(torch.uint8) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                           out2.view(torch.uint8) if out2.dtype == torch.bfloat16 else out2.view(torch.int32)), \
            "prefill_chunk differs from prefill_select + chunk_attn"
    lg, vt = logits.cpu().numpy(), vote.cpu().numpy()
    si_h, sc_h = sel_idx.cpu().numpy(), sel_count.cpu().numpy()
    G = H // geo.num_kv_heads
    L, V, T = [], [], []
    off = 0
    for r in range(b):
        P = past[r]
        blk = lg[off * H: off * H + H * P].reshape(geo.num_kv_heads, P, G)
        L.append(np.ascontiguousarray(blk.transpose(0, 2, 1)).reshape(H, P))
        V.append(vt[off: off + P])
        assert sc_h[r] == min(k, P), (r, sc_h[r], k, P)
        T.append(si_h[r, : sc_h[r]].astype(np.int64))
        off += P
    return PrefillOut(L, stats.cpu().numpy().reshape(b, H, 2), V, T, np32(out),
                      dict(sel_idx=sel_idx, sel_count=sel_count, out=out))


def check_prefill_selection(po: PrefillOut, r: int, cb: wl.ChunkBatch, geo: wl.Geometry, top_k=None,
                            score_scale=1.0):
    """Logits, stats, votes and TopK of request r against the oracle run with the
    exact fp64 mean query over the past."""
    from oracle import prefill_oracle as pre
    k = geo.top_k if top_k is None else top_k
    req = cb.paged.requests[r]
    c = int(cb.chunk_lens[r])
    P = int(cb.seq_lens[r]) - c
    if P == 0:
        assert po.T[r].size == 0
        return dict(n_diff=0)
    Qc = np32(cb.q_chunk[r, :c])
    K = np32(req.k[:, :P])
    qbar = pre.chunk_mean_query(Qc)
    sel = ora.select(qbar, K, k, score_scale)
    check_logits(po.logits[r], qbar, K, sel["z"], score_scale)
    check_stats(po.stats[r], sel, qbar, K, score_scale)
    rel, n_loose = check_vote(po.vote[r], sel, qbar, K, score_scale)
    n_diff = check_topk(po.T[r], po.vote[r], sel, rel, k)
    return dict(n_diff=n_diff, n_loose=n_loose, T_ora=sel["T"])


def check_chunk_attention(po: PrefillOut, r: int, cb: wl.ChunkBatch, geo: wl.Geometry, T,
                          n_local=None, rows=None, fp32_factor=1.0):
    """Chunk attention of request r (rows j of the chunk, all by default) against the
    oracle over the attended sets built from T."""
    from oracle import prefill_oracle as pre
    L = geo.n_local if n_local is None else n_local
    req = cb.paged.requests[r]
    c = int(cb.chunk_lens[r])
    N = int(cb.seq_lens[r])
    P = N - c
    K, V = np32(req.k[:, :N]), np32(req.v[:, :N])
    Qc = np32(cb.q_chunk[r, :c])
    sets = pre.chunk_sets(T, P, c, L)
    fp32 = geo.dtype == "f32"
    worst = 0.0
    for j in (range(c) if rows is None else rows):
        ref = ora.sparse_attention(Qc[j], K, V, sets[j], geo.attn_scale)
        err = np.abs(po.out[r, j].astype(np.float64) - ref)
        if fp32:
            lim = 1e-4 + fp32_factor * tol.attn_budget(Qc[j], K, V, sets[j], geo.attn_scale, ref)
        else:
            lim = 2e-2
        assert np.all(err <= lim), f"chunk row {j}: max-abs {err.max():.3e} (limit {np.max(lim):.3e})"
        worst = max(worst, float(err.max()))
    # rows past the chunk are untouched
    if c < po.out.shape[1]:
        assert np.isnan(po.out[r, c:]).all(), "rows past the chunk were written"
    return worst
