"""First-order fp32 error budgets used when comparing a GPU run with the oracle.

TEST INFRASTRUCTURE ONLY (same import rule as the oracle module).

The selection softmax runs on raw inner products, whose magnitude grows with
the per-head key scale. A logit computed in fp32 carries an absolute error of
about u * sum_d |q_d k_d| (u = 2^-24), and a softmax weight inherits that
absolute logit error as a relative error. For keys scaled by up to 1000 the raw
logits reach ~1e5, so an elementwise relative 1e-4 bound is below what fp32
can deliver for tokens whose vote comes from mid-weight contributions of the
large-scale heads. The budgets below add that first-order term to the relative
bound; fp32 underflow (the oracle keeps values down to 1e-308, fp32 flushes
below 2^-126) adds H * 2^-126.
"""
from __future__ import annotations

import numpy as np

U32 = 2.0 ** -24
FP32_TINY = 2.0 ** -126


def abs_dot(q, K) -> np.ndarray:
    """A[h][i] = sum_d |q_hd| * |K_{g(h)}[i][d]| (G = H / H_kv contiguous groups)."""
    q = np.abs(np.asarray(q, dtype=np.float64))
    H = q.shape[0]
    Hkv, N, _ = K.shape
    G = H // Hkv
    out = np.empty((H, N), dtype=np.float64)
    for g in range(Hkv):
        Kg = np.abs(np.asarray(K[g], dtype=np.float64))
        out[g * G:(g + 1) * G] = (Kg @ q[g * G:(g + 1) * G].T).T
    return out


def vote_budget(q, K, z, p, M, score_scale: float = 1.0) -> np.ndarray:
    """e_i = 4u * sum_h p_h(i) (|z_hi| + |M_h| + score_scale * A_hi) + H * 2^-126."""
    A = abs_dot(q, K)
    H = p.shape[0]
    t = p * (np.abs(z) + np.abs(M)[:, None] + abs(score_scale) * A)
    return 4.0 * U32 * t.sum(axis=0) + H * FP32_TINY


def vote_within(v_gpu, v_ora, budget, rel: float = 1e-4):
    """Band (a): |v_gpu - v_ora| <= rel * v_ora + e_i, elementwise. Returns (ok mask, excess)."""
    v_gpu = np.asarray(v_gpu, dtype=np.float64)
    err = np.abs(v_gpu - v_ora)
    lim = rel * np.abs(v_ora) + budget
    return err <= lim, err - lim


def ambiguous_positions(v_ora, budget, k: int, rel: float = 1e-4) -> np.ndarray:
    """Band (b): positions whose oracle vote lies within tolerance of the k-th vote.

    Position i is ambiguous if |v(i) - v(k-th)| <= rel * v(k-th) + e_i + e_k, with
    e_k the budget of the k-th position itself. Returns a boolean mask.
    """
    v = np.asarray(v_ora, dtype=np.float64)
    N = v.shape[0]
    if k >= N:
        return np.zeros(N, dtype=bool)
    order = np.lexsort((np.arange(N), -v))
    kth = order[k - 1]
    vk = v[kth]
    return np.abs(v - vk) <= rel * abs(vk) + budget + budget[kth]


def attn_budget(q, K, V, S, attn_scale: float, out) -> np.ndarray:
    """fp32 first-order budget of sparse attention, per (head, dim).

    b[h][d] = sum_{i in S} w_i * c_i * |V_i[d] - o[h][d]| with
    c_i = 4u * (attn_scale * A_hi + |a_i| + |a_max|).
    """
    q = np.asarray(q, dtype=np.float64)
    H, d = q.shape
    Hkv = K.shape[0]
    G = H // Hkv
    S = np.asarray(S, dtype=np.int64)
    b = np.empty((H, d), dtype=np.float64)
    for h in range(H):
        g = h // G
        Ks = np.asarray(K[g][S], dtype=np.float64)
        Vs = np.asarray(V[g][S], dtype=np.float64)
        a = attn_scale * (Ks @ q[h])
        A = attn_scale * (np.abs(Ks) @ np.abs(q[h]))
        w = np.exp(a - a.max())
        w /= w.sum()
        c = 4.0 * U32 * (A + np.abs(a) + np.abs(a.max()))
        b[h] = (w * c) @ np.abs(Vs - out[h][None, :])
    return b


# ---------------------------------------------------------------- log-domain votes
# A GPU path that keeps the vote as lv = log2(v) does not underflow, so its votes
# are compared in the log domain with a relative budget and no underflow term.
LN2 = 0.6931471805599453


FP64_TINY = 2.0 ** -1074


def vote_rel_budget(q, K, z, p, M, v, score_scale: float = 1.0) -> np.ndarray:
    """Relative error budget of a vote, r_i (inf where v_i == 0).

    r_i = (4u * sum_h p_h(i) (|z_hi| + |M_h| + score_scale A_hi) + H * 2^-1074) / v_i.
    The first term is the fp32 logit error carried into each head weight; the
    second is the oracle's own fp64 underflow: a head weight below 2^-1022 is a
    subnormal with absolute spacing 2^-1074, so votes near 2^-1074 carry only a
    few significant bits in the oracle.
    """
    A = abs_dot(q, K)
    H = p.shape[0]
    t = (p * (np.abs(z) + np.abs(M)[:, None] + abs(score_scale) * A)).sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(v > 0, (4.0 * U32 * t + H * FP64_TINY) / np.where(v > 0, v, 1.0), np.inf)
    return r


def log_vote_within(lv2_gpu, v_ora, rel, rel_tol: float = 1e-4):
    """Band (a) in the log domain: |lv2 ln2 - ln v| <= rel_tol + r_i + 4u |lv2 ln2|.

    Where the fp64 vote underflows to 0 the GPU's log2 vote must lie below -1000.
    Returns (ok mask, excess).
    """
    lg = np.asarray(lv2_gpu, dtype=np.float64) * LN2
    v = np.asarray(v_ora, dtype=np.float64)
    pos = v > 0
    with np.errstate(divide="ignore"):
        lo = np.where(pos, np.log(np.where(pos, v, 1.0)), -np.inf)
    lim = rel_tol + np.where(np.isfinite(rel), rel, 0.0) + 4.0 * U32 * np.abs(lg)
    err = np.where(pos, np.abs(lg - lo), 0.0)
    ok = np.where(pos, err <= lim, lv2_gpu < -1000.0)
    return ok, np.where(pos, err - lim, 0.0)


def ambiguous_positions_log(v_ora, rel, k: int, rel_tol: float = 1e-4) -> np.ndarray:
    """Band (b) in the log domain: |ln v_i - ln v_k| <= rel_tol + r_i + r_k + 4u(|ln v_i| + |ln v_k|).

    v_k is the oracle's k-th largest vote. If it underflowed to 0, every zero vote
    ties with it.
    """
    v = np.asarray(v_ora, dtype=np.float64)
    N = v.shape[0]
    if k >= N:
        return np.zeros(N, dtype=bool)
    order = np.lexsort((np.arange(N), -v))
    kth = order[k - 1]
    if v[kth] == 0.0:
        return v == 0.0
    with np.errstate(divide="ignore"):
        lv = np.where(v > 0, np.log(np.where(v > 0, v, 1.0)), -np.inf)
    r = np.where(np.isfinite(rel), rel, 0.0)
    lim = rel_tol + r + r[kth] + 4.0 * U32 * (np.abs(lv) + abs(lv[kth]))
    return (v > 0) & (np.abs(lv - lv[kth]) <= lim)
