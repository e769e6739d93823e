"""Plain fp64 CPU oracle for the TokenSelect decode step.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module. The product path never
calls it, and it shares no code with the HIP kernels: it reads the logical
(unpaged) arrays the seeded generator draws, converts them to float64 and
follows the pages' definitions step by step, with numpy matmul, exp and sort
as the only library primitives.

Sources (pages of the reference set):
  [DN] "TokenSelect: Efficient Long-Context Inference and Length Extrapolation
       for LLMs via Dynamic Token-Level KV Cache Selection" (papercache
       deepnotes page). Sections: selective sparse attention formalisation
       (SDPA output O and the selected-token output O-hat); selection-function
       design (naive TopK over Q.K^T and the head hard vote); head soft vote
       (T_head-soft-vote = TopK(sum_h softmax(Q^h . K_cache^h^T))); decode
       selection frequency (Selection Cache); appendix Algorithm 1 (Selection
       Cache) and Algorithm 2 (Paged Dot Product Kernel).
  [BL] "TokenSelect: ... 128K->1M 23.84x" (ai-paper-analysis blog page).
       Section 3.1 (head soft vote), section 3.2 (Algorithm 1, Selection
       Cache), section 4.2 / Table 2 (a budget of 2K selected plus 512 local tokens).

Readings taken where the pages are silent (each is listed in the design notes):
  * selection softmax has no 1/sqrt(d): the printed vote equation applies the
    softmax to the raw inner products; ``score_scale`` stays a parameter;
  * GQA: query head h reads KV head h // (H / H_kv); the vote sums all H query
    heads, so the votes sum to H;
  * TopK runs over all N positions; ties go to the lower position; the result
    is returned in ascending order; k >= N selects everything;
  * the selected set is TopK united with the window [N - max(L, 1), N),
    deduplicated: the current token is attended even with L = 0;
  * attention covers the N cached tokens including the current one, with
    scale 1/sqrt(d), no causal mask (a single decode query);
  * the Selection Cache compares with the query stored at the last miss
    (Algorithm 1 stores Q only when it reselects); hit iff cos >= theta; the
    first query, or a zero-norm query, misses; a hit reuses only the TopK part,
    the local window is rebuilt from the current N every step.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- step 1
def score_logits(q, K, score_scale: float = 1.0) -> np.ndarray:
    """Per-head token criticality z[h][i] = score_scale * <q_h, K_{g(h)}[i]>.

    [DN] Algorithm 2 (Paged Dot Product Kernel) computes, per head, the inner
    product of the head's query with every cached key; [DN] head soft vote
    feeds Q^h . K_cache^h^T to the softmax. ``q`` is [H][d], ``K`` is
    [H_kv][N][d]; query head h uses KV head h // G with G = H / H_kv.
    """
    q = _f64(q)
    H, d = q.shape
    Hkv, N, dk = K.shape
    assert dk == d and H % Hkv == 0
    G = H // Hkv
    z = np.empty((H, N), dtype=np.float64)
    for g in range(Hkv):
        Kg = _f64(K[g])                        # [N][d]
        z[g * G:(g + 1) * G] = (Kg @ q[g * G:(g + 1) * G].T).T
    z *= score_scale
    return z


# ---------------------------------------------------------------- step 2
def head_softmax(z) -> tuple:
    """Per-head softmax over all N cached tokens.

    [DN] head soft vote: each head's criticality row is normalised by the
    softmax sigma before the heads are summed. Returns (p, M, Z) with
    M_h = max_i z[h][i], Z_h = sum_i exp(z[h][i] - M_h), p = exp(z - M) / Z.
    """
    z = _f64(z)
    M = z.max(axis=1)
    e = np.exp(z - M[:, None])
    Z = e.sum(axis=1)
    return e / Z[:, None], M, Z


# ---------------------------------------------------------------- step 3
def soft_vote(p) -> np.ndarray:
    """v_i = sum over the H query heads of p[h][i] ([DN] head soft vote)."""
    return _f64(p).sum(axis=0)


# ---------------------------------------------------------------- step 4
def topk_indices(v, k: int) -> np.ndarray:
    """TopK of the vote: the k largest entries, ties to the lower position.

    [DN] head soft vote (TopK of the summed normalised scores). Returned in
    ascending position order. k >= N returns every position.
    """
    v = _f64(v)
    N = v.shape[0]
    if k >= N:
        return np.arange(N, dtype=np.int64)
    order = np.lexsort((np.arange(N), -v))     # v descending, then position ascending
    return np.sort(order[:k]).astype(np.int64)


def union_local(T, N: int, n_local: int) -> np.ndarray:
    """Selected set S = TopK result united with the last max(n_local, 1) positions.

    [BL] section 4.2 and [DN] results paragraph: the budget is k selected
    tokens plus a window of recent local tokens. [DN] selective sparse
    attention formalisation: the attended keys are [K_select, K_current], so
    the current token (position N - 1) belongs to S whatever the window size;
    with n_local = 0 the window is that one position. Ascending, no duplicates.
    """
    width = max(n_local, 1)
    win = np.arange(max(0, N - width), N, dtype=np.int64)
    return np.union1d(np.asarray(T, dtype=np.int64), win)


def select(q, K, k: int, score_scale: float = 1.0) -> dict:
    """Selection function S(Q, k) by head soft vote: steps 1-4 (TopK part)."""
    z = score_logits(q, K, score_scale)
    p, M, Z = head_softmax(z)
    v = soft_vote(p)
    T = topk_indices(v, k)
    return {"z": z, "p": p, "M": M, "Z": Z, "vote": v, "T": T}


def naive_topk(q, K, k: int, score_scale: float = 1.0) -> np.ndarray:
    """Ablation baseline: TopK over the raw logits of all heads at once.

    [DN] selection-function design, T_topk = TopK(Q . K_cache^T). A position's
    score is its largest raw logit over the H heads (the concatenated logits
    reduced to positions). Ascending output.
    """
    return naive_topk_from_logits(score_logits(q, K, score_scale), k)


def naive_topk_from_logits(z, k: int) -> np.ndarray:
    """The naive TopK's selection step on given logits [H][N]: each position scores
    its largest logit over the heads."""
    return topk_indices(_f64(z).max(axis=0), k)


# ---------------------------------------------------------------- step 5
def sparse_attention(q, K, V, S, attn_scale: float) -> np.ndarray:
    """Scaled dot-product attention over the selected positions S only.

    [DN] selective sparse attention formalisation: O-hat uses the softmax of
    Q^h [K_select, K_current]^T / sqrt(d) times [V_select, V_current] per head.
    ``S`` already contains the current token (the window's last position).
    Returns o [H][d].
    """
    q = _f64(q)
    H, d = q.shape
    Hkv = K.shape[0]
    G = H // Hkv
    S = np.asarray(S, dtype=np.int64)
    out = np.empty((H, d), dtype=np.float64)
    for h in range(H):
        g = h // G
        Ks = _f64(K[g][S])
        Vs = _f64(V[g][S])
        a = attn_scale * (Ks @ q[h])
        w = np.exp(a - a.max())
        w /= w.sum()
        out[h] = w @ Vs
    return out


def dense_attention(q, K, V, attn_scale: float) -> np.ndarray:
    """Full SDPA over all N tokens ([DN] formalisation, output O)."""
    return sparse_attention(q, K, V, np.arange(K.shape[1]), attn_scale)


def decode_step(q, K, V, k: int, n_local: int, score_scale: float = 1.0,
                attn_scale: Optional[float] = None) -> dict:
    """One decode step without the cache: select, add the window, attend."""
    d = q.shape[-1]
    if attn_scale is None:
        attn_scale = 1.0 / math.sqrt(d)
    N = K.shape[1]
    sel = select(q, K, k, score_scale)
    S = union_local(sel["T"], N, n_local)
    sel["S"] = S
    sel["out"] = sparse_attention(q, K, V, S, attn_scale)
    return sel


# ---------------------------------------------------------------- step 0
@dataclass
class CacheState:
    """Selection Cache state: validity flag, C_Q and C_T ([DN] Algorithm 1)."""

    valid: bool = False
    cq: Optional[np.ndarray] = None     # fp64, the concatenated query of the last miss
    ct: Optional[np.ndarray] = None     # TopK positions chosen at the last miss


def cache_cosine(Q, CQ) -> float:
    """cos(Q, C_Q) over the concatenated heads, in fp64; nan if a norm is 0."""
    a = _f64(Q).reshape(-1)
    b = _f64(CQ).reshape(-1)
    na = math.sqrt(float(a @ a))
    nb = math.sqrt(float(b @ b))
    if na == 0.0 or nb == 0.0:
        return float("nan")
    return float(a @ b) / (na * nb)


def cache_lookup(state: CacheState, Q, theta: float) -> tuple:
    """Algorithm 1's test: reuse iff the cache holds a query and cos >= theta.

    [DN] appendix Algorithm 1 and [BL] section 3.2: a first query, or
    cos(Q, C_Q) < theta, reselects. A zero-norm query (cosine undefined)
    reselects. Returns (hit, cos).
    """
    if not state.valid:
        return False, float("nan")
    c = cache_cosine(Q, state.cq)
    if math.isnan(c):
        return False, c
    return c >= theta, c


def decode_sequence(qs, K, V, lens, k: int, n_local: int, theta: float,
                    score_scale: float = 1.0, attn_scale: Optional[float] = None,
                    want_outputs: bool = True) -> dict:
    """Consecutive decode steps under the Selection Cache ([DN] Algorithm 1).

    ``qs`` is [steps][H][d]; step t attends the first lens[t] positions of
    K/V (the pool only grows). On a miss the selection is recomputed at the
    current length and C_Q, C_T are replaced; on a hit C_T is reused. The
    window is rebuilt from lens[t] every step.
    """
    d = qs.shape[-1]
    if attn_scale is None:
        attn_scale = 1.0 / math.sqrt(d)
    state = CacheState()
    hits, coss, Ts, outs = [], [], [], []
    for t in range(len(qs)):
        N = int(lens[t])
        Kt, Vt = K[:, :N], V[:, :N]
        hit, c = cache_lookup(state, qs[t], theta)
        if not hit:
            T = select(qs[t], Kt, k, score_scale)["T"]
            state = CacheState(valid=True, cq=_f64(qs[t]).reshape(-1).copy(), ct=T)
        T = state.ct
        hits.append(bool(hit))
        coss.append(c)
        Ts.append(T)
        if want_outputs:
            outs.append(sparse_attention(qs[t], Kt, Vt, union_local(T, N, n_local), attn_scale))
    return {"hit": np.array(hits), "cos": np.array(coss), "T": Ts,
            "out": np.array(outs) if want_outputs else None}


# ---------------------------------------------------------------- dynamic top-p budget
def topp_count(v, p: float, k_max: int) -> int:
    """Budget of the dynamic top-p selection: the smallest m such that the m largest
    votes (ties to the lower position) hold at least p of the total vote mass,
    capped at k_max and at N.

    RTPurbo team post, dynamic token selection: keep the tokens whose cumulative
    score mass reaches p instead of a fixed top-k; UniPrefill page: keep the minimal
    set whose importance sum reaches 99% of the total. Applied to the head soft vote
    (total mass H). 0 < p <= 1.
    """
    v = _f64(v)
    N = v.shape[0]
    if N == 0:
        return 0
    order = np.lexsort((np.arange(N), -v))
    csum = np.cumsum(v[order])
    target = p * csum[-1]
    m = int(np.searchsorted(csum, target, side="left")) + 1
    return min(m, k_max, N)


def topp_indices(v, p: float, k_max: int) -> np.ndarray:
    """The dynamic top-p set: the topp_count(v, p, k_max) largest votes, ascending."""
    return topk_indices(v, topp_count(v, p, k_max))


# ---------------------------------------------------------------- selection-function ablations
def hard_vote_topk(z, k: int) -> np.ndarray:
    """Head hard vote: every head takes its own TopK of its raw logits, a position
    scores the number of heads that picked it, and the TopK of those counts is the
    selection (ties to the lower position, ascending).

    [DN] selection-function design: T_head-vote = TopK(sum_h I(i in TopK(Q^h K^h^T))),
    the improvement over the naive TopK that keeps the heads independent.
    """
    z = _f64(z)
    H, N = z.shape
    counts = np.zeros(N, dtype=np.float64)
    for h in range(H):
        counts[topk_indices(z[h], k)] += 1.0
    return topk_indices(counts, k)


def block_scores(v, block: int) -> np.ndarray:
    """Block criticality for block-level selection: the sum of the head soft votes of
    the block's positions (blocks of ``block`` consecutive positions, the last one
    possibly shorter)."""
    v = _f64(v)
    N = v.shape[0]
    nb = -(-N // block)
    pad = np.zeros(nb * block)
    pad[:N] = v
    return pad.reshape(nb, block).sum(axis=1)


def block_topk(v, k: int, block: int) -> np.ndarray:
    """Block-level selection with a budget of k tokens: the max(1, k // block) blocks
    of largest summed vote (ties to the lower block), expanded to their positions,
    ascending. block = 1 is the token-level TopK.

    [DN] token-level motivation (Fig. 2b) and [BL] section 2: prior methods split
    the cache into non-overlapping blocks and select blocks by an estimated
    criticality; a block with one critical token is kept whole and a critical token
    in a low-scoring block is lost.
    """
    N = len(v)
    nb_sel = max(1, k // block)
    blocks = topk_indices(block_scores(v, block), nb_sel)
    pos = (blocks[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    return pos[pos < N].astype(np.int64)


def recall(selected, reference) -> float:
    """Fraction of the reference positions that the selection contains."""
    reference = np.asarray(reference)
    if reference.size == 0:
        return 1.0
    return float(np.isin(reference, np.asarray(selected)).mean())
