"""Plain fp64 CPU oracle for chunk-wise prefill selection.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module. It shares no code with
the HIP kernels; it reads the logical (unpaged) arrays the seeded generator
draws and follows the pages step by step in numpy float64.

Sources (pages of the reference set):
  [DN] "TokenSelect: Efficient Long-Context Inference and Length Extrapolation
       for LLMs via Dynamic Token-Level KV Cache Selection" (papercache
       deepnotes page), section on the selection frequency of the prefill
       stage: the c queries of a chunk Q_C are averaged, (1/c) sum_i (Q_C)_i,
       and that single mean query goes through the selection function, so the
       whole chunk shares one selection.
  [BL] the ai-paper-analysis blog review of the same paper, section 3.2 (last
       paragraph): prefill does not use the Selection Cache; it selects once per
       chunk from the mean of the chunk's c queries and the chunk shares it.
       Section 3.3, Fig. 5: the chunk-prefill step studied there has chunk
       size 512, 128K cached tokens and 4K attended tokens.

Readings taken where the pages are silent (each is listed in the design notes):
  * the chunk's tokens occupy positions [P, P + c) of the request's cache, the
    P earlier positions are the past; the selection (score, per-head softmax,
    head soft vote, TopK) runs over the past only, with the mean query;
  * the local window is the L past positions just before the chunk,
    [max(0, P - L), P), shared by the whole chunk like the TopK;
  * chunk query j (position P + j) attends the TopK, the window and the chunk
    positions [P, P + j] (causal inside the chunk), i.e. the selected set
    T united with the contiguous range [max(0, P - L), P + j];
  * attention scale 1/sqrt(d); the selection softmax uses the raw inner
    products times score_scale, as in the decode step;
  * P = 0 (the first chunk of a prompt) selects nothing and the chunk attends
    causally to itself only.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from oracle import tokenselect_oracle as ora


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def chunk_mean_query(Qc) -> np.ndarray:
    """Mean of the chunk's c queries, per head: (1/c) sum_j Qc[j].

    [DN] prefill selection frequency: the c x d query block of a chunk is
    averaged into one query before the selection function. ``Qc`` is
    [c][H][d]; returns [H][d].
    """
    Qc = _f64(Qc)
    c = Qc.shape[0]
    assert c >= 1
    return Qc.sum(axis=0) / c


def prefill_select(Qc, K, P: int, k: int, score_scale: float = 1.0) -> dict:
    """Selection of a chunk: the decode selection function run with the mean
    query over the P past positions of K ([DN] prefill selection frequency,
    [DN] head soft vote). Returns the decode oracle's dict plus "qbar"; with
    P = 0 the TopK is empty."""
    qbar = chunk_mean_query(Qc)
    if P == 0:
        return {"qbar": qbar, "T": np.zeros(0, dtype=np.int64)}
    sel = ora.select(qbar, K[:, :P], k, score_scale)
    sel["qbar"] = qbar
    return sel


def chunk_sets(T, P: int, c: int, n_local: int) -> list:
    """Attended positions of each chunk query j: T united with the range
    [max(0, P - L), P + j] (window before the chunk plus the causal part of the
    chunk), ascending and without duplicates."""
    T = np.asarray(T, dtype=np.int64)
    w0 = max(0, P - n_local)
    return [np.union1d(T, np.arange(w0, P + j + 1, dtype=np.int64)) for j in range(c)]


def chunk_attention(Qc, K, V, T, P: int, n_local: int, attn_scale: float) -> np.ndarray:
    """SDPA of every chunk query over its attended set ([DN] selective sparse
    attention formalisation, with the chunk's causal structure). ``Qc`` is
    [c][H][d], K and V are [H_kv][P + c][d]; returns [c][H][d]."""
    Qc = _f64(Qc)
    c = Qc.shape[0]
    sets = chunk_sets(T, P, c, n_local)
    return np.stack([ora.sparse_attention(Qc[j], K, V, sets[j], attn_scale) for j in range(c)])


def prefill_chunk(Qc, K, V, P: int, k: int, n_local: int, score_scale: float = 1.0,
                  attn_scale: Optional[float] = None) -> dict:
    """One chunk of prefill: select from the past with the mean query, then
    attend every chunk query over TopK, window and the causal chunk part."""
    d = Qc.shape[-1]
    if attn_scale is None:
        attn_scale = 1.0 / math.sqrt(d)
    sel = prefill_select(Qc, K, P, k, score_scale)
    sel["out"] = chunk_attention(Qc, K, V, sel["T"], P, n_local, attn_scale)
    return sel
