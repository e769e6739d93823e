"""Workload recipes and the seeded generator.

The shapes follow the TokenSelect pages: Llama-3-8B and Qwen2-7B head geometry
(32/8 and 28/4 query/KV heads, head dim 128), contexts of 128K and 1M tokens,
a budget of 2K selected plus 512 local tokens ("TokenSelect" deepnotes page,
quick-read results paragraph; blog page section 4.2, Table 2), a cosine
threshold of 0.9 (blog page section 6), consecutive-query cosine around 0.945
(blog page section 2, Fig. 3a) and a three-decade spread of per-head logit
norms (blog page section 2, Fig. 2c).

Draw order inside one request is fixed: per-KV-head scales, queries, background
keys, values, planted positions, planted noise. The page permutation is drawn
afterwards, once per batch. Everything comes from one ``torch.Generator`` on
the device the tensors are made on, so the same seed reproduces the same
tensors on the same kind of device.

Nothing here evaluates a score, a softmax, a vote, a top-k or an attention.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch


@dataclass(frozen=True)
class Geometry:
    """One workload's shapes and selection parameters."""

    name: str
    dtype: str            # "f32" or "bf16": q, K/V pool and output element type
    num_q_heads: int      # H
    num_kv_heads: int     # H_kv; query head h reads KV head h // (H / H_kv)
    head_dim: int         # d
    page_size: int        # P tokens per page
    top_k: int            # k
    n_local: int          # L most recent tokens always attended
    n_planted: int        # planted critical tokens per KV head (per request)
    seq_len: int          # N (first step for the multi-step workload)
    batch: int = 1
    min_len: int = 0      # ragged batch: N_r drawn log-uniform in [min_len, max_len]
    max_len: int = 0
    layers: int = 1       # independent layers (seeds base + l)
    steps: int = 1        # consecutive decode steps (selection cache workload)
    cos_threshold: float = 0.9
    seed: int = 0
    scale_lo: float = 1.0
    scale_hi: float = 1000.0
    chunk: int = 0        # prefill chunk size c (chunk workloads); seq_len counts the chunk

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def attn_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# The five workloads. Seeds: the tiny case uses 0; the others use 1000*X + layer.
CONFIGS = {
    "tiny-f32-8k": Geometry(
        name="tiny-f32-8k", dtype="f32", num_q_heads=8, num_kv_heads=2, head_dim=128,
        page_size=16, top_k=256, n_local=64, n_planted=32, seq_len=8192, seed=0),
    "llama3-8b-128k": Geometry(
        name="llama3-8b-128k", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
        page_size=16, top_k=2048, n_local=512, n_planted=64, seq_len=131072, seed=1000),
    "llama3-8b-1m": Geometry(
        name="llama3-8b-1m", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
        page_size=16, top_k=2048, n_local=512, n_planted=128, seq_len=1048576,
        layers=32, seed=2000),
    "llama3-8b-ragged16": Geometry(
        name="llama3-8b-ragged16", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
        page_size=16, top_k=2048, n_local=512, n_planted=64, seq_len=0, batch=16,
        min_len=32768, max_len=262144, seed=3000),
    "qwen2-7b-cache256": Geometry(
        name="qwen2-7b-cache256", dtype="bf16", num_q_heads=28, num_kv_heads=4, head_dim=128,
        page_size=16, top_k=2048, n_local=512, n_planted=64, seq_len=131072, steps=256,
        cos_threshold=0.9, seed=4000),
    # Chunk-wise prefill (blog page section 3.3, Fig. 5: chunk 512, 128K cached tokens,
    # 4K attended = 3072 selected + 512 local + the 512-token chunk; Fig. 7c: 1M
    # cached tokens with a 2048-token selection budget).
    "prefill-tiny-f32": Geometry(
        name="prefill-tiny-f32", dtype="f32", num_q_heads=8, num_kv_heads=2, head_dim=128,
        page_size=16, top_k=256, n_local=64, n_planted=32, seq_len=8192, chunk=64, seed=5000),
    "prefill-llama3-128k": Geometry(
        name="prefill-llama3-128k", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
        page_size=16, top_k=3072, n_local=512, n_planted=64, seq_len=131072, chunk=512,
        layers=8, seed=6000),
    "prefill-llama3-1m": Geometry(
        name="prefill-llama3-1m", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
        page_size=16, top_k=2048, n_local=512, n_planted=128, seq_len=1048576, chunk=512,
        seed=7000),
}

# Spread of a chunk's queries around their shared master query: q_j = q_master +
# CHUNK_SIGMA * eps_j, eps_j ~ N(0, I_d), so neighbouring queries have cosine
# about 1 / (1 + CHUNK_SIGMA^2) = 0.945 (blog page section 2, Fig. 3a).
CHUNK_SIGMA = 0.24


def workload(name: str, **overrides) -> Geometry:
    """Return a named workload, optionally with fields replaced (smaller N, etc.)."""
    g = CONFIGS[name]
    if overrides:
        d = dict(g.__dict__)
        d.update(overrides)
        g = Geometry(**d)
    return g


@dataclass
class Request:
    """One request's logical (unpaged) inputs, as stored (already rounded)."""

    q: torch.Tensor             # [H][d]
    k: torch.Tensor             # [H_kv][N][d]
    v: torch.Tensor             # [H_kv][N][d]
    planted_pos: torch.Tensor   # int64 [H_kv][n_p]: logical positions
    planted_head: torch.Tensor  # int64 [H_kv][n_p]: query head each planted key targets
    scales: torch.Tensor        # fp32 [H_kv]: per-KV-head key scale s_g
    q_master: Optional[torch.Tensor] = None  # fp64 [H][d] unrounded query (AR(1) state)

    @property
    def seq_len(self) -> int:
        return int(self.k.shape[1])


@dataclass
class PagedBatch:
    """A batch laid out in a shared page pool."""

    q: torch.Tensor              # [b][H][d]
    k_pool: torch.Tensor         # [pages][H_kv][P][d]
    v_pool: torch.Tensor         # [pages][H_kv][P][d]
    block_table: torch.Tensor    # int32 [b][stride]
    seq_lens: torch.Tensor       # int32 [b]
    token_offsets: torch.Tensor  # int64 [b+1], prefix sums of seq_lens
    requests: List[Request] = field(default_factory=list)

    @property
    def total_tokens(self) -> int:
        return int(self.token_offsets[-1])


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def make_request(gen: torch.Generator, geo: Geometry, seq_len: int, device,
                 scale_spread: bool = True, extra_tokens: int = 0,
                 q_master: Optional[torch.Tensor] = None) -> Request:
    """Draw one request.

    q_h ~ N(0, I_d). Background keys and all values ~ N(0, I_d). Each KV head g
    gets a scale s_g = exp(U[ln lo, ln hi)) (s_g = 1 when ``scale_spread`` is
    off). Planted token j of KV head g sits at a distinct uniform position in
    [0, seq_len) and targets query head g*G + (j mod G): its unscaled key is
    8 * q_h / |q_h| + 0.1 * N(0, I_d). The whole KV head, planted rows included,
    is multiplied by s_g and then rounded to the storage type.

    ``extra_tokens`` appends that many background tokens after ``seq_len``
    (the tokens a multi-step decode appends later). ``q_master`` (fp64 [H][d])
    replaces the drawn query, for AR(1) sequences.
    """
    H, Hkv, d, G = geo.num_q_heads, geo.num_kv_heads, geo.head_dim, geo.group
    n_total = seq_len + extra_tokens
    f32 = torch.float32
    # 1. per-KV-head scales
    u = torch.rand(Hkv, generator=gen, device=device, dtype=torch.float64)
    lo, hi = math.log(geo.scale_lo), math.log(geo.scale_hi)
    scales = torch.exp(lo + (hi - lo) * u).to(f32)
    if not scale_spread:
        scales = torch.ones_like(scales)
    # 2. queries
    qm = torch.randn(H, d, generator=gen, device=device, dtype=torch.float64)
    if q_master is not None:
        qm = q_master.to(device=device, dtype=torch.float64)
    q = qm.to(geo.torch_dtype)
    # 3. background keys, 4. values
    k0 = torch.randn(Hkv, n_total, d, generator=gen, device=device, dtype=f32)
    v = torch.randn(Hkv, n_total, d, generator=gen, device=device, dtype=f32)
    # 5. planted positions (distinct per KV head, uniform over [0, seq_len))
    n_p = min(geo.n_planted, seq_len)
    pos = torch.empty(Hkv, n_p, dtype=torch.int64, device=device)
    for g in range(Hkv):
        pos[g] = torch.randperm(seq_len, generator=gen, device=device)[:n_p]
    # 6. planted noise
    noise = torch.randn(Hkv, n_p, d, generator=gen, device=device, dtype=f32)
    heads = (torch.arange(Hkv, device=device)[:, None] * G
             + torch.arange(n_p, device=device)[None, :] % G)
    qs = q.to(f32)
    qhat = qs / torch.linalg.vector_norm(qs, dim=1, keepdim=True)
    for g in range(Hkv):
        k0[g, pos[g]] = 8.0 * qhat[heads[g]] + 0.1 * noise[g]
    k0.mul_(scales[:, None, None])
    k = k0.to(geo.torch_dtype)
    del k0
    v = v.to(geo.torch_dtype)
    return Request(q=q, k=k, v=v, planted_pos=pos, planted_head=heads, scales=scales,
                   q_master=qm)


def request_lengths(gen: torch.Generator, geo: Geometry, device) -> List[int]:
    """Ragged lengths N_r = floor(exp(U[ln min_len, ln max_len])), one per request."""
    u = torch.rand(geo.batch, generator=gen, device=device, dtype=torch.float64).cpu()
    lo, hi = math.log(geo.min_len), math.log(geo.max_len)
    return [int(math.floor(math.exp(lo + (hi - lo) * float(x)))) for x in u]


def page_requests(requests: List[Request], geo: Geometry, gen: Optional[torch.Generator],
                  device, permute: bool = True, pad_value: float = float("nan"),
                  spare_pages: int = 0, stride: Optional[int] = None,
                  pools: Optional[tuple] = None) -> PagedBatch:
    """Lay requests out in one pool of pages [pages][H_kv][P][d].

    Token i of request r lives at pool page block_table[r][i // P], slot i % P.
    Pool pages are handed out by one random permutation of the pool (identity
    when ``permute`` is off). Slots past a request's last token, and
    ``spare_pages`` unused pages, hold ``pad_value`` so that a kernel reading
    them into a result shows up. Block-table entries past a request's last page
    are -1. ``pools`` = (k_pool, v_pool) fills caller-allocated pools of the
    right shape instead of allocating new ones.
    """
    P = geo.page_size
    Hkv, d = geo.num_kv_heads, geo.head_dim
    n_pages = [-(-r.k.shape[1] // P) for r in requests]
    total_pages = sum(n_pages) + spare_pages
    if permute:
        perm = torch.randperm(total_pages, generator=gen, device=device)
    else:
        perm = torch.arange(total_pages, device=device)
    stride = stride or max(n_pages)
    if pools is None:
        k_pool = torch.full((total_pages, Hkv, P, d), pad_value, dtype=geo.torch_dtype, device=device)
        v_pool = torch.full_like(k_pool, pad_value)
    else:
        k_pool, v_pool = pools
        assert k_pool.shape == (total_pages, Hkv, P, d) and v_pool.shape == k_pool.shape
        assert k_pool.dtype == geo.torch_dtype and v_pool.dtype == geo.torch_dtype
        k_pool.fill_(pad_value)
        v_pool.fill_(pad_value)
    bt = torch.full((len(requests), stride), -1, dtype=torch.int32, device=device)
    base = 0
    for r, req in enumerate(requests):
        n = req.k.shape[1]
        npg = n_pages[r]
        ids = perm[base:base + npg]
        base += npg
        bt[r, :npg] = ids.to(torch.int32)
        for src, pool in ((req.k, k_pool), (req.v, v_pool)):
            padded = torch.full((Hkv, npg * P, d), pad_value, dtype=src.dtype, device=device)
            padded[:, :n] = src
            pool[ids] = padded.view(Hkv, npg, P, d).permute(1, 0, 2, 3)
    seq = torch.tensor([r.k.shape[1] for r in requests], dtype=torch.int32, device=device)
    offs = torch.zeros(len(requests) + 1, dtype=torch.int64, device=device)
    offs[1:] = torch.cumsum(seq.to(torch.int64), 0)
    q = torch.stack([r.q for r in requests])
    return PagedBatch(q=q, k_pool=k_pool, v_pool=v_pool, block_table=bt, seq_lens=seq,
                      token_offsets=offs, requests=list(requests))


def make_batch(geo: Geometry, device="cpu", layer: int = 0, permute: bool = True,
               scale_spread: bool = True, pad_value: float = float("nan"),
               seq_len: Optional[int] = None, pools: Optional[tuple] = None) -> PagedBatch:
    """Draw a whole workload (one layer) and page it.

    Workloads with a length range (min_len) draw every request's length first,
    then each request in order; the others use ``seq_len`` (default the
    workload's N) for every request.
    """
    gen = _gen(geo.seed + layer, device)
    if geo.min_len and not seq_len:
        lens = request_lengths(gen, geo, device)
    else:
        lens = [seq_len or geo.seq_len] * geo.batch
    reqs = [make_request(gen, geo, n, device, scale_spread=scale_spread) for n in lens]
    return page_requests(reqs, geo, gen, device, permute=permute, pad_value=pad_value, pools=pools)


def ar1_queries(geo: Geometry, q0_master: torch.Tensor, steps: int, seed: int, device="cpu"):
    """AR(1) query sequence q_t = rho_t q_{t-1} + sqrt(1 - rho_t^2) eps_t.

    rho_t is 0.97 with probability 0.8 and 0.5 with probability 0.2, drawn per
    step; eps_t ~ N(0, I). The recursion runs on the fp64 master copy; each
    step's stored query is that master rounded to the storage type. Returns
    (stored [steps][H][d], rho [steps]); step 0 is q0 itself (rho_0 = nan).
    """
    gen = _gen(seed, device)
    H, d = q0_master.shape
    qs = torch.empty(steps, H, d, dtype=geo.torch_dtype, device=device)
    rhos = torch.full((steps,), float("nan"), dtype=torch.float64)
    cur = q0_master.to(device=device, dtype=torch.float64).clone()
    qs[0] = cur.to(geo.torch_dtype)
    for t in range(1, steps):
        u = float(torch.rand(1, generator=gen, device=device, dtype=torch.float64))
        rho = 0.97 if u < 0.8 else 0.5
        eps = torch.randn(H, d, generator=gen, device=device, dtype=torch.float64)
        cur = rho * cur + math.sqrt(1.0 - rho * rho) * eps
        qs[t] = cur.to(geo.torch_dtype)
        rhos[t] = rho
    return qs, rhos


@dataclass
class ChunkBatch:
    """A prefill chunk per request: the paged cache (chunk tokens included) and the
    chunk's queries."""

    paged: PagedBatch
    q_chunk: torch.Tensor        # [b][c][H][d]
    chunk_lens: torch.Tensor     # int32 [b]
    seq_lens: torch.Tensor       # int32 [b]: P_r + c_r
    past_lens: List[int] = field(default_factory=list)


def make_chunk_batch(geo: Geometry, device="cpu", layer: int = 0, permute: bool = True,
                     pad_value: float = float("nan"), seq_len: Optional[int] = None,
                     chunk_lens: Optional[List[int]] = None,
                     pools: Optional[tuple] = None, scale_spread: bool = True) -> ChunkBatch:
    """Draw a prefill-chunk workload and page it.

    Request r has N_r = seq_len tokens (ragged workloads draw N_r as in decode); its
    last c = geo.chunk tokens are the chunk and its first N_r - c the past, which
    holds the planted critical tokens. The c chunk queries are q_master + CHUNK_SIGMA
    * eps_j, drawn after the request and rounded to the storage type. ``chunk_lens``
    shortens the chunk of some requests to c_r <= c (their last c - c_r drawn tokens
    stay in the pool, unused).
    """
    gen = _gen(geo.seed + layer, device)
    c = geo.chunk
    assert c >= 1
    if geo.min_len and not seq_len:
        lens = request_lengths(gen, geo, device)
    else:
        lens = [seq_len or geo.seq_len] * geo.batch
    assert all(n >= c for n in lens)
    reqs, qcs = [], []
    for n in lens:
        req = make_request(gen, geo, n - c, device, extra_tokens=c, scale_spread=scale_spread)
        eps = torch.randn(c, geo.num_q_heads, geo.head_dim, generator=gen, device=device,
                          dtype=torch.float64)
        qcs.append((req.q_master[None] + CHUNK_SIGMA * eps).to(geo.torch_dtype))
        reqs.append(req)
    paged = page_requests(reqs, geo, gen, device, permute=permute, pad_value=pad_value, pools=pools)
    cl = list(chunk_lens) if chunk_lens is not None else [c] * len(lens)
    assert len(cl) == len(lens) and all(1 <= x <= c for x in cl)
    past = [n - c for n in lens]
    seq = torch.tensor([p + x for p, x in zip(past, cl)], dtype=torch.int32, device=device)
    return ChunkBatch(paged=paged, q_chunk=torch.stack(qcs), chunk_lens=torch.tensor(cl, dtype=torch.int32,
                      device=device), seq_lens=seq, past_lens=past)
