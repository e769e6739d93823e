"""Randomised GPU parity: seeded draws of the shape and selection parameters of the
decode path (batch, ragged lengths, k, L, head grouping, dtype, top-p) and of the
prefill path (chunk lengths, past lengths), each compared with the oracle under the
same bands as the targeted tests. The seeds are fixed, so every run checks the same
cases; each case prints its parameters first.
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
GROUPS = [(8, 8), (16, 8), (12, 4), (32, 8), (20, 4), (24, 4), (28, 4), (64, 8)]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ts.load_library()


def _draw(seed):
    rng = np.random.default_rng(seed)
    H, Hkv = GROUPS[int(rng.integers(len(GROUPS)))]
    b = int(rng.integers(1, 6))
    lo = int(rng.integers(1, 3000))
    hi = lo + int(rng.integers(1, 9000))
    k = int(rng.choice([1, 7, 64, 300, 1024, 5000]))
    L = int(rng.choice([0, 1, 33, 512]))
    dtype = "f32" if rng.random() < 0.3 else "bf16"
    return dict(H=H, Hkv=Hkv, b=b, lo=lo, hi=hi, k=k, L=L, dtype=dtype,
                scale_spread=bool(rng.random() < 0.7))


@pytest.mark.parametrize("seed", range(8100, 8112))
def test_random_decode(seed):
    d = _draw(seed)
    gh.log(f"[random decode seed {seed}] {d}")
    geo = wl.workload("llama3-8b-ragged16", num_q_heads=d["H"], num_kv_heads=d["Hkv"], batch=d["b"],
                      min_len=d["lo"], max_len=d["hi"], top_k=d["k"], n_local=d["L"], dtype=d["dtype"],
                      n_planted=8, seed=seed)
    batch = wl.make_batch(geo, device=DEV, scale_spread=d["scale_spread"])
    po = gh.run_path(batch, geo)
    for r, req in enumerate(batch.requests):
        gh.check_request(po, r, req, geo)


@pytest.mark.parametrize("seed", range(8200, 8208))
def test_random_prefill(seed):
    rng = np.random.default_rng(seed)
    d = _draw(seed)
    c = int(rng.choice([1, 5, 64, 100, 257]))
    lo = max(d["lo"], c)
    geo = wl.workload("prefill-tiny-f32", num_q_heads=d["H"], num_kv_heads=d["Hkv"], batch=d["b"],
                      min_len=lo, max_len=lo + d["hi"] - d["lo"], top_k=d["k"], n_local=d["L"],
                      dtype=d["dtype"], chunk=c, n_planted=8, seed=seed)
    lens = [int(x) for x in rng.integers(1, c + 1, d["b"])]
    gh.log(f"[random prefill seed {seed}] {d} chunk {c} chunk_lens {lens}")
    cb = wl.make_chunk_batch(geo, DEV, chunk_lens=lens)
    po = gh.run_prefill(cb, geo)
    for r in range(d["b"]):
        gh.check_prefill_selection(po, r, cb, geo)
        rows = None if lens[r] <= 64 else sorted({0, 1, lens[r] // 2, lens[r] - 1})
        gh.check_chunk_attention(po, r, cb, geo, po.T[r], rows=rows)


@pytest.mark.parametrize("seed", range(8300, 8306))
def test_random_top_p(seed):
    from tests.test_gpu_topp import _check_request, _run
    rng = np.random.default_rng(seed)
    d = _draw(seed)
    p = float(rng.choice([0.1, 0.5, 0.8, 0.95, 1.0]))
    gh.log(f"[random top-p seed {seed}] {d} p {p}")
    geo = wl.workload("llama3-8b-ragged16", num_q_heads=d["H"], num_kv_heads=d["Hkv"], batch=d["b"],
                      min_len=d["lo"], max_len=d["hi"], top_k=d["k"], n_local=d["L"], dtype=d["dtype"],
                      n_planted=8, seed=seed)
    batch = wl.make_batch(geo, device=DEV, scale_spread=d["scale_spread"])
    lv, si, sc = _run(batch, geo, p)
    offs = batch.token_offsets.cpu().tolist()
    for r in range(d["b"]):
        n = int(batch.seq_lens[r])
        req = batch.requests[r]
        sel = ora.select(gh.np32(req.q), gh.np32(req.k), geo.top_k)
        m = int(sc[r])
        _check_request(lv[offs[r]: offs[r] + n], si[r, :m].astype(np.int64), m, p, geo.top_k, sel["vote"])
