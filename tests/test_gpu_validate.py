"""tokenselect_validate against a direct host evaluation of the input contract:
request lengths within their block-table rows, page ids within the pool."""
import numpy as np
import pytest
import torch

import token_level_sparse_amd as ts
from synth import workloads as wl
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ts.load_library()


def _expected(bt, lens, pool_pages):
    b, stride = bt.shape
    viol, keys, nlen = 0, [], 0
    for r in range(b):
        n = int(lens[r])
        if n < 0 or n > stride * 16:
            viol += 1
            nlen += 1
            keys.append((r << 32) | 0xFFFFFFFF)
        reach = min(-(-n // 16) if n > 0 else 0, stride)
        for p in range(reach):
            v = int(bt[r, p])
            if v < 0 or v >= pool_pages:
                viol += 1
                keys.append((r << 32) | p)
    first = min(keys) if keys else (1 << 64) - 1
    return [viol, first, nlen, int(sum(max(int(n), 0) for n in lens))]


def _report(rep):
    return [int(x) & ((1 << 64) - 1) for x in rep.cpu().tolist()]


def test_validate_clean_and_planted_violations():
    geo = wl.workload("llama3-8b-ragged16", batch=5, min_len=100, max_len=9000, seed=4400)
    gh.log("[validate] 5 ragged requests")
    batch = wl.make_batch(geo, device=DEV)
    b, stride = batch.block_table.shape
    pool_pages = batch.k_pool.shape[0]
    shape = ts.make_shape(geo.num_q_heads, geo.num_kv_heads, b, stride, batch.total_tokens, geo.torch_dtype)
    rep = ts.validate(shape, batch.block_table, batch.seq_lens, pool_pages)
    torch.cuda.synchronize()
    got = _report(rep)
    bt_h, lens_h = batch.block_table.cpu().numpy(), batch.seq_lens.cpu().numpy()
    assert got == _expected(bt_h, lens_h, pool_pages)
    assert got[0] == 0 and got[3] == batch.total_tokens

    # planted: a page id past the pool, a negative page id, an over-long and a negative request
    bt = batch.block_table.clone()
    lens = batch.seq_lens.clone()
    bt[1, 2] = pool_pages + 5
    bt[2, 0] = -1
    lens[3] = stride * 16 + 1
    lens[4] = -3
    rep = ts.validate(shape, bt, lens, pool_pages, report=rep)
    torch.cuda.synchronize()
    got = _report(rep)
    want = _expected(bt.cpu().numpy(), lens.cpu().numpy(), pool_pages)
    gh.log(f"  report {got}")
    assert got == want
    assert got[0] >= 4 and got[2] == 2 and got[1] == (1 << 32) | 2


def _expected_selection(idx, cnt, lens, top_k):
    viol, keys, nc, total = 0, [], 0, 0
    for r in range(len(lens)):
        n, c = int(lens[r]), int(cnt[r])
        cap = min(top_k, max(n, 0))
        ok = 0 <= c <= cap
        if not ok:
            viol += 1
            nc += 1
            keys.append((r << 32) | 0xFFFFFFFF)
        else:
            total += c
        m = c if ok else min(max(c, 0), top_k)
        for e in range(m):
            v = int(idx[r, e])
            if not (0 <= v < n) or (e > 0 and not int(idx[r, e - 1]) < v):
                viol += 1
                keys.append((r << 32) | e)
    first = min(keys) if keys else (1 << 64) - 1
    return [viol, first, nc, total]


def test_validate_selection_clean_and_planted_violations():
    # the decode TopK of a ragged batch is a valid selection; then planted faults:
    # an entry past N_r, a repeated entry, a descending pair, a negative entry, a count
    # above top_k and a count above N_r
    geo = wl.workload("llama3-8b-ragged16", batch=6, min_len=100, max_len=6000, top_k=128, seed=4500)
    gh.log("[validate selection] 6 ragged requests")
    batch = wl.make_batch(geo, device=DEV)
    po = gh.run_path(batch, geo)
    si, sc = po.raw["sel_idx"], po.raw["sel_count"]
    b = si.shape[0]
    shape = ts.make_shape(geo.num_q_heads, geo.num_kv_heads, b, batch.block_table.shape[1],
                          batch.total_tokens, geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local)
    rep = ts.validate_selection(shape, sel, batch.seq_lens, si, sc)
    torch.cuda.synchronize()
    got = _report(rep)
    lens_h = batch.seq_lens.cpu().numpy()
    assert got == _expected_selection(si.cpu().numpy(), sc.cpu().numpy(), lens_h, geo.top_k)
    assert got[0] == 0 and got[3] == sum(min(geo.top_k, int(n)) for n in lens_h)

    si2, sc2 = si.clone(), sc.clone()
    si2[0, 5] = int(lens_h[0]) + 3          # past N_0 (and breaks ascending after it)
    si2[1, 7] = si2[1, 6]                   # repeated
    si2[2, 10], si2[2, 11] = si2[2, 11].clone(), si2[2, 10].clone()   # descending pair
    si2[3, 0] = -1                          # negative
    sc2[4] = geo.top_k + 1                  # above top_k
    lens2 = batch.seq_lens.clone()
    lens2[5] = 3                            # count above N_5
    rep = ts.validate_selection(shape, sel, lens2, si2, sc2, report=rep)
    torch.cuda.synchronize()
    got = _report(rep)
    want = _expected_selection(si2.cpu().numpy(), sc2.cpu().numpy(), lens2.cpu().numpy(), geo.top_k)
    gh.log(f"  report {got}")
    assert got == want
    assert got[2] == 2 and got[1] == (0 << 32) | 5
