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
