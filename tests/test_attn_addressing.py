"""Address arithmetic of the decode attention kernel, emulated on the CPU.

The attention kernel gathers one key row and one value row per selected slot
through the block table. This test restates, slot by slot, how the kernel picks
the token of each gathering lane (TopK slots, window slots, masked slots) and
which block-table entry and pool row that token reaches, and checks on inputs a
caller may legally pass that every gather stays inside the request's reached
pages and the pool: a request with N_r = 0 whose block-table row is all -1, TopK
entries that are stale or negative, window sizes of 0.
"""
import numpy as np
import pytest

PAGE = 16
ATTN_SPLIT = 32            # selected slots per wave
ATTN_TILE = 4 * ATTN_SPLIT  # slots per workgroup


def attn_splits(top_k, window):
    return -(-top_k // ATTN_TILE) + -(-window // ATTN_TILE)


def kernel_gathers(seq_lens, sel_idx, sel_count, block_table, Hkv, top_k, n_local):
    """Yield (r, bt_index) for every block-table read and (r, phys) for every row
    gather the attention kernel issues, following its slot-to-token rule."""
    b, sel_stride = sel_idx.shape
    window = max(1, n_local)                    # the library's decode window
    S = attn_splits(top_k, window)
    nT = -(-top_k // ATTN_TILE)
    reads, gathers = [], []
    for blk in range(b * Hkv * S):
        s = blk % S
        r = (blk // S) // Hkv
        N = int(seq_lens[r])
        if N <= 0:
            continue                            # the workgroup writes the empty partial only
        lstart = max(0, N - window)
        cnt = min(int(sel_count[r]), sel_stride) if s < nT else 0
        for wave in range(4):
            for lane in range(ATTN_SPLIT):
                tok = N - 1
                if s < nT:
                    e = s * ATTN_TILE + wave * ATTN_SPLIT + lane
                    cand = int(sel_idx[r, min(e, sel_stride - 1)])
                    if e < cnt and 0 <= cand < lstart:
                        tok = cand
                else:
                    t = lstart + (s - nT) * ATTN_TILE + wave * ATTN_SPLIT + lane
                    if t < N:
                        tok = t
                reads.append((r, tok // PAGE))
                gathers.append((r, int(block_table[r, tok // PAGE])))
    return reads, gathers


@pytest.mark.parametrize("n_local", [0, 1, 8, 512])
def test_every_gather_stays_in_reached_pages(n_local):
    rng = np.random.default_rng(5)
    pool_pages, stride, top_k = 400, 40, 300
    lens = np.array([0, 17, 1, 640, 0, 300])
    b = len(lens)
    bt = np.full((b, stride), -1, dtype=np.int64)       # unreached entries are invalid
    perm = rng.permutation(pool_pages)
    used = 0
    for r, n in enumerate(lens):
        pages = -(-n // PAGE)
        bt[r, :pages] = perm[used:used + pages]
        used += pages
    sel_idx = rng.integers(-50, 1000, size=(b, top_k))  # stale, negative and past-N entries
    sel_count = np.array([top_k, 5, 0, top_k, 7, 299])
    reads, gathers = kernel_gathers(lens, sel_idx, sel_count, bt, 2, top_k, n_local)
    assert reads, "no gathers emulated"
    for (r, p), (_, phys) in zip(reads, gathers):
        assert lens[r] > 0
        assert 0 <= p < -(-lens[r] // PAGE), (r, p)
        assert 0 <= phys < pool_pages, (r, p, phys)
    # the empty requests' rows (all -1) are never read
    assert not any(r in (0, 4) for r, _ in reads)


def test_current_token_is_gathered_with_no_window():
    # n_local = 0: the window slot is the current token N - 1 for every request
    lens = np.array([5, 33])
    bt = np.arange(2 * 3).reshape(2, 3)
    sel_idx = np.zeros((2, 4), dtype=np.int64)
    sel_count = np.array([0, 0])
    reads, _ = kernel_gathers(lens, sel_idx, sel_count, bt, 1, 4, 0)
    # the one window workgroup per request has its slot 0 at token N - 1; the
    # other slots are masked and also gather N - 1
    assert set(reads) == {(0, 0), (1, 2)}
