"""The chunk attention's search for the TopK entries below the window start,
emulated on the CPU.

Every wave of a chunk-attention workgroup counts the entries of the request's
ascending TopK list that lie below the window start w0 with a 64-way search: each
round probes the 64 entries lo + step (l + 1) - 1 of the run [lo, hi) that holds the
answer, the probes below w0 form a prefix of k lanes, and the run shrinks to
[lo + k step, min(hi, lo + (k + 1) step - 1)). This test restates those rounds
lane by lane and checks the count against a plain count on sorted inputs of every
size class, including the empty list, all entries below and none below.
"""
import bisect

import numpy as np
import pytest

WAVE = 64


def count_below(a, n, x):
    lo, hi, rounds = 0, n, 0
    while lo < hi:
        step = (hi - lo + WAVE - 1) // WAVE
        below = [(lo + step * (l + 1) - 1) < hi and a[lo + step * (l + 1) - 1] < x for l in range(WAVE)]
        k = sum(below)
        assert below == [True] * k + [False] * (WAVE - k)      # a prefix of lanes
        nlo = lo + step * k
        hi = min(hi, nlo + step - 1)
        lo = nlo
        if step == 1:
            hi = lo
        rounds += 1
    return lo, rounds


@pytest.mark.parametrize("n", [0, 1, 2, 63, 64, 65, 100, 2048, 3072, 4095, 4096, 4097, 70000])
def test_count_matches_plain_count(n):
    rng = np.random.default_rng(n)
    a = np.sort(rng.choice(10 * n + 10, size=n, replace=False)).tolist()
    xs = {-1, 0, 10 * n + 11} | set(rng.integers(0, 10 * n + 11, size=20).tolist())
    xs |= {v for v in a[:3] + a[-3:]} | {v + 1 for v in a[:3] + a[-3:]}
    for x in xs:
        got, rounds = count_below(a, n, x)
        assert got == bisect.bisect_left(a, x), (n, x)
        assert rounds <= (2 if n <= 4096 else 3)
