"""Host logic of bench.py that its figures rest on.

The decode leg's roofline divides the bytes the step must move by its time,
and those bytes follow from how many entries each stream's cache holds when a
step attends.  bench.decode_lengths gets that count in closed form from the
separator flags; here it is checked step by step against the oracle's cache
simulator, which keeps the cache's contents one token at a time.
"""
import numpy as np
import pytest

import bench
from oracle import sepllm_oracle as orc
from separator_kv_cache_amd import synth

# (a, s, n, c, p, T, B): the Llama decode geometry, a past window (c > a + s + n,
# including the pages' c = 800 on a short window), no sinks, no separator block,
# n = 1, and flag rates 0 and 1
CASES = [
    (4, 64, 256, 0, 0.12, 1200, 3),
    (4, 64, 256, 800, 0.12, 2400, 2),
    (2, 5, 7, 30, 0.4, 300, 4),
    (0, 3, 5, 0, 0.5, 200, 3),
    (3, 0, 4, 12, 0.3, 200, 3),
    (1, 2, 1, 0, 0.6, 100, 2),
    (1, 2, 1, 9, 0.6, 100, 2),
    (4, 8, 16, 0, 0.0, 150, 2),
    (4, 8, 16, 40, 1.0, 300, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_decode_lengths_match_the_cache_simulator(case):
    a, s, n, c, p, T, B = case
    wl = synth.LLAMA_DECODE.with_(a=a, s=s, n=n, p=p, T=T, B=B)
    flags = wl.flags(7)
    got = bench.decode_lengths(wl, flags, c)
    assert got.shape == (T, B)
    for b in range(B):
        sim = orc.SepCacheSim(a, s, n, c if c > a + s + n else None)
        for t in range(T):
            # a step appends, evicts (no past window) and then attends
            sim.append(int(flags[t, b]))
            sim.evict()
            assert got[t, b] == len(sim.order()), (b, t)


def test_decode_bytes_counts_every_cached_row_once_per_step():
    wl = synth.LLAMA_DECODE.with_(T=40, B=3)
    flags = wl.flags(3)
    length = bench.decode_lengths(wl, flags)
    row = wl.Hkv * wl.d * 2  # one token's K (or V) over the KV heads, bf16
    per_step = [sum(int(length[t, b]) * 2 * row for b in range(wl.B)) + wl.B * (2 * wl.Hq * wl.d * 2 + 2 * row)
                for t in range(wl.T)]
    assert bench.decode_bytes(wl, length) == float(sum(per_step))
