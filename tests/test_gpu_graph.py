"""Graph-captured SepCache steps (as the benchmark replays them) reproduce
eager execution bit for bit, on every replay."""
import numpy as np
import pytest
import torch

from separator_kv_cache_amd import binding as sa
from separator_kv_cache_amd import synth
from tests.util import say

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    say("graph-replay")
    wl = synth.DecodeWorkload("graph", 72, B=4, Hq=8, Hkv=2, d=128, a=2, s=6, n=10, T=96, p=0.3)
    CH = 8
    flags = torch.from_numpy(wl.flags(0)).cuda()
    k, v = wl.kv_steps(0, CH)
    kp = torch.from_numpy(k).to(torch.bfloat16).cuda()
    vp = torch.from_numpy(v).to(torch.bfloat16).cuda()
    qp = torch.from_numpy(wl.q_steps(range(CH))).to(torch.bfloat16).cuda()

    def make():
        return [sa.SepCache(wl.B, wl.Hkv, wl.d, wl.a, wl.s, wl.n, wl.theta) for _ in range(2)]

    # eager reference
    eager = make()
    ref = []
    for t in range(wl.T):
        outs = []
        for c in eager:
            outs.append(c.step(kp[t % CH], vp[t % CH], flags[t], qp[t % CH]).clone())
        ref.append(outs)
    torch.cuda.synchronize()

    caches = make()
    fl_static = torch.zeros((CH, wl.B), dtype=torch.uint8, device="cuda")
    out_static = [[torch.empty((wl.B, wl.Hq, wl.d), dtype=torch.bfloat16, device="cuda") for _ in caches]
                  for _ in range(CH)]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(CH):
            for ci, c in enumerate(caches):
                c.step(kp[i], vp[i], fl_static[i], qp[i], out=out_static[i][ci])
    for c in caches:  # capture does not run the work; start from empty caches
        c.reset()
    torch.cuda.synchronize()
    for chunk in range(wl.T // CH):
        fl_static.copy_(flags[chunk * CH:(chunk + 1) * CH])
        g.replay()
        torch.cuda.synchronize()
        for i in range(CH):
            for ci in range(len(caches)):
                assert torch.equal(out_static[i][ci], ref[chunk * CH + i][ci]), (chunk, i, ci)
        # eager work between replays
        _ = (fl_static.float() * 2).sum().item()
