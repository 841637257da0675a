"""SepCache manager and decode on the GPU against the oracle's simulator."""
import math

import numpy as np
import pytest
import torch

from oracle import sepllm_oracle as orc
from separator_kv_cache_amd import binding as sa
from separator_kv_cache_amd import synth
from tests.util import TOL_BF16, as_f64, cache_k_rows, max_abs, say

pytestmark = pytest.mark.gpu


def _bf(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def _setup(wl, seed=0):
    flags = wl.flags(seed)
    k, v = wl.kv_steps(0, wl.T, seed)
    kb, vb = _bf(k), _bf(v)
    return flags, kb, vb


def _check_state(cache, sims, kb, vb, t):
    """Order, length and the K/V bytes of every occupied slot, bit-exact."""
    pos, ln = cache.export_order()
    pos, ln = pos.cpu().numpy(), ln.cpu().numpy()
    spos = cache.slot_pos.cpu().numpy()          # [B, Hkv, slots]
    state = cache.state.cpu().numpy()
    kc, vc = cache_k_rows(cache.k.cpu(), cache.slots), cache.v.cpu()
    for b, sim in enumerate(sims):
        order = sim.order()
        assert ln[b] == len(order), (t, b)
        assert pos[b, :len(order)].tolist() == order, (t, b)
        assert np.all(pos[b, len(order):] == -1)
        for h in range(cache.Hkv):
            assert np.array_equal(state[b, h], state[b, 0]), (t, b, h)
            occ = np.nonzero(spos[b, h] >= 0)[0]
            assert sorted(spos[b, h, occ].tolist()) == order, (t, b, h)
            src = spos[b, h, occ]
            assert torch.equal(kc[b, h, occ], kb[src, b, h]), (t, b, h)
            assert torch.equal(vc[b, h, occ], vb[src, b, h]), (t, b, h)


SMALL = [
    # B, Hq, Hkv, d, a, s, n, T, p, shift, api ("push", "split" = append+evict, "step" = fused)
    (3, 4, 2, 64, 2, 3, 5, 60, 0.4, True, "push"),
    (3, 4, 2, 128, 2, 3, 5, 60, 0.4, False, "split"),
    (3, 4, 2, 128, 2, 3, 5, 60, 0.4, False, "step"),
    (2, 8, 1, 128, 0, 4, 1, 40, 0.5, True, "step"),
    (2, 2, 2, 64, 4, 0, 6, 50, 0.5, True, "split"),
    (2, 16, 2, 128, 3, 5, 7, 45, 1.0, True, "push"),
    (2, 16, 2, 128, 3, 5, 7, 45, 1.0, True, "step"),
    (2, 4, 4, 64, 1, 8, 3, 45, 0.0, False, "push"),
    (2, 8, 2, 64, 4, 200, 300, 700, 0.3, True, "step"),   # 505 slots: one workgroup of 32 tiles
    (1, 4, 1, 128, 4, 400, 500, 1000, 0.4, True, "step"),  # 905 slots: two, merged through the workspace
    (1, 4, 2, 64, 2, 700, 400, 400, 0.5, False, "push"),   # 1103 slots: the split-and-merge kernels
    (1, 32, 8, 128, 4, 64, 256, 400, 0.12, True, "push"),
    (1, 32, 8, 128, 4, 64, 256, 400, 0.12, True, "step"),
    # slots a multiple of 16: K has no padding rows, the appended row opens a tile
    (2, 8, 2, 128, 4, 11, 16, 90, 0.4, True, "step"),      # 32 slots
    (2, 4, 2, 64, 2, 13, 16, 90, 0.3, False, "split"),     # 32 slots
    # with a capacity c > a + s + n (a past window of c - a - s - n entries);
    # the last field is c
    (3, 4, 2, 64, 2, 3, 5, 90, 0.4, True, "step", 16),
    (3, 4, 2, 128, 2, 3, 5, 90, 0.4, False, "push", 16),
    (2, 4, 2, 64, 2, 3, 5, 90, 0.5, True, "split", 14),
    (2, 8, 2, 128, 3, 0, 4, 70, 0.5, True, "step", 12),    # s = 0: the flush drops everything
    (2, 8, 1, 128, 1, 2, 1, 60, 0.6, False, "step", 9),    # n = 1
    (2, 8, 2, 128, 4, 64, 256, 1300, 0.12, True, "step", 800),  # c = 800: 801 slots, two workgroups
    (1, 4, 2, 64, 2, 300, 400, 900, 0.5, False, "push", 1100),  # 1101 slots: the split-and-merge kernels
    (2, 8, 2, 128, 2, 5, 9, 90, 0.5, True, "step", 47),    # 48 slots: no K padding, with a past window
]


@pytest.mark.parametrize("case", SMALL, ids=[f"cache{i}" for i in range(len(SMALL))])
def test_cache_steps_against_simulator(case):
    B, Hq, Hkv, d, a, s, n, T, p, shift, api = case[:11]
    cap = case[11] if len(case) > 11 else None
    say("cache", case)
    wl = synth.DecodeWorkload("small", 70, B=B, Hq=Hq, Hkv=Hkv, d=d, a=a, s=s, n=n, T=T, p=p, shift=shift)
    flags, kb, vb = _setup(wl)
    qb = _bf(wl.q_steps(range(T)))
    cache = sa.SepCache(B, Hkv, d, a, s, n, wl.theta, cap=cap or 0)
    sims = [orc.SepCacheSim(a, s, n, cap) for _ in range(B)]
    sc = 1 / math.sqrt(d)
    outs = []
    for t in range(T):
        fl = torch.from_numpy(flags[t]).cuda()
        if api == "step":
            outs.append(cache.step(kb[t].cuda(), vb[t].cuda(), fl, qb[t].cuda(), sc, shift=shift))
        else:
            if api == "split":
                cache.append(kb[t].cuda(), vb[t].cuda(), fl)
                cache.evict()
            else:
                cache.push(kb[t].cuda(), vb[t].cuda(), fl)
            outs.append(cache.decode(qb[t].cuda(), sc, shift=shift))
        for b in range(B):
            sims[b].append(int(flags[t, b]))
            sims[b].evict()
        if t < 12 or t % 7 == 0 or t == T - 1 or cache.slots <= 64:
            torch.cuda.synchronize()
            _check_state(cache, sims, kb, vb, t)
    torch.cuda.synchronize()
    ref, _ = orc.decode_run(as_f64(qb), as_f64(kb), as_f64(vb), flags, a, s, n, wl.theta, shift, sc, c=cap)
    for t in range(T):
        assert max_abs(as_f64(outs[t]), ref[t]) <= TOL_BF16, t
    assert int(cache.state[..., 6].abs().sum().cpu()) == 0  # no overflow flag


# Consecutive fused steps with the window full, the state checked after each:
# the evicted row walks over tiles held by different waves.
RUN = list(range(600, 624))


@pytest.mark.parametrize("shift", [True, False], ids=["shift", "original-positions"])
def test_llama_decode_full_run_sampled(shift):
    """The whole 8192-step Llama decode (16 streams, 32 q / 8 KV heads, d = 128,
    a = 4, s = 64, n = 256) through the fused step, with positions shifted to
    ranks in the cache and with original positions (plain RoPE, whose angles
    reach 8191 times the base frequency at the last steps)."""
    wl = synth.LLAMA_DECODE.with_(shift=shift)
    say("cache", wl.name, "shift" if shift else "original positions")
    flags, kb, vb = _setup(wl)
    sample = sorted({0, 1, 3, 4, 5, 100, 259, 260, 261, 793, 1500, 2048, 4095, 6000, 8000, 8001, 8100, 8190,
                     8191, *RUN})
    qb = _bf(wl.q_steps(sample))
    kd, vd = kb.cuda(), vb.cuda()
    fd = torch.from_numpy(flags).cuda()
    cache = sa.SepCache(wl.B, wl.Hkv, wl.d, wl.a, wl.s, wl.n, wl.theta)
    sims = [orc.SepCacheSim(wl.a, wl.s, wl.n) for _ in range(wl.B)]
    sc = 1 / math.sqrt(wl.d)
    outs = {}
    for t in range(wl.T):
        if t in sample:
            outs[t] = cache.step(kd[t], vd[t], fd[t], qb[sample.index(t)].cuda(), sc, shift=shift)
        else:
            cache.push(kd[t], vd[t], fd[t])
        for b in range(wl.B):
            sims[b].append(int(flags[t, b]))
            sims[b].evict()
        if t in sample:
            if t in (0, 5, 261, 793, 4095, 8000, 8191) or t in RUN:
                torch.cuda.synchronize()
                _check_state(cache, sims, kb, vb, t)
    torch.cuda.synchronize()
    assert all(len(s.order()) == wl.a + wl.s + wl.n for s in sims)
    qfull = np.zeros((wl.T, wl.B, wl.Hq, wl.d))
    qfull[sample] = as_f64(qb)
    ref, _ = orc.decode_run(qfull, as_f64(kb), as_f64(vb), flags, wl.a, wl.s, wl.n, wl.theta, shift, sc,
                            out_steps=sample)
    for t in sample:
        assert max_abs(as_f64(outs[t]), ref[t]) <= TOL_BF16, t


def test_full_batch_steps_move_rows():
    """The Llama decode geometry at its full batch (16 streams x 8 KV heads,
    one workgroup each, 21 tiles of 16 rows) with many separators, so that
    most window evictions move a row into the separator block (and, once
    that block is full, drop its oldest).  Every fused step from the point
    where the window is full is checked bit-exactly: the rows a step writes
    (the appended token's slot, freed by the previous eviction, and the
    moved row's destination) are ones it does not attend, while it reads the
    moved row's old K/V wherever that row's tile lies."""
    L = synth.LLAMA_DECODE
    T0, T = 300, 396
    wl = synth.DecodeWorkload("move-rows", 72, B=L.B, Hq=L.Hq, Hkv=L.Hkv, d=L.d, a=L.a, s=L.s, n=L.n, T=T, p=0.6)
    say("cache-move-rows")
    flags, kb, vb = _setup(wl)
    steps = list(range(T0, T))
    qb = _bf(wl.q_steps(steps)).cuda()
    kd, vd, fd = kb.cuda(), vb.cuda(), torch.from_numpy(flags).cuda()
    cache = sa.SepCache(wl.B, wl.Hkv, wl.d, wl.a, wl.s, wl.n, wl.theta)
    sims = [orc.SepCacheSim(wl.a, wl.s, wl.n) for _ in range(wl.B)]
    sc = 1 / math.sqrt(wl.d)
    outs = {}
    for t in range(T):
        if t >= T0:
            outs[t] = cache.step(kd[t], vd[t], fd[t], qb[t - T0], sc, shift=True)
        else:
            cache.push(kd[t], vd[t], fd[t])
        for b in range(wl.B):
            sims[b].append(int(flags[t, b]))
            sims[b].evict()
        if t >= T0:
            torch.cuda.synchronize()
            _check_state(cache, sims, kb, vb, t)
    qfull = np.zeros((T, wl.B, wl.Hq, wl.d))
    qfull[steps] = as_f64(qb.cpu())
    ref, _ = orc.decode_run(qfull, as_f64(kb), as_f64(vb), flags, wl.a, wl.s, wl.n, wl.theta, True, sc,
                            out_steps=steps[::8])
    for t in steps[::8]:
        assert max_abs(as_f64(outs[t]), ref[t]) <= TOL_BF16, t


def test_cache_resume_and_determinism():
    wl = synth.DecodeWorkload("resume", 71, B=4, Hq=8, Hkv=2, d=128, a=4, s=16, n=32, T=200, p=0.2)
    say("cache-resume")
    flags, kb, vb = _setup(wl)
    qb = _bf(wl.q_steps(range(wl.T))).cuda()
    kd, vd, fd = kb.cuda(), vb.cuda(), torch.from_numpy(flags).cuda()

    def run(cache, t0, t1):
        out = []
        for t in range(t0, t1):
            out.append(cache.step(kd[t], vd[t], fd[t], qb[t]))
        return out

    c1 = sa.SepCache(wl.B, wl.Hkv, wl.d, wl.a, wl.s, wl.n, wl.theta)
    straight = run(c1, 0, wl.T)
    c2 = sa.SepCache(wl.B, wl.Hkv, wl.d, wl.a, wl.s, wl.n, wl.theta)
    run(c2, 0, 100)
    snap = [t.clone() for t in (c2.k, c2.v, c2.slot_pos, c2.slot_sep, c2.state)]
    run(c2, 100, 150)  # diverge, then restore
    for dst, src in zip((c2.k, c2.v, c2.slot_pos, c2.slot_sep, c2.state), snap):
        dst.copy_(src)
    resumed = run(c2, 100, wl.T)
    torch.cuda.synchronize()
    for t in range(100, wl.T):
        assert torch.equal(straight[t], resumed[t - 100]), t


def test_append_without_evict_sets_overflow_flag():
    say("cache-overflow")
    B, Hkv, d = 2, 2, 64
    cache = sa.SepCache(B, Hkv, d, 1, 2, 2, 10000.0)
    k = torch.zeros((B, Hkv, d), dtype=torch.bfloat16, device="cuda")
    f = torch.zeros(B, dtype=torch.uint8, device="cuda")
    for _ in range(4):  # sink + window of 2 + spare slot, then one too many
        cache.append(k, k, f)
    cache.append(k, k, f)
    torch.cuda.synchronize()
    st = cache.state.cpu().numpy()
    assert np.all(st[..., 6] & 1)
    assert np.all(st[..., 0] == 4)  # the last token was not taken
