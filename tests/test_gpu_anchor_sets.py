"""Anchor-set variants on the GPU against the oracle: fixed-interval anchors
(FixLLM, [HUB] third reviewer A2) and separator subsets ([HUB] first reviewer
A6).  Only the flags change; the metadata, forward, backward and cache
kernels are the ones of the separator mask."""
import math

import numpy as np
import pytest
import torch

from oracle import sepllm_oracle as orc
from separator_kv_cache_amd import binding as sa
from separator_kv_cache_amd import synth
from tests.util import TOL_BF16, TOL_LSE_BF16, as_f64, inputs, max_abs, say, edge_excess

pytestmark = pytest.mark.gpu


def _check_meta(m, f, a, n):
    B, L = f.shape
    idx, cnt = orc.separator_index(f, a)
    assert np.array_equal(m.is_sep.cpu().numpy(), f)
    assert np.array_equal(m.sep_cnt.cpu().numpy(), cnt)
    assert np.array_equal(m.sep_idx.cpu().numpy(), idx)
    assert np.array_equal(m.sep_before.cpu().numpy(), orc.separator_prefix(f, a))
    plain = np.full((B, L), L, dtype=np.int32)
    pc = np.zeros(B, dtype=np.int32)
    for b in range(B):
        lst = [j for j in range(a, L) if not f[b, j]]
        plain[b, :len(lst)] = lst
        pc[b] = len(lst)
    assert np.array_equal(m.plain_cnt.cpu().numpy(), pc)
    assert np.array_equal(m.plain_idx.cpu().numpy(), plain)
    if L <= 40000:
        assert np.array_equal(m.kept.cpu().numpy(), orc.kept_pairs(f, a, n))


FIXED = [
    # B, L, a, n, delta
    (2, 1, 4, 1, 1),
    (2, 300, 4, 16, 8),
    (1, 1001, 3, 17, 1),      # every token an anchor: causal
    (1, 1001, 3, 17, 2000),   # no anchor: sinks + window
    (3, 2048, 0, 64, 5),
    (1, 32768, 4, 4096, 8),   # the Llama prefill length, one anchor in 8
]


@pytest.mark.parametrize("case", FIXED, ids=[f"fixed{i}" for i in range(len(FIXED))])
def test_fixed_anchor_metadata_bit_exact(case):
    B, L, a, n, delta = case
    say("fixed-meta", case)
    m = sa.build_mask_fixed(B, L, delta, a, n)
    torch.cuda.synchronize()
    _check_meta(m, orc.fixed_flags(B, L, delta), a, n)


def _fwd_bwd(wl, m, f, seed):
    tok_d, (q, k, v), (qh, kh, vh), _ = inputs(wl, seed)
    do = torch.from_numpy(wl.dout(seed)).to(torch.bfloat16)
    sc = 1.0 / math.sqrt(wl.d)
    o, lse = sa.sepattn_fwd(q, k, v, m, sc)
    dq, dk, dv = sa.sepattn_bwd(q, k, v, o, lse, do.cuda(), m, sc)
    torch.cuda.synchronize()
    ro, rl = orc.attn_fwd(qh, kh, vh, f, wl.a, wl.n, sc)
    assert max_abs(as_f64(o), ro) <= TOL_BF16
    assert max_abs(as_f64(lse), rl) <= TOL_LSE_BF16
    rq, rk, rv = orc.attn_bwd(qh, kh, vh, as_f64(do), f, wl.a, wl.n, sc)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        assert edge_excess(as_f64(got), ref) <= 0.0, name


@pytest.mark.parametrize("delta,n", [(8, 40), (3, 300), (16, 4)])
def test_fixed_anchor_forward_backward(delta, n):
    B, Hq, Hkv, L, d, a = 2, 4, 2, 333, 128, 4
    say("fixed-fwd-bwd", delta, n)
    wl = synth.PrefillWorkload("fixed", 54, B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, a=a, n=n, p=0.0, dtype="bf16",
                               qkv_scale=0.5)
    m = sa.build_mask_fixed(B, L, delta, a, n)
    _fwd_bwd(wl, m, orc.fixed_flags(B, L, delta), seed=7)


@pytest.mark.parametrize("subset", [synth.SEP_IDS[:2], synth.SEP_IDS[3:8], synth.SEP_IDS[-1:]])
def test_separator_subset(subset):
    B, Hq, Hkv, L, d, a, n = 2, 4, 2, 400, 128, 4, 32
    say("subset", subset)
    wl = synth.PrefillWorkload("subset", 55, B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, a=a, n=n, p=0.4, dtype="bf16",
                               qkv_scale=0.5)
    tok = wl.tokens(9)
    m = sa.build_mask(torch.from_numpy(tok).cuda(), subset, a, n)
    torch.cuda.synchronize()
    f = orc.separator_flags(tok, subset)
    _check_meta(m, f, a, n)
    _fwd_bwd(wl, m, f, seed=9)


def test_fixed_anchor_streaming_cache():
    """A streaming cache fed FixLLM flags (token t is an anchor iff delta
    divides t + 1) keeps them in its separator block, like separators."""
    B, Hq, Hkv, d, a, s, n, T, delta = 2, 8, 2, 128, 4, 6, 10, 120, 5
    say("fixed-cache")
    rng = np.random.default_rng(12)
    flags = np.ascontiguousarray(orc.fixed_flags(B, T, delta).T)  # [T, B]
    kb = torch.from_numpy(rng.standard_normal((T, B, Hkv, d), dtype=np.float32)).to(torch.bfloat16)
    vb = torch.from_numpy(rng.standard_normal((T, B, Hkv, d), dtype=np.float32)).to(torch.bfloat16)
    qb = torch.from_numpy(rng.standard_normal((T, B, Hq, d), dtype=np.float32)).to(torch.bfloat16)
    cache = sa.SepCache(B, Hkv, d, a, s, n, 10000.0)
    fd = torch.from_numpy(flags).cuda()
    sc = 1 / math.sqrt(d)
    outs = [cache.step(kb[t].cuda(), vb[t].cuda(), fd[t], qb[t].cuda(), sc, shift=True) for t in range(T)]
    torch.cuda.synchronize()
    ref, orders = orc.decode_run(as_f64(qb), as_f64(kb), as_f64(vb), flags, a, s, n, 10000.0, True, sc,
                                 order_steps=[T - 1])
    pos, ln = cache.export_order()
    for b in range(B):
        assert pos[b, :ln[b]].cpu().tolist() == orders[T - 1][b]
        assert all((j + 1) % delta == 0 for j in orders[T - 1][b][a:-n])  # the anchors kept outside the window
    for t in range(T):
        assert max_abs(as_f64(outs[t]), ref[t]) <= TOL_BF16, t
