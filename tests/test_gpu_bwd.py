"""Backward on the GPU against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

from oracle import sepllm_oracle as orc
from separator_kv_cache_amd import binding as sa
from separator_kv_cache_amd import synth
from tests.util import TOL_BF16, TOL_LSE_BF16, as_f64, edge_excess, inputs, max_abs, say

pytestmark = pytest.mark.gpu


def _run(wl, seed=0):
    tok_d, (q, k, v), host, tok = inputs(wl, seed)
    do = torch.from_numpy(wl.dout(seed)).to(torch.bfloat16)
    m = sa.build_mask(tok_d, synth.SEP_IDS, wl.a, wl.n)
    sc = 1.0 / math.sqrt(wl.d)
    o, lse = sa.sepattn_fwd(q, k, v, m, sc)
    dq, dk, dv = sa.sepattn_bwd(q, k, v, o, lse, do.cuda(), m, sc)
    torch.cuda.synchronize()
    f = orc.separator_flags(tok, synth.SEP_IDS)
    return (dq, dk, dv), host + (as_f64(do),), f, (o, lse)


@pytest.mark.parametrize("wl", synth.PYTHIA_BWD, ids=lambda w: w.name)
def test_bwd_pythia_shape(wl):
    """The Pythia-160M-shaped forward and backward (8 sequences x 12 heads,
    L = 2048, d = 64): O, LSE, dQ, dK and dV of every (sequence, head)
    against the oracle, element by element."""
    say("bwd", wl.name)
    (dq, dk, dv), (q, k, v, do), f, (o, lse) = _run(wl)
    sc = 1 / math.sqrt(wl.d)
    ro, rl = orc.attn_fwd(q, k, v, f, wl.a, wl.n, sc)
    err_o, err_l = max_abs(as_f64(o), ro), max_abs(as_f64(lse), rl)
    print(wl.name, "o max-abs", err_o, "lse max-abs", err_l)
    assert err_o <= TOL_BF16 and err_l <= TOL_LSE_BF16
    rq, rk, rv = orc.attn_bwd(q, k, v, do, f, wl.a, wl.n, sc)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        err = max_abs(as_f64(got), ref)
        print(wl.name, name, "max-abs", err)
        assert err <= TOL_BF16, name


@pytest.fixture(scope="module")
def llama_bwd():
    """The Llama-3-8B-shaped forward and backward (L = 32768, 32 q / 8 KV
    heads, d = 128, n = 4096, clustered separators, dO ~ N(0, 1)) run once on
    the GPU, gradients on the host."""
    wl = synth.LLAMA_PREFILL
    say("bwd", wl.name)
    (dq, dk, dv), host, f, _ = _run(wl)
    return wl, (as_f64(dq), as_f64(dk), as_f64(dv)), host, f


def test_bwd_llama_prefill_invariants(llama_bwd):
    """Every KV head: rows of P sum to one, so the keys' dV sum to the rows'
    dO and the keys' dK sum to zero; sampled dQ rows of every q head."""
    wl, (dqg, dkg, dvg), (q, k, v, do), f = llama_bwd
    assert np.isfinite(dqg).all() and np.isfinite(dkg).all() and np.isfinite(dvg).all()
    sc = 1 / math.sqrt(wl.d)
    g = wl.Hq // wl.Hkv
    for kh in range(wl.Hkv):
        want = do[0, kh * g:(kh + 1) * g].sum(axis=(0, 1))
        assert max_abs(dvg[0, kh].sum(axis=0), want) < 1.0, kh
        assert np.abs(dkg[0, kh].sum(axis=0)).max() < 1.0, kh
    rng = np.random.default_rng(2)
    for h in range(wl.Hq):
        rows = np.concatenate([[0, 4, 4096, wl.L - 1], rng.integers(0, wl.L, 3)])
        rq = orc.attn_bwd_rows(q, k, v, do, f, wl.a, wl.n, sc, 0, h, rows)
        assert max_abs(dqg[0, h, rows], rq) <= TOL_BF16, h


@pytest.mark.parametrize("kv", [0, synth.LLAMA_PREFILL.Hkv - 1], ids=lambda i: f"kv{i}")
def test_bwd_llama_prefill_full_size(llama_bwd, kv):
    """dQ of the KV group's four q heads and its dK, dV, every row, against
    the oracle."""
    wl, (dqg, dkg, dvg), (q, k, v, do), f = llama_bwd
    g = wl.Hq // wl.Hkv
    hs = slice(kv * g, (kv + 1) * g)
    rq, rk, rv = orc.attn_bwd(q[:, hs], k[:, kv:kv + 1], v[:, kv:kv + 1], do[:, hs], f, wl.a, wl.n,
                              1 / math.sqrt(wl.d), block=512)
    for name, got, ref in (("dq", dqg[:, hs], rq), ("dk", dkg[:, kv:kv + 1], rk), ("dv", dvg[:, kv:kv + 1], rv)):
        err = max_abs(got, ref)
        print("kv", kv, name, "max-abs", err)
        assert err <= TOL_BF16, name


EDGE = [
    # B, Hq, Hkv, L, d, a, n, p
    (2, 4, 2, 333, 128, 4, 40, 0.15),
    (1, 2, 1, 1, 64, 4, 1, 0.5),
    (2, 2, 2, 300, 64, 0, 1, 0.2),
    (1, 3, 1, 97, 128, 200, 5, 0.3),
    (1, 2, 2, 200, 64, 4, 200, 0.3),
    (2, 4, 1, 257, 64, 4, 8, 1.0),
    (2, 4, 1, 257, 128, 4, 8, 0.0),
    (1, 8, 2, 700, 128, 2, 300, 0.12),
    (1, 2, 1, 1500, 64, 4, 1000, 0.05),
    (1, 2, 2, 129, 64, 1, 3, 0.4),
    # 256-row query tiles (n > 256): one or two key tiles, rows past L, no sinks
    (2, 4, 2, 260, 128, 4, 257, 0.2),
    (1, 2, 1, 64, 128, 4, 300, 0.3),
    (1, 4, 4, 1030, 64, 0, 600, 0.25),
]


@pytest.mark.parametrize("case", EDGE, ids=[f"edge{i}" for i in range(len(EDGE))])
def test_bwd_edge_cases(case):
    B, Hq, Hkv, L, d, a, n, p = case
    say("bwd-edge", case)
    wl = synth.PrefillWorkload("edge", 52, B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, a=a, n=n, p=p, dtype="bf16",
                               qkv_scale=0.5)
    (dq, dk, dv), (q, k, v, do), f, _ = _run(wl, seed=5)
    rq, rk, rv = orc.attn_bwd(q, k, v, do, f, a, n, 1 / math.sqrt(d))
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        err = max_abs(as_f64(got), ref)
        print(name, "max-abs", err, "max |ref|", float(np.abs(ref).max()))
        assert edge_excess(as_f64(got), ref) <= 0.0, (name, err)


def test_bwd_deterministic_and_strided():
    B, Hq, Hkv, L, d, a, n = 2, 4, 2, 400, 128, 4, 64
    wl = synth.PrefillWorkload("strided", 53, B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, a=a, n=n, p=0.2, dtype="bf16",
                               qkv_scale=0.5)
    say("bwd-strided")
    (dq1, dk1, dv1), _, _, (o, lse) = _run(wl, seed=6)
    (dq2, dk2, dv2), (q, k, v, do), f, _ = _run(wl, seed=6)
    assert torch.equal(dq1, dq2) and torch.equal(dk1, dk2) and torch.equal(dv1, dv2)
    qd, kd, vd = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (q, k, v))
    perm = lambda t: t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    dod = perm(torch.from_numpy(do).to(torch.bfloat16).cuda())
    tok_d = torch.from_numpy(wl.tokens(6)).cuda()
    m = sa.build_mask(tok_d, synth.SEP_IDS, a, n)
    qs, ks, vs = perm(qd), perm(kd), perm(vd)
    os_ = perm(o)
    dq3, dk3, dv3 = sa.sepattn_bwd(qs, ks, vs, os_, lse, dod, m)
    torch.cuda.synchronize()
    assert torch.equal(dq3, dq1) and torch.equal(dk3, dk1) and torch.equal(dv3, dv1)
