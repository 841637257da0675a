"""Forward on the GPU against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

from oracle import sepllm_oracle as orc
from separator_kv_cache_amd import binding as sa
from separator_kv_cache_amd import synth
from tests.util import TOL_BF16, TOL_F32, TOL_LSE_BF16, as_f64, inputs, max_abs, say

pytestmark = pytest.mark.gpu


def _run(wl, seed=0):
    tok_d, (q, k, v), host, tok = inputs(wl, seed)
    m = sa.build_mask(tok_d, synth.SEP_IDS, wl.a, wl.n)
    o, lse = sa.sepattn_fwd(q, k, v, m, 1.0 / math.sqrt(wl.d))
    torch.cuda.synchronize()
    f = orc.separator_flags(tok, synth.SEP_IDS)
    return o, lse, host, f


def _tol(wl):
    return (TOL_F32, TOL_F32) if wl.dtype == "f32" else (TOL_BF16, TOL_LSE_BF16)


def test_fwd_tiny_f32_full():
    wl = synth.TINY_F32
    say("fwd", wl.name)
    o, lse, (q, k, v), f = _run(wl)
    ro, rl = orc.attn_fwd(q, k, v, f, wl.a, wl.n, 1 / math.sqrt(wl.d))
    assert max_abs(as_f64(o), ro) <= TOL_F32
    assert max_abs(as_f64(lse), rl) <= TOL_F32


@pytest.mark.parametrize("wl", [synth.PYTHIA_FWD, synth.PYTHIA_FWD_N64, synth.PYTHIA_FWD_FULL],
                         ids=lambda w: w.name)
def test_fwd_pythia_shape(wl):
    say("fwd", wl.name)
    o, lse, (q, k, v), f = _run(wl)
    og, lg = as_f64(o), as_f64(lse)
    sc = 1 / math.sqrt(wl.d)
    # two whole (sequence, head) slices ...
    for b, h in ((0, 0), (wl.B - 1, wl.Hq - 1)):
        ro, rl = orc.attn_fwd(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                              f[b:b + 1], wl.a, wl.n, sc)
        assert max_abs(og[b, h], ro[0, 0]) <= TOL_BF16, (b, h)
        assert max_abs(lg[b, h], rl[0, 0]) <= TOL_LSE_BF16, (b, h)
    # ... and sampled rows of every (sequence, head)
    rng = np.random.default_rng(0)
    for b in range(wl.B):
        for h in range(wl.Hq):
            rows = np.concatenate([[0, wl.L - 1], rng.integers(0, wl.L, 6)])
            ro, rl = orc.attn_fwd_rows(q, k, v, f, wl.a, wl.n, sc, b, h, rows)
            assert max_abs(og[b, h, rows], ro) <= TOL_BF16, (b, h)
            assert max_abs(lg[b, h, rows], rl) <= TOL_LSE_BF16, (b, h)


@pytest.fixture(scope="module")
def llama_fwd():
    """The Llama-3-8B-shaped forward (L = 32768, 32 q / 8 KV heads, d = 128,
    n = 4096, clustered separators) run once on the GPU, outputs on the host."""
    wl = synth.LLAMA_PREFILL
    say("fwd", wl.name)
    o, lse, host, f = _run(wl)
    return wl, as_f64(o), as_f64(lse), host, f


@pytest.mark.parametrize("kv", range(synth.LLAMA_PREFILL.Hkv), ids=lambda i: f"kv{i}")
def test_fwd_llama_prefill_full_size(llama_fwd, kv):
    """Every row of the KV group's four q heads against the oracle."""
    wl, og, lg, (q, k, v), f = llama_fwd
    g = wl.Hq // wl.Hkv
    hs = slice(kv * g, (kv + 1) * g)
    ro, rl = orc.attn_fwd(q[:, hs], k[:, kv:kv + 1], v[:, kv:kv + 1], f, wl.a, wl.n, 1 / math.sqrt(wl.d))
    err_o, err_l = max_abs(og[:, hs], ro), max_abs(lg[:, hs], rl)
    print("kv", kv, "o max-abs", err_o, "lse max-abs", err_l)
    assert err_o <= TOL_BF16 and err_l <= TOL_LSE_BF16


EDGE = [
    # B, Hq, Hkv, L, d, a, n, p, dtype
    (2, 4, 2, 333, 128, 4, 40, 0.15, "bf16"),
    (1, 2, 1, 1, 64, 4, 1, 0.5, "bf16"),
    (2, 2, 2, 300, 64, 0, 1, 0.2, "bf16"),
    (1, 3, 1, 97, 128, 200, 5, 0.3, "bf16"),
    (1, 2, 2, 200, 64, 4, 200, 0.3, "f32"),
    (2, 4, 1, 257, 64, 4, 8, 1.0, "bf16"),
    (2, 4, 1, 257, 128, 4, 8, 0.0, "f32"),
    (1, 8, 2, 700, 128, 2, 300, 0.12, "bf16"),
    (1, 2, 1, 1500, 64, 4, 1000, 0.05, "f32"),
]


@pytest.mark.parametrize("case", EDGE, ids=[f"edge{i}" for i in range(len(EDGE))])
def test_fwd_edge_cases(case):
    B, Hq, Hkv, L, d, a, n, p, dt = case
    say("fwd-edge", case)
    wl = synth.PrefillWorkload("edge", 50, B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, a=a, n=n, p=p, dtype=dt)
    o, lse, (q, k, v), f = _run(wl, seed=3)
    ro, rl = orc.attn_fwd(q, k, v, f, a, n, 1 / math.sqrt(d))
    tol, tl = _tol(wl)
    assert max_abs(as_f64(o), ro) <= tol
    assert max_abs(as_f64(lse), rl) <= tl


def test_fwd_strided_layout_and_determinism():
    # [B, L, H, d] storage viewed as [B, H, L, d]
    B, Hq, Hkv, L, d, a, n = 2, 4, 2, 400, 128, 4, 64
    wl = synth.PrefillWorkload("strided", 51, B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, a=a, n=n, p=0.2, dtype="bf16")
    say("fwd-strided")
    tok_d, (q, k, v), (qh, kh, vh), tok = inputs(wl, 4)
    qs = q.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    ks = k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    vs = v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    m = sa.build_mask(tok_d, synth.SEP_IDS, a, n)
    out = torch.empty((B, L, Hq, d), dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
    o1, _ = sa.sepattn_fwd(qs, ks, vs, m, out=out)
    o2, _ = sa.sepattn_fwd(q, k, v, m)
    o3, _ = sa.sepattn_fwd(q, k, v, m)
    torch.cuda.synchronize()
    assert torch.equal(o2, o3)
    assert torch.equal(o1, o2)
    f = orc.separator_flags(tok, synth.SEP_IDS)
    ro, _ = orc.attn_fwd(qh, kh, vh, f, a, n, 1 / math.sqrt(d))
    assert max_abs(as_f64(o1), ro) <= TOL_BF16
