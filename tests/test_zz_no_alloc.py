"""sepattn_bwd_noalloc (the backward with the library's static workspace, for
callers that cannot allocate) against sepattn_bwd, through the C ABI: two
calls in a row, the second smaller than the first, each bit-identical to
the workspace entry point's gradients and within the per-element bf16 bound
of the oracle."""
import ctypes
import math

import numpy as np
import pytest
import torch

from oracle import sepllm_oracle as orc
from separator_kv_cache_amd import _lib
from separator_kv_cache_amd import binding as sa
from separator_kv_cache_amd import synth
from tests.util import as_f64, edge_excess, inputs, say

pytestmark = pytest.mark.gpu

CASES = [
    # a larger call first, then a smaller one: the static array keeps the
    # first call's D values past the second call's rows
    synth.PrefillWorkload("noalloc-1", 56, B=2, Hq=8, Hkv=2, L=1100, d=128, a=4, n=300, p=0.15, dtype="bf16",
                          qkv_scale=0.5),
    synth.PrefillWorkload("noalloc-2", 57, B=1, Hq=4, Hkv=2, L=333, d=64, a=2, n=40, p=0.2, dtype="bf16",
                          qkv_scale=0.5),
]


def test_noalloc_backward_matches_workspace_backward():
    lib = _lib.load()
    for wl in CASES:
        say("bwd-noalloc", wl.name)
        tok_d, (q, k, v), host, tok = inputs(wl, 8)
        do = torch.from_numpy(wl.dout(8)).to(torch.bfloat16).cuda()
        m = sa.build_mask(tok_d, synth.SEP_IDS, wl.a, wl.n)
        sc = 1.0 / math.sqrt(wl.d)
        o, lse = sa.sepattn_fwd(q, k, v, m, sc)
        ref = sa.sepattn_bwd(q, k, v, o, lse, do, m, sc)
        got = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
        s = sa._shape(q, k, v, o)
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = lib.sepattn_bwd_noalloc(ctypes.byref(s), _lib.BF16, m.ref(), *(ctypes.c_void_p(t.data_ptr()) for t in
                                     (q, k, v, o, lse, do)), sc, *(ctypes.c_void_p(t.data_ptr()) for t in got),
                                     stream)
        assert rc == _lib.OK, lib.sepattn_last_error()
        torch.cuda.synchronize()
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(g, r), (wl.name, name)
        f = orc.separator_flags(tok, synth.SEP_IDS)
        rq, rk, rv = orc.attn_bwd(*host, as_f64(do), f, wl.a, wl.n, sc)
        # cases off the stated workloads (four q heads summed into dK/dV, whose
        # entries reach about 4): the per-element bf16 bound
        for name, g, r in zip(("dq", "dk", "dv"), got, (rq, rk, rv)):
            assert edge_excess(as_f64(g), r) <= 0.0, (wl.name, name)
