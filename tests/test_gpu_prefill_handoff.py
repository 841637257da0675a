"""Prompt hand-off from prefill into a SepCache on the GPU: sepcache_prefill
against pushing the prompt token by token (every array bit-exact), against the
oracle's simulator, and decode steps after it against the oracle's decode of
the whole sequence."""
import math

import numpy as np
import pytest
import torch

from oracle import sepllm_oracle as orc
from separator_kv_cache_amd import binding as sa
from separator_kv_cache_amd import synth
from tests.test_gpu_cache import _check_state
from tests.util import TOL_BF16, as_f64, max_abs, say

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, d, a, s, n, c, L (prompt), T (steps after), p, shift, strided K/V
    (2, 8, 2, 128, 4, 6, 10, 0, 1, 20, 0.3, True, False),     # a one-token prompt (a sink)
    (2, 8, 2, 128, 4, 6, 10, 0, 3, 20, 0.3, True, False),     # shorter than the sinks
    (2, 8, 2, 64, 4, 6, 10, 0, 12, 20, 0.3, False, False),    # the window not yet full
    (3, 4, 2, 128, 4, 6, 10, 0, 200, 40, 0.3, True, True),    # many separators gone; strided K/V
    (2, 8, 2, 128, 2, 3, 5, 16, 150, 40, 0.4, True, False),   # with a past window (c > a + s + n)
    (2, 8, 2, 64, 0, 0, 4, 12, 77, 30, 0.5, False, False),    # a = 0, s = 0, past window
    (16, 32, 8, 128, 4, 64, 256, 0, 4096, 16, 0.12, True, False),  # Llama decode geometry, 4096-token prompt
]


def _bf(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


@pytest.mark.parametrize("case", CASES, ids=[f"handoff{i}" for i in range(len(CASES))])
def test_prefill_handoff(case):
    B, Hq, Hkv, d, a, s, n, cap, L, T, p, shift, strided = case
    say("handoff", case)
    rng = np.random.default_rng(1000 + 7 * L + B)
    tok = synth.tokens_iid(0, 80 + L, B, L, p)
    f_prompt = orc.separator_flags(tok, synth.SEP_IDS).astype(np.uint8)  # [B, L]
    f_dec = (rng.random((T, B)) < p).astype(np.uint8)
    flags = np.concatenate([f_prompt.T, f_dec], axis=0)  # [L + T, B]
    kb = _bf(rng.standard_normal((L + T, B, Hkv, d), dtype=np.float32))  # token-major, as the simulator checks
    vb = _bf(rng.standard_normal((L + T, B, Hkv, d), dtype=np.float32))
    qb = _bf(rng.standard_normal((T, B, Hq, d), dtype=np.float32))
    kd, vd = kb.cuda(), vb.cuda()
    if strided:  # [B, L, Hkv, d] storage viewed as [B, Hkv, L, d]
        kp = kd[:L].permute(1, 0, 2, 3).contiguous().permute(0, 2, 1, 3)
        vp = vd[:L].permute(1, 0, 2, 3).contiguous().permute(0, 2, 1, 3)
    else:
        kp = kd[:L].permute(1, 2, 0, 3).contiguous()
        vp = vd[:L].permute(1, 2, 0, 3).contiguous()
    m = sa.build_mask(torch.from_numpy(tok).cuda(), synth.SEP_IDS, a, 8)
    a_cache = sa.SepCache(B, Hkv, d, a, s, n, 10000.0, cap=cap)
    a_cache.prefill(kp, vp, m)
    b_cache = sa.SepCache(B, Hkv, d, a, s, n, 10000.0, cap=cap)
    fd = torch.from_numpy(flags).cuda()
    for t in range(L):
        b_cache.push(kd[t], vd[t], fd[t])
    torch.cuda.synchronize()
    for name in ("k", "v", "slot_pos", "slot_sep", "state"):
        assert torch.equal(getattr(a_cache, name), getattr(b_cache, name)), name
    sims = [orc.SepCacheSim(a, s, n, cap or None) for _ in range(B)]
    for t in range(L):
        for bb in range(B):
            sims[bb].append(int(flags[t, bb]))
            sims[bb].evict()
    _check_state(a_cache, sims, kb, vb, L - 1)
    # decode on from the handed-over cache
    sc = 1 / math.sqrt(d)
    outs = []
    for i in range(T):
        outs.append(a_cache.step(kd[L + i], vd[L + i], fd[L + i], qb[i].cuda(), sc, shift=shift))
    torch.cuda.synchronize()
    q_all = np.zeros((L + T, B, Hq, d))
    q_all[L:] = as_f64(qb)
    ref, _ = orc.decode_run(q_all, as_f64(kb), as_f64(vb), flags, a, s, n, 10000.0, shift, sc,
                            out_steps=range(L, L + T), c=cap or None)
    for i in range(T):
        assert max_abs(as_f64(outs[i]), ref[L + i]) <= TOL_BF16, i
