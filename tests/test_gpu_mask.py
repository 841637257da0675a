"""Mask metadata on the GPU against the oracle: bit-exact."""
import numpy as np
import pytest
import torch

from oracle import sepllm_oracle as orc
from separator_kv_cache_amd import binding as sa
from separator_kv_cache_amd import synth
from tests.util import say

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, L, a, n, p, clustered
    ("tiny-f32-shape", 1, 256, 4, 32, 0.15, False),
    ("pythia-n128", 8, 2048, 4, 128, 0.15, False),
    ("pythia-n64-p10", 8, 2048, 4, 64, 0.10, False),
    ("pythia-full", 8, 2048, 4, 2048, 0.20, False),
    ("llama-L32768", 1, 32768, 4, 4096, 0.12, True),
    ("ragged", 3, 1001, 3, 17, 0.3, False),
    ("L1", 2, 1, 4, 1, 0.5, False),
    ("a0-n1", 2, 300, 0, 1, 0.2, False),
    ("a-over-L", 2, 50, 60, 5, 0.5, False),
    ("all-sep", 2, 257, 4, 8, 1.0, False),
    ("no-sep", 2, 257, 4, 8, 0.0, False),
    ("n-over-L", 1, 100, 2, 500, 0.3, False),
    ("long-B2", 2, 70001, 4, 777, 0.12, True),
]


def _gpu_mask(tok, a, n):
    m = sa.build_mask(torch.from_numpy(tok).cuda(), synth.SEP_IDS, a, n)
    torch.cuda.synchronize()
    return m


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mask_metadata_bit_exact(case):
    name, B, L, a, n, p, clustered = case
    say("mask", name, B, L, a, n, p)
    tok = (synth.tokens_clustered if clustered else synth.tokens_iid)(11, 40, B, L, p)
    m = _gpu_mask(tok, a, n)
    f = orc.separator_flags(tok, synth.SEP_IDS)
    idx, cnt = orc.separator_index(f, a)
    pre = orc.separator_prefix(f, a)
    assert np.array_equal(m.is_sep.cpu().numpy(), f)
    assert np.array_equal(m.sep_cnt.cpu().numpy(), cnt)
    assert np.array_equal(m.sep_idx.cpu().numpy(), idx)
    assert np.array_equal(m.sep_before.cpu().numpy(), pre)
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


BIT_CASES = [c for c in CASES if c[2] <= 32768]


@pytest.mark.parametrize("case", BIT_CASES, ids=[c[0] for c in BIT_CASES])
def test_mask_expansion_matches_definition(case):
    """The dense mask as the forward kernel's traversal walks it (gathered
    anchors, then the band with its element test), every row, against the
    definition; up to the L = 32768 Llama-shaped sequence."""
    name, B, L, a, n, p, clustered = case
    say("mask-bits", name)
    tok = (synth.tokens_clustered if clustered else synth.tokens_iid)(12, 41, B, L, p)
    m = _gpu_mask(tok, a, n)
    bits = sa.mask_bits(m).cpu().numpy().view(np.uint32)
    f = orc.separator_flags(tok, synth.SEP_IDS)
    W = (L + 31) // 32
    for b in range(B):
        for r0 in range(0, L, 1024):
            r1 = min(L, r0 + 1024)
            M = orc.mask_rows(f[b], a, n, r0, r1)
            pad = np.zeros((r1 - r0, W * 32), dtype=bool)
            pad[:, :L] = M
            want = np.packbits(pad.reshape(r1 - r0, W, 32)[:, :, ::-1], axis=-1, bitorder="big")
            want = want.view(">u4").reshape(r1 - r0, W).astype(np.uint32)
            assert np.array_equal(bits[b, r0:r1], want), (name, b, r0)


@pytest.mark.parametrize("case", BIT_CASES, ids=[c[0] for c in BIT_CASES])
def test_tile_descriptors_bit_exact(case):
    """Per-query-tile (sink_vis, sep_vis, band_lo, band_hi) as the kernels
    derive them, against the oracle's reading of the mask: the forward's own
    tile size for the window and other tile sizes (ragged last tiles)."""
    name, B, L, a, n, p, clustered = case
    say("tile-desc", name)
    tok = (synth.tokens_clustered if clustered else synth.tokens_iid)(13, 43, B, L, p)
    m = _gpu_mask(tok, a, n)
    f = orc.separator_flags(tok, synth.SEP_IDS)
    fwd_rows = sa.fwd_tile_rows(n)
    assert fwd_rows == (64 if n <= 256 else 256)
    sizes = [256] if L > 4096 else sorted({1, 7, 64, 256, fwd_rows})
    for rows in sizes:
        got = sa.tile_desc(m, rows).cpu().numpy()
        want = orc.tile_descriptors(f, a, n, rows)
        assert np.array_equal(got, want), (name, rows)


def test_mask_deterministic():
    tok = synth.tokens_iid(3, 42, 4, 5000, 0.2)
    m1 = _gpu_mask(tok, 4, 100)
    m2 = _gpu_mask(tok, 4, 100)
    for name in ("is_sep", "sep_idx", "sep_before", "sep_cnt", "plain_idx", "plain_cnt", "kept"):
        assert torch.equal(getattr(m1, name), getattr(m2, name)), name
