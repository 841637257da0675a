"""The C ABI library loads, exports every declared entry point, and rejects
bad arguments with status codes (validation precedes any HIP call, so these
run without a GPU)."""
import ctypes
import os
import re

import pytest

from separator_kv_cache_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "sepattn.h")).read()
    return sorted(set(re.findall(r"SEPATTN_API\s+[\w\s\*]+?\b((?:sepattn|sepcache)_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for want in ("sepattn_build_mask", "sepattn_fwd", "sepattn_bwd", "sepcache_append", "sepcache_evict",
                 "sepcache_decode"):
        assert want in names
    assert set(names) == set(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.sepattn_version() >= 10000


def _shape(B=1, Hq=4, Hkv=2, L=64, d=64):
    s = _lib.SepattnShape()
    s.B, s.Hq, s.Hkv, s.L, s.d = B, Hq, Hkv, L, d
    for f in ("q_stride", "k_stride", "v_stride", "o_stride"):
        arr = getattr(s, f)
        H = Hq if f in ("q_stride", "o_stride") else Hkv
        arr[0], arr[1], arr[2] = H * L * d, L * d, d
    return s


def _mask(B=1, L=64, a=4, n=8):
    m = _lib.SepattnMask()
    buf = ctypes.create_string_buffer(_lib.load().sepattn_mask_bytes(B, L) + 256)
    base = (ctypes.addressof(buf) + 255) & ~255
    rc = _lib.load().sepattn_mask_carve(ctypes.byref(m), B, L, a, n, ctypes.c_void_p(base),
                                        _lib.load().sepattn_mask_bytes(B, L))
    assert rc == _lib.OK
    return m, buf


def test_argument_validation_without_gpu():
    lib = _lib.load()
    m, _keep = _mask()
    assert lib.sepattn_mask_bytes(0, 10) == 0
    m2 = _lib.SepattnMask()
    assert lib.sepattn_mask_carve(ctypes.byref(m2), 0, 5, 1, 1, ctypes.c_void_p(256), 10) == _lib.EINVAL
    assert lib.sepattn_mask_carve(ctypes.byref(m2), 1, 5, 1, 0, ctypes.c_void_p(256), 10 ** 6) == _lib.EINVAL
    assert lib.sepattn_mask_carve(ctypes.byref(m2), 1, 5, -1, 3, ctypes.c_void_p(256), 10 ** 6) == _lib.EINVAL
    assert lib.sepattn_mask_carve(ctypes.byref(m2), 2, 100, 1, 3, ctypes.c_void_p(256), 64) == _lib.ESPACE
    assert b"bytes" in lib.sepattn_last_error()
    ids = (ctypes.c_int32 * 1)(5)
    assert lib.sepattn_build_mask(None, ids, 1, ctypes.byref(m), None) == _lib.EINVAL
    assert lib.sepattn_build_mask(ctypes.c_void_p(256), ids, 0, ctypes.byref(m), None) == _lib.EINVAL
    assert lib.sepattn_build_mask(ctypes.c_void_p(256), ids, 65, ctypes.byref(m), None) == _lib.EINVAL
    p = ctypes.c_void_p(4096)
    s = _shape(Hq=3, Hkv=2)
    assert lib.sepattn_fwd(ctypes.byref(s), _lib.BF16, ctypes.byref(m), p, p, p, 0.1, p, None, None) == _lib.EINVAL
    assert b"multiple" in lib.sepattn_last_error()
    s = _shape(d=96)
    assert lib.sepattn_fwd(ctypes.byref(s), _lib.BF16, ctypes.byref(m), p, p, p, 0.1, p, None, None) == _lib.ENOTSUP
    s = _shape()
    assert lib.sepattn_fwd(ctypes.byref(s), 7, ctypes.byref(m), p, p, p, 0.1, p, None, None) == _lib.ENOTSUP
    assert lib.sepattn_fwd(ctypes.byref(s), _lib.BF16, ctypes.byref(m), None, p, p, 0.1, p, None, None) == _lib.EINVAL
    assert lib.sepattn_fwd(ctypes.byref(s), _lib.BF16, ctypes.byref(m), ctypes.c_void_p(4098), p, p, 0.1, p,
                           None, None) == _lib.EINVAL
    assert lib.sepattn_fwd(ctypes.byref(s), _lib.BF16, ctypes.byref(m), p, p, p, float("nan"), p, None,
                           None) == _lib.EINVAL
    s = _shape(L=65)
    assert lib.sepattn_fwd(ctypes.byref(s), _lib.BF16, ctypes.byref(m), p, p, p, 0.1, p, None, None) == _lib.EINVAL
    s = _shape()
    s.q_stride[2] = 3
    assert lib.sepattn_fwd(ctypes.byref(s), _lib.BF16, ctypes.byref(m), p, p, p, 0.1, p, None, None) == _lib.EINVAL
    s = _shape()
    s.o_stride[1] = 0  # every head's output rows on top of each other
    assert lib.sepattn_fwd(ctypes.byref(s), _lib.BF16, ctypes.byref(m), p, p, p, 0.1, p, None, None) == _lib.EINVAL
    assert b"overlap" in lib.sepattn_last_error()
    s = _shape()
    s.o_stride[2] = 32  # token rows of 64 elements, 32 apart
    assert lib.sepattn_fwd(ctypes.byref(s), _lib.BF16, ctypes.byref(m), p, p, p, 0.1, p, None, None) == _lib.EINVAL
    s = _shape()
    s.o_stride[0], s.o_stride[1], s.o_stride[2] = 64, 64 * 1, 64 * 4  # [B, L, H, d] storage: rows apart
    assert lib.sepattn_fwd(ctypes.byref(s), 7, ctypes.byref(m), p, p, p, 0.1, p, None, None) == _lib.ENOTSUP
    s = _shape()
    need = lib.sepattn_bwd_workspace_size(ctypes.byref(s))
    assert lib.sepattn_bwd(ctypes.byref(s), _lib.F32, ctypes.byref(m), p, p, p, p, p, p, 0.1, p, p, p, p,
                           need, None) == _lib.ENOTSUP  # the backward is bf16 only
    s.k_stride[1] = 0  # dK would take K's strides: an expanded K is refused
    assert lib.sepattn_bwd(ctypes.byref(s), _lib.BF16, ctypes.byref(m), p, p, p, p, p, p, 0.1, p, p, p, p,
                           need, None) == _lib.EINVAL
    assert b"overlap" in lib.sepattn_last_error()
    # the no-allocation backward: its static workspace bounds B * Hq * L
    mb, _keep_b = _mask(L=2048)
    s = _shape(Hq=4096, Hkv=1, L=2048)
    assert 4096 * 2048 > _lib.BWD_NOALLOC_MAX_ROWS
    assert lib.sepattn_bwd_noalloc(ctypes.byref(s), _lib.BF16, ctypes.byref(mb), p, p, p, p, p, p, 0.1, p, p, p,
                                   None) == _lib.ESPACE
    assert b"static workspace" in lib.sepattn_last_error()
    s = _shape()
    assert lib.sepattn_bwd_noalloc(ctypes.byref(s), _lib.F32, ctypes.byref(m), p, p, p, p, p, p, 0.1, p, p, p,
                                   None) == _lib.ENOTSUP
    assert lib.sepattn_bwd_noalloc(ctypes.byref(s), _lib.BF16, ctypes.byref(m), p, p, p, p, p, p, 0.1, None, p, p,
                                   None) == _lib.EINVAL
    s = _shape()
    need = lib.sepattn_bwd_workspace_size(ctypes.byref(s))
    assert need == 1 * 4 * 64 * 4 + 1024  # D rounded up to 256 bytes, then the dK/dV tile counters
    assert lib.sepattn_bwd(ctypes.byref(s), _lib.BF16, ctypes.byref(m), p, p, p, p, p, p, 0.1, p, p, p, p,
                           need - 1, None) == _lib.ESPACE
    assert lib.sepcache_slots(4, 64, 256, 0) == 325
    assert lib.sepcache_slots(4, 64, 256, 324) == 325
    assert lib.sepcache_slots(4, 64, 256, 800) == 801  # a past window of 476 entries
    assert lib.sepcache_slots(4, 64, 256, 300) == -1   # capacity below a + s + n
    assert lib.sepcache_slots(4, 64, 0, 0) == -1
    c = _lib.SepCacheStruct()
    c.B, c.Hkv, c.d, c.a, c.s, c.n = 2, 2, 64, 4, 8, 0
    assert lib.sepcache_reset(ctypes.byref(c), None) == _lib.EINVAL
    c.n, c.d = 16, 80
    assert lib.sepcache_reset(ctypes.byref(c), None) == _lib.ENOTSUP
    c.d = 64
    assert lib.sepcache_reset(ctypes.byref(c), None) == _lib.EINVAL  # null arrays
    c.k = c.v = c.slot_pos = c.slot_sep = c.state = 4096
    assert lib.sepcache_decode(ctypes.byref(c), 4, p, 0.1, 1, p, p, 10 ** 6, None) == _lib.EINVAL  # theta 0
    c.theta = 10000.0
    assert lib.sepcache_decode(ctypes.byref(c), 3, p, 0.1, 1, p, p, 10 ** 6, None) == _lib.EINVAL
    assert lib.sepcache_decode(ctypes.byref(c), 32, p, 0.1, 1, p, p, 10 ** 6, None) == _lib.ENOTSUP
    assert lib.sepcache_decode_workspace_size(ctypes.byref(c), 4) == 0  # small cache: one kernel
    c.s = 2000  # large cache: split path with a workspace
    need = lib.sepcache_decode_workspace_size(ctypes.byref(c), 4)
    assert need > 0
    assert lib.sepcache_decode(ctypes.byref(c), 4, p, 0.1, 1, p, p, need - 1, None) == _lib.ESPACE
    c.s = 8
    c.c = 20  # below a + s + n = 28
    assert lib.sepcache_reset(ctypes.byref(c), None) == _lib.EINVAL
    assert b"capacity" in lib.sepattn_last_error()
    c.c = 0
    assert lib.sepcache_step(ctypes.byref(c), None, p, p, 4, p, 0.1, 1, p, None, 0, None) == _lib.EINVAL
    # prompt hand-off: the mask must describe the cache's streams and sinks
    st3 = (ctypes.c_int64 * 3)(0, 0, 64)
    mk = _lib.SepattnMask()
    assert lib.sepcache_prefill(ctypes.byref(c), p, p, st3, st3, None, None) == _lib.EINVAL
    mk.B, mk.L, mk.a, mk.n = 2, 10, 4, 3
    mk.is_sep = mk.sep_idx = mk.sep_before = mk.sep_cnt = mk.plain_idx = mk.plain_cnt = mk.kept = 4096
    mk.a = 3
    assert lib.sepcache_prefill(ctypes.byref(c), p, p, st3, st3, ctypes.byref(mk), None) == _lib.EINVAL
    assert b"a=" in lib.sepattn_last_error()
    mk.a, mk.B = 4, 3
    assert lib.sepcache_prefill(ctypes.byref(c), p, p, st3, st3, ctypes.byref(mk), None) == _lib.EINVAL
    mk.B = 2
    assert lib.sepcache_prefill(ctypes.byref(c), None, p, st3, st3, ctypes.byref(mk), None) == _lib.EINVAL
    bad = (ctypes.c_int64 * 3)(0, 0, 65)
    assert lib.sepcache_prefill(ctypes.byref(c), p, p, bad, st3, ctypes.byref(mk), None) == _lib.EINVAL


def test_mask_rebuild_target_must_match():
    """build_mask(out=...) rebuilds into an existing Mask only if it
    describes the same B, L, a and n; a mismatch is refused before any
    device call (here on CPU tensors)."""
    import torch
    from separator_kv_cache_amd import binding as sa
    tok = torch.zeros((2, 40), dtype=torch.int32)
    m = sa.Mask(2, 40, 4, 8, device="cpu")
    for bad in (sa.Mask(1, 40, 4, 8, device="cpu"), sa.Mask(2, 41, 4, 8, device="cpu"),
                sa.Mask(2, 40, 3, 8, device="cpu"), sa.Mask(2, 40, 4, 9, device="cpu")):
        with pytest.raises(ValueError, match="out mask"):
            sa.build_mask(tok, [5], 4, 8, out=bad)
    assert (m.B, m.L, m.a, m.n) == (2, 40, 4, 8)


def test_tiled_key_layout():
    """sepcache_k_rows pads a slice to whole 16-row tiles, and the header's
    chunk formula (what tests.util.cache_k_rows reads back) is a bijection
    from (slot, dim) onto the padded slice."""
    import torch
    from tests.util import cache_k_rows
    lib = _lib.load()
    assert [lib.sepcache_k_rows(x) for x in (1, 15, 16, 17, 325, 65536)] == [16, 16, 16, 32, 336, 65536]
    assert lib.sepcache_k_rows(0) == -1 and lib.sepcache_k_rows(65537) == -1
    for slots, d in ((325, 128), (37, 64)):
        R, nch = lib.sepcache_k_rows(slots), d // 8
        flat = torch.full((R * d,), -1, dtype=torch.int64)
        for r in range(slots):
            for e in range(d):
                ch = e // 8
                idx = (((r // 16) * nch + ch) * 16 + r % 16) * 8 + e % 8
                assert flat[idx] == -1
                flat[idx] = r * d + e
        rows = cache_k_rows(flat.view(1, 1, R, d), slots)[0, 0]
        assert torch.equal(rows, torch.arange(slots * d).view(slots, d))


def test_binding_refuses_host_memory_and_bad_outputs():
    """The binding hands the kernels device pointers only: host tensors, a
    host-memory mask or cache, and outputs, log-sum-exps or output gradients
    that do not match what the entry points assume are refused before any
    call (here on CPU tensors, so nothing reaches a kernel)."""
    import torch
    from separator_kv_cache_amd import binding as sa
    with pytest.raises(ValueError, match="device tensor"):
        sa._ptr(torch.zeros(4))
    assert sa._ptr(None).value is None
    tok = torch.zeros((1, 32), dtype=torch.int32)
    with pytest.raises(ValueError, match="device tensor"):
        sa.build_mask(tok, [5], 4, 8)
    m = sa.Mask(1, 32, 4, 8, device="cpu")
    with pytest.raises(ValueError, match="device memory"):
        m.ref()
    with pytest.raises(ValueError, match="device memory"):
        sa.SepCache(1, 1, 64, 4, 8, 16, device="cpu")
    q = torch.zeros((1, 2, 32, 64), dtype=torch.bfloat16)
    kv = torch.zeros((1, 1, 32, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="q's dtype"):
        sa.sepattn_fwd(q, kv, kv, m, out=torch.zeros(q.shape, dtype=torch.float32))
    with pytest.raises(ValueError, match="lse must be"):
        sa.sepattn_fwd(q, kv, kv, m, lse=torch.zeros((1, 2, 31)))
    with pytest.raises(ValueError, match="lse must be"):
        sa.sepattn_bwd(q, kv, kv, q, torch.zeros((1, 2, 32), dtype=torch.float64), q, m)
    with pytest.raises(ValueError, match="o's shape"):
        sa.sepattn_bwd(q, kv, kv, q, torch.zeros((1, 2, 32)), q[:, :1], m)
    with pytest.raises(ValueError, match="q's dtype"):
        sa.sepattn_bwd(q, kv, kv, q, torch.zeros((1, 2, 32)), q.float(), m)


def test_binding_output_layouts():
    """The gradients take the strides of q, k and v: the binding recognises
    layouts whose rows overlap (an expanded view) and copies those inputs to
    contiguous tensors before the backward."""
    import torch
    from separator_kv_cache_amd import binding as sa
    kv = torch.zeros((2, 1, 32, 64), dtype=torch.bfloat16)
    assert sa._rows_apart(kv)
    assert not sa._rows_apart(kv.expand(2, 4, 32, 64))           # head stride 0
    assert sa._rows_apart(torch.zeros((2, 32, 4, 64)).permute(0, 2, 1, 3))  # [B, L, H, d] storage
    assert not sa._rows_apart(torch.zeros(256).as_strided((1, 1, 2, 64), (128, 128, 32, 1)))  # rows 32 apart
    assert sa._rows_apart(torch.zeros((1, 1, 1, 64)).expand(3, 1, 1, 64)[:1])
