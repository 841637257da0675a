"""Thin torch-facing binding of the C ABI: argument marshalling only.

Tensors are PyTorch device tensors; work is enqueued on torch's current
stream.  Every computation happens in the HIP kernels of libsepattn.so; if
the library is missing, the first call raises.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import BF16, F32, SepattnMask, SepattnShape, SepCacheStruct, check

_DT = {torch.bfloat16: BF16, torch.float32: F32}


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    if t is not None and not t.is_cuda:
        # the kernels dereference every pointer on the device
        raise ValueError(f"expected a device tensor, got one on {t.device}")
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _check_lse(lse: torch.Tensor, B: int, Hq: int, L: int):
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, L) or not lse.is_contiguous():
        raise ValueError(f"lse must be contiguous fp32 [{B}, {Hq}, {L}]")


class Mask:
    """Mask metadata for B sequences of L tokens in one device buffer."""

    def __init__(self, B: int, L: int, a: int, n: int, device="cuda"):
        lib = _lib.load()
        nbytes = lib.sepattn_mask_bytes(B, L)
        if nbytes == 0:
            raise ValueError(f"bad mask size B={B} L={L}")
        self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.c = SepattnMask()
        # carving only computes the fields' addresses inside the buffer
        check(lib.sepattn_mask_carve(ctypes.byref(self.c), B, L, a, n, ctypes.c_void_p(self.buffer.data_ptr()),
                                     nbytes))
        self.B, self.L, self.a, self.n = B, L, a, n

    def ref(self):
        """The struct for a call that runs on the device."""
        if not self.buffer.is_cuda:
            raise ValueError(f"mask metadata must be in device memory, not on {self.buffer.device}")
        return ctypes.byref(self.c)

    def _view(self, field: str, dtype, shape):
        off = getattr(self.c, field) - self.buffer.data_ptr()
        count = math.prod(shape)
        nbytes = count * torch.empty((), dtype=dtype).element_size()
        return self.buffer[off:off + nbytes].view(dtype).view(shape)

    @property
    def is_sep(self): return self._view("is_sep", torch.uint8, (self.B, self.L))
    @property
    def sep_idx(self): return self._view("sep_idx", torch.int32, (self.B, self.L))
    @property
    def sep_before(self): return self._view("sep_before", torch.int32, (self.B, self.L + 1))
    @property
    def sep_cnt(self): return self._view("sep_cnt", torch.int32, (self.B,))
    @property
    def plain_idx(self): return self._view("plain_idx", torch.int32, (self.B, self.L))
    @property
    def plain_cnt(self): return self._view("plain_cnt", torch.int32, (self.B,))
    @property
    def kept(self): return self._view("kept", torch.int64, (self.B,))


def build_mask(tok: torch.Tensor, sep_ids, a: int, n: int, out: Mask | None = None) -> Mask:
    """sepattn_build_mask: tok int32 [B, L] on the device.  With `out` (a
    Mask of the same B, L, a, n) the metadata is rebuilt in its buffer, so a
    loop that rebuilds masks allocates nothing."""
    if tok.dtype != torch.int32 or tok.dim() != 2 or not tok.is_contiguous():
        raise ValueError("tok must be a contiguous int32 [B, L] tensor")
    B, L = tok.shape
    if out is not None:
        if (out.B, out.L, out.a, out.n) != (B, L, a, n):
            raise ValueError(f"out mask is B={out.B} L={out.L} a={out.a} n={out.n}, need {B} {L} {a} {n}")
        m = out
    else:
        m = Mask(B, L, a, n, tok.device)
    ids = (ctypes.c_int32 * len(sep_ids))(*[int(x) for x in sep_ids])
    check(_lib.load().sepattn_build_mask(_ptr(tok), ids, len(sep_ids), m.ref(), _stream()))
    return m


def build_mask_fixed(B: int, L: int, delta: int, a: int, n: int, device="cuda") -> Mask:
    """sepattn_build_mask_fixed: fixed-interval anchors, token j kept outside
    the window iff (j + 1) % delta == 0."""
    m = Mask(B, L, a, n, device)
    check(_lib.load().sepattn_build_mask_fixed(int(delta), m.ref(), _stream()))
    return m


def mask_bits(m: Mask) -> torch.Tensor:
    """sepattn_mask_bits: the dense mask as uint32 words [B, L, ceil(L/32)]
    (int32 storage holding the same bits)."""
    words = (m.L + 31) // 32
    bits = torch.empty((m.B, m.L, words), dtype=torch.int32, device=m.buffer.device)
    check(_lib.load().sepattn_mask_bits(m.ref(), _ptr(bits), _stream()))
    return bits


def fwd_tile_rows(n: int) -> int:
    """sepattn_fwd_tile_rows: query rows per tile of the forward (and dQ)."""
    return int(_lib.load().sepattn_fwd_tile_rows(int(n)))


def tile_desc(m: Mask, tile_rows: int) -> torch.Tensor:
    """sepattn_tile_desc: int32 [B, ceil(L / tile_rows), 4] of (sink_vis,
    sep_vis, band_lo, band_hi) per query tile."""
    n_tiles = (m.L + tile_rows - 1) // tile_rows
    desc = torch.empty((m.B, n_tiles, 4), dtype=torch.int32, device=m.buffer.device)
    check(_lib.load().sepattn_tile_desc(m.ref(), int(tile_rows), _ptr(desc), _stream()))
    return desc


def _shape(q, k, v, o) -> SepattnShape:
    for t in (q, k, v, o):
        if t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError("attention tensors must be 4-d [B, H, L, d] with a contiguous last dimension")
    s = SepattnShape()
    s.B, s.Hq, s.L, s.d = q.shape
    s.Hkv = k.shape[1]
    if k.shape != (s.B, s.Hkv, s.L, s.d) or v.shape != k.shape or o.shape != q.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)} o{tuple(o.shape)}")
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", o)):
        arr = getattr(s, name)
        for i in range(3):
            arr[i] = t.stride(i)
    return s


def sepattn_fwd(q, k, v, m: Mask, scale: float | None = None, out: torch.Tensor | None = None,
                lse: torch.Tensor | None = None, want_lse: bool = True):
    """sepattn_fwd: returns (O, LSE) with O like q and LSE fp32 [B, Hq, L]."""
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype bf16 or fp32")
    if out is not None and out.dtype != q.dtype:
        raise ValueError("out must have q's dtype")
    o = torch.empty_like(q) if out is None else out
    B, Hq, L, d = q.shape
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    if want_lse:
        _check_lse(lse, B, Hq, L)
    s = _shape(q, k, v, o)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    check(_lib.load().sepattn_fwd(ctypes.byref(s), _DT[q.dtype], m.ref(), _ptr(q), _ptr(k), _ptr(v),
                                  sc, _ptr(o), _ptr(lse if want_lse else None), _stream()))
    return o, lse


def _rows_apart(t: torch.Tensor) -> bool:
    """No two rows of a [B, H, L, d] tensor (last dimension contiguous) share
    memory: the layout the ABI requires of an output."""
    span = t.shape[-1]
    for size, stride in sorted(((t.shape[i], t.stride(i)) for i in range(3) if t.shape[i] > 1),
                               key=lambda x: x[1]):
        if stride < span:
            return False
        span += (size - 1) * stride
    return True


def bwd_workspace_bytes(q, k, v, o) -> int:
    """sepattn_bwd_workspace_size for these tensors."""
    return int(_lib.load().sepattn_bwd_workspace_size(ctypes.byref(_shape(q, k, v, o))))


def _grad_outputs(grads, q, k, v):
    """dq, dk, dv laid out like q, k, v: the caller's tensors (checked) or new ones."""
    outs = []
    for g, t in zip(grads, (q, k, v)):
        if g is None:
            g = torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device)
        elif g.shape != t.shape or g.stride() != t.stride() or g.dtype != t.dtype:
            raise ValueError("gradient outputs must match q, k and v in shape, strides and dtype")
        outs.append(g)
    return outs


def sepattn_bwd(q, k, v, o, lse, dout, m: Mask, scale: float | None = None, workspace=None,
                dq=None, dk=None, dv=None):
    """sepattn_bwd: returns (dQ, dK, dV), laid out like q, k and v (a q, k or
    v whose rows overlap, e.g. an expanded view, is copied to a contiguous
    tensor first, since the gradients take its strides).  Outputs and a
    workspace given by the caller are used in place (a loop that passes them
    allocates nothing)."""
    q, k, v = (t if _rows_apart(t) else t.contiguous() for t in (q, k, v))
    if dout.shape != o.shape or dout.stride() != o.stride():
        raise ValueError("dout must have o's shape and strides")
    if o.dtype != q.dtype or dout.dtype != q.dtype:
        raise ValueError("o and dout must have q's dtype")
    s = _shape(q, k, v, o)
    _check_lse(lse, s.B, s.Hq, s.L)
    lib = _lib.load()
    need = lib.sepattn_bwd_workspace_size(ctypes.byref(s))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq, dk, dv = _grad_outputs((dq, dk, dv), q, k, v)
    sc = 1.0 / math.sqrt(q.shape[-1]) if scale is None else float(scale)
    check(lib.sepattn_bwd(ctypes.byref(s), _DT[q.dtype], m.ref(), _ptr(q), _ptr(k), _ptr(v),
                          _ptr(o), _ptr(lse), _ptr(dout), sc, _ptr(dq), _ptr(dk), _ptr(dv),
                          _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))
    return dq, dk, dv


def sepattn_bwd_noalloc(q, k, v, o, lse, dout, m: Mask, scale: float | None = None, dq=None, dk=None, dv=None):
    """sepattn_bwd_noalloc: sepattn_bwd with the library's static workspace
    (B * Hq * L <= BWD_NOALLOC_MAX_ROWS).  Outputs given by the caller are
    written in place (the call then allocates nothing); missing ones are
    allocated here like q, k and v."""
    if dout.shape != o.shape or dout.stride() != o.stride():
        raise ValueError("dout must have o's shape and strides")
    if o.dtype != q.dtype or dout.dtype != q.dtype:
        raise ValueError("o and dout must have q's dtype")
    s = _shape(q, k, v, o)
    _check_lse(lse, s.B, s.Hq, s.L)
    outs = _grad_outputs((dq, dk, dv), q, k, v)
    sc = 1.0 / math.sqrt(q.shape[-1]) if scale is None else float(scale)
    check(_lib.load().sepattn_bwd_noalloc(ctypes.byref(s), _DT[q.dtype], m.ref(), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(o), _ptr(lse), _ptr(dout), sc, _ptr(outs[0]), _ptr(outs[1]),
                                          _ptr(outs[2]), _stream()))
    return tuple(outs)


class SepCache:
    """A SepCache for B streams (bf16 K/V); cap is the capacity c (0 or
    a + s + n: no past window)."""

    def __init__(self, B: int, Hkv: int, d: int, a: int, s: int, n: int, theta: float = 500000.0,
                 cap: int = 0, device="cuda"):
        if torch.device(device).type != "cuda":
            raise ValueError("a SepCache lives in device memory")
        lib = _lib.load()
        slots = lib.sepcache_slots(a, s, n, cap)
        if slots < 0:
            raise ValueError(f"bad cache sizes a={a} s={s} n={n} c={cap}")
        self.B, self.Hkv, self.d, self.a, self.s, self.n, self.slots = B, Hkv, d, a, s, n, slots
        self.cap = slots - 1
        # K in the library's tiled layout: sepcache_k_rows(slots) rows per
        # (stream, KV head), 16-row tiles stored chunk-major (sepattn.h)
        self.k = torch.zeros((B, Hkv, lib.sepcache_k_rows(slots), d), dtype=torch.bfloat16, device=device)
        self.v = torch.zeros((B, Hkv, slots, d), dtype=torch.bfloat16, device=device)
        self.slot_pos = torch.empty((B, Hkv, slots), dtype=torch.int32, device=device)
        self.slot_sep = torch.empty((B, Hkv, slots), dtype=torch.uint8, device=device)
        self.state = torch.empty((B, Hkv, 8), dtype=torch.int32, device=device)
        c = SepCacheStruct()
        c.B, c.Hkv, c.d, c.a, c.s, c.n = B, Hkv, d, a, s, n
        c.k, c.v = self.k.data_ptr(), self.v.data_ptr()
        c.slot_pos, c.slot_sep, c.state = (self.slot_pos.data_ptr(), self.slot_sep.data_ptr(),
                                           self.state.data_ptr())
        c.theta = float(theta)
        c.c = int(cap)
        self.c = c
        self._ws = None
        self.reset()

    def reset(self):
        check(_lib.load().sepcache_reset(ctypes.byref(self.c), _stream()))

    def _kvf(self, k_new, v_new, is_sep):
        for t in (k_new, v_new):
            if t.dtype != torch.bfloat16 or t.shape != (self.B, self.Hkv, self.d) or not t.is_contiguous():
                raise ValueError("k_new/v_new must be contiguous bf16 [B, Hkv, d]")
        if is_sep.dtype != torch.uint8 or is_sep.shape != (self.B,):
            raise ValueError("is_sep must be uint8 [B]")

    def append(self, k_new, v_new, is_sep):
        self._kvf(k_new, v_new, is_sep)
        check(_lib.load().sepcache_append(ctypes.byref(self.c), _ptr(k_new), _ptr(v_new), _ptr(is_sep), _stream()))

    def evict(self):
        check(_lib.load().sepcache_evict(ctypes.byref(self.c), _stream()))

    def push(self, k_new, v_new, is_sep):
        self._kvf(k_new, v_new, is_sep)
        check(_lib.load().sepcache_push(ctypes.byref(self.c), _ptr(k_new), _ptr(v_new), _ptr(is_sep), _stream()))

    def workspace(self, Hq: int) -> torch.Tensor:
        need = _lib.load().sepcache_decode_workspace_size(ctypes.byref(self.c), Hq)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=self.k.device)
        return self._ws

    def decode(self, q, scale: float | None = None, shift: bool = True, out=None):
        """sepcache_decode: q bf16 [B, Hq, d] -> o bf16 [B, Hq, d]."""
        o = self._q_out(q, out)
        ws = self.workspace(q.shape[1])
        sc = 1.0 / math.sqrt(self.d) if scale is None else float(scale)
        check(_lib.load().sepcache_decode(ctypes.byref(self.c), q.shape[1], _ptr(q), sc, 1 if shift else 0,
                                          _ptr(o), _ptr(ws), ws.numel(), _stream()))
        return o

    def step(self, k_new, v_new, is_sep, q, scale: float | None = None, shift: bool = True, out=None):
        """sepcache_step: append + evict + decode."""
        self._kvf(k_new, v_new, is_sep)
        o = self._q_out(q, out)
        ws = self.workspace(q.shape[1])
        sc = 1.0 / math.sqrt(self.d) if scale is None else float(scale)
        check(_lib.load().sepcache_step(ctypes.byref(self.c), _ptr(k_new), _ptr(v_new), _ptr(is_sep), q.shape[1],
                                        _ptr(q), sc, 1 if shift else 0, _ptr(o), _ptr(ws), ws.numel(),
                                        _stream()))
        return o

    def _q_out(self, q, out):
        if q.dtype != torch.bfloat16 or q.dim() != 3 or q.shape[0] != self.B or q.shape[2] != self.d \
                or not q.is_contiguous():
            raise ValueError("q must be contiguous bf16 [B, Hq, d]")
        if out is not None and (out.dtype != q.dtype or out.shape != q.shape or not out.is_contiguous()):
            raise ValueError("out must be a contiguous tensor like q")
        return torch.empty_like(q) if out is None else out

    def prefill(self, k, v, m: Mask):
        """sepcache_prefill: seed every stream with a prompt of m.L tokens
        (k, v bf16 [B, Hkv, L, d], keys before RoPE; m its mask metadata)."""
        for t in (k, v):
            if (t.dtype != torch.bfloat16 or t.dim() != 4 or t.shape[0] != self.B or t.shape[1] != self.Hkv
                    or t.shape[2] != m.L or t.shape[3] != self.d or t.stride(-1) != 1):
                raise ValueError("k/v must be bf16 [B, Hkv, L, d] with a contiguous last dimension")
        ks = (ctypes.c_int64 * 3)(*k.stride()[:3])
        vs = (ctypes.c_int64 * 3)(*v.stride()[:3])
        check(_lib.load().sepcache_prefill(ctypes.byref(self.c), _ptr(k), _ptr(v), ks, vs, m.ref(),
                                           _stream()))

    def export_order(self):
        """sepcache_export_order: (pos int32 [B, slots - 1], len int32 [B])."""
        pos = torch.empty((self.B, self.cap), dtype=torch.int32, device=self.k.device)
        ln = torch.empty((self.B,), dtype=torch.int32, device=self.k.device)
        check(_lib.load().sepcache_export_order(ctypes.byref(self.c), _ptr(pos), _ptr(ln), _stream()))
        return pos, ln
