"""Helpers shared by the GPU parity tests."""
from __future__ import annotations

import sys

import numpy as np
import torch

from separator_kv_cache_amd import synth

# Tolerances (max-abs against the fp64 oracle).  fp32: 1e-4 on outputs.  bf16
# inputs with fp32 accumulation: 2e-2 on outputs and gradients (P is rounded
# to bf16 before the PV product, about 2^-9 relative per probability).
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
TOL_LSE_BF16 = 2e-3


def edge_excess(got, ref) -> float:
    """For bf16 results on inputs outside the stated workloads, where single
    elements can grow large (e.g. sinks absorbing all attention mass): the
    largest amount by which |got - ref| exceeds its own element's bound
    2e-2 + 2^-8 |ref_ij| (<= 0 when every element is within it).  The
    per-element term covers rounding that element to bf16 (2^-9 relative)
    and the bf16 rounding of P and dS in its fp32-accumulated products
    (2^-9 relative per term); small elements keep the flat 2e-2."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not ref.size:
        return -1.0
    bound = TOL_BF16 + 2.0 ** -8 * np.abs(ref)
    return float(np.max(np.abs(got - ref) - bound))


def say(*a):
    """Names the case before each GPU step (flushed, so it survives a crash)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def round_bf16(x: np.ndarray) -> torch.Tensor:
    """fp32 numpy -> bf16 CPU tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def inputs(wl: synth.PrefillWorkload, seed: int = 0, device="cuda"):
    """(tok, q, k, v) on the device in the workload's dtype, plus the same
    values as fp64 numpy arrays for the oracle."""
    tok = wl.tokens(seed)
    q, k, v = wl.qkv(seed)
    if wl.dtype == "bf16":
        tq, tk, tv = round_bf16(q), round_bf16(k), round_bf16(v)
    else:
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    host = (as_f64(tq), as_f64(tk), as_f64(tv))
    dev = tuple(t.to(device) for t in (tq, tk, tv))
    return torch.from_numpy(tok).to(device), dev, host, tok


def max_abs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def cache_k_rows(k, slots):
    """The keys of a SepCache K buffer as rows [B, Hkv, slots, d], from the
    tiled layout the C header documents (sepcache_k_rows): 16-byte chunk ch of
    slot r at chunk index ((r / 16) * (d / 8) + ch) * 16 + r % 16."""
    B, H, R, d = k.shape
    t = k.reshape(B, H, R // 16, d // 8, 16, 8)  # [tile, chunk, row in tile, 8]
    return t.permute(0, 1, 2, 4, 3, 5).reshape(B, H, R, d)[:, :, :slots]
