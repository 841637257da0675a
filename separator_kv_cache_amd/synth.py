"""Seeded synthetic inputs for the separator-mask attention path.

This module draws random numbers and nothing else: token streams with a
chosen separator rate, Gaussian Q/K/V/dO tensors, and per-step decode inputs.
It holds none of the method's arithmetic (no flags, masks, softmax or cache
logic), so both the fp64 oracle and the HIP path can take their inputs from
here without sharing any computation.

Every draw comes from ``numpy.random.default_rng(SeedSequence(seed,
spawn_key=(workload_id, tensor_id)))`` so each tensor of each workload has its
own reproducible stream.

Token streams stand in for tokenised text (the pages evaluate on Pile, PG19,
GSM8K; none of that data is used or reproduced).  The nine separator ids are
arbitrary fixed ids in a 50k vocabulary: the mask depends only on whether a
token is in the separator set, and the pages name the separators as
characters (". , ? ! ; :" space, tab, newline), not as tokenizer ids.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

VOCAB = 50_000
# Nine distinct, deliberately non-contiguous ids: one per separator character
# ('.', ',', '?', '!', ';', ':', ' ', '\t', '\n').
SEP_IDS = (7, 1013, 4099, 12007, 20011, 27077, 33331, 41017, 49999)

# tensor ids used in spawn keys
T_TOK, T_Q, T_K, T_V, T_DO, T_DEC_Q, T_DEC_K, T_DEC_V, T_DEC_F = range(9)


def _rng(seed: int, wid: int, tid: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(wid, tid)))


def _non_separator_ids() -> np.ndarray:
    allowed = np.ones(VOCAB, dtype=bool)
    allowed[list(SEP_IDS)] = False
    return np.nonzero(allowed)[0].astype(np.int32)


def tokens_iid(seed: int, wid: int, B: int, L: int, p: float) -> np.ndarray:
    """Token ids int32 [B, L]: each position is a separator with probability p
    (id uniform over the nine separator ids), otherwise uniform over the rest
    of the vocabulary, so the separator indicator is exactly Bernoulli(p)."""
    rng = _rng(seed, wid, T_TOK)
    is_sep = rng.random((B, L)) < p
    sep_pick = rng.integers(0, len(SEP_IDS), size=(B, L))
    other = _non_separator_ids()
    oth_pick = rng.integers(0, len(other), size=(B, L))
    tok = np.where(is_sep, np.asarray(SEP_IDS, dtype=np.int32)[sep_pick], other[oth_pick])
    return tok.astype(np.int32)


def tokens_clustered(seed: int, wid: int, B: int, L: int, p: float,
                     mean_segment: float = 8.0) -> np.ndarray:
    """Token ids int32 [B, L] with separators in runs, mimicking sentence
    structure: alternating non-separator segments (geometric lengths, support
    >= 1, mean ``mean_segment``) and separator runs (geometric, support >= 1,
    mean ``mean_segment * p / (1 - p)``), so the long-run separator rate is p.
    The first segment's kind is drawn with probability p of being a run."""
    rng = _rng(seed, wid, T_TOK)
    other = _non_separator_ids()
    sep_arr = np.asarray(SEP_IDS, dtype=np.int32)
    mean_run = mean_segment * p / (1.0 - p)
    out = np.empty((B, L), dtype=np.int32)
    for b in range(B):
        is_sep = np.empty(L, dtype=bool)
        pos = 0
        in_run = bool(rng.random() < p)
        while pos < L:
            mean = mean_run if in_run else mean_segment
            length = int(rng.geometric(1.0 / mean))
            is_sep[pos:pos + length] = in_run
            pos += length
            in_run = not in_run
        sep_pick = rng.integers(0, len(sep_arr), size=L)
        oth_pick = rng.integers(0, len(other), size=L)
        out[b] = np.where(is_sep, sep_arr[sep_pick], other[oth_pick])
    return out


def gaussian(seed: int, wid: int, tid: int, shape, scale: float = 1.0) -> np.ndarray:
    """float32 N(0, 1) * scale.  Rounding to bf16 is the caller's cast."""
    rng = _rng(seed, wid, tid)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def bernoulli(seed: int, wid: int, tid: int, shape, p: float) -> np.ndarray:
    rng = _rng(seed, wid, tid)
    return (rng.random(shape) < p).astype(np.uint8)


# --------------------------------------------------------------------------
# Workloads.  Shapes follow the pages' models (Pythia-160M: 12 heads of 64;
# Llama-3-8B: 32 query heads, 8 KV heads of 128) at the sizes stated for
# each workload.
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    wid: int
    B: int
    Hq: int
    Hkv: int
    L: int
    d: int
    a: int
    n: int
    p: float
    dtype: str              # "f32" or "bf16"
    qkv_scale: float = 1.0
    clustered: bool = False
    backward: bool = False

    def tokens(self, seed: int = 0) -> np.ndarray:
        if self.clustered:
            return tokens_clustered(seed, self.wid, self.B, self.L, self.p)
        return tokens_iid(seed, self.wid, self.B, self.L, self.p)

    def qkv(self, seed: int = 0):
        """fp32 arrays q [B,Hq,L,d], k/v [B,Hkv,L,d] (not yet rounded)."""
        q = gaussian(seed, self.wid, T_Q, (self.B, self.Hq, self.L, self.d), self.qkv_scale)
        k = gaussian(seed, self.wid, T_K, (self.B, self.Hkv, self.L, self.d), self.qkv_scale)
        v = gaussian(seed, self.wid, T_V, (self.B, self.Hkv, self.L, self.d), self.qkv_scale)
        return q, k, v

    def dout(self, seed: int = 0) -> np.ndarray:
        return gaussian(seed, self.wid, T_DO, (self.B, self.Hq, self.L, self.d), 1.0)

    def with_(self, **kw) -> "PrefillWorkload":
        d = dict(self.__dict__)
        d.update(kw)
        return PrefillWorkload(**d)


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    wid: int
    B: int
    Hq: int
    Hkv: int
    d: int
    a: int
    s: int
    n: int
    T: int
    p: float
    theta: float = 500000.0
    shift: bool = True

    @property
    def slots(self) -> int:
        return self.a + self.s + self.n

    def flags(self, seed: int = 0) -> np.ndarray:
        """Separator indicator per (step, stream): uint8 [T, B], i.i.d. Bernoulli(p)."""
        return bernoulli(seed, self.wid, T_DEC_F, (self.T, self.B), self.p)

    def _step(self, seed: int, tid: int, t: int, shape) -> np.ndarray:
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(self.wid, tid, t)))
        return rng.standard_normal(size=shape, dtype=np.float32)

    def q_steps(self, steps, seed: int = 0) -> np.ndarray:
        """fp32 queries N(0,1) of the given steps: [len(steps), B, Hq, d].
        Each step has its own stream, so any subset is reproducible."""
        return np.stack([self._step(seed, T_DEC_Q, int(t), (self.B, self.Hq, self.d)) for t in steps])

    def kv_steps(self, t0: int, t1: int, seed: int = 0):
        """fp32 new keys and values N(0,1) of steps [t0, t1): [t1-t0, B, Hkv, d] each."""
        k = np.stack([self._step(seed, T_DEC_K, t, (self.B, self.Hkv, self.d)) for t in range(t0, t1)])
        v = np.stack([self._step(seed, T_DEC_V, t, (self.B, self.Hkv, self.d)) for t in range(t0, t1)])
        return k, v

    def with_(self, **kw) -> "DecodeWorkload":
        d = dict(self.__dict__)
        d.update(kw)
        return DecodeWorkload(**d)


# Sep-mask forward, fp32, tiny: the correctness workload.
TINY_F32 = PrefillWorkload("sep-fwd-f32-L256", 1, B=1, Hq=2, Hkv=2, L=256, d=64,
                           a=4, n=32, p=0.15, dtype="f32")
# Pythia-160M-shaped forward, bf16 (n=128); run 2 uses n=64 plus a full layer.
PYTHIA_FWD = PrefillWorkload("pythia160m-fwd-n128", 2, B=8, Hq=12, Hkv=12, L=2048, d=64,
                             a=4, n=128, p=0.15, dtype="bf16", qkv_scale=0.5)
PYTHIA_FWD_N64 = PYTHIA_FWD.with_(name="pythia160m-fwd-n64", n=64)
PYTHIA_FWD_FULL = PYTHIA_FWD.with_(name="pythia160m-fwd-full", n=2048)
# Pythia-160M-shaped forward + backward, four (n, p) runs.
PYTHIA_BWD = [PYTHIA_FWD.with_(name=f"pythia160m-bwd-n{n}-p{int(p*100):02d}", wid=3,
                               n=n, p=p, backward=True)
              for n in (64, 128) for p in (0.10, 0.20)]
# Llama-3-8B-shaped SepCache decode.
LLAMA_DECODE = DecodeWorkload("llama3-8b-sepcache-decode", 4, B=16, Hq=32, Hkv=8, d=128,
                              a=4, s=64, n=256, T=8192, p=0.12)
# Llama-3-8B-shaped long prefill, clustered separators, fwd + bwd.
LLAMA_PREFILL = PrefillWorkload("llama3-8b-prefill-L32768", 5, B=1, Hq=32, Hkv=8, L=32768,
                                d=128, a=4, n=4096, p=0.12, dtype="bf16", qkv_scale=0.5,
                                clustered=True, backward=True)
