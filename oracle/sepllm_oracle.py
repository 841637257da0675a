"""Plain, slow fp64 CPU oracle for SepLLM separator-mask attention and SepCache.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it, and it imports nothing from the GPU path (the two share only the
seeded input generators, which hold no arithmetic of the method).

Sources (the pages about SepLLM, arXiv 2412.12094):
  [ANTH]  anthology-of-the-sota record LIT-748, "Key takeaways": the mask
          bullet (initial tokens, preceding separators, n nearest tokens, same
          in every head; the nine separators) and the streaming bullet.
  [PITH]  pith.science verdict for 2412.12094, pith_extraction.key_machinery:
          the binary mask M over (i) the first a tokens, (ii) separators seen so
          far, (iii) the n nearest preceding tokens; the streaming cache of
          initial / separator / local-window / past-window blocks under a
          capacity, where leaving tokens are dropped unless they are
          separators, which move into the separator cache.
  [HUB]   paperhub.cn author responses, second reviewer, answer A1: RoPE with
          positions taken inside the cache (the worked example: a cache
          holding tokens 0,1,2,3,6,7,8 while decoding token 9 uses positions
          0..7); plain RoPE without shifting for training-length inputs.
          Same page, second reviewer A2: without separators SepLLM becomes
          StreamingLLM.

Readings where the pages leave a step open (each is listed with its reason in
the design notes of the repository):
  * the n-token window includes the query itself: j in (i-n, i];
  * separators listed in sep_idx are positions j >= a (a sink is a sink);
  * softmax scale 1/sqrt(d); GQA q head h reads KV head h // (Hq/Hkv);
  * RoPE pairs dimension i with i + d/2, frequency theta^(-2i/d);
  * per decode step: append the token, evict from the window if it holds
    more than n entries (separator -> separator FIFO of capacity s, whose
    oldest entry is dropped on overflow; other tokens are dropped), attend;
  * with a capacity c > a + s + n, the past-window block holds the
    c - a - s - n = P tokens that left the local window most recently; the
    window and the past window form one queue of at most n + P tokens, and
    once it is full, the next token first makes its oldest P + 1 leave (the
    separators among them join the separator FIFO in order, the others are
    dropped), so the queue keeps n tokens with the new one;
  * in-cache positions are ranks in the order sinks, separators, past
    window, window.

Everything is float64 (integers are exact).  Rows of the attention are
computed in groups only to vectorise: every column left out of a group is one
the mask definition rejects for every row of that group, and the mask is
evaluated from its definition on every column that is kept.
"""
from __future__ import annotations

from collections import deque

import numpy as np

# --------------------------------------------------------------------------
# Mask side
# --------------------------------------------------------------------------


def separator_flags(tok: np.ndarray, sep_ids) -> np.ndarray:
    """f[b, j] = 1 iff token j is one of the separator ids.  [ANTH] mask bullet."""
    return np.isin(np.asarray(tok), np.asarray(list(sep_ids))).astype(np.uint8)


def fixed_flags(B: int, L: int, delta: int) -> np.ndarray:
    """FixLLM anchors, [HUB] third reviewer A2: every delta-th token is kept
    outside the neighbouring window, in place of the separators.  Read as the
    delta-th, 2*delta-th, ... token counting from one: f[b, j] = 1 iff delta
    divides j + 1, for every sequence."""
    if delta < 1:
        raise ValueError("delta >= 1")
    j = np.arange(L)
    return np.ascontiguousarray(np.broadcast_to(((j + 1) % delta == 0).astype(np.uint8), (B, L)))


def mask_rows(f_b: np.ndarray, a: int, n: int, r0: int, r1: int, c1: int | None = None) -> np.ndarray:
    """Rows [r0, r1) of the SepLLM mask of one sequence, columns [0, c1).

    M[i, j] = (j <= i) and (j < a  or  i - j < n  or  f[j] = 1)
    ([ANTH] mask bullet; [PITH] key_machinery (i)-(iii)).
    """
    L = f_b.shape[0]
    c1 = L if c1 is None else c1
    i = np.arange(r0, r1)[:, None]
    j = np.arange(c1)[None, :]
    sep = f_b[:c1].astype(bool)[None, :]
    return (j <= i) & ((j < a) | (i - j < n) | sep)


def mask_dense(f: np.ndarray, a: int, n: int) -> np.ndarray:
    """The full mask M [B, L, L] (bool); for small L only."""
    B, L = f.shape
    return np.stack([mask_rows(f[b], a, n, 0, L) for b in range(B)])


def separator_index(f: np.ndarray, a: int):
    """Ascending positions j >= a with f[j] = 1, per sequence.

    Returns (sep_idx int32 [B, L] with the unused tail set to L, sep_cnt int32
    [B]).  Sinks are never listed, even when their token is a separator.
    """
    B, L = f.shape
    idx = np.full((B, L), L, dtype=np.int32)
    cnt = np.zeros(B, dtype=np.int32)
    for b in range(B):
        pos = [j for j in range(a, L) if f[b, j]]
        idx[b, :len(pos)] = pos
        cnt[b] = len(pos)
    return idx, cnt


def separator_prefix(f: np.ndarray, a: int) -> np.ndarray:
    """sep_before[b, j] = number of separators at positions k >= a with k < j,
    for j in [0, L] (an exclusive prefix count; int32 [B, L+1])."""
    B, L = f.shape
    out = np.zeros((B, L + 1), dtype=np.int32)
    for b in range(B):
        run = 0
        for j in range(L):
            out[b, j] = run
            if j >= a and f[b, j]:
                run += 1
        out[b, L] = run
    return out


def tile_descriptors(f: np.ndarray, a: int, n: int, rows: int) -> np.ndarray:
    """Per query tile of ``rows`` rows, [q0, q1), read off the mask M itself:
    band_lo = max(0, q0 - n + 1) is the first key any row of the tile keeps
    through its window and band_hi = q1; left of band_lo the tile keeps
    exactly the keys every one of its rows keeps (checked here), counted as
    sinks (j < a) and separators (j >= a).  Returns int32 [B, n_tiles, 4] of
    (sink_vis, sep_vis, band_lo, band_hi).  [ANTH] mask bullet."""
    B, L = f.shape
    n_tiles = (L + rows - 1) // rows
    out = np.zeros((B, n_tiles, 4), dtype=np.int32)
    for b in range(B):
        for t in range(n_tiles):
            q0, q1 = t * rows, min(L, (t + 1) * rows)
            lo = max(0, q0 - n + 1)
            m = mask_rows(f[b], a, n, q0, q1, lo)  # rows of the tile, keys left of the band
            seen = m.any(axis=0)
            if not np.array_equal(seen, m.all(axis=0)):
                raise AssertionError("a key left of the band is kept by some rows of the tile only")
            out[b, t] = (int(seen[:a].sum()), int(seen[a:].sum()), lo, q1)
    return out


def kept_pairs(f: np.ndarray, a: int, n: int, block: int = 512) -> np.ndarray:
    """Number of kept (query, key) pairs per sequence: the popcount of M.
    int64 [B].  Rows are counted in groups of ``block``."""
    B, L = f.shape
    out = np.zeros(B, dtype=np.int64)
    for b in range(B):
        tot = 0
        for r0 in range(0, L, block):
            r1 = min(L, r0 + block)
            tot += int(mask_rows(f[b], a, n, r0, r1, r1).sum())
        out[b] = tot
    return out


# --------------------------------------------------------------------------
# Attention under M (prefill / training)
# --------------------------------------------------------------------------


def _row_groups(L: int, block: int):
    for r0 in range(0, L, block):
        yield r0, min(L, r0 + block)


def attn_fwd(q, k, v, f, a: int, n: int, scale: float, block: int = 256):
    """O = softmax(scale * Q K^T, masked by M) V and LSE = log-sum-exp (natural
    log) of each row's kept scores.  q [B,Hq,L,d], k/v [B,Hkv,L,d]; returns
    O float64 [B,Hq,L,d] and LSE float64 [B,Hq,L].  [ANTH] mask bullet."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    o = np.zeros((B, Hq, L, d))
    lse = np.zeros((B, Hq, L))
    for b in range(B):
        for r0, r1 in _row_groups(L, block):
            m = mask_rows(f[b], a, n, r0, r1, r1)
            cols = np.nonzero(m.any(axis=0))[0]
            mc = m[:, cols]
            for h in range(Hq):
                kh = h // g
                s = scale * (q[b, h, r0:r1] @ k[b, kh, cols].T)
                s = np.where(mc, s, -np.inf)
                mx = s.max(axis=1, keepdims=True)
                p = np.exp(s - mx)
                l = p.sum(axis=1, keepdims=True)
                o[b, h, r0:r1] = (p / l) @ v[b, kh, cols]
                lse[b, h, r0:r1] = (mx + np.log(l))[:, 0]
    return o, lse


def attn_fwd_rows(q, k, v, f, a: int, n: int, scale: float, b: int, h: int, rows):
    """O and LSE for selected rows of one (sequence, q head), each row computed
    alone from its kept keys (for spot checks at large L)."""
    Hq, Hkv = q.shape[1], k.shape[1]
    kh = h // (Hq // Hkv)
    rows = np.asarray(rows)
    d = q.shape[-1]
    o = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    for t, i in enumerate(rows):
        m = mask_rows(f[b], a, n, int(i), int(i) + 1, int(i) + 1)[0]
        cols = np.nonzero(m)[0]
        s = scale * (k[b, kh, cols].astype(np.float64) @ q[b, h, i].astype(np.float64))
        mx = s.max()
        p = np.exp(s - mx)
        l = p.sum()
        o[t] = (p / l) @ v[b, kh, cols].astype(np.float64)
        lse[t] = mx + np.log(l)
    return o, lse


def attn_bwd(q, k, v, do, f, a: int, n: int, scale: float, block: int = 256, heads=None):
    """Gradients of the masked attention for upstream dO.

    P = softmax(scale*QK^T masked by M);  O = P V;  D_i = sum_d dO_i O_i;
    dV = P^T dO;  dP = dO V^T;  dS = P * (dP - D);  dQ = scale dS K;
    dK = scale dS^T Q.  dK and dV of a KV head sum over the q heads that read
    it.  ``heads`` restricts the work to a list of KV heads (the other
    outputs stay zero).  Returns dq, dk, dv (float64).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    kv_heads = range(Hkv) if heads is None else heads
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for r0, r1 in _row_groups(L, block):
            m = mask_rows(f[b], a, n, r0, r1, r1)
            cols = np.nonzero(m.any(axis=0))[0]
            mc = m[:, cols]
            for kh in kv_heads:
                kc = k[b, kh, cols]
                vc = v[b, kh, cols]
                for h in range(kh * g, (kh + 1) * g):
                    s = scale * (q[b, h, r0:r1] @ kc.T)
                    s = np.where(mc, s, -np.inf)
                    mx = s.max(axis=1, keepdims=True)
                    p = np.exp(s - mx)
                    p /= p.sum(axis=1, keepdims=True)
                    o = p @ vc
                    dob = do[b, h, r0:r1]
                    D = (dob * o).sum(axis=1, keepdims=True)
                    dp = dob @ vc.T
                    ds = p * (dp - D)
                    dq[b, h, r0:r1] = scale * (ds @ kc)
                    dk[b, kh, cols] += scale * (ds.T @ q[b, h, r0:r1])
                    dv[b, kh, cols] += p.T @ dob
    return dq, dk, dv


def attn_bwd_rows(q, k, v, do, f, a: int, n: int, scale: float, b: int, h: int, rows):
    """dQ for selected rows of one (sequence, q head), each row computed alone:
    P_i over the row's kept keys, O_i = P_i V, D_i = dO_i . O_i,
    dS_i = P_i (dO_i V^T - D_i), dQ_i = scale dS_i K."""
    Hq, Hkv = q.shape[1], k.shape[1]
    kh = h // (Hq // Hkv)
    rows = np.asarray(rows)
    out = np.zeros((len(rows), q.shape[-1]))
    for t, i in enumerate(rows):
        m = mask_rows(f[b], a, n, int(i), int(i) + 1, int(i) + 1)[0]
        cols = np.nonzero(m)[0]
        kc = k[b, kh, cols].astype(np.float64)
        vc = v[b, kh, cols].astype(np.float64)
        s = scale * (kc @ q[b, h, i].astype(np.float64))
        p = np.exp(s - s.max())
        p /= p.sum()
        dob = do[b, h, i].astype(np.float64)
        D = dob @ (p @ vc)
        ds = p * (vc @ dob - D)
        out[t] = scale * (ds @ kc)
    return out


# --------------------------------------------------------------------------
# RoPE and the streaming SepCache
# --------------------------------------------------------------------------


def rope(x, pos, theta: float):
    """Rotary position embedding, half-split pairing: for i < d/2 with
    w_i = theta^(-2i/d), (x_i, x_{i+d/2}) is rotated by the angle pos * w_i.
    x [..., d]; pos broadcastable to x.shape[:-1].  [HUB] A1 ("we just adopt
    RoPE")."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    w = theta ** (-2.0 * np.arange(half) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * w
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


class SepCacheSim:
    """Bookkeeping of one stream's SepCache: which original positions it holds
    and in what order.  [PITH] key_machinery (initial, separator, local-window
    and past-window blocks under a capacity c; once the cache is full, the
    past window's separators move to the separator cache and its other
    tokens are dropped, a periodic evolution), [ANTH] streaming bullet
    (fixed-size cache).  The separator block keeps its s most recent
    separators (oldest dropped first).

    c = None or a + s + n: no past window, so a token leaving the window is
    classified at once (evict()).  c > a + s + n: the window and the past
    window are one queue ``win`` of at most n + P tokens, P = c - a - s - n;
    an append to a full queue first makes its oldest P + 1 tokens leave."""

    def __init__(self, a: int, s: int, n: int, c: int | None = None):
        if n < 1 or a < 0 or s < 0:
            raise ValueError("need n >= 1, a >= 0, s >= 0")
        if c is not None and c < a + s + n:
            raise ValueError("need c >= a + s + n")
        self.a, self.s, self.n = a, s, n
        self.P = 0 if c is None else c - a - s - n
        self.t = 0
        self.sinks: list[int] = []
        self.sep: deque[int] = deque()
        self.win: deque[int] = deque()
        self.flag: dict[int, int] = {}

    def _leave(self, e: int) -> None:
        """Token e leaves the window: a separator joins the separator FIFO,
        anything else is dropped."""
        if self.flag[e]:
            self.sep.append(e)
            if len(self.sep) > self.s:
                self.sep.popleft()

    def append(self, flag: int) -> None:
        t = self.t
        self.flag[t] = int(flag)
        if t < self.a:
            self.sinks.append(t)
        else:
            if self.P > 0 and len(self.win) == self.n + self.P:
                for _ in range(self.P + 1):
                    self._leave(self.win.popleft())
            self.win.append(t)
        self.t += 1

    def evict(self) -> None:
        # without a past window: the oldest of n + 1 window tokens leaves
        if len(self.win) > self.n + self.P:
            self._leave(self.win.popleft())

    def order(self) -> list[int]:
        """Original positions held, in the cache's logical order."""
        return list(self.sinks) + list(self.sep) + list(self.win)

    def positions(self, shift: bool) -> tuple[np.ndarray, int]:
        """(key positions, query position) for the entries of ``order()``;
        the query is the newest entry.  With shift, positions are ranks inside
        the cache ([HUB] A1 worked example); without, original positions."""
        ordr = self.order()
        if shift:
            return np.arange(len(ordr)), len(ordr) - 1
        return np.asarray(ordr), self.t - 1


def decode_run(q_all, k_all, v_all, flags, a: int, s: int, n: int, theta: float,
               shift: bool, scale: float, out_steps=None, order_steps=(), c: int | None = None):
    """Streaming decode over a SepCache, one simulator per stream.

    q_all [T,B,Hq,d], k_all/v_all [T,B,Hkv,d] (keys pre-RoPE), flags [T,B].
    Each step t: append token t, evict, then attend with the rotated query
    over every cached entry (keys rotated at their positions).  Returns
    (outputs {t: o [B,Hq,d] float64} for t in out_steps (all if None),
     orders {t: [order per stream]} for t in order_steps).
    """
    T, B, Hq, d = q_all.shape
    Hkv = k_all.shape[2]
    g = Hq // Hkv
    sims = [SepCacheSim(a, s, n, c) for _ in range(B)]
    want = set(range(T)) if out_steps is None else set(out_steps)
    want_order = set(order_steps)
    outs, orders = {}, {}
    for t in range(T):
        for b in range(B):
            sims[b].append(int(flags[t, b]))
            sims[b].evict()
        if t in want_order:
            orders[t] = [sims[b].order() for b in range(B)]
        if t not in want:
            continue
        o = np.zeros((B, Hq, d))
        for b in range(B):
            ordr = np.asarray(sims[b].order())
            kpos, qpos = sims[b].positions(shift)
            for kh in range(Hkv):
                kk = rope(k_all[ordr, b, kh], kpos, theta)
                vv = np.asarray(v_all[ordr, b, kh], dtype=np.float64)
                for h in range(kh * g, (kh + 1) * g):
                    qq = rope(q_all[t, b, h], qpos, theta)
                    sc = scale * (kk @ qq)
                    mx = sc.max()
                    p = np.exp(sc - mx)
                    o[b, h] = (p / p.sum()) @ vv
        outs[t] = o
    return outs, orders
