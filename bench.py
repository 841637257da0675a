"""Benchmark of the SepLLM hot path on one MI355X.

One step = the whole path over one batch of synthetic input:
  prefill leg (Llama-3-8B shape: B=1, 32 q / 8 KV heads, d=128, L=32768,
    a=4, n=4096, clustered separators at p=0.12): mask build, forward,
    backward (dO given);
  decode leg (Llama-3-8B shape SepCache: 16 streams, 32 q / 8 KV heads,
    d=128, a=4, s=64, n=256, 8192 tokens per stream, separators p=0.12):
    every token is pushed into and decoded against the cache of each of
    `--layers` layers (32 by default, as in Llama-3-8B), so the caches'
    working set (~680 MB) exceeds the 256 MB Infinity Cache.  Each token has
    its own q/k/v (N(0,1), drawn per step from the seed and resident on the
    device before timing); tokens run as replays of a HIP graph of 64 tokens,
    whose input buffers are refilled from the resident arrays per replay.

Prints one JSON line.  `value` is the prefill leg's kept-FLOP rate (forward
4*d*kept + backward 10*d*kept per q head, kept pairs counted by the mask
kernel); the decode leg's algorithmic HBM rate is reported beside it.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from separator_kv_cache_amd import binding as sa  # noqa: E402
from separator_kv_cache_amd import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CHUNK = 64                  # tokens per decode graph


class PrefillLeg:
    def __init__(self, wl: synth.PrefillWorkload, seed: int = 0):
        self.wl = wl
        dev = "cuda"
        self.tok = torch.from_numpy(wl.tokens(seed)).to(dev)
        q, k, v = wl.qkv(seed)
        self.q, self.k, self.v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (q, k, v))
        del q, k, v
        self.do = torch.from_numpy(wl.dout(seed)).to(torch.bfloat16).to(dev)
        self.scale = 1.0 / math.sqrt(wl.d)
        self.mask = sa.build_mask(self.tok, synth.SEP_IDS, wl.a, wl.n)
        self.o, self.lse = sa.sepattn_fwd(self.q, self.k, self.v, self.mask, self.scale)
        # the backward's outputs and workspace, allocated once: no allocation in the timed region
        self.dq, self.dk, self.dv = (torch.empty_like(t) for t in (self.q, self.k, self.v))
        self.ws = torch.empty(sa.bwd_workspace_bytes(self.q, self.k, self.v, self.o), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        self.kept_per_seq = int(self.mask.kept.sum().cpu())
        self.fwd_flops = 4.0 * wl.d * self.kept_per_seq * wl.Hq
        self.bwd_flops = 10.0 * wl.d * self.kept_per_seq * wl.Hq
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def step(self):
        wl, e = self.wl, self.ev
        e[0].record()
        sa.build_mask(self.tok, synth.SEP_IDS, wl.a, wl.n, out=self.mask)  # rebuilt in place
        e[1].record()
        sa.sepattn_fwd(self.q, self.k, self.v, self.mask, self.scale, out=self.o, lse=self.lse)
        e[2].record()
        sa.sepattn_bwd(self.q, self.k, self.v, self.o, self.lse, self.do, self.mask, self.scale, workspace=self.ws,
                       dq=self.dq, dk=self.dk, dv=self.dv)
        e[3].record()

    def times_ms(self):
        e = self.ev
        return e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])


def decode_lengths(wl: synth.DecodeWorkload, flags: np.ndarray, cap: int = 0) -> np.ndarray:
    """Entries each stream's cache holds when step t attends, [T, B].  They
    follow from the flags: sinks, separators that left the window queue (at
    most s), and the queue, which holds the last L tokens: with P past-window
    entries (capacity c = a + s + n + P) L counts up to n + P and then cycles
    n, ..., n + P (a full queue empties to n - 1 before the next token)."""
    T = flags.shape[0]
    P = max(0, cap - (wl.a + wl.s + wl.n))
    t = np.arange(T)
    f = flags.astype(np.int64)
    f_after_sinks = np.where(t[:, None] >= wl.a, f, 0)
    csum = np.cumsum(f_after_sinks, axis=0)  # separators at positions <= t
    x = np.maximum(t + 1 - wl.a, 0)  # tokens that entered the queue
    L = np.where(x <= wl.n + P, x, wl.n + (x - wl.n - P - 1) % (P + 1))
    last_left = t - L  # tokens at positions <= t - L have left the queue
    left = np.where(last_left[:, None] >= 0, csum[np.clip(last_left, 0, None)], 0)
    return np.minimum(t + 1, wl.a)[:, None] + np.minimum(left, wl.s) + L[:, None]


def decode_bytes(wl: synth.DecodeWorkload, length: np.ndarray) -> float:
    """Bytes one layer's decode must move over the steps of `length`: every
    cached K and V row read once per token, plus q, o and the new K/V row (the
    separator move is an implementation choice and not counted)."""
    row = wl.Hkv * wl.d * 2
    return float(length.sum()) * row * 2 + length.shape[0] * wl.B * (2 * wl.Hq * wl.d * 2 + 2 * row)


class DecodeLeg:
    def __init__(self, wl: synth.DecodeWorkload, layers: int, seed: int = 0, cap: int = 0):
        self.wl, self.layers, self.cap = wl, layers, cap
        dev = "cuda"
        self.flags_np = wl.flags(seed)
        self.flags = torch.from_numpy(self.flags_np).to(dev)
        # every token's own q, k, v (bf16), resident on the device
        self.q_all = torch.empty((wl.T, wl.B, wl.Hq, wl.d), dtype=torch.bfloat16, device=dev)
        self.k_all = torch.empty((wl.T, wl.B, wl.Hkv, wl.d), dtype=torch.bfloat16, device=dev)
        self.v_all = torch.empty_like(self.k_all)
        for t0 in range(0, wl.T, CHUNK):
            t1 = min(wl.T, t0 + CHUNK)
            k, v = wl.kv_steps(t0, t1, seed)
            self.k_all[t0:t1].copy_(torch.from_numpy(k).to(torch.bfloat16))
            self.v_all[t0:t1].copy_(torch.from_numpy(v).to(torch.bfloat16))
            self.q_all[t0:t1].copy_(torch.from_numpy(wl.q_steps(range(t0, t1), seed)).to(torch.bfloat16))
        # the graph's input buffers, refilled before each replay
        self.kp = torch.empty((CHUNK,) + self.k_all.shape[1:], dtype=torch.bfloat16, device=dev)
        self.vp = torch.empty_like(self.kp)
        self.qp = torch.empty((CHUNK,) + self.q_all.shape[1:], dtype=torch.bfloat16, device=dev)
        self.scale = 1.0 / math.sqrt(wl.d)
        self.caches = [sa.SepCache(wl.B, wl.Hkv, wl.d, wl.a, wl.s, wl.n, wl.theta, cap=cap) for _ in range(layers)]
        self.out = torch.empty((layers, wl.B, wl.Hq, wl.d), dtype=torch.bfloat16, device=dev)
        self.fl_static = torch.zeros((CHUNK, wl.B), dtype=torch.uint8, device=dev)
        for c in self.caches:  # each cache's step workspace, zero-filled before the graph is captured
            c.workspace(wl.Hq)
        torch.cuda.synchronize()
        self.stream = torch.cuda.Stream()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph, stream=self.stream):
            for i in range(CHUNK):
                for li, c in enumerate(self.caches):
                    c.step(self.kp[i], self.vp[i], self.fl_static[i], self.qp[i], self.scale, shift=wl.shift,
                           out=self.out[li])
        torch.cuda.synchronize()
        self.n_chunks = wl.T // CHUNK
        assert self.n_chunks * CHUNK == wl.T
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        self.bytes = self._algorithmic_bytes()

    def _algorithmic_bytes(self) -> float:
        length = decode_lengths(self.wl, self.flags_np, self.cap)
        self.mean_len = float(length.mean())
        return decode_bytes(self.wl, length) * self.layers

    def step(self):
        for c in self.caches:
            c.reset()
        self.ev[0].record()
        for ch in range(self.n_chunks):
            sl = slice(ch * CHUNK, (ch + 1) * CHUNK)
            self.fl_static.copy_(self.flags[sl])
            self.kp.copy_(self.k_all[sl])
            self.vp.copy_(self.v_all[sl])
            self.qp.copy_(self.q_all[sl])
            self.graph.replay()
        self.ev[1].record()

    def time_ms(self):
        return self.ev[0].elapsed_time(self.ev[1])


def _rows_for_budget(run, L: int, first: int, budget_s: float) -> tuple[int, float]:
    """Rows of the prefix sample: time `run(first)`, then grow the prefix so
    that the timed call takes about budget_s (the work grows about as
    rows^1.25 over this range: fixed costs weigh on short prefixes)."""
    t0 = time.perf_counter()
    run(first)
    t_small = time.perf_counter() - t0
    rows = int(first * (budget_s / max(t_small, 1e-3)) ** (1 / 1.25)) // 256 * 256
    return max(first, min(L, rows)), t_small


def cpu_baseline(pre: PrefillLeg, dwl: synth.DecodeWorkload, seed: int, budget_s: float = 8.0) -> dict:
    """The fp64 oracle, as it stands, on bounded samples of the workloads,
    timed on this host's cores: the forward and the backward of one q head
    over a prefix of the L = 32768 sequence (a causal prefix is itself a
    prefill of that length), and the decode simulation over the first steps
    of the 16-stream decode with outputs over a window of steady-state steps.
    Flags and inputs come from the seeded generators, never from the GPU."""
    from oracle import sepllm_oracle as orc
    wl = pre.wl
    cores = len(os.sched_getaffinity(0))
    f = orc.separator_flags(wl.tokens(seed), synth.SEP_IDS)
    q, k, v = wl.qkv(seed)
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()
    q, k, v = bf(q[:, :1]), bf(k[:, :1]), bf(v[:, :1])
    do = bf(wl.dout(seed)[:, :1])
    sc = pre.scale
    out = {}
    fwd = lambda r: orc.attn_fwd(q[:, :, :r], k[:, :, :r], v[:, :, :r], f[:, :r], wl.a, wl.n, sc)
    bwd = lambda r: orc.attn_bwd(q[:, :, :r], k[:, :, :r], v[:, :, :r], do[:, :, :r], f[:, :r], wl.a, wl.n, sc)
    for name, run, per_pair in (("fwd", fwd, 4.0), ("bwd", bwd, 10.0)):
        rows, _ = _rows_for_budget(run, wl.L, 2048, budget_s)
        t0 = time.perf_counter()
        run(rows)
        dt = time.perf_counter() - t0
        kept = int(orc.kept_pairs(f[:, :rows], wl.a, wl.n).sum())
        out[name] = {"value": per_pair * wl.d * kept / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
                     "kind": "oracle",
                     "sample": f"fp64 numpy {name} of 1 of {wl.Hq} q heads (d={wl.d}), rows 0..{rows - 1} "
                               f"of {wl.L}: {kept} kept pairs in {dt:.1f} s"}
    # decode: the simulator from an empty cache, outputs over steady-state steps
    t_first, n_out = 800, 48
    T = t_first + n_out
    flags = dwl.flags(seed)[:T]
    kk, vv = dwl.kv_steps(0, T, seed)
    qq = dwl.q_steps(range(T), seed)
    rnd = lambda x: torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    kk, vv, qq = rnd(kk), rnd(vv), rnd(qq)
    steps = list(range(t_first, T))
    t0 = time.perf_counter()
    orc.decode_run(qq, kk, vv, flags, dwl.a, dwl.s, dwl.n, dwl.theta, dwl.shift, 1.0 / math.sqrt(dwl.d),
                   out_steps=steps)
    dt = time.perf_counter() - t0
    nbytes = decode_bytes(dwl, decode_lengths(dwl, flags)[t_first:])
    out["decode"] = {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
                     "sample": f"fp64 numpy SepCache simulator, {dwl.B} streams x {T} steps from empty, outputs "
                               f"of steps {t_first}..{T - 1} (one layer, {dwl.Hq}/{dwl.Hkv} heads, d={dwl.d}): "
                               f"{nbytes / 1e6:.1f} MB of algorithmic bytes in {dt:.1f} s"}
    fl = pre.fwd_flops / pre.kept_per_seq / wl.Hq, pre.bwd_flops / pre.kept_per_seq / wl.Hq
    t_pair = fl[0] / (out["fwd"]["value"] * 1e12) + fl[1] / (out["bwd"]["value"] * 1e12)
    return {"value": (fl[0] + fl[1]) / t_pair / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "prefill forward + backward kept-FLOP rate combined from the two samples below",
            "fwd": out["fwd"], "bwd": out["bwd"], "decode": out["decode"]}


def kernel_sources_sha256() -> str:
    """sha256 over the kernel sources (every file of separator_kv_cache_amd/csrc,
    by name), to tell whether a stored counter profile still describes them."""
    import hashlib
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "separator_kv_cache_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic() -> dict:
    """HBM bytes per launch (fetched + written) per kernel from the committed
    counter profile (profiles/hbm_traffic_per_launch.txt: FETCH_SIZE and
    WRITE_SIZE passes scaled by a device copy's readings).  Empty when the
    kernel sources changed since the profile was taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "hbm_traffic_per_launch.txt")
    if not os.path.exists(path):
        return {}
    sha, out = None, {}
    for line in open(path):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        if f[0] == "sources_sha256":
            sha = f[1]
        elif len(f) == 3:
            out[f[0]] = int(f[1]) + int(f[2])
    return out if sha == kernel_sources_sha256() else {}


def fixllm_leg(pre: PrefillLeg, delta: int, reps: int) -> dict:
    """The prefill forward and backward with fixed-interval anchors (FixLLM:
    one anchor every delta tokens in place of the separators) on the prefill
    leg's own tensors, event-timed; kept-FLOP rates as for the separator mask."""
    wl = pre.wl
    m = sa.build_mask_fixed(wl.B, wl.L, delta, wl.a, wl.n)
    o, lse = sa.sepattn_fwd(pre.q, pre.k, pre.v, m, pre.scale)
    grads = dict(workspace=pre.ws, dq=pre.dq, dk=pre.dk, dv=pre.dv)
    sa.sepattn_bwd(pre.q, pre.k, pre.v, o, lse, pre.do, m, pre.scale, **grads)
    torch.cuda.synchronize()
    kept = int(m.kept.sum().cpu())
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    tf = tb = 0.0
    for _ in range(reps):
        e[0].record()
        sa.sepattn_fwd(pre.q, pre.k, pre.v, m, pre.scale, out=o, lse=lse)
        e[1].record()
        sa.sepattn_bwd(pre.q, pre.k, pre.v, o, lse, pre.do, m, pre.scale, **grads)
        e[2].record()
        torch.cuda.synchronize()
        tf += e[0].elapsed_time(e[1])
        tb += e[1].elapsed_time(e[2])
    tf, tb = tf / reps, tb / reps
    fwd = 4.0 * wl.d * kept * wl.Hq / (tf * 1e-3) / 1e12
    bwd = 10.0 * wl.d * kept * wl.Hq / (tb * 1e-3) / 1e12
    return {"delta": delta, "kept_pairs_per_head": kept, "fwd_ms": round(tf, 4), "bwd_ms": round(tb, 4),
            "fwd_tflops": round(fwd, 2), "bwd_tflops": round(bwd, 2),
            "fwd_util": round(fwd / PEAK_BF16_TFLOPS, 4), "bwd_util": round(bwd / PEAK_BF16_TFLOPS, 4)}


def handoff_leg(wl: synth.DecodeWorkload, L: int, seed: int, sets: int = 8, rounds: int = 6) -> dict:
    """sepcache_prefill of an L-token prompt into one layer's caches.  The
    calls rotate over `sets` distinct (prompt K/V, cache) pairs, whose bytes
    touched per call (~43 MB each) together exceed the 256 MB Infinity Cache,
    so each call reads and writes HBM rather than cache-resident lines.  Its
    algorithmic bytes: the K/V rows of the entries kept (read once) and every
    slot's K/V and metadata and the counters (written once); the few mask
    words it reads per (stream, KV head) are left out."""
    dev = "cuda"
    tok = torch.from_numpy(synth.tokens_iid(seed, 90, wl.B, L, wl.p)).to(dev)
    m = sa.build_mask(tok, synth.SEP_IDS, wl.a, wl.n)
    gen = torch.Generator(device=dev).manual_seed(seed)
    prompts = [tuple(torch.randn((wl.B, wl.Hkv, L, wl.d), generator=gen, device=dev).to(torch.bfloat16)
                     for _ in range(2)) for _ in range(sets)]
    caches = [sa.SepCache(wl.B, wl.Hkv, wl.d, wl.a, wl.s, wl.n, wl.theta) for _ in range(sets)]
    caches[0].prefill(*prompts[0], m)
    torch.cuda.synchronize()
    entries = int((caches[0].slot_pos[:, 0] >= 0).sum())  # over streams, one KV head
    # the calls run as one graph replay, back to back on the device: timed
    # call by call from Python, the host's launch rate would be measured
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(rounds):
            for (k, v), c in zip(prompts, caches):
                c.prefill(k, v, m)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    calls = rounds * sets
    us = e0.elapsed_time(e1) * 1e3 / calls
    row = wl.d * 2
    nbytes = entries * wl.Hkv * row * 2 + wl.B * wl.Hkv * (caches[0].slots * (row * 2 + 5) + 32)
    return {"config": {"B": wl.B, "Hkv": wl.Hkv, "d": wl.d, "a": wl.a, "s": wl.s, "n": wl.n, "prompt": L,
                       "distinct_sets": sets, "calls": calls},
            "us": round(us, 3), "bytes": nbytes, "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "entries": entries}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--layers", type=int, default=32, help="decode layer caches")
    ap.add_argument("--decode-tokens", type=int, default=None,
                    help="tokens per stream (default: the workload's 8192; fewer only for profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-copy-mb", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (a known-size kernel that "
                         "calibrates HBM byte counters in a profiler run)")
    ap.add_argument("--general-tokens", type=int, default=4096,
                    help="tokens of the capacity-800 cache leg (the pages' streaming capacity; 0 skips it)")
    ap.add_argument("--general-layers", type=int, default=8, help="layer caches of that leg")
    ap.add_argument("--resident-tokens", type=int, default=2048,
                    help="tokens of the one-layer (cache-resident) decode leg (0 skips it)")
    ap.add_argument("--fixllm-delta", type=int, default=8,
                    help="anchor interval of the FixLLM prefill leg (0 skips it)")
    ap.add_argument("--handoff-tokens", type=int, default=4096,
                    help="prompt length of the prefill-to-cache hand-off leg (0 skips it)")
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the SepLLM path here runs on a single MI355X "
              "(multi-GPU sharding is a design note, not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    pre = PrefillLeg(synth.LLAMA_PREFILL, args.seed)
    dwl = synth.LLAMA_DECODE
    if args.decode_tokens is not None:
        dwl = dwl.with_(T=args.decode_tokens)
    dec = DecodeLeg(dwl, args.layers, args.seed)

    if args.profile_copy_mb > 0:
        src = torch.empty(args.profile_copy_mb << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # The decode leg is enqueued first, so the prefill's first event and its
    # mask build are queued behind it and start when it ends: started on an
    # idle stream, the first event would also time the host's enqueue latency.
    for _ in range(args.warmup):
        dec.step()
        pre.step()
    torch.cuda.synchronize()

    t_mask = t_fwd = t_bwd = t_dec = 0.0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dec.step()
        pre.step()
        torch.cuda.synchronize()
        a, b, c = pre.times_ms()
        t_mask += a
        t_fwd += b
        t_bwd += c
        t_dec += dec.time_ms()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # The same decode with one layer's caches (21 MB, resident in the 256 MB
    # Infinity Cache between tokens), beside the 32-layer figure above.
    res_out = None
    if args.resident_tokens > 0:
        res = DecodeLeg(dwl.with_(T=args.resident_tokens), 1, args.seed)
        res.step()
        torch.cuda.synchronize()
        t_res = 0.0
        for _ in range(args.steps):
            res.step()
            torch.cuda.synchronize()
            t_res += res.time_ms()
        t_res /= args.steps
        gbs = res.bytes / (t_res * 1e-3) / 1e9
        res_out = {"layers": 1, "tokens": res.wl.T, "ms": round(t_res, 3), "gbs": round(gbs, 1),
                   "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                   "us_per_token_layer": round(t_res * 1e3 / res.wl.T, 3)}
        del res
    # The four-block cache at capacity c = 800 (a past window of 476 entries)
    # on the same decode geometry: timed on its own, outside the step.
    gen_out = None
    if args.general_tokens > 0:
        gen = DecodeLeg(synth.LLAMA_DECODE.with_(T=args.general_tokens), args.general_layers, args.seed, cap=800)
        gen.step()
        torch.cuda.synchronize()
        t_gen = 0.0
        for _ in range(args.steps):
            gen.step()
            torch.cuda.synchronize()
            t_gen += gen.time_ms()
        t_gen /= args.steps
        gbs = gen.bytes / (t_gen * 1e-3) / 1e9
        gen_out = {"config": {"B": gen.wl.B, "Hq": gen.wl.Hq, "Hkv": gen.wl.Hkv, "d": gen.wl.d, "a": gen.wl.a,
                              "s": gen.wl.s, "n": gen.wl.n, "c": 800, "tokens": gen.wl.T,
                              "layers": args.general_layers, "p": gen.wl.p, "shift": gen.wl.shift},
                   "ms": round(t_gen, 3), "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                   "bytes": gen.bytes, "mean_cache_len": round(gen.mean_len, 2),
                   "us_per_token_layer": round(t_gen * 1e3 / (gen.wl.T * args.general_layers), 3)}
        del gen
    # Prompt hand-off: seed the Llama decode caches (16 streams x 8 KV heads,
    # 324 entries) from a prompt's K/V and mask metadata, timed on its own.
    fix_out = fixllm_leg(pre, args.fixllm_delta, args.steps) if args.fixllm_delta > 0 else None
    hand_out = None
    if args.handoff_tokens > 0:
        hand_out = handoff_leg(synth.LLAMA_DECODE, args.handoff_tokens, args.seed)
    K = args.steps
    t_mask, t_fwd, t_bwd, t_dec = t_mask / K, t_fwd / K, t_bwd / K, t_dec / K
    pre_ms = t_mask + t_fwd + t_bwd
    value = (pre.fwd_flops + pre.bwd_flops) / (pre_ms * 1e-3) / 1e12
    fwd_tf = pre.fwd_flops / (t_fwd * 1e-3) / 1e12
    bwd_tf = pre.bwd_flops / (t_bwd * 1e-3) / 1e12
    dec_gbs = dec.bytes / (t_dec * 1e-3) / 1e9
    launches = dec.wl.T * args.layers
    wl = pre.wl
    out = {
        "metric": "kept-FLOP TFLOP/s (MFMA util) sep-attn prefill + decode HBM GB/s, Llama-3-8B",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama3-8b sep-attn prefill L=32768 fwd+bwd + sepcache decode 8192 tokens x "
                        f"{args.layers} layers",
            "prefill": {"B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "L": wl.L, "d": wl.d, "a": wl.a, "n": wl.n,
                        "p": wl.p, "separators": "clustered"},
            "decode": {"B": dec.wl.B, "Hq": dec.wl.Hq, "Hkv": dec.wl.Hkv, "d": dec.wl.d, "a": dec.wl.a,
                       "s": dec.wl.s, "n": dec.wl.n, "tokens": dec.wl.T, "p": dec.wl.p,
                       "layers": args.layers, "shift": dec.wl.shift,
                       "inputs": "each token its own q/k/v, N(0,1) per step from the seed, bf16, resident in HBM"},
        },
        "prefill": {
            "kept_pairs_per_head": pre.kept_per_seq,
            "kept_fraction_of_causal": round(pre.kept_per_seq / (wl.L * (wl.L + 1) / 2), 4),
            "mask_ms": round(t_mask, 4), "fwd_ms": round(t_fwd, 4), "bwd_ms": round(t_bwd, 4),
            "fwd_tflops": round(fwd_tf, 2), "bwd_tflops": round(bwd_tf, 2),
            "fwd_util": round(fwd_tf / PEAK_BF16_TFLOPS, 4), "bwd_util": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
        },
        "decode": {
            "ms": round(t_dec, 3), "gbs": round(dec_gbs, 1), "frac_of_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4),
            "bytes": dec.bytes, "mean_cache_len": round(dec.mean_len, 2), "launches": launches,
            "us_per_token_layer": round(t_dec * 1e3 / (dec.wl.T * args.layers), 3),
        },
        "roofline": None,
        "rooflines": None,
    }
    if res_out is not None:
        out["decode_resident"] = res_out
    if gen_out is not None:
        out["decode_c800"] = gen_out
    if hand_out is not None:
        out["prefill_handoff"] = hand_out
    if fix_out is not None:
        out["prefill_fixllm"] = fix_out
    traffic = measured_traffic()
    dec_launch_us = t_dec * 1e3 / (dec.wl.T * args.layers)
    per_launch_bytes = dec.bytes / (dec.wl.T * args.layers)
    r_dec = {"kernel": "decode_tiles (SepCache step: append, evict, attend; one layer, d=128, 4 q heads per KV head)",
             "bound": "hbm", "achieved": round(per_launch_bytes / (dec_launch_us * 1e-6) / 1e9, 1),
             "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(per_launch_bytes / (dec_launch_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
             "traffic": traffic.get("decode_tiles"),
             "per_launch_bytes": round(per_launch_bytes), "avg_launch_us": round(dec_launch_us, 3)}
    r_fwd = {"kernel": "fwd_pp_kernel (bf16, d=128)", "bound": "mfma", "achieved": round(fwd_tf, 2),
             "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
             "traffic": traffic.get("fwd_pp_kernel"), "per_launch_flops": pre.fwd_flops,
             "avg_launch_ms": round(t_fwd, 4)}
    r_bwd = {"kernel": "dq_kernel + dkdv_kernel (bf16, d=128)", "bound": "mfma", "achieved": round(bwd_tf, 2),
             "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
             "traffic": (traffic["dq_kernel"] + traffic["dkdv_kernel"]
                         if "dq_kernel" in traffic and "dkdv_kernel" in traffic else None),
             "per_launch_flops": pre.bwd_flops, "avg_launch_ms": round(t_bwd, 4)}
    # the kernel that dominates a step's time carries the headline roofline
    out["roofline"] = r_dec if t_dec > pre_ms else r_fwd
    out["rooflines"] = [r_fwd, r_bwd, r_dec]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(pre, synth.LLAMA_DECODE, args.seed)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
