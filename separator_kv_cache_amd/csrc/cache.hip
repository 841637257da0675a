// SepCache: the streaming cache of SepLLM and decode over it.
//
// The cache (pith.science verdict for 2412.12094, key_machinery; anthology
// record LIT-748, "Key takeaways", streaming bullet) keeps a initial tokens,
// a separator block and a window.  A token leaving the window moves to the
// separator block if it is a separator, otherwise it is dropped.  Here the
// separator block holds s entries first-in first-out, and the window holds n
// entries counting the newest token.  Keys are stored before RoPE and rotated
// at decode time, by their rank inside the cache when positions are shifted
// (paperhub.cn author responses, second reviewer, A1) or by their original
// position otherwise.
//
// Physical slots of a (stream, KV head): [0, a) sinks, [a, a+s) separator
// ring, [a+s, a+s+n+1) window ring (one spare slot holds the appended token
// until eviction).  Each (stream, KV head) has its own counters and slot
// metadata.  The counters also carry the separator flag of the window's
// oldest entry, so a step's transition needs no lookup into the slots.
#include <math.h>

#include "common.h"

namespace {

enum { ST_T = 0, ST_NSINK, ST_SEPH, ST_SEPC, ST_WINH, ST_WINC, ST_FLAGS, ST_OLDSEP };
constexpr int FLAG_WINDOW_OVERFLOW = 1;

// n is the window queue's capacity: the window plus the past window (P
// entries, 0 without one).  The step logic below (append, evict, ranks) only
// needs that capacity; the flush of a full queue alone needs P.
struct CacheParams {
  bf16* k;
  bf16* v;
  int32_t* slot_pos;
  uint8_t* slot_sep;
  int32_t* state;
  int B, Hkv, d, a, s, n, slots, P;
};

// K of one (stream, KV head) is stored per 16-row tile, chunk-major: 16-byte
// chunk ch of row r sits at chunk index ((r / 16) * nch + ch) * 16 + r % 16
// of the slice, which has sepcache_k_rows_of(slots) rows.  The decode's
// score operand of a 16-row tile (lane (g, col) holds chunk 4m + g of row
// 16t + col) is then 1 KB contiguous per load.  V is row-major.
__device__ __forceinline__ size_t k_at(int row, int ch, int nch) {  // element offset of chunk ch of row
  return ((((size_t)(row >> 4) * nch + ch) << 4) + (size_t)(row & 15)) * 8;
}

int past_entries(const sepcache* c) { return c->c > c->a + c->s + c->n ? c->c - (c->a + c->s + c->n) : 0; }

CacheParams make_params(const sepcache* c) {
  CacheParams p;
  p.k = (bf16*)c->k; p.v = (bf16*)c->v;
  p.slot_pos = c->slot_pos; p.slot_sep = c->slot_sep; p.state = c->state;
  p.P = past_entries(c);
  p.B = c->B; p.Hkv = c->Hkv; p.d = c->d; p.a = c->a; p.s = c->s; p.n = c->n + p.P;
  p.slots = c->a + c->s + p.n + 1;
  return p;
}

struct Counters {
  int t, nsink, seph, sepc, winh, winc, flags, oldsep;
};

__device__ __forceinline__ Counters load_counters(const int32_t* st) {
  Counters c;
  c.t = st[ST_T]; c.nsink = st[ST_NSINK]; c.seph = st[ST_SEPH]; c.sepc = st[ST_SEPC];
  c.winh = st[ST_WINH]; c.winc = st[ST_WINC]; c.flags = st[ST_FLAGS]; c.oldsep = st[ST_OLDSEP];
  return c;
}

__device__ __forceinline__ void store_counters(int32_t* st, const Counters& c) {
  st[ST_T] = c.t; st[ST_NSINK] = c.nsink; st[ST_SEPH] = c.seph; st[ST_SEPC] = c.sepc;
  st[ST_WINH] = c.winh; st[ST_WINC] = c.winc; st[ST_FLAGS] = c.flags; st[ST_OLDSEP] = c.oldsep;
}

// The effect of appending one token (app) and evicting (ev) on the counters.
// app_slot: where the token goes (-1: dropped because the window was full);
// ev_src/ev_dst: the slot leaving the window and where it goes (-1: none or
// dropped); sep_drop: the separator ring's oldest entry was dropped.  When
// the window's oldest entry changes to an older resident, its flag must be
// read from slot_sep (refresh_oldsep); after.oldsep is then stale.
struct Transition {
  Counters after;
  int app_slot, ev_src, ev_dst;
  bool evicted, sep_drop, refresh_oldsep;
};

__device__ __forceinline__ Transition transition(const Counters& c0, int a, int s, int n, bool app, bool new_sep,
                                                 bool ev) {
  Transition tr;
  Counters c = c0;
  tr.app_slot = tr.ev_src = tr.ev_dst = -1;
  tr.evicted = tr.sep_drop = tr.refresh_oldsep = false;
  const int W = n + 1;
  if (app) {
    if (c.t < a) {
      tr.app_slot = c.t;
      c.nsink = c.t + 1;
      ++c.t;
    } else if (c.winc <= n) {
      tr.app_slot = a + s + (c.winh + c.winc) % W;
      if (c.winc == 0) c.oldsep = new_sep ? 1 : 0;
      ++c.winc;
      ++c.t;
    } else {
      c.flags |= FLAG_WINDOW_OVERFLOW;
    }
  }
  if (ev && c.winc > n) {
    tr.evicted = true;
    tr.ev_src = a + s + c.winh;  // never the token appended in this step
    if (c.oldsep && s > 0) {
      if (c.sepc < s) {
        tr.ev_dst = a + (c.seph + c.sepc) % s;
        ++c.sepc;
      } else {
        tr.ev_dst = a + c.seph;
        c.seph = (c.seph + 1) % s;
        tr.sep_drop = true;
      }
    }
    c.winh = (c.winh + 1) % W;
    --c.winc;
    if (c.winc > 0) {
      if (a + s + c.winh == tr.app_slot) c.oldsep = new_sep ? 1 : 0;
      else tr.refresh_oldsep = true;
    }
  }
  tr.after = c;
  return tr;
}

// Slot metadata and counters after a transition (one thread; the caller has
// finished every read of the old metadata).  ev_pos: original position of
// the evicted token; new_oldsep: flag of the new oldest window entry when
// tr.refresh_oldsep.
__device__ __forceinline__ void commit(const Transition& tr, int32_t* st, int32_t* spos, uint8_t* ssep,
                                       bool new_sep, int ev_pos, int new_oldsep) {
  if (tr.app_slot >= 0) {
    spos[tr.app_slot] = tr.after.t - 1;
    ssep[tr.app_slot] = new_sep ? 1 : 0;
  }
  if (tr.evicted) {
    if (tr.ev_dst >= 0) {
      spos[tr.ev_dst] = ev_pos;
      ssep[tr.ev_dst] = 1;
    }
    spos[tr.ev_src] = -1;
    ssep[tr.ev_src] = 0;
  }
  Counters c = tr.after;
  if (tr.refresh_oldsep) c.oldsep = new_oldsep;
  store_counters(st, c);
}

constexpr int MAX_HALF = 64;  // d/2 for d = 128

// RoPE revolutions per position of each frequency: theta^(-2i/d) / (2 pi).
struct RopeFreqs {
  double rev[MAX_HALF];
};

RopeFreqs rope_freqs(const sepcache* c) {
  RopeFreqs f;
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < MAX_HALF; ++i) f.rev[i] = i < c->d / 2 ? pow((double)c->theta, -2.0 * i / c->d) / two_pi : 0.0;
  return f;
}

__global__ void reset_kernel(CacheParams p) {
  const size_t bh = blockIdx.x;
  for (int i = threadIdx.x; i < p.slots; i += blockDim.x) {
    p.slot_pos[bh * p.slots + i] = -1;
    p.slot_sep[bh * p.slots + i] = 0;
  }
  // K and V of every slot to zero: decode multiplies the rows that hold no
  // entry by a zero probability, which must not meet a non-finite value
  // (K's slice includes the padding rows of its last tile)
  const size_t kchunks = (size_t)sepcache_k_rows_of(p.slots) * p.d / 8, vchunks = (size_t)p.slots * p.d / 8;
  const u32x4 z = {0u, 0u, 0u, 0u};
  bf16* kz = p.k + bh * sepcache_k_rows_of(p.slots) * p.d;
  for (size_t i = threadIdx.x; i < kchunks; i += blockDim.x) st16(kz + i * 8, z);
  for (size_t i = threadIdx.x; i < vchunks; i += blockDim.x) st16(p.v + bh * p.slots * p.d + i * 8, z);
  if (threadIdx.x < 8) p.state[bh * 8 + threadIdx.x] = 0;
}

// Seeds one (stream, KV head) with the state that L pushes from empty leave:
// a prompt handed over from prefill.  Every slot's content is a closed form
// of L.  Ring token j (token a + j) always goes to ring slot j mod W (each
// append goes to head + count, which departures leave unchanged), and
// separator push i to ring slot i mod s; the queue holds its last Lq tokens
// and the separator ring the last min(s, cnt) of the cnt separators that
// left the queue.  A ring slot that holds no entry keeps the K/V of its last
// occupant (departures clear only the slot's metadata); other empty slots
// were never written since the reset and hold zeros.
// one 16-byte chunk of K and one of V per thread: the most workgroups per
// (stream, KV head) (kernel trace of the prompt hand-off on the Llama decode
// geometry, 4096 tokens: 8.2 us per call, against 9.7 us with 4 per thread)
constexpr int PF_THREADS = 256, PF_PER_THREAD = 1, PF_CHUNKS = PF_THREADS * PF_PER_THREAD;

__global__ __launch_bounds__(PF_THREADS) void prefill_kernel(CacheParams p, const bf16* k, const bf16* v, int64_t ksb,
                                                      int64_t ksh, int64_t kst, int64_t vsb, int64_t vsh,
                                                      int64_t vst, int L, const uint8_t* is_sep,
                                                      const int32_t* sep_idx, const int32_t* sep_before) {
  const int bh = blockIdx.x, b = bh / p.Hkv, h = bh % p.Hkv;
  const int W = p.n + 1, P = p.P, n = p.n - p.P, NCH = p.d / 8;
  const int x = max(0, L - p.a);  // tokens that entered the queue
  const int Lq = x <= n + P ? x : n + (x - n - P - 1) % (P + 1);
  const int cnt = sep_before[(size_t)b * (L + 1) + (L - Lq)];  // separators that left it
  const int sepc = min(p.s, cnt);
  const uint8_t* fl = is_sep + (size_t)b * L;
  const int32_t* si = sep_idx + (size_t)b * L;
  const bf16* kp = k + b * ksb + h * ksh;
  const bf16* vp = v + b * vsb + h * vsh;
  int32_t* spos = p.slot_pos + (size_t)bh * p.slots;
  uint8_t* ssep = p.slot_sep + (size_t)bh * p.slots;
  bf16* kc = p.k + (size_t)bh * sepcache_k_rows_of(p.slots) * p.d;
  bf16* vc = p.v + (size_t)bh * p.slots * p.d;
  auto token_of = [&](int slot) -> int {
    if (slot < p.a) return slot < L ? slot : -1;
    if (slot < p.a + p.s) {
      if (sepc == 0) return -1;
      const int base = cnt - sepc;
      const int i = base + ((slot - p.a - base) % p.s + p.s) % p.s;
      return i < cnt ? si[i] : -1;
    }
    if (Lq == 0) return -1;
    const int base = x - Lq;
    const int j = base + ((slot - p.a - p.s - base) % W + W) % W;
    return j < x ? p.a + j : -1;
  };
  // the token whose K/V a slot holds: its entry, or for an empty ring slot
  // the last token that left it (the largest j < base congruent to it)
  auto content_of = [&](int slot) -> int {
    const int tok = token_of(slot);
    if (tok >= 0 || slot < p.a + p.s) return tok;
    const int base = x - Lq;
    const int j = base - 1 - ((base - 1 - (slot - p.a - p.s)) % W + W) % W;
    return j >= 0 ? p.a + j : -1;
  };
  // workgroup y of the pair's grid row takes chunks [y, y + 1) * PF_CHUNKS
  // of the K/V rows (16 bytes each, PF_PER_THREAD per thread, all loads
  // issued before the stores) and, the first, the metadata and counters
  const int i0 = (int)blockIdx.y * PF_CHUNKS + (int)threadIdx.x;
  const u32x4 z = {0u, 0u, 0u, 0u};
  u32x4 kx[PF_PER_THREAD], vx[PF_PER_THREAD];
#pragma unroll
  for (int u = 0; u < PF_PER_THREAD; ++u) {
    const int i = i0 + u * PF_THREADS;
    const int slot = i / NCH, ch = i % NCH;
    const int tok = i < p.slots * NCH ? content_of(slot) : -1;
    kx[u] = tok >= 0 ? ld16(kp + tok * kst + ch * 8) : z;
    vx[u] = tok >= 0 ? ld16(vp + tok * vst + ch * 8) : z;
  }
#pragma unroll
  for (int u = 0; u < PF_PER_THREAD; ++u) {
    const int i = i0 + u * PF_THREADS;
    if (i < p.slots * NCH) {
      st16(kc + k_at(i / NCH, i % NCH, NCH), kx[u]);
      st16(vc + (size_t)(i / NCH) * p.d + (i % NCH) * 8, vx[u]);
    }
  }
  if (blockIdx.y != 0) return;
  for (int slot = threadIdx.x; slot < p.slots; slot += blockDim.x) {
    const int tok = token_of(slot);
    spos[slot] = tok;
    ssep[slot] = tok >= 0 ? fl[tok] : 0;
  }
  if (threadIdx.x == 0) {
    Counters c;
    c.t = L;
    c.nsink = min(p.a, L);
    c.seph = p.s > 0 ? max(0, cnt - p.s) % p.s : 0;
    c.sepc = sepc;
    c.winh = (x - Lq) % W;
    c.winc = Lq;
    c.flags = 0;
    c.oldsep = Lq > 0 ? fl[p.a + x - Lq] : 0;
    store_counters(p.state + (size_t)bh * 8, c);
  }
}

// Stores a new row (d elements of K and of V, contiguous) into slot `dst`
// with the workgroup's threads: K into the tiled slice, V row-major.
__device__ __forceinline__ void store_row(int d, const bf16* ks, const bf16* vs, bf16* kslice, int dst, bf16* vd) {
  const int ch = d / 8;
  for (int i = threadIdx.x; i < 2 * ch; i += blockDim.x) {
    if (i < ch) st16(kslice + k_at(dst, i, ch), ld16(ks + i * 8));
    else st16(vd + (i - ch) * 8, ld16(vs + (i - ch) * 8));
  }
}

// Moves the row of slot `src` to slot `dst` (K in the tiled slice, V
// row-major) with the workgroup's threads.
__device__ __forceinline__ void move_row(int d, bf16* kslice, int src, int dst, const bf16* vs, bf16* vd) {
  const int ch = d / 8;
  for (int i = threadIdx.x; i < 2 * ch; i += blockDim.x) {
    if (i < ch) st16(kslice + k_at(dst, i, ch), ld16(kslice + k_at(src, i, ch)));
    else st16(vd + (i - ch) * 8, ld16(vs + (i - ch) * 8));
  }
}

// Append and/or evict for one (stream, KV head).
__global__ __launch_bounds__(64) void update_kernel(CacheParams p, const bf16* k_new, const bf16* v_new,
                                                    const uint8_t* is_sep, int do_append, int do_evict) {
  const int bh = blockIdx.x;
  const int b = bh / p.Hkv;
  int32_t* st = p.state + (size_t)bh * 8;
  int32_t* spos = p.slot_pos + (size_t)bh * p.slots;
  uint8_t* ssep = p.slot_sep + (size_t)bh * p.slots;
  const Counters c0 = load_counters(st);
  const bool new_sep = do_append ? is_sep[b] != 0 : false;
  const Transition tr = transition(c0, p.a, p.s, p.n, do_append, new_sep, do_evict);
  const int ev_pos = tr.evicted ? spos[tr.ev_src] : -1;
  const int new_oldsep = tr.refresh_oldsep ? ssep[p.a + p.s + tr.after.winh] : 0;
  bf16* kb = p.k + (size_t)bh * sepcache_k_rows_of(p.slots) * p.d;
  bf16* vb = p.v + (size_t)bh * p.slots * p.d;
  if (tr.app_slot >= 0)
    store_row(p.d, k_new + (size_t)bh * p.d, v_new + (size_t)bh * p.d, kb, tr.app_slot, vb + (size_t)tr.app_slot * p.d);
  if (tr.ev_dst >= 0) move_row(p.d, kb, tr.ev_src, tr.ev_dst, vb + (size_t)tr.ev_src * p.d, vb + (size_t)tr.ev_dst * p.d);
  __syncthreads();
  if (threadIdx.x == 0) commit(tr, st, spos, ssep, new_sep, ev_pos, new_oldsep);
}

// With a past window (P >= 1): before a token is appended to a full window
// queue (n + P entries), its oldest P + 1 entries leave it in order.  The
// separators among them join the separator ring, which keeps its s most
// recent; the others are dropped; the queue keeps its newest n - 1.  One wave
// per (stream, KV head); nothing happens unless the queue is full.
__global__ __launch_bounds__(64) void flush_kernel(CacheParams p) {
  const int bh = blockIdx.x, lane = threadIdx.x;
  int32_t* st = p.state + (size_t)bh * 8;
  int32_t* spos = p.slot_pos + (size_t)bh * p.slots;
  uint8_t* ssep = p.slot_sep + (size_t)bh * p.slots;
  bf16* kb = p.k + (size_t)bh * sepcache_k_rows_of(p.slots) * p.d;
  bf16* vb = p.v + (size_t)bh * p.slots * p.d;
  const Counters c = load_counters(st);
  if (c.winc < p.n) return;  // p.n = n + P, the queue's capacity
  const int W = p.n + 1, m = p.P + 1, q0 = p.a + p.s;
  auto qslot = [&](int e) { return q0 + (c.winh + e) % W; };
  // the number of separators among the leaving entries
  int M = 0;
  for (int e0 = 0; e0 < m; e0 += 64) {
    const bool sep = e0 + lane < m && ssep[qslot(e0 + lane)] != 0;
    M += __popcll(__ballot(sep));
  }
  // separator i (in order) goes to ring slot (seph + sepc + i) mod s; of
  // more than s, only the last s survive, so only those are written and
  // every ring slot is written once
  const int keep_from = max(0, M - p.s);
  int before = 0;
  for (int e0 = 0; e0 < m; e0 += 64) {
    const int e = e0 + lane;
    const int src = qslot(e < m ? e : 0);
    const bool sep = e < m && ssep[src] != 0;
    const uint64_t bal = __ballot(sep);
    const int i = before + __popcll(bal & ((1ull << lane) - 1ull));
    if (sep && p.s > 0 && i >= keep_from) {
      const int dst = p.a + (c.seph + c.sepc + i) % p.s;
      for (int ch = 0; ch < p.d / 8; ++ch) {
        st16(kb + k_at(dst, ch, p.d / 8), ld16(kb + k_at(src, ch, p.d / 8)));
        st16(vb + (size_t)dst * p.d + ch * 8, ld16(vb + (size_t)src * p.d + ch * 8));
      }
      spos[dst] = spos[src];
      ssep[dst] = 1;
    }
    before += __popcll(bal);
  }
  // the leaving entries' slots now hold none (this wave read them above)
  for (int e = lane; e < m; e += 64) {
    spos[qslot(e)] = -1;
    ssep[qslot(e)] = 0;
  }
  if (lane == 0) {
    Counters c1 = c;
    if (p.s > 0) {
      c1.seph = (c.seph + max(0, c.sepc + M - p.s)) % p.s;
      c1.sepc = min(p.s, c.sepc + M);
    }
    c1.winh = (c.winh + m) % W;
    c1.winc = c.winc - m;
    c1.oldsep = c1.winc > 0 ? ssep[q0 + c1.winh] : 0;  // a slot that stays
    store_counters(st, c1);
  }
}

__global__ void export_kernel(CacheParams p, int32_t* pos, int32_t* len) {
  const int b = blockIdx.x;
  const size_t bh = (size_t)b * p.Hkv;  // KV head 0's copy
  const Counters c = load_counters(p.state + bh * 8);
  const int cap = p.a + p.s + p.n;
  const int W = p.n + 1;
  for (int i = threadIdx.x; i < cap; i += blockDim.x) pos[(size_t)b * cap + i] = -1;
  __syncthreads();
  for (int slot = threadIdx.x; slot < p.slots; slot += blockDim.x) {
    int r = -1;
    if (slot < p.a) r = slot < c.nsink ? slot : -1;
    else if (slot < p.a + p.s) {
      const int off = (slot - p.a - c.seph + p.s) % p.s;
      r = off < c.sepc ? c.nsink + off : -1;
    } else {
      const int off = (slot - p.a - p.s - c.winh + W) % W;
      r = off < c.winc ? c.nsink + c.sepc + off : -1;
    }
    if (r >= 0 && r < cap) pos[(size_t)b * cap + r] = p.slot_pos[bh * p.slots + slot];
  }
  if (threadIdx.x == 0) len[b] = c.nsink + c.sepc + c.winc;
}

// ---------------------------------------------------------------- attention
//
// Caches of at most DT_MAX_ROWS rows (the physical slots, plus the appended
// token's row in a step) run as one kernel, decode_tiles, with one workgroup
// per (stream, KV head).  Larger caches split their rows over several
// attend_part workgroups that each write an (o, sum, max) partial, and
// attend_merge combines them.

struct AttendParams {
  CacheParams c;
  const bf16* q;
  bf16* o;
  const bf16* k_new;
  const bf16* v_new;
  const uint8_t* is_sep;
  float* part;  // workspace: partial results (and, tiled path, tickets)
  int Hq, shift, split, tiled;
  float scale_log2;
  float rev_log2_step;   // -2 log2(theta) / d: frequency i turns 2^(i * step) / (2 pi) per position
  double rev[MAX_HALF];  // theta^(-2i/d) / (2 pi): RoPE revolutions per position
};

// cos and sin of 2 pi * frac(pos * rev).  Positions inside the cache (ranks,
// below 2^16) reduce in fp32: the product's absolute error stays below 2^-8
// times the rank's ulp share, about 1e-5 of a turn at rank 1000; original
// positions (any size) reduce in double precision.
template <bool SMALL>
__device__ __forceinline__ void rope_cs(int pos, double rev, float rev32, float& c, float& s) {
  float f;
  if constexpr (SMALL) {
    f = __builtin_amdgcn_fractf((float)pos * rev32);
  } else {
    double x = (double)pos * rev;
    x -= floor(x);
    f = (float)x;
  }
  c = __builtin_amdgcn_cosf(f);
  s = __builtin_amdgcn_sinf(f);
}

// Rank after the step of physical row `row` (row == slots: the appended
// token), or -1 if the row holds no entry then.
template <bool UPDATE>
__device__ __forceinline__ int row_rank(int row, const Counters& c0, const Transition& tr, int a, int s, int n,
                                        int slots) {
  const Counters& c1 = tr.after;
  if (row >= slots) return (UPDATE && row == slots && tr.app_slot >= 0) ? c1.nsink + c1.sepc + c1.winc - 1 : -1;
  if (row < a) return row < c0.nsink ? row : -1;
  if (row < a + s) {
    int off = row - a - c0.seph;
    if (off < 0) off += s;
    if (off >= c0.sepc) return -1;
    if (tr.sep_drop) return off == 0 ? -1 : c1.nsink + off - 1;
    return c1.nsink + off;
  }
  int off = row - a - s - c0.winh;
  if (off < 0) off += n + 1;
  if (off >= c0.winc) return -1;
  if (tr.evicted) {
    if (off == 0) return tr.ev_dst >= 0 ? c1.nsink + c1.sepc - 1 : -1;
    return c1.nsink + c1.sepc + off - 1;
  }
  return c1.nsink + c1.sepc + off;
}

// ---- split path: workgroup = (stream, KV head, split) over at most 64 (d=128)
// or 128 (d=64) rows.  A group of D/8 lanes takes one row; lane li holds
// dimensions [4li, 4li+4) and their RoPE partners [D/2 + 4li, D/2 + 4li + 4).
// Every load is issued before the counters are used, and RoPE angles are
// computed in the kernel, so a split costs one memory round trip.  For a
// step, the lanes holding the new token and the evicted separator also write
// those rows to their new slots (slots no other split reads this step);
// attend_merge commits the slot metadata and counters.

constexpr int SPLIT_THREADS = 256;  // rows per split = 256/(d/8) * 4
constexpr int SPLIT_MAXR = 4;

template <int D, int G, bool UPDATE, bool SHIFT>
__global__ __launch_bounds__(SPLIT_THREADS) void attend_part(AttendParams p) {
  constexpr int LPR = D / 8;
  constexpr int GROUPS = SPLIT_THREADS / LPR;
  constexpr int HALF = D / 2;
  constexpr int NW = SPLIT_THREADS / 64;
  constexpr int MAXR = SPLIT_MAXR;
  __shared__ float sc[G][GROUPS * MAXR];
  __shared__ float red[NW][G];
  __shared__ float mstat[G];
  __shared__ float acc[NW][G][D];

  const CacheParams& c = p.c;
  const int split = blockIdx.x % p.split;
  const int bh = blockIdx.x / p.split;
  const int b = bh / c.Hkv, kvh = bh % c.Hkv;
  const int li = threadIdx.x % LPR, grp = threadIdx.x / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  bf16* kb = c.k + (size_t)bh * sepcache_k_rows_of(c.slots) * D;
  bf16* vb = c.v + (size_t)bh * c.slots * D;
  const int rows = c.slots + (UPDATE ? 1 : 0);
  const int per = (rows + p.split - 1) / p.split;
  const int row0 = split * per, row1 = min(rows, row0 + per);

  // ---- every load first: slot positions (no shift), K/V rows, queries
  int spos_r[MAXR];
  if constexpr (!SHIFT) {
#pragma unroll
    for (int r = 0; r < MAXR; ++r)
      spos_r[r] = c.slot_pos[(size_t)bh * c.slots + min(row0 + grp + r * GROUPS, c.slots - 1)];
  }
  bf16x4 klo[MAXR], khi[MAXR], vlo[MAXR], vhi[MAXR];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    const int row = min(row0 + grp + r * GROUPS, rows - 1);
    const bool cached = row < c.slots;
    const bf16* kn = p.k_new + (size_t)bh * D;
    const bf16* vs = cached ? vb + (size_t)row * D : p.v_new + (size_t)bh * D;
    // dims li * 4 .. + 3 and HALF + li * 4 .. + 3 (each inside one 16-byte chunk)
    klo[r] = *(const bf16x4*)(cached ? kb + k_at(row, li / 2, D / 8) + (li & 1) * 4 : kn + li * 4);
    khi[r] = *(const bf16x4*)(cached ? kb + k_at(row, (HALF + li * 4) / 8, D / 8) + (li & 1) * 4 : kn + HALF + li * 4);
    vlo[r] = *(const bf16x4*)(vs + li * 4);
    vhi[r] = *(const bf16x4*)(vs + HALF + li * 4);
  }
  bf16x4 qlo_b[G], qhi_b[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const bf16* qr = p.q + ((size_t)b * p.Hq + kvh * G + h) * D;
    qlo_b[h] = *(const bf16x4*)(qr + li * 4);
    qhi_b[h] = *(const bf16x4*)(qr + HALF + li * 4);
  }
  double rev[4];
  float rev32[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    rev[e] = p.rev[li * 4 + e];
    rev32[e] = (float)rev[e];
  }
  const bool new_sep = UPDATE ? p.is_sep[b] != 0 : false;

  // ---- counters after the step and the rows' positions
  const Counters c0 = load_counters(c.state + (size_t)bh * 8);
  const Transition tr = transition(c0, c.a, c.s, c.n, UPDATE, new_sep, UPDATE);
  const Counters c1 = tr.after;
  const int total = c1.nsink + c1.sepc + c1.winc;
  int kpos[MAXR];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    const int row = row0 + grp + r * GROUPS;
    const int rk = row < row1 ? row_rank<UPDATE>(row, c0, tr, c.a, c.s, c.n, c.slots) : -1;
    if constexpr (SHIFT) kpos[r] = rk;
    else kpos[r] = rk < 0 ? -1 : (row < c.slots ? spos_r[r] : c1.t - 1);
  }

  // ---- query, rotated at its position, scaled into the log2 domain
  const int qpos = SHIFT ? total - 1 : c1.t - 1;
  float qlo[G][4], qhi[G][4];
  {
    float cv[4], sv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) rope_cs<SHIFT>(qpos, rev[e], rev32[e], cv[e], sv[e]);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x1 = bf2f(qlo_b[h][e]), x2 = bf2f(qhi_b[h][e]);
        qlo[h][e] = (x1 * cv[e] - x2 * sv[e]) * p.scale_log2;
        qhi[h][e] = (x2 * cv[e] + x1 * sv[e]) * p.scale_log2;
      }
  }

  // ---- scores
  float mloc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mloc[h] = -INFINITY;
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    const int pos = kpos[r];
    float part[G];
#pragma unroll
    for (int h = 0; h < G; ++h) part[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float cv, sv;
      rope_cs<SHIFT>(pos < 0 ? 0 : pos, rev[e], rev32[e], cv, sv);
      const float x1 = bf2f(klo[r][e]), x2 = bf2f(khi[r][e]);
      const float y1 = x1 * cv - x2 * sv, y2 = x2 * cv + x1 * sv;
#pragma unroll
      for (int h = 0; h < G; ++h) part[h] += qlo[h][e] * y1 + qhi[h][e] * y2;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float x = group_sum<LPR>(part[h]);
      if (pos < 0) x = -INFINITY;
      part[h] = x;
      mloc[h] = fmaxf(mloc[h], x);
    }
    if (li == 0)
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h][grp + r * GROUPS] = part[h];
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = mloc[h];
    for (int off = LPR; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    if (lane == 0) red[wave][h] = x;
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float m = -INFINITY;
    for (int w = 0; w < NW; ++w) m = fmaxf(m, red[w][threadIdx.x]);
    mstat[threadIdx.x] = m;
  }
  __syncthreads();
  // probabilities, once per (row, head)
  for (int idx = threadIdx.x; idx < G * GROUPS * MAXR; idx += SPLIT_THREADS) {
    const int h = idx / (GROUPS * MAXR), rr = idx % (GROUPS * MAXR);
    sc[h][rr] = fast_exp2(sc[h][rr] - mstat[h]);
  }
  __syncthreads();

  // ---- P V and the probability sum
  float olo[G][4], ohi[G][4], lsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) olo[h][e] = ohi[h][e] = 0.f;
  }
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    if (kpos[r] < 0) continue;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pr = sc[h][grp + r * GROUPS];
      lsum[h] += pr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        olo[h][e] += pr * bf2f(vlo[r][e]);
        ohi[h][e] += pr * bf2f(vhi[r][e]);
      }
    }
  }
  // reduce over the row groups: in-wave by shuffles, then across waves
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = olo[h][e], y = ohi[h][e];
      for (int off = LPR; off < 64; off <<= 1) {
        x += __shfl_xor(x, off, 64);
        y += __shfl_xor(y, off, 64);
      }
      olo[h][e] = x;
      ohi[h][e] = y;
    }
    float l = li == 0 ? lsum[h] : 0.f;
    for (int off = 1; off < 64; off <<= 1) l += __shfl_xor(l, off, 64);
    lsum[h] = l;
  }
  __syncthreads();
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[wave][h][li * 4 + e] = olo[h][e];
        acc[wave][h][HALF + li * 4 + e] = ohi[h][e];
      }
  }
  if (lane == 0)
#pragma unroll
    for (int h = 0; h < G; ++h) red[wave][h] = lsum[h];
  __syncthreads();
  float* out = p.part + ((size_t)bh * p.split + split) * G * (D + 2);
  for (int idx = threadIdx.x; idx < G * (D + 2); idx += SPLIT_THREADS) {
    const int h = idx / (D + 2), dd = idx % (D + 2);
    float v;
    if (dd < D) {
      v = 0.f;
      for (int w = 0; w < NW; ++w) v += acc[w][h][dd];
    } else if (dd == D) {
      v = 0.f;
      for (int w = 0; w < NW; ++w) v += red[w][h];
    } else {
      v = mstat[h];
    }
    out[idx] = v;
  }

  // ---- a step moves the new token and the evicted separator from registers
  if constexpr (UPDATE) {
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      const int row = row0 + grp + r * GROUPS;
      int dst = -1;
      if (row < row1) {
        if (row == c.slots) dst = tr.app_slot;
        else if (row == tr.ev_src) dst = tr.ev_dst;
      }
      if (dst >= 0) {
        bf16* vd = vb + (size_t)dst * D;
        *(bf16x4*)(kb + k_at(dst, li / 2, D / 8) + (li & 1) * 4) = klo[r];
        *(bf16x4*)(kb + k_at(dst, (HALF + li * 4) / 8, D / 8) + (li & 1) * 4) = khi[r];
        *(bf16x4*)(vd + li * 4) = vlo[r];
        *(bf16x4*)(vd + HALF + li * 4) = vhi[r];
      }
    }
  }
}

constexpr int MERGE_THREADS = 256;
constexpr int MERGE_MAXS = 16;  // splits whose partials are requested together

template <int D, int G, bool UPDATE>
__global__ __launch_bounds__(MERGE_THREADS) void attend_merge(AttendParams p) {
  __shared__ float mmax[G], linv[G];
  __shared__ float wgt[MERGE_MAXS][G];
  const CacheParams& c = p.c;
  const int bh = blockIdx.x;
  const int b = bh / c.Hkv, kvh = bh % c.Hkv;
  const float* part = p.part + (size_t)bh * p.split * G * (D + 2);
  const int nsp = min(p.split, MERGE_MAXS);

  // the partials' maxima and sums, all requested at once
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float ms[MERGE_MAXS], ls[MERGE_MAXS];
#pragma unroll
    for (int sp = 0; sp < MERGE_MAXS; ++sp) {
      ms[sp] = sp < nsp ? part[(sp * G + h) * (D + 2) + D + 1] : -INFINITY;
      ls[sp] = sp < nsp ? part[(sp * G + h) * (D + 2) + D] : 0.f;
    }
    float m = -INFINITY;
    for (int sp = 0; sp < p.split; ++sp)
      m = fmaxf(m, sp < MERGE_MAXS ? ms[sp] : part[(sp * G + h) * (D + 2) + D + 1]);
    float l = 0.f;
#pragma unroll
    for (int sp = 0; sp < MERGE_MAXS; ++sp) {
      const float w = ms[sp] == -INFINITY ? 0.f : fast_exp2(ms[sp] - m);
      wgt[sp][h] = w;
      l += w * ls[sp];
    }
    for (int sp = MERGE_MAXS; sp < p.split; ++sp) {
      const float msp = part[(sp * G + h) * (D + 2) + D + 1];
      l += (msp == -INFINITY ? 0.f : fast_exp2(msp - m)) * part[(sp * G + h) * (D + 2) + D];
    }
    mmax[h] = m;
    linv[h] = l > 0.f ? 1.f / l : (l != l ? l : 0.f);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += MERGE_THREADS) {
    const int h = idx / D, dd = idx % D;
    float vals[MERGE_MAXS];
#pragma unroll
    for (int sp = 0; sp < MERGE_MAXS; ++sp) vals[sp] = sp < nsp ? part[(sp * G + h) * (D + 2) + dd] : 0.f;
    float o = 0.f;
#pragma unroll
    for (int sp = 0; sp < MERGE_MAXS; ++sp) o += wgt[sp][h] * vals[sp];
    for (int sp = MERGE_MAXS; sp < p.split; ++sp) {  // very large caches only
      const float msp = part[(sp * G + h) * (D + 2) + D + 1];
      o += (msp == -INFINITY ? 0.f : fast_exp2(msp - mmax[h])) * part[(sp * G + h) * (D + 2) + dd];
    }
    p.o[((size_t)b * p.Hq + kvh * G + h) * D + dd] = (bf16)(o * linv[h]);
  }
  if constexpr (UPDATE) {
    if (threadIdx.x == 0) {
      int32_t* st = c.state + (size_t)bh * 8;
      int32_t* spos = c.slot_pos + (size_t)bh * c.slots;
      uint8_t* ssep = c.slot_sep + (size_t)bh * c.slots;
      const Counters c0 = load_counters(st);
      const bool new_sep = p.is_sep[b] != 0;
      const Transition tr = transition(c0, c.a, c.s, c.n, true, new_sep, true);
      const int ev_pos = tr.evicted ? spos[tr.ev_src] : -1;
      const int new_oldsep = tr.refresh_oldsep ? ssep[c.a + c.s + tr.after.winh] : 0;
      commit(tr, st, spos, ssep, new_sep, ev_pos, new_oldsep);
    }
  }
}

// ---- tiled path
//
// Workgroups of 16 waves; the rows of one (stream, KV head) are cut into
// tiles of 16, held by one workgroup of at most DT_TPW tiles or shared by
// two (larger caches).  Per tile:
//  * scores S = K Q^T on 16x16x32 bf16 MFMAs, keys along the rows: lane
//    (g, col) (g = lane / 16) loads row 16t + col, dimensions 32m + 8g .. +7
//    for m < D/32, so each RoPE pair (i, i + D/2) lies in one lane; query
//    heads along the columns.  S lands as lane (g, h): rows 4g .. 4g+3 of
//    head h, which is also the operand layout P needs below.
//  * O += P V on 16x16x16 bf16 MFMAs: lane (g, c) loads rows 16t + 4g .. +3,
//    dimensions 8c .. 8c+7 and transposes that 4x8 block in registers, so
//    MFMA e takes dimension 8c + e of each column c.
// K/V addresses are physical rows, so every wave issues all its loads right
// after one barrier at entry.  The counters and the row intervals that
// follow from them are computed once, by wave 0, which holds no tile unless
// the others are full; it publishes them in LDS behind a flag that the
// other waves poll.  No barrier sits between the loads and the scores: a
// compute unit keeps only so many loads in flight, so waves that are still
// blocked issuing theirs would hold back those whose data has arrived.  A
// wave keeps the scores of its tiles and takes one maximum over them; the
// waves' (o, sum, max) merge through LDS after the one barrier at the end.
// With two workgroups per (stream, KV head), each writes that triple to the
// workspace and the last to arrive (an atomic ticket per (stream, KV head),
// reset by that workgroup) merges them, writes o and, for a step, commits
// the slot metadata.
//
// RoPE with positions shifted to ranks.  A row's rank is its physical index
// plus an offset that is constant on a few intervals of rows: the sinks, the
// two sides of each ring's wrap point, the evicted row that moves to the
// separator block, and the appended token.  Rotations about the same planes
// compose, so for row 16t + col of interval k, with rank 16t + col + delta_k,
//     R(rank) k . R(p_q) q  =  R(col) k . R(p_q - delta_k - 16t) q.
// Keys turn by their column's angle (a 16-row table in LDS, so a lane's angles
// are the same for all its tiles) and the query by the rest: a wave turns
// its own copy of the query for each (interval, tile) pair it scores, into
// its slice of LDS.  A tile that meets several intervals runs its score
// MFMAs once per interval and keeps each row's own result.  With original
// positions, keys turn by their own angle and the query is one copy.
//
// Rows that hold no entry get probability zero; a non-finite value in such a
// slot would still reach the output through 0 * V in the MFMA, so
// sepcache_reset zeroes every slot and slots only receive tokens' K and V.

constexpr int DT_WAVES = 16;
constexpr int DT_THREADS = 64 * DT_WAVES;
constexpr int DT_ROWS = 16;   // rows per tile
constexpr int DT_MAXT = 2;    // tiles per wave
constexpr int DT_TPW = DT_WAVES * DT_MAXT;  // tiles per workgroup
constexpr int DT_MAX_SPLIT = 2;
constexpr int DT_MAX_ROWS = DT_MAX_SPLIT * DT_TPW * DT_ROWS;
static_assert(DT_MAX_ROWS == 1024, "the tiled decode covers caches of up to 1024 rows");
constexpr int DT_NCLS = 7;    // intervals of constant rank offset
constexpr size_t DT_TICKET_BYTES = 256;            // per 64 (stream, KV head) pairs

typedef short i16x4_t __attribute__((ext_vector_type(4)));

// Row intervals [lo, hi) of constant rank - row = delta; a row of interval k
// holds an entry iff its rank lies in [vlo, vhi).
struct RowClasses {
  int lo[DT_NCLS], hi[DT_NCLS], delta[DT_NCLS], vlo[DT_NCLS], vhi[DT_NCLS];
};

template <bool UPDATE>
__device__ __forceinline__ RowClasses row_classes(const Counters& c0, const Transition& tr, int a, int s, int n,
                                                  int slots) {
  const Counters& c1 = tr.after;
  const int drop = tr.sep_drop ? 1 : 0, ev = tr.evicted ? 1 : 0;
  const int sep0 = a + c0.seph, win0 = a + s + c0.winh;
  const int sep_rank = c1.nsink, win_rank = c1.nsink + c1.sepc;
  const int dsep = sep_rank - sep0 - drop, dwin = win_rank - ev - win0;
  const bool moved = tr.evicted && tr.ev_dst >= 0;
  const bool app = UPDATE && tr.app_slot >= 0;
  const int total = c1.nsink + c1.sepc + c1.winc;
  RowClasses rc;
  // sinks; separator ring past / before its head; window ring past / before
  // its head; the evicted row moving to the separator block; the appended token
  const int lo[DT_NCLS] = {0, a, sep0, a + s, win0 + ev, win0, slots};
  const int hi[DT_NCLS] = {a, sep0, a + s, win0, slots, win0 + (moved ? 1 : 0), slots + (app ? 1 : 0)};
  const int dl[DT_NCLS] = {0, dsep + s, dsep, dwin + n + 1, dwin, win_rank - 1 - win0, total - 1 - slots};
  const int vl[DT_NCLS] = {0, sep_rank, sep_rank, win_rank, win_rank, win_rank - 1, total - 1};
  const int vh[DT_NCLS] = {c0.nsink, sep_rank + c0.sepc - drop, sep_rank + c0.sepc - drop,
                           win_rank + c0.winc - ev, win_rank + c0.winc - ev, win_rank, total};
#pragma unroll
  for (int k = 0; k < DT_NCLS; ++k) {
    rc.lo[k] = lo[k];
    rc.hi[k] = hi[k];
    rc.delta[k] = dl[k];
    rc.vlo[k] = vl[k];
    rc.vhi[k] = vh[k];
  }
  return rc;
}

__device__ __forceinline__ float lo_bf(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf(float x, float y) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(bf16)x, (bf16)y};
  return __builtin_bit_cast(uint32_t, v);
}

// max(x[l], x[l ^ 16]): v_permlane16_swap exchanges the odd 16-lane rows of
// its first register with the even rows of its second.
__device__ __forceinline__ float max_xor16(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

// Workspace of the tiled path: tickets, then [B * Hkv][split][G][D + 2]
// partials (o, sum, max).
__host__ __device__ inline size_t dt_ticket_bytes(int bh) {
  return ((size_t)bh * 4 + DT_TICKET_BYTES - 1) / DT_TICKET_BYTES * DT_TICKET_BYTES;
}

// What a wave needs before it issues its loads comes as leading scalar
// arguments, which the dispatcher preloads into registers (the struct is read
// from memory): dims0 = B * Hkv | Hkv << 16 | workgroups per pair << 24,
// dims1 = slots | Hq << 16.
template <int D, int G, bool UPDATE, bool SHIFT>
__global__ __launch_bounds__(DT_THREADS) void decode_tiles(const int32_t* state, bf16* kc, bf16* vc, const bf16* qg,
                                                           const uint8_t* is_sep, uint32_t dims0, uint32_t dims1,
                                                           float rev_log2_step, AttendParams p) {
  constexpr int NM = D / 32;  // score MFMAs per tile (k = 32 dimensions each)
  constexpr int NP = NM / 2;  // chunks m < NP pair with m + NP
  constexpr int NCH = D / 8;  // 16-byte chunks per row
  constexpr int HALF = D / 2;
  constexpr int QSTR = D + 8;  // LDS row of one head of a query copy; the pad spreads banks
  constexpr int TSTR = HALF + 2;  // LDS row of the column angles, likewise
  // each wave's query copy and output (apart, so that a wave writes its
  // output while others still score)
  __shared__ __attribute__((aligned(16))) bf16 qc_all[DT_WAVES * G * QSTR];
  __shared__ __attribute__((aligned(16))) float o_w[DT_WAVES][G][D];
  __shared__ __attribute__((aligned(16))) float2 tcol[SHIFT ? DT_ROWS * TSTR : 1];
  __shared__ __attribute__((aligned(16))) u32x4 newrow[2][NCH];  // appended token's K and V (step)
  __shared__ float m_w[DT_WAVES][G], l_w[DT_WAVES][G];
  // published by wave 0: per interval, the rows [x, y) that hold an entry and
  // rank - row (z); then the query position and the rows that move
  __shared__ __attribute__((aligned(16))) int4 cls_tab[8];
  __shared__ int info[4];
  __shared__ double rev_lds[SHIFT ? 1 : HALF];
  __shared__ int ready, last_s;

  const CacheParams& c = p.c;
  const int BH = (int)(dims0 & 0xffffu), Hkv = (int)((dims0 >> 16) & 0xffu), nsplit = (int)(dims0 >> 24);
  const int Hq = (int)(dims1 >> 16);
  const int bh = blockIdx.x % BH, split = blockIdx.x / BH;  // splits of one pair are BH apart
  const int b = bh / Hkv, kvh = bh % Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: tile branches stay scalar
  const int g = lane >> 4, col = lane & 15;
  const int slots = (int)(dims1 & 0xffffu);
  const int rows = slots + (UPDATE ? 1 : 0);
  const int n_tiles = (rows + DT_ROWS - 1) / DT_ROWS;
  const int tps = (n_tiles + nsplit - 1) / nsplit;
  const int t_lo = split * tps, t_hi = min(t_lo + tps, n_tiles);  // this workgroup's tiles
  const uint32_t row_bytes = D * 2;
  bf16* kb = kc + (size_t)bh * sepcache_k_rows_of(slots) * D;
  bf16* vb = vc + (size_t)bh * slots * D;
  const bool lead = wave == 0;

  // ---- the counters (lane i: word i) and the separator flag go out first,
  // as vector loads: a scalar load would be waited for by every later wait
  // on a kernel argument or an LDS access
  // (every wave issues them, so that no load is conditional: the waits on
  // the loads after them stay counted)
  const int st_l = bld4(make_rsrc(state + (size_t)bh * 8, 32), lane < 8 ? (uint32_t)lane * 4u : BUF_OOB);
  const int is_sep_b = UPDATE ? (int)is_sep[b] : 0;
  if (tid == 0) ready = 0;
  // the column angles (shifted positions): no memory involved
  if constexpr (SHIFT) {
    for (int idx = tid; idx < DT_ROWS * HALF; idx += DT_THREADS) {
      const int i = idx % HALF;
      float cs, sn;
      rope_cs<true>(idx / HALF, 0.0, fast_exp2((float)i * rev_log2_step) * 0.15915494309189535f, cs, sn);
      tcol[(idx / HALF) * TSTR + i] = make_float2(cs, sn);
    }
  }
  // the only barrier before the merge (the waves start together).  A bare
  // barrier after an LDS-only wait: __syncthreads' fence would also wait for
  // the loads just issued.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---- loads: the query (lane l < D/2: dimensions 2l, 2l + 1 of each head,
  // so that lane l ^ D/4 holds their RoPE partners), its frequencies, then the
  // K/V tiles.  Tiles go, from the last down, to waves 1, 2, ..., 15 in
  // turn, and to wave 0, which does the counters, only once those are full.
  // In a step the last tile, which holds the appended token's row, is wave
  // 1's first in the last workgroup; wave 1 stages that row through LDS, one
  // 16-byte chunk per lane.
  constexpr int QL = HALF / 2;
  uint32_t q_own[G];
  {
    const rsrc_t qrs = make_rsrc(qg + ((size_t)b * Hq + kvh * G) * D, G * D * 2);
#pragma unroll
    for (int h = 0; h < G; ++h) q_own[h] = (uint32_t)bld4(qrs, lane < HALF ? (uint32_t)(h * D + 2 * lane) * 2u : BUF_OOB);
  }
  const int fi = 2 * (lane % QL);  // this lane's frequencies fi, fi + 1
  const double rv0 = p.rev[fi], rv1 = p.rev[fi + 1];
  auto tile_of = [&](int j) {
    const int k = lead ? (DT_WAVES - 1) * DT_MAXT + j : (DT_WAVES - 1) * j + wave - 1;
    const int t = t_hi - 1 - k;
    return t >= t_lo ? t : -1;
  };
  const bool holds_new = UPDATE && wave == 1 && t_hi == n_tiles;
  u32x4 nk, nv;
  const rsrc_t krs = make_rsrc(kb, (uint32_t)sepcache_k_rows_of(slots) * row_bytes);
  const rsrc_t vrs = make_rsrc(vb, (uint32_t)slots * row_bytes);
  const rsrc_t prs = make_rsrc(c.slot_pos + (size_t)bh * slots, (uint32_t)slots * 4);
  // (the tile rows are read once per step, with the non-temporal hint: the
  // other layers' caches pass through the caches before this one is read
  // again; measured 9.04 -> 8.78 us per layer-token on the Llama step)
  u32x4 kr[DT_MAXT][NM], vr[DT_MAXT][4];
  int spos[DT_MAXT];
  // An absent tile (t = -1) sets the offsets' top bit arithmetically rather
  // than by a select, so the compiler neither branches on it nor merges the
  // identical loads it would produce (either would put a wait here).
#pragma unroll
  for (int j = 0; j < DT_MAXT; ++j) {
    const int t = tile_of(j);
    const uint32_t absent = (uint32_t)(t >> 31) & BUF_OOB;
    const int krow = t * DT_ROWS + col;
#pragma unroll
    for (int m = 0; m < NM; ++m)  // tile-major K: 1 KB contiguous per load; rows past the slots read as zeros
      kr[j][m] = bld16_nt(krs, ((uint32_t)(t * DT_ROWS) * row_bytes + (uint32_t)(((4 * m + g) << 4) + col) * 16) |
                                   absent | (((uint32_t)(slots - 1 - krow) >> 31) << 31));
    if constexpr (!SHIFT) spos[j] = bld4(prs, ((uint32_t)krow * 4) | absent);
  }
  // The scores need only K, so every K tile goes out before any V tile: a
  // wait for a tile's K then covers no V load (measured 8.79 -> 8.68 us per
  // layer-token on the Llama step).  The appended row's pointers come from
  // the struct, so its loads wait for that read; after the K tiles, the wait
  // holds back no K load.
  if (holds_new) {
    nk = bld16(make_rsrc(p.k_new + (size_t)bh * D, row_bytes), lane < NCH ? lane * 16 : BUF_OOB);
    nv = bld16(make_rsrc(p.v_new + (size_t)bh * D, row_bytes),
               lane >= 32 && lane - 32 < NCH ? (lane - 32) * 16 : BUF_OOB);
  }
#pragma unroll
  for (int j = 0; j < DT_MAXT; ++j) {
    const int t = tile_of(j);
    const uint32_t absent = (uint32_t)(t >> 31) & BUF_OOB;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      vr[j][u] = bld16_nt(vrs, col < NCH ? ((uint32_t)(t * DT_ROWS + 4 * g + u) * row_bytes + col * 16) | absent : BUF_OOB);
  }

  // ---- wave 0: the counters after the step and the row intervals,
  // published in LDS
  // used by the commit only (thread 0, in wave 0): no defaults on the other
  // waves' path, which would make wave 0 wait here for the loads below
  int ev_pos, new_oldsep;
  Transition tr;
  bool new_sep;
  if (lead) {
    if constexpr (!SHIFT) {
      if (lane < HALF) rev_lds[lane] = p.rev[lane];
    }
    Counters c0;
    c0.t = __builtin_amdgcn_readlane(st_l, ST_T);
    c0.nsink = __builtin_amdgcn_readlane(st_l, ST_NSINK);
    c0.seph = __builtin_amdgcn_readlane(st_l, ST_SEPH);
    c0.sepc = __builtin_amdgcn_readlane(st_l, ST_SEPC);
    c0.winh = __builtin_amdgcn_readlane(st_l, ST_WINH);
    c0.winc = __builtin_amdgcn_readlane(st_l, ST_WINC);
    c0.flags = __builtin_amdgcn_readlane(st_l, ST_FLAGS);
    c0.oldsep = __builtin_amdgcn_readlane(st_l, ST_OLDSEP);
    new_sep = __builtin_amdgcn_readfirstlane(is_sep_b) != 0;
    tr = transition(c0, c.a, c.s, c.n, UPDATE, new_sep, UPDATE);
    const Counters& c1 = tr.after;
    const RowClasses rc = row_classes<UPDATE>(c0, tr, c.a, c.s, c.n, slots);
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < DT_NCLS; ++k)
        cls_tab[k] = make_int4(max(rc.lo[k], rc.vlo[k] - rc.delta[k]), min(rc.hi[k], rc.vhi[k] - rc.delta[k]),
                               rc.delta[k], 0);
      cls_tab[DT_NCLS] = make_int4(0, 0, 0, 0);
      // shifted: the query's rank; original positions: its position
      info[0] = SHIFT ? c1.nsink + c1.sepc + c1.winc - 1 : c1.t - 1;
      info[1] = UPDATE ? tr.app_slot : -1;
      info[2] = UPDATE ? tr.ev_src : -1;
      info[3] = UPDATE ? tr.ev_dst : -1;
    }
    // the LDS writes above complete before the flag (an LDS wait only: the
    // tile loads stay in flight)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    if (lane == 0) __hip_atomic_store(&ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if constexpr (UPDATE) {
      // read by the commit at the end; vector loads, so nothing here waits for them
      ev_pos = bld4(prs, tr.evicted ? (uint32_t)tr.ev_src * 4u : BUF_OOB);
      new_oldsep = (int)__builtin_amdgcn_raw_buffer_load_b8(
          make_rsrc(c.slot_sep + (size_t)bh * slots, (uint32_t)slots),
          tr.refresh_oldsep ? (uint32_t)(c.a + c.s + c1.winh) : BUF_OOB, 0, 0);
    }
  } else {
    // wave 0 always sets the flag, so this wait ends
    while (__hip_atomic_load(&ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int4 ct = cls_tab[lane & 7];  // lanes k < 7: interval k
  const int q_pos = __builtin_amdgcn_readfirstlane(info[0]);
  const int app_slot = __builtin_amdgcn_readfirstlane(info[1]);
  const int ev_src = __builtin_amdgcn_readfirstlane(info[2]);
  const int ev_dst = __builtin_amdgcn_readfirstlane(info[3]);

  // ---- this wave's query copy: turned to `pos`, scaled into the log2
  // domain; lane l < D/2 writes dimensions 2l, 2l + 1 of each head.  Lanes
  // l < D/4 hold the first element x1 of their pairs, lanes D/4 <= l < D/2
  // the second x2:   y1 = x1 cos - x2 sin,   y2 = x2 cos + x1 sin.
  bf16* const qc = qc_all + wave * (G * QSTR);
  uint32_t q_oth[G];
#pragma unroll
  for (int h = 0; h < G; ++h) q_oth[h] = (uint32_t)__shfl_xor((int)q_own[h], QL, 64);
  const float sgn = (lane & QL) ? p.scale_log2 : -p.scale_log2;
  auto build_copy = [&](int pos) {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // after the previous pass's reads
    float cs0, sn0, cs1, sn1;
    rope_cs<SHIFT>(pos, rv0, (float)rv0, cs0, sn0);
    rope_cs<SHIFT>(pos, rv1, (float)rv1, cs1, sn1);
    cs0 *= p.scale_log2;
    cs1 *= p.scale_log2;
    sn0 *= sgn;
    sn1 *= sgn;
    if (lane < HALF)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float y0 = lo_bf(q_own[h]) * cs0 + lo_bf(q_oth[h]) * sn0;
        const float y1 = hi_bf(q_own[h]) * cs1 + hi_bf(q_oth[h]) * sn1;
        *(uint32_t*)(qc + h * QSTR + 2 * lane) = pack_bf(y0, y1);
      }
    // read back by this wave only: its LDS accesses complete in order
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  if constexpr (!SHIFT) build_copy(q_pos);

  // this lane's key angles (shifted positions): column col, frequencies
  // i = 32 m + 8 g + e, m < NP
  const float2* kcs = tcol + col * TSTR + 8 * g;

  // ---- scores of this wave's tiles
  f32x4 sco[DT_MAXT];
#pragma unroll
  for (int j = 0; j < DT_MAXT; ++j) {
    const int t = tile_of(j);
    sco[j] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (t < 0) continue;
    const int row0 = t * DT_ROWS;
    const int krow = row0 + col;
    if (j == 0 && holds_new) {  // rows past the cache read as zeros; fill row `slots`
      if (lane < NCH) newrow[0][lane] = nk;
      if (lane >= 32 && lane - 32 < NCH) newrow[1][lane - 32] = nv;
      if (krow == slots)
#pragma unroll
        for (int m = 0; m < NM; ++m) kr[0][m] = newrow[0][4 * m + g];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (row0 + 4 * g + u == slots && col < NCH) vr[0][u] = newrow[1][col];
    }

    if constexpr (UPDATE) {  // rows that move: raw K/V to their new slots
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int src = w == 0 ? slots : ev_src;
        const int dst = w == 0 ? app_slot : ev_dst;
        if (dst >= 0 && src >= row0 && src < row0 + DT_ROWS) {
          if (krow == src)
#pragma unroll
            for (int m = 0; m < NM; ++m) st16(kb + k_at(dst, 4 * m + g, NCH), kr[j][m]);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (row0 + 4 * g + u == src && col < NCH) st16(vb + (size_t)dst * D + col * 8, vr[j][u]);
        }
      }
    }

    // K turned: pairs (m, e) and (m + NP, e), packed chunk pair by chunk pair
    bf16x8 ka[NM];
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      u32x4 w1o, w2o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float y1[2], y2[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int e = 2 * q + h2;
          const uint32_t w1 = kr[j][m][q], w2 = kr[j][m + NP][q];
          const float x1 = h2 ? hi_bf(w1) : lo_bf(w1);
          const float x2 = h2 ? hi_bf(w2) : lo_bf(w2);
          float cs, sn;
          if constexpr (SHIFT) {
            const float2 a = kcs[32 * m + e];
            cs = a.x;
            sn = a.y;
          } else {
            const int pos = krow == slots ? q_pos : spos[j];
            rope_cs<false>(pos, rev_lds[32 * m + 8 * g + e], 0.f, cs, sn);
          }
          y1[h2] = x1 * cs - x2 * sn;
          y2[h2] = x2 * cs + x1 * sn;
        }
        w1o[q] = pack_bf(y1[0], y1[1]);
        w2o[q] = pack_bf(y2[0], y2[1]);
      }
      ka[m] = __builtin_bit_cast(bf16x8, w1o);
      ka[m + NP] = __builtin_bit_cast(bf16x8, w2o);
    }

    // the tile's rows per interval (lanes k < 7), one pass per interval it
    // meets: each row keeps its own interval's score, rows that hold no
    // entry keep -inf
    const int lo = max(ct.x, row0) - row0, hi = min(ct.y, row0 + DT_ROWS) - row0;
    const uint32_t mk = (lane < DT_NCLS && hi > lo) ? (((1u << hi) - 1u) & ~((1u << lo) - 1u)) : 0u;
    f32x4 s = sco[j];
    auto pass = [&](uint32_t rows_mask) {
      const bf16* qv = qc + (col & (G - 1)) * QSTR;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const bf16x8 qb = *(const bf16x8*)(qv + (4 * m + g) * 8);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[m], qb, acc, 0, 0, 0);
      }
      const uint32_t mine = rows_mask >> (4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if ((mine >> r) & 1u) s[r] = acc[r];
    };
    if constexpr (SHIFT) {
      uint64_t todo = __builtin_amdgcn_ballot_w64(mk != 0);
      while (todo) {
        const int k = (int)__builtin_ctzll(todo);
        todo &= todo - 1;
        const uint32_t mkk = (uint32_t)__builtin_amdgcn_readlane((int)mk, k);
        // rank = row + delta_k, so row 16t + col turns by col and the query by the rest
        build_copy(q_pos - __builtin_amdgcn_readlane(ct.z, k) - row0);
        pass(mkk);
      }
    } else {
      uint32_t all = 0;
#pragma unroll
      for (int k = 0; k < DT_NCLS; ++k) all |= (uint32_t)__builtin_amdgcn_readlane((int)mk, k);
      if (all) pass(all);
    }
    sco[j] = s;
  }

  // ---- this wave's maximum per head (lanes (g, h) hold head h)
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < DT_MAXT; ++j) mx = fmaxf(mx, fmaxf(fmaxf(sco[j][0], sco[j][1]), fmaxf(sco[j][2], sco[j][3])));
  mx = max_xor16(mx);
  mx = max_xor32(mx);
  const float mu = mx == -INFINITY ? 0.f : mx;

  // ---- P V
  f32x4 oacc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) oacc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
#pragma unroll
  for (int j = 0; j < DT_MAXT; ++j) {
    if (tile_of(j) < 0) continue;
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = fast_exp2(sco[j][r] - mu);
      lsum += pr[r];
    }
    const u32x2 pw = {pack_bf(pr[0], pr[1]), pack_bf(pr[2], pr[3])};
    const i16x4_t pa = __builtin_bit_cast(i16x4_t, pw);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const u32x2 vw = {__builtin_amdgcn_perm(vr[j][1][e >> 1], vr[j][0][e >> 1], sel),
                        __builtin_amdgcn_perm(vr[j][3][e >> 1], vr[j][2][e >> 1], sel)};
      oacc[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, __builtin_bit_cast(i16x4_t, vw), oacc[e], 0, 0, 0);
    }
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);

  // ---- merge the waves, then the workgroups of this (stream, KV head)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * g + r;
    if (h < G && col < NCH)
#pragma unroll
      for (int e = 0; e < 8; ++e) o_w[wave][h][8 * col + e] = oacc[e][r];
  }
  if (g == 0 && col < G) {
    m_w[wave][col] = mx;
    l_w[wave][col] = lsum;
  }
  __syncthreads();
  bf16* out = p.o + ((size_t)b * Hq + kvh * G) * D;
  // (max, sum, o) of output (h, d) over the waves.  The 64 lanes of a wave
  // hold 64 consecutive d of one head (D >= 64), so lane l computes the
  // factor of wave l % DT_WAVES once and the others read it.
  auto merge_waves = [&](int h, int d, float& M, float& L, float& O) {
    const int wl = lane % DT_WAVES;
    const float mw = m_w[wl][h];
    M = group_max<DT_WAVES>(mw);
    const float f = M == -INFINITY ? 0.f : fast_exp2(mw - M);
    L = group_sum<DT_WAVES>(f * l_w[wl][h]);
    O = 0.f;
#pragma unroll
    for (int w = 0; w < DT_WAVES; ++w)
      O += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), w)) * o_w[w][h][d];
  };
  if (nsplit == 1) {
    for (int idx = tid; idx < G * D; idx += DT_THREADS) {
      float M, L, O;
      merge_waves(idx / D, idx % D, M, L, O);
      out[idx] = (bf16)(L > 0.f ? O / L : 0.f);
    }
  } else {
    int* ticket = (int*)p.part;
    float* part = (float*)((char*)p.part + dt_ticket_bytes(BH)) + (size_t)bh * nsplit * G * (D + 2);
    for (int idx = tid; idx < G * D; idx += DT_THREADS) {
      const int h = idx / D, d = idx % D;
      float M, L, O;
      merge_waves(h, d, M, L, O);
      // the partials and the ticket are agent-scope atomics: they are
      // performed at the device's coherence point, with no cache-wide
      // write-back or invalidation
      float* ps = part + ((size_t)split * G + h) * (D + 2);
      __hip_atomic_store(ps + d, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d == 0) {
        __hip_atomic_store(ps + D, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ps + D + 1, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // every store of this workgroup has completed (reached the coherence
    // point) before the ticket is taken; the fence keeps the compiler from
    // moving them past the wait
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const int seen = __hip_atomic_fetch_add(ticket + bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = seen == nsplit - 1;
      if (last) __hip_atomic_store(ticket + bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_s = last;
    }
    __syncthreads();
    if (!last_s) return;
    auto rd = [](const float* x) { return __hip_atomic_load(x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    for (int idx = tid; idx < G * D; idx += DT_THREADS) {
      const int h = idx / D, d = idx % D;
      float ms[DT_MAX_SPLIT], ls[DT_MAX_SPLIT], os[DT_MAX_SPLIT];
      float M = -INFINITY;
#pragma unroll
      for (int sp = 0; sp < DT_MAX_SPLIT; ++sp) {
        if (sp < nsplit) {
          const float* ps = part + ((size_t)sp * G + h) * (D + 2);
          ms[sp] = rd(ps + D + 1);
          ls[sp] = rd(ps + D);
          os[sp] = rd(ps + d);
        } else {
          ms[sp] = -INFINITY;
          ls[sp] = os[sp] = 0.f;
        }
        M = fmaxf(M, ms[sp]);
      }
      float L = 0.f, O = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int sp = 0; sp < DT_MAX_SPLIT; ++sp) {
          const float f = fast_exp2(ms[sp] - M);
          L += f * ls[sp];
          O += f * os[sp];
        }
      }
      out[idx] = (bf16)(L > 0.f ? O / L : 0.f);
    }
  }
  if constexpr (UPDATE) {
    // every workgroup of this (stream, KV head) read the old metadata before
    // its ticket (or, with one workgroup, before the barrier above); thread 0
    // belongs to wave 0, which holds the step's transition
    if (tid == 0) {
      // opaque here, so that the compiler keeps the commit's selects on these
      // loaded values down here instead of waiting for the loads early
      asm volatile("" : "+v"(ev_pos), "+v"(new_oldsep));
      commit(tr, c.state + (size_t)bh * 8, c.slot_pos + (size_t)bh * slots, c.slot_sep + (size_t)bh * slots,
             new_sep, ev_pos, new_oldsep);
    }
  }
}

// Tiled path: workgroups per (stream, KV head), 0 if the cache is too large.
int dt_split(int rows) {
  const int n_tiles = (rows + DT_ROWS - 1) / DT_ROWS;
  const int sp = (n_tiles + DT_TPW - 1) / DT_TPW;
  return sp <= DT_MAX_SPLIT ? sp : 0;
}

int attend_rows(const sepcache* c, bool update) { return make_params(c).slots + (update ? 1 : 0); }
// Workgroups per (stream, KV head) of the tiled path, 0 if it does not apply:
// the cache is too large, or a size does not fit the kernel's packed
// arguments (B * Hkv, slots and Hq in 16 bits, Hkv in 8).
int tiled_split(const sepcache* c, int Hq, bool update) {
  if (c->B * c->Hkv >= 65536 || c->Hkv >= 256 || Hq >= 65536) return 0;
  return dt_split(attend_rows(c, update));
}
// split path: workgroups per (stream, KV head)
int attend_split(const sepcache* c, bool update) {
  const int per_split = SPLIT_THREADS / (c->d / 8) * SPLIT_MAXR;
  return (attend_rows(c, update) + per_split - 1) / per_split;
}

template <int D, int G, bool UPDATE, bool SHIFT>
void launch_attend_t(const AttendParams& p, hipStream_t st) {
  if (p.tiled) {
    const uint32_t dims0 = (uint32_t)(p.c.B * p.c.Hkv) | (uint32_t)p.c.Hkv << 16 | (uint32_t)p.split << 24;
    const uint32_t dims1 = (uint32_t)p.c.slots | (uint32_t)p.Hq << 16;
    hipLaunchKernelGGL((decode_tiles<D, G, UPDATE, SHIFT>), dim3(p.c.B * p.c.Hkv * p.split), dim3(DT_THREADS), 0,
                       st, p.c.state, p.c.k, p.c.v, p.q, p.is_sep, dims0, dims1, p.rev_log2_step, p);
  } else {
    hipLaunchKernelGGL((attend_part<D, G, UPDATE, SHIFT>), dim3(p.c.B * p.c.Hkv * p.split), dim3(SPLIT_THREADS), 0,
                       st, p);
    hipLaunchKernelGGL((attend_merge<D, G, UPDATE>), dim3(p.c.B * p.c.Hkv), dim3(MERGE_THREADS), 0, st, p);
  }
}

template <int D, int G>
int launch_attend(const AttendParams& p, bool update, hipStream_t st) {
  if (update) {
    if (p.shift) launch_attend_t<D, G, true, true>(p, st);
    else launch_attend_t<D, G, true, false>(p, st);
  } else {
    if (p.shift) launch_attend_t<D, G, false, true>(p, st);
    else launch_attend_t<D, G, false, false>(p, st);
  }
  return sepattn_hip_check(hipGetLastError(), update ? "step launch" : "decode launch");
}

int dispatch_attend(const AttendParams& p, int G, bool update, hipStream_t st) {
#define SEPATTN_DISPATCH_G(DD)                                 \
  switch (G) {                                                 \
    case 1: return launch_attend<DD, 1>(p, update, st);        \
    case 2: return launch_attend<DD, 2>(p, update, st);        \
    case 4: return launch_attend<DD, 4>(p, update, st);        \
    case 8: return launch_attend<DD, 8>(p, update, st);        \
    default: return sepattn_fail(SEPATTN_ENOTSUP, "decode: %d q heads per KV head", G); \
  }
  if (p.c.d == 128) { SEPATTN_DISPATCH_G(128) }
  SEPATTN_DISPATCH_G(64)
#undef SEPATTN_DISPATCH_G
}

AttendParams attend_params(const sepcache* c, int Hq, const void* q, float scale, int shift, void* o, void* ws,
                           bool update) {
  AttendParams p;
  p.c = make_params(c);
  p.q = (const bf16*)q; p.o = (bf16*)o;
  p.k_new = p.v_new = nullptr; p.is_sep = nullptr;
  p.Hq = Hq; p.shift = shift;
  const int sp = tiled_split(c, Hq, update);
  p.tiled = sp > 0;
  p.split = p.tiled ? sp : attend_split(c, update);
  // both paths keep the tickets' area, so one workspace serves either
  p.part = (float*)ws;
  if (!p.tiled && ws) p.part = (float*)((char*)ws + dt_ticket_bytes(c->B * c->Hkv));
  p.scale_log2 = scale * 1.4426950408889634f;
  p.rev_log2_step = (float)(-2.0 * log2((double)c->theta) / c->d);
  const RopeFreqs f = rope_freqs(c);
  for (int i = 0; i < MAX_HALF; ++i) p.rev[i] = f.rev[i];
  return p;
}

}  // namespace

int sepcache_launch_reset(const sepcache* c, hipStream_t st) {
  hipLaunchKernelGGL(reset_kernel, dim3(c->B * c->Hkv), dim3(256), 0, st, make_params(c));
  return sepattn_hip_check(hipGetLastError(), "reset launch");
}

int sepcache_launch_prefill(const sepcache* c, const void* k, const void* v, const int64_t* ks, const int64_t* vs,
                            const sepattn_mask* m, hipStream_t st) {
  const CacheParams cp = make_params(c);
  const int wgs = (cp.slots * (c->d / 8) + PF_CHUNKS - 1) / PF_CHUNKS;  // per (stream, KV head)
  hipLaunchKernelGGL(prefill_kernel, dim3(c->B * c->Hkv, wgs), dim3(PF_THREADS), 0, st, cp, (const bf16*)k,
                     (const bf16*)v, ks[0], ks[1], ks[2], vs[0], vs[1], vs[2], m->L, (const uint8_t*)m->is_sep,
                     (const int32_t*)m->sep_idx, (const int32_t*)m->sep_before);
  return sepattn_hip_check(hipGetLastError(), "prefill launch");
}

// With a past window, an append first flushes a full window queue.
static int launch_flush(const sepcache* c, hipStream_t st) {
  if (past_entries(c) == 0) return SEPATTN_OK;
  hipLaunchKernelGGL(flush_kernel, dim3(c->B * c->Hkv), dim3(64), 0, st, make_params(c));
  return sepattn_hip_check(hipGetLastError(), "flush launch");
}

int sepcache_launch_update(const sepcache* c, const void* k_new, const void* v_new, const uint8_t* is_sep,
                           int do_append, int do_evict, hipStream_t st) {
  if (do_append) SEPATTN_TRY(launch_flush(c, st));
  hipLaunchKernelGGL(update_kernel, dim3(c->B * c->Hkv), dim3(64), 0, st, make_params(c), (const bf16*)k_new,
                     (const bf16*)v_new, is_sep, do_append, do_evict);
  return sepattn_hip_check(hipGetLastError(), "update launch");
}

size_t sepcache_decode_ws_bytes(const sepcache* c, int Hq) {
  const size_t BH = (size_t)c->B * c->Hkv, G = Hq / c->Hkv;
  size_t need = 0;
  for (int update = 0; update < 2; ++update) {
    const int sp = tiled_split(c, Hq, update);
    size_t b;
    if (sp == 1) b = 0;
    else if (sp > 1) b = dt_ticket_bytes((int)BH) + BH * sp * G * (c->d + 2) * 4;
    else b = dt_ticket_bytes((int)BH) + BH * attend_split(c, update) * G * (c->d + 2) * 4;
    need = need > b ? need : b;
  }
  return need;
}

int sepcache_launch_decode(const sepcache* c, int Hq, const void* q, float scale, int shift, void* o, void* ws,
                           hipStream_t st) {
  const AttendParams p = attend_params(c, Hq, q, scale, shift, o, ws, false);
  return dispatch_attend(p, Hq / c->Hkv, false, st);
}

int sepcache_launch_step(const sepcache* c, const void* k_new, const void* v_new, const uint8_t* is_sep, int Hq,
                         const void* q, float scale, int shift, void* o, void* ws, hipStream_t st) {
  SEPATTN_TRY(launch_flush(c, st));
  AttendParams p = attend_params(c, Hq, q, scale, shift, o, ws, true);
  p.k_new = (const bf16*)k_new; p.v_new = (const bf16*)v_new; p.is_sep = is_sep;
  return dispatch_attend(p, Hq / c->Hkv, true, st);
}

int sepcache_launch_export(const sepcache* c, int32_t* pos, int32_t* len, hipStream_t st) {
  hipLaunchKernelGGL(export_kernel, dim3(c->B), dim3(256), 0, st, make_params(c), pos, len);
  return sepattn_hip_check(hipGetLastError(), "export launch");
}
