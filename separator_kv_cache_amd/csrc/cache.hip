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

struct CacheParams {
  bf16* k;
  bf16* v;
  int32_t* slot_pos;
  uint8_t* slot_sep;
  int32_t* state;
  int B, Hkv, d, a, s, n, slots;
};

CacheParams make_params(const sepcache* c) {
  CacheParams p;
  p.k = (bf16*)c->k; p.v = (bf16*)c->v;
  p.slot_pos = c->slot_pos; p.slot_sep = c->slot_sep; p.state = c->state;
  p.B = c->B; p.Hkv = c->Hkv; p.d = c->d; p.a = c->a; p.s = c->s; p.n = c->n;
  p.slots = c->a + c->s + c->n + 1;
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

__global__ void reset_kernel(CacheParams p) {
  const size_t bh = blockIdx.x;
  for (int i = threadIdx.x; i < p.slots; i += blockDim.x) {
    p.slot_pos[bh * p.slots + i] = -1;
    p.slot_sep[bh * p.slots + i] = 0;
  }
  if (threadIdx.x < 8) p.state[bh * 8 + threadIdx.x] = 0;
}

// Copies one row (d elements of K and of V) with the workgroup's threads.
__device__ __forceinline__ void copy_row(int d, const bf16* ks, const bf16* vs, bf16* kd, bf16* vd) {
  const int ch = d / 8;
  for (int i = threadIdx.x; i < 2 * ch; i += blockDim.x) {
    if (i < ch) st16(kd + i * 8, ld16(ks + i * 8));
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
  bf16* kb = p.k + (size_t)bh * p.slots * p.d;
  bf16* vb = p.v + (size_t)bh * p.slots * p.d;
  if (tr.app_slot >= 0)
    copy_row(p.d, k_new + (size_t)bh * p.d, v_new + (size_t)bh * p.d, kb + (size_t)tr.app_slot * p.d,
             vb + (size_t)tr.app_slot * p.d);
  if (tr.ev_dst >= 0)
    copy_row(p.d, kb + (size_t)tr.ev_src * p.d, vb + (size_t)tr.ev_src * p.d, kb + (size_t)tr.ev_dst * p.d,
             vb + (size_t)tr.ev_dst * p.d);
  __syncthreads();
  if (threadIdx.x == 0) commit(tr, st, spos, ssep, new_sep, ev_pos, new_oldsep);
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
// Two kernels per decode (or step):
//  * attend_part: workgroup = (stream, KV head, split) over at most 64 (d=128)
//    or 128 (d=64) rows.  Rows are the physical slots plus, for a step, one
//    virtual row holding the new token (read from the inputs).  A group of
//    D/8 lanes takes one row; lane li holds dimensions [4li, 4li+4) and their
//    RoPE partners [D/2 + 4li, D/2 + 4li + 4).  Every load is issued before
//    the counters are used (none of the addresses depends on them), and RoPE
//    angles are computed in the kernel, so a split costs one memory round
//    trip.  Each split writes its (o, sum, max) partial; for a step, the
//    lanes holding the new token and the evicted separator also write those
//    rows to their new slots (slots no other split needs in this step).
//  * attend_merge: workgroup = (stream, KV head): merges the partials in split
//    order and writes o; for a step it then commits slot metadata and
//    counters.

constexpr int SPLIT_THREADS = 256;   // split path: rows per split = 256/(d/8) * 4
constexpr int SPLIT_MAXR = 4;
constexpr int FUSED_THREADS = 512;   // fused path: up to 512/(d/8) * 12 rows
constexpr int FUSED_MAXR = 12;
constexpr int MAX_HALF = 64;    // d/2 for d = 128

struct AttendParams {
  CacheParams c;
  const bf16* q;
  bf16* o;
  const bf16* k_new;
  const bf16* v_new;
  const uint8_t* is_sep;
  float* part;  // [B, Hkv, split, G, D + 2]: o, sum, max
  int Hq, shift, split;
  float scale_log2;
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

// FUSED: one workgroup holds every row of its (stream, KV head) (split ==
// 1): it normalises and writes o itself and, for a step, commits the slot
// metadata and counters after its last read of them.
template <int D, int G, bool UPDATE, bool SHIFT, int NT, int MAXR, bool FUSED>
__global__ __launch_bounds__(NT) void attend_part(AttendParams p) {
  constexpr int AT_THREADS = NT;
  constexpr int AT_MAXR = MAXR;
  constexpr int LPR = D / 8;
  constexpr int GROUPS = AT_THREADS / LPR;
  constexpr int HALF = D / 2;
  constexpr int NW = AT_THREADS / 64;
  __shared__ float sc[G][GROUPS * AT_MAXR];
  __shared__ float red[NW][G];
  __shared__ float mstat[G];
  __shared__ float acc[NW][G][D];

  const CacheParams& c = p.c;
  const int split = blockIdx.x % p.split;
  const int bh = blockIdx.x / p.split;
  const int b = bh / c.Hkv, kvh = bh % c.Hkv;
  const int li = threadIdx.x % LPR, grp = threadIdx.x / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  bf16* kb = c.k + (size_t)bh * c.slots * D;
  bf16* vb = c.v + (size_t)bh * c.slots * D;
  const int rows = c.slots + (UPDATE ? 1 : 0);
  const int per = (rows + p.split - 1) / p.split;
  const int row0 = split * per, row1 = min(rows, row0 + per);

  // ---- every load first: slot positions (no shift), K/V rows, queries
  int spos_r[AT_MAXR];
  if constexpr (!SHIFT) {
#pragma unroll
    for (int r = 0; r < AT_MAXR; ++r)
      spos_r[r] = c.slot_pos[(size_t)bh * c.slots + min(row0 + grp + r * GROUPS, c.slots - 1)];
  }
  bf16x4 klo[AT_MAXR], khi[AT_MAXR], vlo[AT_MAXR], vhi[AT_MAXR];
#pragma unroll
  for (int r = 0; r < AT_MAXR; ++r) {
    const int row = min(row0 + grp + r * GROUPS, rows - 1);
    const bool cached = row < c.slots;
    const bf16* ks = cached ? kb + (size_t)row * D : p.k_new + (size_t)bh * D;
    const bf16* vs = cached ? vb + (size_t)row * D : p.v_new + (size_t)bh * D;
    klo[r] = *(const bf16x4*)(ks + li * 4);
    khi[r] = *(const bf16x4*)(ks + HALF + li * 4);
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
  const int W = c.n + 1;
  // offsets within a ring without integer division: x lies in (-m, m)
  auto wrap = [](int x, int m) { return x < 0 ? x + m : x; };
  auto rank_of = [&](int row) -> int {
    if (row >= c.slots) return (UPDATE && tr.app_slot >= 0) ? total - 1 : -1;  // the new token
    if (row < c.a) return row < c0.nsink ? row : -1;
    if (row < c.a + c.s) {
      const int off = wrap(row - c.a - c0.seph, c.s);
      if (off >= c0.sepc) return -1;
      if (tr.sep_drop) return off == 0 ? -1 : c1.nsink + off - 1;
      return c1.nsink + off;
    }
    const int off = wrap(row - c.a - c.s - c0.winh, W);
    if (off >= c0.winc) return -1;
    if (tr.evicted) {
      if (off == 0) return tr.ev_dst >= 0 ? c1.nsink + c1.sepc - 1 : -1;
      return c1.nsink + c1.sepc + off - 1;
    }
    return c1.nsink + c1.sepc + off;
  };
  int ev_pos = -1, new_oldsep = 0;
  if constexpr (FUSED && UPDATE) {
    if (threadIdx.x == 0) {
      if (tr.evicted) ev_pos = c.slot_pos[(size_t)bh * c.slots + tr.ev_src];
      if (tr.refresh_oldsep) new_oldsep = c.slot_sep[(size_t)bh * c.slots + c.a + c.s + c1.winh];
    }
  }
  int kpos[AT_MAXR];
#pragma unroll
  for (int r = 0; r < AT_MAXR; ++r) {
    const int row = row0 + grp + r * GROUPS;
    const int rk = row < row1 ? rank_of(row) : -1;
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
  for (int r = 0; r < AT_MAXR; ++r) {
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
  for (int idx = threadIdx.x; idx < G * GROUPS * AT_MAXR; idx += AT_THREADS) {
    const int h = idx / (GROUPS * AT_MAXR), rr = idx % (GROUPS * AT_MAXR);
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
  for (int r = 0; r < AT_MAXR; ++r) {
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
  if constexpr (FUSED) {
    for (int idx = threadIdx.x; idx < G * D; idx += AT_THREADS) {
      const int h = idx / D, dd = idx % D;
      float v = 0.f, l = 0.f;
      for (int w = 0; w < NW; ++w) {
        v += acc[w][h][dd];
        l += red[w][h];
      }
      p.o[((size_t)b * p.Hq + kvh * G + h) * D + dd] = (bf16)(l > 0.f ? v / l : 0.f);
    }
  }
  float* out = p.part + ((size_t)bh * p.split + split) * G * (D + 2);
  for (int idx = threadIdx.x; !FUSED && idx < G * (D + 2); idx += AT_THREADS) {
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
    for (int r = 0; r < AT_MAXR; ++r) {
      const int row = row0 + grp + r * GROUPS;
      int dst = -1;
      if (row < row1) {
        if (row == c.slots) dst = tr.app_slot;
        else if (row == tr.ev_src) dst = tr.ev_dst;
      }
      if (dst >= 0) {
        bf16* kd = kb + (size_t)dst * D;
        bf16* vd = vb + (size_t)dst * D;
        *(bf16x4*)(kd + li * 4) = klo[r];
        *(bf16x4*)(kd + HALF + li * 4) = khi[r];
        *(bf16x4*)(vd + li * 4) = vlo[r];
        *(bf16x4*)(vd + HALF + li * 4) = vhi[r];
      }
    }
    if constexpr (FUSED) {
      // every read of the old metadata (ranks, positions) happened before the
      // barriers above; thread 0 holds the two values the commit needs
      if (threadIdx.x == 0)
        commit(tr, c.state + (size_t)bh * 8, c.slot_pos + (size_t)bh * c.slots, c.slot_sep + (size_t)bh * c.slots,
               new_sep, ev_pos, new_oldsep);
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

int attend_rows(const sepcache* c, bool update) { return c->a + c->s + c->n + 1 + (update ? 1 : 0); }
bool attend_fused(const sepcache* c, bool update) {
  return attend_rows(c, update) <= FUSED_THREADS / (c->d / 8) * FUSED_MAXR;
}
int attend_split(const sepcache* c, bool update) {
  if (attend_fused(c, update)) return 1;
  const int per_split = SPLIT_THREADS / (c->d / 8) * SPLIT_MAXR;
  return (attend_rows(c, update) + per_split - 1) / per_split;
}

template <int D, int G, bool UPDATE, bool SHIFT>
void launch_attend_t(const AttendParams& p, bool fused, hipStream_t st) {
  if (fused) {
    hipLaunchKernelGGL((attend_part<D, G, UPDATE, SHIFT, FUSED_THREADS, FUSED_MAXR, true>),
                       dim3(p.c.B * p.c.Hkv), dim3(FUSED_THREADS), 0, st, p);
  } else {
    hipLaunchKernelGGL((attend_part<D, G, UPDATE, SHIFT, SPLIT_THREADS, SPLIT_MAXR, false>),
                       dim3(p.c.B * p.c.Hkv * p.split), dim3(SPLIT_THREADS), 0, st, p);
    hipLaunchKernelGGL((attend_merge<D, G, UPDATE>), dim3(p.c.B * p.c.Hkv), dim3(MERGE_THREADS), 0, st, p);
  }
}

template <int D, int G>
int launch_attend(const AttendParams& p, bool update, hipStream_t st) {
  const bool fused = p.split == 1;
  if (update) {
    if (p.shift) launch_attend_t<D, G, true, true>(p, fused, st);
    else launch_attend_t<D, G, true, false>(p, fused, st);
  } else {
    if (p.shift) launch_attend_t<D, G, false, true>(p, fused, st);
    else launch_attend_t<D, G, false, false>(p, fused, st);
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
  p.part = (float*)ws;
  p.Hq = Hq; p.shift = shift;
  p.split = attend_split(c, update);
  p.scale_log2 = scale * 1.4426950408889634f;
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < MAX_HALF; ++i)
    p.rev[i] = i < c->d / 2 ? pow((double)c->theta, -2.0 * i / c->d) / two_pi : 0.0;
  return p;
}

}  // namespace

int sepcache_launch_reset(const sepcache* c, hipStream_t st) {
  hipLaunchKernelGGL(reset_kernel, dim3(c->B * c->Hkv), dim3(256), 0, st, make_params(c));
  return sepattn_hip_check(hipGetLastError(), "reset launch");
}

int sepcache_launch_update(const sepcache* c, const void* k_new, const void* v_new, const uint8_t* is_sep,
                           int do_append, int do_evict, hipStream_t st) {
  hipLaunchKernelGGL(update_kernel, dim3(c->B * c->Hkv), dim3(64), 0, st, make_params(c), (const bf16*)k_new,
                     (const bf16*)v_new, is_sep, do_append, do_evict);
  return sepattn_hip_check(hipGetLastError(), "update launch");
}

size_t sepcache_decode_ws_bytes(const sepcache* c, int Hq) {
  const int split = attend_split(c, true);  // the larger of the two
  if (split == 1 && attend_split(c, false) == 1) return 0;
  return (size_t)c->B * c->Hkv * split * (Hq / c->Hkv) * (c->d + 2) * 4;
}

int sepcache_launch_decode(const sepcache* c, int Hq, const void* q, float scale, int shift, void* o, void* ws,
                           hipStream_t st) {
  const AttendParams p = attend_params(c, Hq, q, scale, shift, o, ws, false);
  return dispatch_attend(p, Hq / c->Hkv, false, st);
}

int sepcache_launch_step(const sepcache* c, const void* k_new, const void* v_new, const uint8_t* is_sep, int Hq,
                         const void* q, float scale, int shift, void* o, void* ws, hipStream_t st) {
  AttendParams p = attend_params(c, Hq, q, scale, shift, o, ws, true);
  p.k_new = (const bf16*)k_new; p.v_new = (const bf16*)v_new; p.is_sep = is_sep;
  return dispatch_attend(p, Hq / c->Hkv, true, st);
}

int sepcache_launch_export(const sepcache* c, int32_t* pos, int32_t* len, hipStream_t st) {
  hipLaunchKernelGGL(export_kernel, dim3(c->B), dim3(256), 0, st, make_params(c), pos, len);
  return sepattn_hip_check(hipGetLastError(), "export launch");
}
