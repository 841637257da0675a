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
// Physical slots of a stream: [0, a) sinks, [a, a+s) separator ring,
// [a+s, a+s+n+1) window ring (one spare slot holds the appended token until
// eviction).  All KV heads of a stream share the slot structure.
#include "common.h"

namespace {

enum { ST_T = 0, ST_NSINK, ST_SEPH, ST_SEPC, ST_WINH, ST_WINC, ST_FLAGS, ST_RES };
constexpr int FLAG_WINDOW_OVERFLOW = 1;

struct CacheParams {
  bf16* k;
  bf16* v;
  int32_t* slot_pos;
  uint8_t* slot_sep;
  int32_t* state;
  const float* rope;
  int rope_len;
  int B, Hkv, d, a, s, n, slots;
};

CacheParams make_params(const sepcache* c) {
  CacheParams p;
  p.k = (bf16*)c->k; p.v = (bf16*)c->v;
  p.slot_pos = c->slot_pos; p.slot_sep = c->slot_sep; p.state = c->state;
  p.rope = c->rope; p.rope_len = c->rope_len;
  p.B = c->B; p.Hkv = c->Hkv; p.d = c->d; p.a = c->a; p.s = c->s; p.n = c->n;
  p.slots = c->a + c->s + c->n + 1;
  return p;
}

__global__ void reset_kernel(CacheParams p) {
  const int b = blockIdx.x;
  for (int i = threadIdx.x; i < p.slots; i += blockDim.x) {
    p.slot_pos[(size_t)b * p.slots + i] = -1;
    p.slot_sep[(size_t)b * p.slots + i] = 0;
  }
  if (threadIdx.x < 8) p.state[b * 8 + threadIdx.x] = 0;
}

// Copies row `src` (or the new token) to row `dst` of every KV head of stream b.
__device__ __forceinline__ void copy_rows(const CacheParams& p, int b, const bf16* src_k, const bf16* src_v,
                                          int64_t src_head_stride, int dst) {
  const int chunks = p.d / 8;  // 16-byte chunks per row
  const int total = p.Hkv * chunks;
  for (int i = threadIdx.x; i < 2 * total; i += blockDim.x) {
    const bool isv = i >= total;
    const int ii = isv ? i - total : i;
    const int h = ii / chunks, c = ii % chunks;
    const bf16* src = (isv ? src_v : src_k) + (int64_t)h * src_head_stride + c * 8;
    bf16* dstp = (isv ? p.v : p.k) + (((size_t)b * p.Hkv + h) * p.slots + dst) * p.d + c * 8;
    st16(dstp, ld16(src));
  }
}

// One workgroup per stream: append the new token, then evict (either step
// optional).  Every thread reads the counters first; thread 0 writes the new
// counters and slot metadata after a barrier.
__global__ __launch_bounds__(256) void update_kernel(CacheParams p, const bf16* k_new, const bf16* v_new,
                                                     const uint8_t* is_sep, int do_append, int do_evict) {
  const int b = blockIdx.x;
  int32_t* st = p.state + b * 8;
  int t = st[ST_T], nsink = st[ST_NSINK], seph = st[ST_SEPH], sepc = st[ST_SEPC];
  int winh = st[ST_WINH], winc = st[ST_WINC], flags = st[ST_FLAGS];
  int32_t* spos = p.slot_pos + (size_t)b * p.slots;
  uint8_t* ssep = p.slot_sep + (size_t)b * p.slots;
  const int W = p.n + 1;  // window ring capacity

  int app_slot = -1, app_flag = 0;
  if (do_append) {
    if (t < p.a) {
      app_slot = t;
      nsink = t + 1;
    } else if (winc <= p.n) {
      app_slot = p.a + p.s + (winh + winc) % W;
      ++winc;
    } else {
      flags |= FLAG_WINDOW_OVERFLOW;  // append without evict: token dropped
    }
    if (app_slot >= 0) {
      app_flag = is_sep[b] ? 1 : 0;
      const int64_t hs = p.d;  // k_new [B, Hkv, d]
      copy_rows(p, b, k_new + (size_t)b * p.Hkv * p.d, v_new + (size_t)b * p.Hkv * p.d, hs, app_slot);
      ++t;
    }
  }
  int ev_src = -1, ev_dst = -1, ev_pos = -1;
  if (do_evict && winc > p.n) {
    ev_src = p.a + p.s + winh;
    const bool sep = ev_src == app_slot ? app_flag : ssep[ev_src] != 0;
    ev_pos = spos[ev_src];
    if (sep && p.s > 0) {
      if (sepc < p.s) {
        ev_dst = p.a + (seph + sepc) % p.s;
        ++sepc;
      } else {
        ev_dst = p.a + seph;
        seph = (seph + 1) % p.s;
      }
      const int64_t hs = (int64_t)p.slots * p.d;
      copy_rows(p, b, p.k + ((size_t)b * p.Hkv * p.slots + ev_src) * p.d,
                p.v + ((size_t)b * p.Hkv * p.slots + ev_src) * p.d, hs, ev_dst);
    }
    winh = (winh + 1) % W;
    --winc;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (app_slot >= 0) {
      spos[app_slot] = t - 1;
      ssep[app_slot] = (uint8_t)app_flag;
    }
    if (ev_src >= 0) {
      if (ev_dst >= 0) {
        spos[ev_dst] = ev_pos;
        ssep[ev_dst] = 1;
      }
      spos[ev_src] = -1;
      ssep[ev_src] = 0;
    }
    st[ST_T] = t; st[ST_NSINK] = nsink; st[ST_SEPH] = seph; st[ST_SEPC] = sepc;
    st[ST_WINH] = winh; st[ST_WINC] = winc; st[ST_FLAGS] = flags;
  }
}

// Logical rank of physical slot `p` (or -1 if empty).
__device__ __forceinline__ int slot_rank(int slot, int a, int s, int n, int nsink, int seph, int sepc, int winh,
                                         int winc) {
  if (slot < a) return slot < nsink ? slot : -1;
  if (slot < a + s) {
    const int off = (slot - a - seph + s) % s;
    return off < sepc ? nsink + off : -1;
  }
  const int off = (slot - a - s - winh + (n + 1)) % (n + 1);
  return off < winc ? nsink + sepc + off : -1;
}

__global__ void export_kernel(CacheParams p, int32_t* pos, int32_t* len) {
  const int b = blockIdx.x;
  const int32_t* st = p.state + b * 8;
  const int nsink = st[ST_NSINK], seph = st[ST_SEPH], sepc = st[ST_SEPC], winh = st[ST_WINH], winc = st[ST_WINC];
  const int cap = p.a + p.s + p.n;
  for (int i = threadIdx.x; i < cap; i += blockDim.x) pos[(size_t)b * cap + i] = -1;
  __syncthreads();
  for (int slot = threadIdx.x; slot < p.slots; slot += blockDim.x) {
    const int r = slot_rank(slot, p.a, p.s, p.n, nsink, seph, sepc, winh, winc);
    if (r >= 0 && r < cap) pos[(size_t)b * cap + r] = p.slot_pos[(size_t)b * p.slots + slot];
  }
  if (threadIdx.x == 0) len[b] = nsink + sepc + winc;
}

// ---------------------------------------------------------------- decode
//
// Workgroup = (stream b, KV head, split).  Each 16-lane group of a wave
// handles one slot (row) at a time; lane li holds dimensions [4li, 4li+4) and
// their RoPE partners [d/2 + 4li, d/2 + 4li + 4) of K, V and the G queries.
// Pass 1 scores every row of the split, pass 2 accumulates P V; partials
// (max, sum, o) of the splits are merged by the last workgroup to finish.

constexpr int DEC_THREADS = 256;
constexpr int DEC_MAXR = 4;  // rows per 16-lane group per split
constexpr int DEC_ROWS = DEC_THREADS / 16 * DEC_MAXR;  // rows per split (d = 128)

struct DecodeParams {
  CacheParams c;
  const bf16* q;
  bf16* o;
  float* part;       // [B, Hkv, split, G, d + 2]
  int32_t* counter;  // [B, Hkv]
  int Hq, G, split, shift;
  float scale_log2;
};

template <int D, int G>
__global__ __launch_bounds__(DEC_THREADS) void decode_kernel(DecodeParams p) {
  constexpr int LPR = D / 8;                 // lanes per row
  constexpr int GROUPS = DEC_THREADS / LPR;  // rows in flight per pass
  constexpr int HALF = D / 2;
  __shared__ float sc[G][GROUPS * DEC_MAXR];
  __shared__ float red[DEC_THREADS / 64][G];
  __shared__ float stat[2][G];
  __shared__ int last_flag;

  const CacheParams& c = p.c;
  const int split = blockIdx.x % p.split;
  const int kvh = (blockIdx.x / p.split) % c.Hkv;
  const int b = blockIdx.x / (p.split * c.Hkv);
  const int li = threadIdx.x % LPR, grp = threadIdx.x / LPR;
  const int32_t* st = c.state + b * 8;
  const int t = st[ST_T], nsink = st[ST_NSINK], seph = st[ST_SEPH], sepc = st[ST_SEPC];
  const int winh = st[ST_WINH], winc = st[ST_WINC];
  const int total = nsink + sepc + winc;
  const int rows_per = (c.slots + p.split - 1) / p.split;
  const int row0 = split * rows_per, row1 = min(c.slots, row0 + rows_per);

  // query position and rotated queries (fp32) for this lane's 8 dims
  const int qpos = p.shift ? total - 1 : t - 1;
  const bool qpos_ok = qpos >= 0 && qpos < c.rope_len;
  float qlo[G][4], qhi[G][4];
  {
    const float* cs = c.rope + (size_t)(qpos_ok ? qpos : 0) * HALF * 2 + li * 8;
    const f32x4 c01 = *(const f32x4*)cs, c23 = *(const f32x4*)(cs + 4);
    const float cosv[4] = {c01[0], c01[2], c23[0], c23[2]}, sinv[4] = {c01[1], c01[3], c23[1], c23[3]};
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const bf16* qr = p.q + ((size_t)b * p.Hq + kvh * G + h) * D;
      const bf16x4 lo = *(const bf16x4*)(qr + li * 4), hi = *(const bf16x4*)(qr + HALF + li * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x1 = bf2f(lo[e]), x2 = bf2f(hi[e]);
        qlo[h][e] = (x1 * cosv[e] - x2 * sinv[e]) * p.scale_log2;
        qhi[h][e] = (x2 * cosv[e] + x1 * sinv[e]) * p.scale_log2;
      }
    }
  }

  // ---- loads: K, V and rank for this lane's rows
  const bf16* kb = c.k + ((size_t)b * c.Hkv + kvh) * c.slots * D;
  const bf16* vb = c.v + ((size_t)b * c.Hkv + kvh) * c.slots * D;
  const int32_t* spos = c.slot_pos + (size_t)b * c.slots;
  bf16x4 klo[DEC_MAXR], khi[DEC_MAXR], vlo[DEC_MAXR], vhi[DEC_MAXR];
  int kpos[DEC_MAXR];
#pragma unroll
  for (int r = 0; r < DEC_MAXR; ++r) {
    const int slot = row0 + grp + r * GROUPS;
    int rank = -1;
    if (slot < row1) rank = slot_rank(slot, c.a, c.s, c.n, nsink, seph, sepc, winh, winc);
    kpos[r] = rank < 0 ? -1 : (p.shift ? rank : spos[slot]);
    if (rank >= 0) {
      klo[r] = *(const bf16x4*)(kb + (size_t)slot * D + li * 4);
      khi[r] = *(const bf16x4*)(kb + (size_t)slot * D + HALF + li * 4);
      vlo[r] = *(const bf16x4*)(vb + (size_t)slot * D + li * 4);
      vhi[r] = *(const bf16x4*)(vb + (size_t)slot * D + HALF + li * 4);
    }
  }

  // ---- pass 1: scores (log2 domain) of every row, kept in LDS
  float mloc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mloc[h] = -INFINITY;
#pragma unroll
  for (int r = 0; r < DEC_MAXR; ++r) {
    float part[G];
#pragma unroll
    for (int h = 0; h < G; ++h) part[h] = 0.f;
    const int pos = kpos[r];
    if (pos >= 0) {
      const int pp = pos < c.rope_len ? pos : 0;
      const float* cs = c.rope + (size_t)pp * HALF * 2 + li * 8;
      const f32x4 c01 = *(const f32x4*)cs, c23 = *(const f32x4*)(cs + 4);
      const float cosv[4] = {c01[0], c01[2], c23[0], c23[2]}, sinv[4] = {c01[1], c01[3], c23[1], c23[3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x1 = bf2f(klo[r][e]), x2 = bf2f(khi[r][e]);
        const float y1 = x1 * cosv[e] - x2 * sinv[e], y2 = x2 * cosv[e] + x1 * sinv[e];
#pragma unroll
        for (int h = 0; h < G; ++h) part[h] += qlo[h][e] * y1 + qhi[h][e] * y2;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float x = part[h];
#pragma unroll
      for (int off = 1; off < LPR; off <<= 1) x += __shfl_xor(x, off, 64);
      if (pos < 0) x = -INFINITY;
      if (pos >= c.rope_len || !qpos_ok) x = NAN;  // position outside the RoPE table
      part[h] = x;
      mloc[h] = fmaxf(mloc[h], x);
    }
    if (li == 0)
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h][grp + r * GROUPS] = part[h];
  }
  // workgroup max per head
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = mloc[h];
    for (int off = 32; off >= LPR; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    if (lane == 0) red[wave][h] = x;
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float m = -INFINITY;
    for (int w = 0; w < DEC_THREADS / 64; ++w) m = fmaxf(m, red[w][threadIdx.x]);
    stat[0][threadIdx.x] = m;
  }
  __syncthreads();

  // ---- pass 2: P V
  float olo[G][4], ohi[G][4], lsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) olo[h][e] = ohi[h][e] = 0.f;
  }
#pragma unroll
  for (int r = 0; r < DEC_MAXR; ++r) {
    if (kpos[r] < 0) continue;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m = stat[0][h];
      const float pr = fast_exp2(sc[h][grp + r * GROUPS] - (m == -INFINITY ? 0.f : m));
      lsum[h] += pr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        olo[h][e] += pr * bf2f(vlo[r][e]);
        ohi[h][e] += pr * bf2f(vhi[r][e]);
      }
    }
  }
  // reduce over the row groups through LDS
  float* outp = p.part + ((((size_t)b * c.Hkv + kvh) * p.split + split) * G) * (D + 2);
  __shared__ float acc[GROUPS][G][D + 1];
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[grp][h][li * 4 + e] = olo[h][e];
      acc[grp][h][HALF + li * 4 + e] = ohi[h][e];
    }
  if (li == 0)
#pragma unroll
    for (int h = 0; h < G; ++h) acc[grp][h][D] = lsum[h];
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * (D + 1); idx += DEC_THREADS) {
    const int h = idx / (D + 1), dd = idx % (D + 1);
    float s = 0.f;
    for (int g2 = 0; g2 < GROUPS; ++g2) s += acc[g2][h][dd];
    if (p.split == 1) {
      // single split: normalise and write the output directly
      acc[0][h][dd] = s;
    } else {
      outp[h * (D + 2) + dd] = s;  // o[0..D), l at D
      if (dd == 0) outp[h * (D + 2) + D + 1] = stat[0][h];
    }
  }
  if (p.split == 1) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += DEC_THREADS) {
      const int h = idx / D, dd = idx % D;
      const float l = acc[0][h][D];
      p.o[((size_t)b * p.Hq + kvh * G + h) * D + dd] = (bf16)(l > 0.f ? acc[0][h][dd] / l : 0.f);
    }
    return;
  }
  // ---- last workgroup of this (stream, KV head) merges the splits
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(p.counter + b * c.Hkv + kvh, 1);
    last_flag = prev == p.split - 1;
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  const float* base = p.part + (((size_t)b * c.Hkv + kvh) * p.split) * G * (D + 2);
  for (int idx = threadIdx.x; idx < G * D; idx += DEC_THREADS) {
    const int h = idx / D, dd = idx % D;
    float m = -INFINITY;
    for (int sp = 0; sp < p.split; ++sp) m = fmaxf(m, __builtin_nontemporal_load(base + (sp * G + h) * (D + 2) + D + 1));
    const float mu = m == -INFINITY ? 0.f : m;
    float l = 0.f, o = 0.f;
    for (int sp = 0; sp < p.split; ++sp) {
      const float* pp = base + (sp * G + h) * (D + 2);
      const float w = fast_exp2(__builtin_nontemporal_load(pp + D + 1) - mu);
      l += w * __builtin_nontemporal_load(pp + D);
      o += w * __builtin_nontemporal_load(pp + dd);
    }
    p.o[((size_t)b * p.Hq + kvh * G + h) * D + dd] = (bf16)(l > 0.f ? o / l : 0.f);
  }
  if (threadIdx.x == 0) p.counter[b * c.Hkv + kvh] = 0;
}

int decode_split(const sepcache* c) {
  const int slots = c->a + c->s + c->n + 1;
  const int rows_per_split = DEC_ROWS * 128 / c->d;  // GROUPS * MAXR
  return (slots + rows_per_split - 1) / rows_per_split;
}

template <int D, int G>
int launch_decode(const DecodeParams& p, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<D, G>), dim3(p.c.B * p.c.Hkv * p.split), dim3(DEC_THREADS), 0, st, p);
  return sepattn_hip_check(hipGetLastError(), "decode launch");
}

}  // namespace

int sepcache_launch_reset(const sepcache* c, hipStream_t st) {
  hipLaunchKernelGGL(reset_kernel, dim3(c->B), dim3(256), 0, st, make_params(c));
  return sepattn_hip_check(hipGetLastError(), "reset launch");
}

int sepcache_launch_update(const sepcache* c, const void* k_new, const void* v_new, const uint8_t* is_sep,
                           int do_append, int do_evict, hipStream_t st) {
  hipLaunchKernelGGL(update_kernel, dim3(c->B), dim3(256), 0, st, make_params(c), (const bf16*)k_new,
                     (const bf16*)v_new, is_sep, do_append, do_evict);
  return sepattn_hip_check(hipGetLastError(), "update launch");
}

size_t sepcache_decode_ws_bytes(const sepcache* c, int Hq) {
  const int split = decode_split(c);
  const int G = Hq / c->Hkv;
  const size_t part = (size_t)c->B * c->Hkv * split * G * (c->d + 2) * 4;
  const size_t counters = (size_t)c->B * c->Hkv * 4;
  return ((part + 255) & ~(size_t)255) + counters;
}

int sepcache_launch_decode(const sepcache* c, int Hq, const void* q, float scale, int shift, void* o, void* ws,
                           hipStream_t st) {
  DecodeParams p;
  p.c = make_params(c);
  p.q = (const bf16*)q;
  p.o = (bf16*)o;
  p.Hq = Hq;
  p.G = Hq / c->Hkv;
  p.split = decode_split(c);
  p.shift = shift;
  p.scale_log2 = scale * 1.4426950408889634f;
  const size_t part = (size_t)c->B * c->Hkv * p.split * p.G * (c->d + 2) * 4;
  p.part = (float*)ws;
  p.counter = (int32_t*)((char*)ws + ((part + 255) & ~(size_t)255));
  const int G = p.G;
#define DISPATCH(DD)                                       \
  switch (G) {                                             \
    case 1: return launch_decode<DD, 1>(p, st);            \
    case 2: return launch_decode<DD, 2>(p, st);            \
    case 4: return launch_decode<DD, 4>(p, st);            \
    case 8: return launch_decode<DD, 8>(p, st);            \
    default: return sepattn_fail(SEPATTN_ENOTSUP, "decode: %d q heads per KV head", G); \
  }
  if (c->d == 128) { DISPATCH(128) }
  DISPATCH(64)
#undef DISPATCH
}

int sepcache_launch_export(const sepcache* c, int32_t* pos, int32_t* len, hipStream_t st) {
  hipLaunchKernelGGL(export_kernel, dim3(c->B), dim3(256), 0, st, make_params(c), pos, len);
  return sepattn_hip_check(hipGetLastError(), "export launch");
}
