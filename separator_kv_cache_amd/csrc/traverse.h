// Key traversal of one query tile under the SepLLM mask.
//
// The mask (anthology record LIT-748, "Key takeaways", mask bullet; pith.science
// key_machinery (i)-(iii)) keeps, for query i, key j <= i when j < a (sink),
// i - j < n (window, the query included) or token j is a separator.
//
// For a tile of rows [q0, q0 + rows) let band_lo = max(0, q0 - n + 1).  A key
// j < band_lo is outside the window of every row of the tile, so the tile sees
// it iff it is a sink or a separator, and then every row sees it.  Those keys
// are a prefix of one ascending list: sinks 0..min(a, band_lo)-1 followed by
// the separators sep_idx[0 .. sep_before[band_lo]).  Keys in [band_lo,
// band_hi) form the band, where the element test decides.
#pragma once

#include "common.h"

struct TileKeys {
  int band_lo, band_hi;  // band [band_lo, band_hi)
  int n_sink;            // gathered sinks: keys 0 .. n_sink-1
  int n_gather;          // gathered keys: n_sink sinks then separators
};

__device__ __forceinline__ TileKeys tile_keys(int q0, int rows, int L, int a, int n,
                                              const int32_t* __restrict__ sep_before_b) {
  TileKeys t;
  t.band_lo = max(0, q0 - n + 1);
  t.band_hi = min(L, q0 + rows);
  t.n_sink = min(a, t.band_lo);
  t.n_gather = t.n_sink + sep_before_b[t.band_lo];
  return t;
}

// Key position of gathered entry c (c < n_gather).
__device__ __forceinline__ int gather_key(int c, int n_sink, const int32_t* __restrict__ sep_idx_b) {
  return c < n_sink ? c : sep_idx_b[c - n_sink];
}

// Element test of the band.
__device__ __forceinline__ bool band_keep(int i, int j, int a, int n, const uint8_t* __restrict__ is_sep_b) {
  return j <= i && (j < a || i - j < n || is_sep_b[j] != 0);
}

// Keys per key tile of the query-major kernels (forward, dQ).
constexpr int KTILE = 64;

// Bits [0, x) set, x clamped to [0, 64].
__device__ __forceinline__ uint64_t below64(int x) {
  return x <= 0 ? 0ull : x >= 64 ? ~0ull : ((1ull << x) - 1ull);
}

// The key tiles of one query tile: tiles [0, n_gt) hold the gathered keys,
// tiles [n_gt, n_tiles) the band.  A thread that moves tile rows rows[u]
// asks keys() for their key positions (-1: absent row, past the end).  The
// sep_idx entries of a gathered tile must have been fetched by issue_idx() at
// least one step earlier, so that no load waits on another inside a loop.
// Loads use buffer resources: an absent row costs neither a branch nor
// memory traffic.
template <int PT>
struct KeyStream {
  TileKeys tk;
  int n_gt, n_tiles;
  rsrc_t irs, frs;
  int raw[PT];

  __device__ __forceinline__ void init(int q0, int rows, int L, int a, int n, const int32_t* sep_before_b,
                                       const int32_t* sep_idx_b, const uint8_t* is_sep_b) {
    tk = tile_keys(q0, rows, L, a, n, sep_before_b);
    n_gt = (tk.n_gather + KTILE - 1) / KTILE;
    n_tiles = n_gt + (tk.band_hi - tk.band_lo + KTILE - 1) / KTILE;
    irs = make_rsrc(sep_idx_b, (uint32_t)L * 4u);
    frs = make_rsrc(is_sep_b, (uint32_t)L);
  }
  __device__ __forceinline__ void issue_idx(int t, const int (&rows)[PT]) {
    if (t < n_gt) {
#pragma unroll
      for (int u = 0; u < PT; ++u) {
        const int c = t * KTILE + rows[u] - tk.n_sink;
        raw[u] = bld4(irs, c >= 0 && c < tk.n_gather - tk.n_sink ? (uint32_t)c * 4u : BUF_OOB);
      }
    }
  }
  __device__ __forceinline__ void keys(int t, const int (&rows)[PT], int (&key)[PT]) const {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      if (t < n_gt) {
        const int c = t * KTILE + rows[u];
        key[u] = c < tk.n_sink ? c : (c < tk.n_gather ? raw[u] : -1);
      } else {
        const int j = tk.band_lo + (t - n_gt) * KTILE + rows[u];
        key[u] = j < tk.band_hi ? j : -1;
      }
    }
  }
  // is_sep of row r of tile t (band tiles; 0 for gathered ones).
  __device__ __forceinline__ uint32_t flag_byte(int t, int r) const {
    return t >= n_gt ? __builtin_amdgcn_raw_buffer_load_b8(frs, tk.band_lo + (t - n_gt) * KTILE + r, 0, 0) : 0u;
  }
  // Whether every key of tile t is kept for rows [r0, r0 + 32).
  __device__ __forceinline__ bool full(int t, int r0, int n) const {
    if (t < n_gt) return (t + 1) * KTILE <= tk.n_gather;
    const int k0 = tk.band_lo + (t - n_gt) * KTILE;
    return (k0 + KTILE <= tk.band_hi) && (k0 + KTILE - 1 <= r0) && (r0 + 31 - k0 < n);
  }
  // Bit kl: key kl of tile t is kept for query row `row`; sep_bits holds the
  // separator flags of a band tile.
  __device__ __forceinline__ uint64_t keep64(int t, int row, int a, int n, uint64_t sep_bits) const {
    if (t < n_gt) return below64(tk.n_gather - t * KTILE);
    const int k0 = tk.band_lo + (t - n_gt) * KTILE;
    const int d = row - k0;  // key kl lies d - kl positions before the row
    const uint64_t causal = below64(min(d, tk.band_hi - 1 - k0) + 1);
    const uint64_t window = ~below64(d - n + 1);
    const uint64_t sinks = below64(a - k0);
    return causal & (window | sinks | sep_bits);
  }
};

// One 64-row tile of a [., D] matrix of T moving global -> registers -> LDS.
// Thread x handles 16-byte chunk x % CH of rows x / CH + u * (NT / CH); a row
// whose key is < 0 loads as zeros.
template <typename T, int D, int NT>
struct RowMover {
  static constexpr int CH = D * (int)sizeof(T) / 16;
  static constexpr int ROWS_PER_PASS = NT / CH;
  static constexpr int PT = KTILE / ROWS_PER_PASS;
  static_assert(NT % CH == 0 && KTILE % ROWS_PER_PASS == 0, "tile chunks must divide the workgroup");
  u32x4 r[PT];

  __device__ static int chunk() { return (int)threadIdx.x % CH; }
  __device__ static void rows(int (&rw)[PT]) {
#pragma unroll
    for (int u = 0; u < PT; ++u) rw[u] = (int)threadIdx.x / CH + u * ROWS_PER_PASS;
  }
  __device__ __forceinline__ void load(rsrc_t rs, uint32_t row_bytes, const int (&key)[PT]) {
#pragma unroll
    for (int u = 0; u < PT; ++u)
      r[u] = bld16(rs, key[u] >= 0 ? (uint32_t)key[u] * row_bytes + chunk() * 16 : BUF_OOB);
  }
  // SWZ: chunk c of row r goes to chunk position c ^ ((r >> 2) & 3) (the
  // reader applies the same map).
  template <int STR, bool SWZ = false>
  __device__ __forceinline__ void store(T* dst) const {
    const int r0 = (int)threadIdx.x / CH;
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int row = r0 + u * ROWS_PER_PASS;
      const int pos = SWZ ? chunk() ^ ((row >> 2) & 3) : chunk();
      st16((char*)(dst + row * STR) + pos * 16, r[u]);
    }
  }
};

// Puts -inf on the scores of keys this lane's row does not keep.  s[kb][r]
// belongs to key 32*kb + 8*(r/4) + 4*hh + r%4 of the tile (the MFMA result
// layout with keys along rows); bit kl of keep64 keeps key kl.
template <int NKB>
__device__ __forceinline__ void mask_scores(f32x16 (&s)[NKB], uint64_t keep64, int hh, float fill) {
  const uint64_t kl = hh ? keep64 >> 4 : keep64;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const uint32_t w = (uint32_t)(kl >> (32 * kb));
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (!((w >> (8 * (r >> 2) + (r & 3))) & 1u)) s[kb][r] = fill;
  }
}

// Rows per query tile of the forward, chosen from the window only so that the
// mask expansion can reproduce the same tiling: short windows take small
// tiles (less band waste), long ones 256 rows (8 waves sharing each K/V tile).
static inline int fwd_tile_rows(int n) { return n <= 256 ? 64 : 256; }

// Workgroup order of a 1-D grid of N = B * Hq * n_qtiles query tiles.  The
// dispatcher hands consecutive workgroups to the chip's 8 XCDs in turn, and
// each XCD has its own L2.  Workgroup i takes logical index
// (i % 8) * (N / 8) + i / 8, so each XCD walks one contiguous range of the
// logical order; in that order the query heads that share a KV head are
// adjacent and on the same query tile, heaviest tile first, so the K/V tiles
// they stream are fetched into one L2 and reused there.
struct TileWork {
  int b, h, qt;
};
__device__ __forceinline__ TileWork tile_work(int i, int N, int Hq, int Hkv, int n_qtiles) {
  constexpr int XCD = 8;
  const int lam = (N % XCD == 0) ? (i % XCD) * (N / XCD) + i / XCD : i;
  const int g = Hq / Hkv;
  const int per = n_qtiles * g;  // workgroups per (sequence, KV head)
  const int bk = lam / per, rem = lam % per;
  TileWork w;
  w.b = bk / Hkv;
  w.h = (bk % Hkv) * g + rem % g;
  w.qt = n_qtiles - 1 - rem / g;
  return w;
}
