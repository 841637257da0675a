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
