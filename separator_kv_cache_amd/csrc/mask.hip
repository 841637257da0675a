// Mask metadata: separator flags, prefix count, compaction, kept-pair count.
//
// The separator set and the mask are those of the anthology record LIT-748
// ("Key takeaways", mask bullet): a token is a separator iff its id is one of
// the given separator ids; query i keeps key j <= i when j < a, i - j < n or
// token j is a separator.
//
// One workgroup of 1024 threads per sequence: each thread owns a contiguous
// run of positions, counts separators and plain tokens in it, a block-wide
// exclusive scan gives every run its output offsets, and a second pass writes
// the compacted lists, the prefix counts and the per-row kept counts.
#include "common.h"
#include "traverse.h"

namespace {

struct SepIds {
  int n;
  int id[SEPATTN_MAX_SEP_IDS];
};

constexpr int kScanThreads = 1024;
constexpr int kWaves = kScanThreads / 64;

__device__ __forceinline__ bool is_separator(int tok, const SepIds& ids) {
  bool f = false;
  for (int k = 0; k < ids.n; ++k) f |= (tok == ids.id[k]);
  return f;
}

// Exclusive scan of two counters over the block; also returns the totals.
__device__ void block_scan2(int x, int y, int* ex, int* ey, int* tx, int* ty) {
  __shared__ int wx[kWaves], wy[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int ix = x, iy = y;
  for (int o = 1; o < 64; o <<= 1) {
    int ux = __shfl_up(ix, o, 64), uy = __shfl_up(iy, o, 64);
    if (lane >= o) { ix += ux; iy += uy; }
  }
  if (lane == 63) { wx[wave] = ix; wy[wave] = iy; }
  __syncthreads();
  int bx = 0, by = 0, sx = 0, sy = 0;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) { bx += wx[w]; by += wy[w]; }
    sx += wx[w]; sy += wy[w];
  }
  *ex = bx + ix - x;
  *ey = by + iy - y;
  *tx = sx;
  *ty = sy;
}

__device__ long long block_sum64(long long v) {
  __shared__ long long ws[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) v += __shfl_down(v, o, 64);
  if (lane == 0) ws[wave] = v;
  __syncthreads();
  long long s = 0;
  if (threadIdx.x == 0)
    for (int w = 0; w < kWaves; ++w) s += ws[w];
  return s;
}

// Anchor flags: token j is a separator (its id is in ids) or, with every > 0,
// j is one of the fixed-interval anchors (j + 1) mod every == 0 (tok unused).
__global__ __launch_bounds__(kScanThreads) void build_mask_kernel(
    const int32_t* __restrict__ tok, SepIds ids, int every, int L, int a, int n,
    uint8_t* __restrict__ is_sep, int32_t* __restrict__ sep_idx, int32_t* __restrict__ sep_before,
    int32_t* __restrict__ sep_cnt, int32_t* __restrict__ plain_idx, int32_t* __restrict__ plain_cnt,
    int64_t* __restrict__ kept) {
  const int b = blockIdx.x;
  const int per = (L + kScanThreads - 1) / kScanThreads;
  const int p0 = min(L, (int)threadIdx.x * per), p1 = min(L, p0 + per);
  const int32_t* tk = every > 0 ? nullptr : tok + (size_t)b * L;
  auto flag = [&](int j) { return every > 0 ? (j + 1) % every == 0 : is_separator(tk[j], ids); };

  int cs = 0, cp = 0;
  for (int j = p0; j < p1; ++j) {
    const bool f = flag(j);
    is_sep[(size_t)b * L + j] = f ? 1 : 0;
    if (j >= a) {
      cs += f ? 1 : 0;
      cp += f ? 0 : 1;
    }
  }
  int os, op, ts, tp;
  block_scan2(cs, cp, &os, &op, &ts, &tp);

  int32_t* sb = sep_before + (size_t)b * (L + 1);
  int32_t* si = sep_idx + (size_t)b * L;
  int32_t* pi = plain_idx + (size_t)b * L;
  long long kl = 0;
  for (int j = p0; j < p1; ++j) {
    const bool f = flag(j);
    sb[j] = os;
    // kept pairs of row j: its sinks and its window positions past the
    // sinks ...
    kl += min(j + 1, a) + max(0, j - max(a, j - n + 1) + 1);
    // ... plus, summed over rows, the separators left of each window:
    // row i contributes sep_before[i - n + 1] for i >= n - 1, i.e. every
    // position x <= L - n contributes sep_before[x] once.
    if (j <= L - n) kl += os;
    if (j >= a) {
      if (f) si[os++] = j;
      else pi[op++] = j;
    }
  }
  for (int j = ts + threadIdx.x; j < L; j += kScanThreads) si[j] = L;
  for (int j = tp + threadIdx.x; j < L; j += kScanThreads) pi[j] = L;
  const long long total = block_sum64(kl);
  if (threadIdx.x == 0) {
    sb[L] = ts;
    sep_cnt[b] = ts;
    plain_cnt[b] = tp;
    kept[b] = total;
  }
}

// One thread per row: walk the row's keys the way the forward tiles do and
// write the row's bit-packed mask.
__global__ __launch_bounds__(256) void mask_bits_kernel(
    const uint8_t* __restrict__ is_sep, const int32_t* __restrict__ sep_idx,
    const int32_t* __restrict__ sep_before, int L, int a, int n, int tile_rows,
    uint32_t* __restrict__ bits) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= L) return;
  const int words = (L + 31) / 32;
  uint32_t* row = bits + ((size_t)b * L + i) * words;
  for (int w = 0; w < words; ++w) row[w] = 0;
  const uint8_t* fs = is_sep + (size_t)b * L;
  const int32_t* si = sep_idx + (size_t)b * L;
  const int q0 = (i / tile_rows) * tile_rows;
  const TileKeys t = tile_keys(q0, tile_rows, L, a, n, sep_before + (size_t)b * (L + 1));
  for (int c = 0; c < t.n_gather; ++c) {
    const int j = gather_key(c, t.n_sink, si);
    row[j >> 5] |= 1u << (j & 31);
  }
  for (int j = t.band_lo; j < t.band_hi; ++j)
    if (band_keep(i, j, a, n, fs)) row[j >> 5] |= 1u << (j & 31);
}

}  // namespace

int sepattn_launch_build_mask(const int32_t* tok, const int32_t* ids, int n_ids, const sepattn_mask* m,
                              hipStream_t st) {
  SepIds s;
  s.n = n_ids;
  for (int k = 0; k < SEPATTN_MAX_SEP_IDS; ++k) s.id[k] = k < n_ids ? ids[k] : 0;
  hipLaunchKernelGGL(build_mask_kernel, dim3(m->B), dim3(kScanThreads), 0, st, tok, s, 0, m->L, m->a, m->n,
                     m->is_sep, m->sep_idx, m->sep_before, m->sep_cnt, m->plain_idx, m->plain_cnt,
                     m->kept);
  return sepattn_hip_check(hipGetLastError(), "build_mask launch");
}

int sepattn_launch_build_mask_fixed(int delta, const sepattn_mask* m, hipStream_t st) {
  SepIds s;
  s.n = 0;
  for (int k = 0; k < SEPATTN_MAX_SEP_IDS; ++k) s.id[k] = 0;
  hipLaunchKernelGGL(build_mask_kernel, dim3(m->B), dim3(kScanThreads), 0, st, (const int32_t*)nullptr, s, delta,
                     m->L, m->a, m->n, m->is_sep, m->sep_idx, m->sep_before, m->sep_cnt, m->plain_idx,
                     m->plain_cnt, m->kept);
  return sepattn_hip_check(hipGetLastError(), "build_mask_fixed launch");
}

int sepattn_launch_mask_bits(const sepattn_mask* m, uint32_t* bits, hipStream_t st) {
  dim3 grid((m->L + 255) / 256, m->B);
  hipLaunchKernelGGL(mask_bits_kernel, grid, dim3(256), 0, st, m->is_sep, m->sep_idx, m->sep_before, m->L,
                     m->a, m->n, fwd_tile_rows(m->n), bits);
  return sepattn_hip_check(hipGetLastError(), "mask_bits launch");
}
