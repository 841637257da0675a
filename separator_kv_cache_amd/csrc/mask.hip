// Mask metadata: separator flags, prefix count, compaction, kept-pair count.
//
// The separator set and the mask are those of the anthology record LIT-748
// ("Key takeaways", mask bullet): a token is a separator iff its id is one of
// the given separator ids; query i keeps key j <= i when j < a, i - j < n or
// token j is a separator.
//
// One workgroup of 1024 threads per sequence walks it in chunks of 1024
// positions, thread x taking position c0 + x, so every load and store of a
// wave is contiguous.  A thread first loads its tokens of up to kBatch chunks
// (one latency for all of them); per chunk, wave ballots rank the separators
// and plain tokens inside each wave, the waves' counts go through a
// double-buffered table in LDS (one barrier per chunk), and a running carry
// gives every position its offsets in the compacted lists.
#include "common.h"
#include "traverse.h"

namespace {

struct SepIds {
  int n;
  int id[SEPATTN_MAX_SEP_IDS];
};

constexpr int kScanThreads = 1024;
constexpr int kWaves = kScanThreads / 64;
constexpr int kBatch = 16;  // chunks whose tokens a thread holds at once

__device__ __forceinline__ bool is_separator(int tok, const SepIds& ids) {
  bool f = false;
  for (int k = 0; k < ids.n; ++k) f |= (tok == ids.id[k]);
  return f;
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
  __shared__ int cnt[2][2][kWaves];  // [chunk parity][separators, plain tokens][wave]
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t* tk = every > 0 ? nullptr : tok + (size_t)b * L;
  uint8_t* fs = is_sep + (size_t)b * L;
  int32_t* sb = sep_before + (size_t)b * (L + 1);
  int32_t* si = sep_idx + (size_t)b * L;
  int32_t* pi = plain_idx + (size_t)b * L;
  const uint64_t below = (1ull << lane) - 1ull;  // lanes under this one

  int carry_s = 0, carry_p = 0;  // separators / plain tokens (positions >= a) before the chunk
  long long kl = 0;
  const int n_chunks = (L + kScanThreads - 1) / kScanThreads;
  for (int c_base = 0; c_base < n_chunks; c_base += kBatch) {
    int tv[kBatch];
    if (every == 0) {
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int j = (c_base + k) * kScanThreads + (int)threadIdx.x;
        tv[k] = j < L ? tk[j] : 0;
      }
    }
    for (int k = 0; k < kBatch; ++k) {
      const int c = c_base + k;
      if (c >= n_chunks) break;  // uniform
      const int j = c * kScanThreads + (int)threadIdx.x;
      const bool in = j < L;
      const bool f = in && (every > 0 ? (j + 1) % every == 0 : is_separator(tv[k], ids));
      const bool cs = f && j >= a, cp = in && !f && j >= a;
      const uint64_t ms = __ballot(cs), mp = __ballot(cp);
      int* t = cnt[c & 1][0];
      if (lane == 0) {
        t[wave] = __popcll(ms);
        cnt[c & 1][1][wave] = __popcll(mp);
      }
      __syncthreads();
      int ws = 0, wp = 0, tot_s = 0, tot_p = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const int xs = cnt[c & 1][0][w], xp = cnt[c & 1][1][w];
        if (w < wave) { ws += xs; wp += xp; }
        tot_s += xs;
        tot_p += xp;
      }
      const int os = carry_s + ws + __popcll(ms & below);  // separators (>= a) before j
      const int op = carry_p + wp + __popcll(mp & below);
      if (in) {
        fs[j] = f ? 1 : 0;
        sb[j] = os;
        // kept pairs of row j: its sinks and its window positions past the
        // sinks ...
        kl += min(j + 1, a) + max(0, j - max(a, j - n + 1) + 1);
        // ... plus, summed over rows, the separators left of each window:
        // row i contributes sep_before[i - n + 1] for i >= n - 1, i.e. every
        // position x <= L - n contributes sep_before[x] once.
        if (j <= L - n) kl += os;
        if (cs) si[os] = j;
        if (cp) pi[op] = j;
      }
      carry_s += tot_s;
      carry_p += tot_p;
    }
  }
  for (int j = carry_s + (int)threadIdx.x; j < L; j += kScanThreads) si[j] = L;
  for (int j = carry_p + (int)threadIdx.x; j < L; j += kScanThreads) pi[j] = L;
  const long long total = block_sum64(kl);
  if (threadIdx.x == 0) {
    sb[L] = carry_s;
    sep_cnt[b] = carry_s;
    plain_cnt[b] = carry_p;
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

// One thread per query tile: the tile's descriptor as the forward and dQ
// kernels derive it (tile_keys), for checks against the mask's definition.
__global__ __launch_bounds__(256) void tile_desc_kernel(const int32_t* __restrict__ sep_before, int L, int a, int n,
                                                        int tile_rows, int n_tiles, int32_t* __restrict__ desc) {
  const int b = blockIdx.y;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_tiles) return;
  const TileKeys k = tile_keys(t * tile_rows, tile_rows, L, a, n, sep_before + (size_t)b * (L + 1));
  int32_t* o = desc + ((size_t)b * n_tiles + t) * 4;
  o[0] = k.n_sink;
  o[1] = k.n_gather - k.n_sink;
  o[2] = k.band_lo;
  o[3] = k.band_hi;
}

}  // namespace

int sepattn_launch_tile_desc(const sepattn_mask* m, int tile_rows, int32_t* desc, hipStream_t st) {
  const int n_tiles = (m->L + tile_rows - 1) / tile_rows;
  dim3 grid((n_tiles + 255) / 256, m->B);
  hipLaunchKernelGGL(tile_desc_kernel, grid, dim3(256), 0, st, m->sep_before, m->L, m->a, m->n, tile_rows,
                     n_tiles, desc);
  return sepattn_hip_check(hipGetLastError(), "tile_desc launch");
}

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
