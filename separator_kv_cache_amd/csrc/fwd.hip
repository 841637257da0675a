// Forward of attention under the SepLLM mask (anthology record LIT-748, "Key
// takeaways", mask bullet): O = softmax(scale * Q K^T on kept pairs) V.
//
// One workgroup per (query tile of 32*WAVES rows, q head, sequence); wave w
// owns rows [q0 + 32w, q0 + 32w + 32).  The tile's keys are visited in tiles
// of 64: first the gathered anchors (sinks and separators left of the band,
// loaded by index), then the contiguous band with the element test (see
// traverse.h).  Online softmax in fp32.
//
// MFMA orientation: S^T = K Q^T (A = 32 keys from LDS, B = 32 queries held in
// registers) puts one query per lane, so softmax statistics are per lane and
// the probabilities are already the B operand of O^T = V^T P^T.  V^T is read
// from the row-major V tile with LDS transposing reads.
#include "common.h"
#include "traverse.h"

namespace {

constexpr int BK = 64;  // keys per tile
constexpr float RESCALE_SLACK = 8.f;  // log2 units

template <typename T, int D>
struct FwdLayout;

template <int D>
struct FwdLayout<bf16, D> {
  static constexpr int KSTR = D + 8;                 // K row stride (elements)
  static constexpr int VSTR = D == 128 ? 160 : 96;   // V row stride: 16 (mod 64) dwords
  static constexpr int K_BYTES = BK * KSTR * 2;
  static constexpr int V_BYTES = BK * VSTR * 2;
  static constexpr int BUF_BYTES = K_BYTES + V_BYTES + 16;  // + separator bits of the tile
};

template <int D>
struct FwdLayout<float, D> {
  static constexpr int KSTR = D + 4;
  static constexpr int VSTR = D + 4;
  static constexpr int K_BYTES = BK * KSTR * 4;
  static constexpr int V_BYTES = BK * VSTR * 4;
  static constexpr int BUF_BYTES = K_BYTES + V_BYTES + 16;  // + separator bits of the tile
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t sq[3], sk[3], sv[3], so[3];
  uint32_t k_span, v_span;  // bytes of one (sequence, KV head) slice of K, V
  const uint8_t* is_sep;
  const int32_t* sep_idx;
  const int32_t* sep_before;
  int B, Hq, Hkv, L, a, n;
  int n_qtiles;
  float scale_log2;  // softmax scale * log2(e)
};

// Moves one 64-key tile (rows of K and V) of the workgroup through registers
// into LDS.  Thread x always handles 16-byte chunk x % CH_PER_ROW of rows
// x / CH_PER_ROW + u * ROWS_PER_PASS.  A row whose key is < 0 loads as zeros.
template <typename T, int D, int NT>
struct TileLoader {
  static constexpr int CH_PER_ROW = D * (int)sizeof(T) / 16;  // 16-byte chunks per row
  static constexpr int ROWS_PER_PASS = NT / CH_PER_ROW;
  static constexpr int PER_THREAD = BK / ROWS_PER_PASS;
  static_assert(NT % CH_PER_ROW == 0 && BK % ROWS_PER_PASS == 0, "tile chunks must divide the workgroup");
  u32x4 kr[PER_THREAD], vr[PER_THREAD];

  __device__ static int row(int u) { return (int)threadIdx.x / CH_PER_ROW + u * ROWS_PER_PASS; }
  __device__ static int chunk() { return (int)threadIdx.x % CH_PER_ROW; }

  __device__ __forceinline__ void load(rsrc_t krs, rsrc_t vrs, uint32_t krow, uint32_t vrow,
                                       const int (&key)[PER_THREAD]) {
    const uint32_t c16 = chunk() * 16;
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
      const bool ok = key[u] >= 0;
      kr[u] = bld16(krs, ok ? (uint32_t)key[u] * krow + c16 : BUF_OOB);
      vr[u] = bld16(vrs, ok ? (uint32_t)key[u] * vrow + c16 : BUF_OOB);
    }
  }
  template <int KSTR, int VSTR>
  __device__ __forceinline__ void store(T* ks, T* vs) {
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
      const int r = row(u), c = chunk();
      st16((char*)(ks + r * KSTR) + c * 16, kr[u]);
      st16((char*)(vs + r * VSTR) + c * 16, vr[u]);
    }
  }
};

// Bits [0, x) set, x clamped to [0, 64].
__device__ __forceinline__ uint64_t below64(int x) {
  return x <= 0 ? 0ull : x >= 64 ? ~0ull : ((1ull << x) - 1ull);
}

template <typename T, int D, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void fwd_kernel(FwdParams p) {
  using LY = FwdLayout<T, D>;
  constexpr int NT = WAVES * 64;
  constexpr int BQ = WAVES * 32;
  constexpr bool BF = sizeof(T) == 2;
  constexpr int KSTR = LY::KSTR, VSTR = LY::VSTR;

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const TileWork tw = tile_work(blockIdx.x, p.B * p.Hq * p.n_qtiles, p.Hq, p.Hkv, p.n_qtiles);
  const int b = tw.b, h = tw.h, qt = tw.qt;
  const int kvh = h / (p.Hq / p.Hkv);
  const int q0 = qt * BQ;
  const int r0 = q0 + wave * 32;
  const int qn = lane & 31, hh = lane >> 5;
  const int my_row = r0 + qn;

  const T* qb = (const T*)p.q + b * p.sq[0] + h * p.sq[1];
  const T* kb = (const T*)p.k + b * p.sk[0] + kvh * p.sk[1];
  const T* vb = (const T*)p.v + b * p.sv[0] + kvh * p.sv[1];
  const uint8_t* fs = p.is_sep + (size_t)b * p.L;
  const int32_t* si = p.sep_idx + (size_t)b * p.L;
  const TileKeys tk = tile_keys(q0, BQ, p.L, p.a, p.n, p.sep_before + (size_t)b * (p.L + 1));
  const int n_gt = (tk.n_gather + BK - 1) / BK;
  const int n_bt = (tk.band_hi - tk.band_lo + BK - 1) / BK;
  const int n_tiles = n_gt + n_bt;

  // ---- queries (B operand) in registers
  constexpr int QREGS = BF ? D / 16 : D / 2;
  using QT = typename std::conditional<BF, bf16x8, float>::type;
  QT qreg[QREGS];
  {
    const bool ok = my_row < p.L;
    const T* qrow = qb + (int64_t)(ok ? my_row : 0) * p.sq[2];
#pragma unroll
    for (int kk = 0; kk < QREGS; ++kk) {
      if constexpr (BF) {
        u32x4 x = ok ? ld16(qrow + kk * 16 + hh * 8) : u32x4{0, 0, 0, 0};
        qreg[kk] = __builtin_bit_cast(bf16x8, x);
      } else {
        qreg[kk] = ok ? qrow[kk * 2 + hh] : 0.f;
      }
    }
  }

  // ---- key schedule.  Gathered tiles take their keys from sep_idx; those
  // indices are loaded one tile ahead of the K/V rows they address, so no
  // load waits on another inside the loop.
  using LD = TileLoader<T, D, NT>;
  constexpr int PT = LD::PER_THREAD;
  const rsrc_t krs = make_rsrc(kb, p.k_span), vrs = make_rsrc(vb, p.v_span);
  const rsrc_t irs = make_rsrc(si, (uint32_t)p.L * 4u);
  const uint32_t krow = (uint32_t)(p.sk[2] * sizeof(T)), vrow = (uint32_t)(p.sv[2] * sizeof(T));
  int raw[PT], key[PT];
  auto issue_idx = [&](int t) {  // sep_idx entries of gathered tile t
    if (t < n_gt) {
#pragma unroll
      for (int u = 0; u < PT; ++u) {
        const int c = t * BK + LD::row(u) - tk.n_sink;
        raw[u] = bld4(irs, c >= 0 && c < tk.n_gather - tk.n_sink ? (uint32_t)c * 4u : BUF_OOB);
      }
    }
  };
  auto keys_of = [&](int t) {  // keys of tile t (raw holds its indices if gathered)
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int r = LD::row(u);
      if (t < n_gt) {
        const int c = t * BK + r;
        key[u] = c < tk.n_sink ? c : (c < tk.n_gather ? raw[u] : -1);
      } else {
        const int j = tk.band_lo + (t - n_gt) * BK + r;
        key[u] = j < tk.band_hi ? j : -1;
      }
    }
  };

  // Separator flags of a band tile travel with it as a 64-bit mask (bit r =
  // is_sep of row r), built by wave 0 with one ballot.
  const rsrc_t frs = make_rsrc(fs, (uint32_t)p.L);
  uint32_t flag = 0;
  auto issue_flag = [&](int t) {
    if (wave == 0) flag = t >= n_gt ? __builtin_amdgcn_raw_buffer_load_b8(frs, tk.band_lo + (t - n_gt) * BK + lane, 0, 0) : 0;
  };

  LD ld;
  auto kbuf = [&](int s) { return (T*)(smem + s * LY::BUF_BYTES); };
  auto vbuf = [&](int s) { return (T*)(smem + s * LY::BUF_BYTES + LY::K_BYTES); };
  auto fbuf = [&](int s) { return (uint64_t*)(smem + s * LY::BUF_BYTES + LY::K_BYTES + LY::V_BYTES); };
  auto store_tile = [&](int s) {
    ld.template store<KSTR, VSTR>(kbuf(s), vbuf(s));
    if (wave == 0) {
      const uint64_t bits = __ballot(flag != 0);
      if (lane == 0) *fbuf(s) = bits;
    }
  };

  // ---- prologue: tile 0 into LDS, indices of tile 1 in flight
  issue_idx(0);
  keys_of(0);
  ld.load(krs, vrs, krow, vrow, key);
  issue_flag(0);
  issue_idx(1);
  store_tile(0);
  __syncthreads();

  constexpr int NKB = BK / 32;  // 32-key blocks per tile
  constexpr int NDB = D / 32;   // 32-dim blocks
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  for (int t = 0; t < n_tiles; ++t) {
    const int cur = t & 1;
    // Tile t + 1 (all-absent past the last tile: zero loads, unused store).
    keys_of(t + 1);
    ld.load(krs, vrs, krow, vrow, key);
    issue_flag(t + 1);
    issue_idx(t + 2);
    const T* ks = kbuf(cur);
    const T* vs = vbuf(cur);

    // ---- S^T = K Q^T
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2) sacc[kb2] = f32x16{};
    if constexpr (BF) {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2) {
          const bf16x8 a = *(const bf16x8*)(ks + (kb2 * 32 + qn) * KSTR + kk * 16 + hh * 8);
          sacc[kb2] = mfma32x16(a, qreg[kk], sacc[kb2]);
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < D / 2; ++kk) {
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2) {
          const float a = ks[(kb2 * 32 + qn) * KSTR + kk * 2 + hh];
          sacc[kb2] = mfma32x2f(a, qreg[kk], sacc[kb2]);
        }
      }
    }

    // ---- mask, online softmax (log2 domain).  The running reference max m_run
    // is raised only when some lane's tile max exceeds it by more than
    // RESCALE_SLACK (a wave-uniform branch), so O and l are rarely rescaled;
    // probabilities stay below 2^RESCALE_SLACK.  O / l and the LSE use the
    // same reference, so the result does not depend on when it moved.
    // Partial tiles: bit kl of keep64 says whether key kl of the tile is kept
    // for this lane's row.
    const bool gathered = t < n_gt;
    const int k0 = tk.band_lo + (t - n_gt) * BK;
    const bool full = gathered ? (t + 1) * BK <= tk.n_gather
                               : (k0 + BK <= tk.band_hi) && (k0 + BK - 1 <= r0) && (r0 + 31 - k0 < p.n);
    if (!full) {
      uint64_t keep64;
      if (gathered) {
        keep64 = below64(tk.n_gather - t * BK);
      } else {
        const int d = my_row - k0;  // key kl lies d - kl rows before this row
        const uint64_t causal = below64(min(d, tk.band_hi - 1 - k0) + 1);
        const uint64_t window = ~below64(d - p.n + 1);
        const uint64_t sinks = below64(p.a - k0);
        keep64 = causal & (window | sinks | *fbuf(cur));
      }
      const uint64_t kl = hh ? keep64 >> 4 : keep64;
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) {
        const uint32_t w = (uint32_t)(kl >> (32 * kb2));
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((w >> (8 * (r >> 2) + (r & 3))) & 1u)) sacc[kb2][r] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb2][r]);
    mx = fmaxf(mx, xor32(mx)) * p.scale_log2;  // the scale is positive
    if (__any(mx > m_run + RESCALE_SLACK)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb2][r] = fast_exp2(__builtin_fmaf(sacc[kb2][r], p.scale_log2, -m_use));

#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2) l_run += tree_sum16(sacc[kb2]);

    // ---- O^T += V^T P^T
    if constexpr (BF) {
      const int g = lane >> 4, li = lane & 15;
#pragma unroll
      for (int c = 0; c < BK / 16; ++c) {
        bf16x8 pb;
#pragma unroll
        for (int s = 0; s < 8; ++s) pb[s] = (bf16)sacc[c >> 1][(c & 1) * 8 + s];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          // lane li of group g reads V[key_base + li/4][dim_base + 4*(li%4)]
          const int dim = db * 32 + 16 * (g & 1) + 4 * (li & 3);
          const int key = 16 * c + 4 * (g >> 1) + (li >> 2);
          const bf16x4 lo = lds_read_tr16(vs + key * VSTR + dim);
          const bf16x4 hi = lds_read_tr16(vs + (key + 8) * VSTR + dim);
          const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[db] = mfma32x16(a, pb, oacc[db]);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < BK / 2; ++c) {
        const int kb2 = c >> 4, rr = c & 15;
        const int key = kb2 * 32 + 8 * (rr >> 2) + 4 * hh + (rr & 3);
        const float pb = sacc[kb2][rr];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const float a = vs[key * VSTR + db * 32 + qn];
          oacc[db] = mfma32x2f(a, pb, oacc[db]);
        }
      }
    }

    store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  const float l_tot = l_run + xor32(l_run);
  const float inv = 1.f / l_tot;
  if (my_row < p.L) {
    T* orow = (T*)p.o + b * p.so[0] + h * p.so[1] + (int64_t)my_row * p.so[2];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dim = db * 32 + 8 * i + 4 * hh;
        if constexpr (BF) {
          bf16x4 w = {(bf16)(oacc[db][4 * i + 0] * inv), (bf16)(oacc[db][4 * i + 1] * inv),
                      (bf16)(oacc[db][4 * i + 2] * inv), (bf16)(oacc[db][4 * i + 3] * inv)};
          *(bf16x4*)(orow + dim) = w;
        } else {
          f32x4 w = {oacc[db][4 * i + 0] * inv, oacc[db][4 * i + 1] * inv, oacc[db][4 * i + 2] * inv,
                     oacc[db][4 * i + 3] * inv};
          *(f32x4*)(orow + dim) = w;
        }
      }
    }
    if (p.lse && hh == 0) {
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      p.lse[((size_t)b * p.Hq + h) * p.L + my_row] = (m_use + __log2f(l_tot)) * 0.69314718055994531f;
    }
  }
}

// ---------------------------------------------------------------- bf16, 8 waves, ping-pong
//
// Same traversal and numerics as fwd_kernel.  The two waves that share a SIMD
// (waves w and w + 4 of the workgroup) alternate between a matrix phase C and
// a vector phase V, so one keeps the matrix core busy while the other runs
// the softmax:
//   C(t): S(t+1) = K(t+1) Q^T and O^T += V(t)^T P(t)^T      (32 MFMAs)
//   V(t): mask, running max, exponentials of S(t+1) -> P(t+1), row sums
// Every wave runs C(t), barrier, V(t), barrier; waves 4-7 pass one extra
// barrier first, so their C(t) runs beside the V(t) of waves 0-3.  In that
// shared interval both groups write their halves of K(t+2) and V(t+1) into
// LDS (group 0 from its V phase, group 1 from its C phase), over the buffers
// of K(t) and V(t-1), which every wave finished reading an interval earlier.
// Each group then starts the global loads of its halves of K(t+3), V(t+2).

// One 64-row tile of one bf16 [., D] matrix moving global -> registers -> LDS.
// Thread x handles 16-byte chunk x % CH of rows x / CH + u * (NT / CH).
template <int D, int NT>
struct RowMover {
  static constexpr int CH = D * 2 / 16;
  static constexpr int ROWS_PER_PASS = NT / CH;
  static constexpr int PT = BK / ROWS_PER_PASS;
  static_assert(NT % CH == 0 && BK % ROWS_PER_PASS == 0, "tile chunks must divide the workgroup");
  u32x4 r[PT];

  __device__ static int row(int u) { return (int)threadIdx.x / CH + u * ROWS_PER_PASS; }
  __device__ static int chunk() { return (int)threadIdx.x % CH; }
  __device__ __forceinline__ void load(rsrc_t rs, uint32_t row_bytes, const int (&key)[PT]) {
#pragma unroll
    for (int u = 0; u < PT; ++u)
      r[u] = bld16(rs, key[u] >= 0 ? (uint32_t)key[u] * row_bytes + chunk() * 16 : BUF_OOB);
  }
  template <int STR>
  __device__ __forceinline__ void store(bf16* dst) {
#pragma unroll
    for (int u = 0; u < PT; ++u) st16((char*)(dst + row(u) * STR) + chunk() * 16, r[u]);
  }
};

template <int D>
__global__ __launch_bounds__(512) void fwd_pp_kernel(FwdParams p) {
  using LY = FwdLayout<bf16, D>;
  constexpr int WAVES = 8, NT = 512, BQ = 256;
  constexpr int KSTR = LY::KSTR, VSTR = LY::VSTR;
  constexpr int NKB = BK / 32;  // 32-key blocks per tile
  constexpr int NDB = D / 32;   // 32-dim blocks
  constexpr int KK = D / 16;    // 16-dim steps of the score product

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = wave >> 2;
  const TileWork tw = tile_work(blockIdx.x, p.B * p.Hq * p.n_qtiles, p.Hq, p.Hkv, p.n_qtiles);
  const int b = tw.b, h = tw.h, qt = tw.qt;
  const int kvh = h / (p.Hq / p.Hkv);
  const int q0 = qt * BQ;
  const int r0 = q0 + wave * 32;
  const int qn = lane & 31, hh = lane >> 5;
  const int my_row = r0 + qn;

  const bf16* qb = (const bf16*)p.q + b * p.sq[0] + h * p.sq[1];
  const bf16* kb = (const bf16*)p.k + b * p.sk[0] + kvh * p.sk[1];
  const bf16* vb = (const bf16*)p.v + b * p.sv[0] + kvh * p.sv[1];
  const uint8_t* fs = p.is_sep + (size_t)b * p.L;
  const int32_t* si = p.sep_idx + (size_t)b * p.L;
  const TileKeys tk = tile_keys(q0, BQ, p.L, p.a, p.n, p.sep_before + (size_t)b * (p.L + 1));
  const int n_gt = (tk.n_gather + BK - 1) / BK;
  const int n_bt = (tk.band_hi - tk.band_lo + BK - 1) / BK;
  const int n_tiles = n_gt + n_bt;

  // ---- queries (B operand of the score product) in registers
  bf16x8 qreg[KK];
  {
    const bool ok = my_row < p.L;
    const bf16* qrow = qb + (int64_t)(ok ? my_row : 0) * p.sq[2];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qreg[kk] = __builtin_bit_cast(bf16x8, ok ? ld16(qrow + kk * 16 + hh * 8) : u32x4{0, 0, 0, 0});
  }

  // ---- key schedule (as in fwd_kernel; sep_idx entries run one tile ahead of K)
  using MV = RowMover<D, NT>;
  constexpr int PT = MV::PT;
  const rsrc_t krs = make_rsrc(kb, p.k_span), vrs = make_rsrc(vb, p.v_span);
  const rsrc_t irs = make_rsrc(si, (uint32_t)p.L * 4u), frs = make_rsrc(fs, (uint32_t)p.L);
  const uint32_t krow = (uint32_t)(p.sk[2] * 2), vrow = (uint32_t)(p.sv[2] * 2);
  int raw[PT], key_k[PT], key_v[PT];
  auto issue_idx = [&](int t) {
    if (t < n_gt) {
#pragma unroll
      for (int u = 0; u < PT; ++u) {
        const int c = t * BK + MV::row(u) - tk.n_sink;
        raw[u] = bld4(irs, c >= 0 && c < tk.n_gather - tk.n_sink ? (uint32_t)c * 4u : BUF_OOB);
      }
    }
  };
  auto keys_of = [&](int t, int (&key)[PT]) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int r = MV::row(u);
      if (t < n_gt) {
        const int c = t * BK + r;
        key[u] = c < tk.n_sink ? c : (c < tk.n_gather ? raw[u] : -1);
      } else {
        const int j = tk.band_lo + (t - n_gt) * BK + r;
        key[u] = j < tk.band_hi ? j : -1;
      }
    }
  };
  uint32_t flag = 0;
  auto issue_flag = [&](int t) {
    if (wave == 0) flag = t >= n_gt ? __builtin_amdgcn_raw_buffer_load_b8(frs, tk.band_lo + (t - n_gt) * BK + lane, 0, 0) : 0;
  };

  auto kbuf = [&](int s) { return (bf16*)(smem + (s & 1) * LY::K_BYTES); };
  auto vbuf = [&](int s) { return (bf16*)(smem + 2 * LY::K_BYTES + (s & 1) * LY::V_BYTES); };
  auto fslot = [&](int t) { return (uint64_t*)(smem + 2 * LY::K_BYTES + 2 * LY::V_BYTES + (t & 3) * 8); };
  auto store_flag = [&](int t) {
    if (wave == 0) {
      const uint64_t bits = __ballot(flag != 0);
      if (lane == 0) *fslot(t) = bits;
    }
  };

  MV mk, mv;
  // Store site of interval t: K(t+2), V(t+1) into LDS, then start K(t+3), V(t+2).
  auto store_and_fetch = [&](int t) {
    mk.template store<KSTR>(kbuf(t + 2));
    mv.template store<VSTR>(vbuf(t + 1));
    store_flag(t + 2);
    keys_of(t + 3, key_k);
    mk.load(krs, krow, key_k);
    mv.load(vrs, vrow, key_v);
    issue_flag(t + 3);
    issue_idx(t + 4);
#pragma unroll
    for (int u = 0; u < PT; ++u) key_v[u] = key_k[u];
  };

  f32x16 sacc[NKB];
  bf16x8 pb[BK / 16];
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // Matrix phase: S(t+1) = K(t+1) Q^T (NS MFMAs) then O^T += V(t)^T P(t)^T
  // (NP MFMAs) as one stream whose LDS operand reads run PD MFMAs ahead, so
  // a wave alone keeps the matrix core fed (sched_barrier pins the order).
  constexpr int NS = KK * NKB, NP = (BK / 16) * NDB, PD = 4;
  auto matrix_phase = [&](const bf16* ks, const bf16* vs) {
    const int g = lane >> 4, li = lane & 15;
    auto opnd = [&](int i) -> bf16x8 {
      if (i < NS) return *(const bf16x8*)(ks + ((i % NKB) * 32 + qn) * KSTR + (i / NKB) * 16 + hh * 8);
      // lane li of group g reads V[key_base + li/4][dim_base + 4*(li%4)]
      const int c = (i - NS) / NDB, db = (i - NS) % NDB;
      const int dim = db * 32 + 16 * (g & 1) + 4 * (li & 3);
      const int key = 16 * c + 4 * (g >> 1) + (li >> 2);
      const bf16x4 lo = lds_read_tr16(vs + key * VSTR + dim);
      const bf16x4 hi = lds_read_tr16(vs + (key + 8) * VSTR + dim);
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    bf16x8 op[NS + NP];
#pragma unroll
    for (int i = 0; i < PD; ++i) op[i] = opnd(i);
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2) sacc[kb2] = f32x16{};
#pragma unroll
    for (int i = 0; i < NS + NP; ++i) {
      if (i + PD < NS + NP) op[i + PD] = opnd(i + PD);
      if (i < NS) {
        sacc[i % NKB] = mfma32x16(op[i], qreg[i / NKB], sacc[i % NKB]);
      } else {
        const int j = i - NS;
        oacc[j % NDB] = mfma32x16(op[i], pb[j / NDB], oacc[j % NDB]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto scores = [&](const bf16* ks) {
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2) sacc[kb2] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) {
        const bf16x8 a = *(const bf16x8*)(ks + (kb2 * 32 + qn) * KSTR + kk * 16 + hh * 8);
        sacc[kb2] = mfma32x16(a, qreg[kk], sacc[kb2]);
      }
  };
  // Softmax of the scores of tile t (in sacc) into pb, updating m, l, O.
  auto softmax = [&](int t) {
    const bool gathered = t < n_gt;
    const int k0 = tk.band_lo + (t - n_gt) * BK;
    const bool full = gathered ? (t + 1) * BK <= tk.n_gather
                               : (k0 + BK <= tk.band_hi) && (k0 + BK - 1 <= r0) && (r0 + 31 - k0 < p.n);
    if (!full) {
      uint64_t keep64;
      if (gathered) {
        keep64 = below64(tk.n_gather - t * BK);
      } else {
        const int d = my_row - k0;  // key kl lies d - kl rows before this row
        const uint64_t causal = below64(min(d, tk.band_hi - 1 - k0) + 1);
        const uint64_t window = ~below64(d - p.n + 1);
        const uint64_t sinks = below64(p.a - k0);
        keep64 = causal & (window | sinks | *fslot(t));
      }
      const uint64_t kl = hh ? keep64 >> 4 : keep64;
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) {
        const uint32_t w = (uint32_t)(kl >> (32 * kb2));
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((w >> (8 * (r >> 2) + (r & 3))) & 1u)) sacc[kb2][r] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb2][r]);
    mx = max_xor32(mx) * p.scale_log2;  // the scale is positive
    if (__any(mx > m_run + RESCALE_SLACK)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb2][r] = fast_exp2(__builtin_fmaf(sacc[kb2][r], p.scale_log2, -m_use));
      l_run += tree_sum16(sacc[kb2]);
    }
#pragma unroll
    for (int c = 0; c < BK / 16; ++c)
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) pb[c][sl] = (bf16)sacc[c >> 1][(c & 1) * 8 + sl];
  };

  // ---- prologue: K(0), V(0), K(1) in LDS, K(2) and V(1) in flight; P(0)
  issue_idx(0);
  keys_of(0, key_k);
  mk.load(krs, krow, key_k);
  mv.load(vrs, vrow, key_k);
  issue_flag(0);
  issue_idx(1);
  mk.template store<KSTR>(kbuf(0));
  mv.template store<VSTR>(vbuf(0));
  store_flag(0);
  keys_of(1, key_v);
  mk.load(krs, krow, key_v);
  issue_flag(1);
  issue_idx(2);
  mk.template store<KSTR>(kbuf(1));
  store_flag(1);
  keys_of(2, key_k);
  mk.load(krs, krow, key_k);
  mv.load(vrs, vrow, key_v);
  issue_flag(2);
  issue_idx(3);
#pragma unroll
  for (int u = 0; u < PT; ++u) key_v[u] = key_k[u];
  __syncthreads();
  scores(kbuf(0));
  softmax(0);

  if (grp == 1) __syncthreads();  // group 1 runs one phase behind
  for (int t = 0; t < n_tiles; ++t) {
    // ---- C(t)
    __builtin_amdgcn_s_setprio(1);
    matrix_phase(kbuf(t + 1), vbuf(t));
    __builtin_amdgcn_s_setprio(0);
    if (grp == 1) store_and_fetch(t);
    __syncthreads();
    // ---- V(t)
    if (t + 1 < n_tiles) softmax(t + 1);
    if (grp == 0) store_and_fetch(t);
    __syncthreads();
  }
  if (grp == 0) __syncthreads();

  // ---- epilogue
  const float l_tot = l_run + xor32(l_run);
  const float inv = 1.f / l_tot;
  if (my_row < p.L) {
    bf16* orow = (bf16*)p.o + b * p.so[0] + h * p.so[1] + (int64_t)my_row * p.so[2];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dim = db * 32 + 8 * i + 4 * hh;
        bf16x4 w = {(bf16)(oacc[db][4 * i + 0] * inv), (bf16)(oacc[db][4 * i + 1] * inv),
                    (bf16)(oacc[db][4 * i + 2] * inv), (bf16)(oacc[db][4 * i + 3] * inv)};
        *(bf16x4*)(orow + dim) = w;
      }
    }
    if (p.lse && hh == 0) {
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      p.lse[((size_t)b * p.Hq + h) * p.L + my_row] = (m_use + __log2f(l_tot)) * 0.69314718055994531f;
    }
  }
}

template <int D>
int launch_fwd_pp(const FwdParams& p, hipStream_t st) {
  using LY = FwdLayout<bf16, D>;
  const int smem = 2 * LY::K_BYTES + 2 * LY::V_BYTES + 32;
  auto kern = fwd_pp_kernel<D>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return sepattn_hip_check(e, "fwd smem attribute");
  hipLaunchKernelGGL(kern, dim3(p.B * p.Hq * p.n_qtiles), dim3(512), smem, st, p);
  return sepattn_hip_check(hipGetLastError(), "fwd launch");
}

template <typename T, int D, int WAVES>
int launch_fwd(const FwdParams& p, hipStream_t st) {
  constexpr int BQ = WAVES * 32;
  const int smem = 2 * FwdLayout<T, D>::BUF_BYTES;
  auto kern = fwd_kernel<T, D, WAVES>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return sepattn_hip_check(e, "fwd smem attribute");
  hipLaunchKernelGGL(kern, dim3(p.B * p.Hq * p.n_qtiles), dim3(WAVES * 64), smem, st, p);
  return sepattn_hip_check(hipGetLastError(), "fwd launch");
}

}  // namespace

int sepattn_launch_fwd(const sepattn_shape* s, int dtype, const sepattn_mask* m, const void* q,
                       const void* k, const void* v, float scale, void* o, float* lse, hipStream_t st) {
  FwdParams p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  for (int i = 0; i < 3; ++i) {
    p.sq[i] = s->q_stride[i]; p.sk[i] = s->k_stride[i]; p.sv[i] = s->v_stride[i]; p.so[i] = s->o_stride[i];
  }
  const int esz = dtype == SEPATTN_BF16 ? 2 : 4;
  p.k_span = (uint32_t)((((int64_t)s->L - 1) * s->k_stride[2] + s->d) * esz);
  p.v_span = (uint32_t)((((int64_t)s->L - 1) * s->v_stride[2] + s->d) * esz);
  p.is_sep = m->is_sep; p.sep_idx = m->sep_idx; p.sep_before = m->sep_before;
  p.B = s->B; p.Hq = s->Hq; p.Hkv = s->Hkv; p.L = s->L; p.a = m->a; p.n = m->n;
  p.scale_log2 = scale * 1.4426950408889634f;
  const int rows = fwd_tile_rows(m->n);
  p.n_qtiles = (s->L + rows - 1) / rows;
  const bool big = rows == 256;
  if (dtype == SEPATTN_BF16) {
    if (s->d == 128) return big ? launch_fwd_pp<128>(p, st) : launch_fwd<bf16, 128, 2>(p, st);
    return big ? launch_fwd_pp<64>(p, st) : launch_fwd<bf16, 64, 2>(p, st);
  }
  if (s->d == 128) return big ? launch_fwd<float, 128, 8>(p, st) : launch_fwd<float, 128, 2>(p, st);
  return big ? launch_fwd<float, 64, 8>(p, st) : launch_fwd<float, 64, 2>(p, st);
}
