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

constexpr int BK = KTILE;             // keys per tile
constexpr float RESCALE_SLACK = 8.f;  // log2 units

template <typename T, int D>
struct FwdLayout;

template <int D>
struct FwdLayout<bf16, D> {
  static constexpr int KSTR = D + 8;                 // K row stride (elements)
  static constexpr int VSTR = D == 128 ? 160 : 96;   // V row stride: 16 (mod 64) dwords
  static constexpr int K_BYTES = BK * KSTR * 2;
  static constexpr int V_BYTES = BK * VSTR * 2;
};

template <int D>
struct FwdLayout<float, D> {
  static constexpr int KSTR = D + 4;
  static constexpr int VSTR = D + 4;
  static constexpr int K_BYTES = BK * KSTR * 4;
  static constexpr int V_BYTES = BK * VSTR * 4;
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

// Lazy online softmax over one key tile, log2 domain.  The running reference
// m is raised only when some lane's tile maximum exceeds it by more than
// RESCALE_SLACK (a wave-uniform branch), so O and l are rarely rescaled and
// probabilities stay below 2^RESCALE_SLACK.  O / l and the LSE use the same
// reference, so the result does not depend on when it moved.  On return s
// holds exp2(scale_log2 * s - m) and l includes their sums.
template <int NKB, int NDB>
__device__ __forceinline__ void softmax_tile(f32x16 (&s)[NKB], f32x16 (&o)[NDB], float& m_run, float& l_run,
                                             float scale_log2) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = max_xor32(mx) * scale_log2;  // the two lanes of a query row; the scale is positive
  if (__any(mx > m_run + RESCALE_SLACK)) {
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
  }
  const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], scale_log2, -m_use));
    l_run += tree_sum16(s[kb]);
  }
}

// O = O^T accumulator / l and the natural-log LSE of one query row.
template <typename T, int NDB>
__device__ __forceinline__ void store_rows(const FwdParams& p, const f32x16 (&o)[NDB], float m_run, float l_run,
                                           int b, int h, int my_row, int hh) {
  const float l_tot = l_run + xor32(l_run);
  const float inv = 1.f / l_tot;
  if (my_row >= p.L) return;
  T* orow = (T*)p.o + b * p.so[0] + h * p.so[1] + (int64_t)my_row * p.so[2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int dim = db * 32 + 8 * i + 4 * hh;
      if constexpr (sizeof(T) == 2) {
        bf16x4 w = {(bf16)(o[db][4 * i + 0] * inv), (bf16)(o[db][4 * i + 1] * inv), (bf16)(o[db][4 * i + 2] * inv),
                    (bf16)(o[db][4 * i + 3] * inv)};
        *(bf16x4*)(orow + dim) = w;
      } else {
        f32x4 w = {o[db][4 * i + 0] * inv, o[db][4 * i + 1] * inv, o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv};
        *(f32x4*)(orow + dim) = w;
      }
    }
  }
  if (p.lse && hh == 0) {
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    p.lse[((size_t)b * p.Hq + h) * p.L + my_row] = (m_use + __log2f(l_tot)) * 0.69314718055994531f;
  }
}

// ---------------------------------------------------------------- lockstep kernel
//
// Every wave loads its share of tile t+1 into registers, computes tile t from
// LDS, and stores tile t+1 into the other buffer before the tile's barrier.
// Used for short windows (64-row tiles, 2 waves) and for fp32.

template <typename T, int D, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void fwd_kernel(FwdParams p) {
  using LY = FwdLayout<T, D>;
  constexpr int NT = WAVES * 64;
  constexpr int BQ = WAVES * 32;
  constexpr bool BF = sizeof(T) == 2;
  constexpr int KSTR = LY::KSTR, VSTR = LY::VSTR;
  constexpr int BUF = LY::K_BYTES + LY::V_BYTES + 16;  // K, V, separator bits
  constexpr int NKB = BK / 32;  // 32-key blocks per tile
  constexpr int NDB = D / 32;   // 32-dim blocks

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const TileWork tw = tile_work(blockIdx.x, p.B * p.Hq * p.n_qtiles, p.Hq, p.Hkv, p.n_qtiles);
  const int b = tw.b, h = tw.h;
  const int kvh = h / (p.Hq / p.Hkv);
  const int q0 = tw.qt * BQ;
  const int r0 = q0 + wave * 32;
  const int qn = lane & 31, hh = lane >> 5;
  const int my_row = r0 + qn;

  const T* qb = (const T*)p.q + b * p.sq[0] + h * p.sq[1];
  const T* kb = (const T*)p.k + b * p.sk[0] + kvh * p.sk[1];
  const T* vb = (const T*)p.v + b * p.sv[0] + kvh * p.sv[1];

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

  using MV = RowMover<T, D, NT>;
  constexpr int PT = MV::PT;
  KeyStream<PT> ks;
  ks.init(q0, BQ, p.L, p.a, p.n, p.sep_before + (size_t)b * (p.L + 1), p.sep_idx + (size_t)b * p.L,
          p.is_sep + (size_t)b * p.L);
  const rsrc_t krs = make_rsrc(kb, p.k_span), vrs = make_rsrc(vb, p.v_span);
  const uint32_t krow = (uint32_t)(p.sk[2] * sizeof(T)), vrow = (uint32_t)(p.sv[2] * sizeof(T));
  int rows[PT], key[PT];
  MV::rows(rows);
  MV mk, mv;
  uint32_t flag = 0;

  auto kbuf = [&](int s) { return (T*)(smem + s * BUF); };
  auto vbuf = [&](int s) { return (T*)(smem + s * BUF + LY::K_BYTES); };
  auto fbuf = [&](int s) { return (uint64_t*)(smem + s * BUF + LY::K_BYTES + LY::V_BYTES); };
  // Separator flags of a band tile travel with it as a 64-bit mask built by
  // wave 0 with one ballot.
  auto fetch = [&](int t) {
    ks.keys(t, rows, key);
    mk.load(krs, krow, key);
    mv.load(vrs, vrow, key);
    if (wave == 0) flag = ks.flag_byte(t, lane);
  };
  auto store = [&](int s) {
    mk.template store<KSTR>(kbuf(s));
    mv.template store<VSTR>(vbuf(s));
    if (wave == 0) {
      const uint64_t bits = __ballot(flag != 0);
      if (lane == 0) *fbuf(s) = bits;
    }
  };

  // ---- prologue: tile 0 into LDS, indices of tile 1 in flight
  ks.issue_idx(0, rows);
  fetch(0);
  ks.issue_idx(1, rows);
  store(0);
  __syncthreads();

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  for (int t = 0; t < ks.n_tiles; ++t) {
    const int cur = t & 1;
    // Tile t + 1 (all-absent past the last tile: zero loads, unused store).
    fetch(t + 1);
    ks.issue_idx(t + 2, rows);
    const T* kt = kbuf(cur);
    const T* vt = vbuf(cur);

    // ---- S^T = K Q^T
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2) sacc[kb2] = f32x16{};
    if constexpr (BF) {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2) {
          const bf16x8 a = *(const bf16x8*)(kt + (kb2 * 32 + qn) * KSTR + kk * 16 + hh * 8);
          sacc[kb2] = mfma32x16(a, qreg[kk], sacc[kb2]);
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < D / 2; ++kk) {
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2) {
          const float a = kt[(kb2 * 32 + qn) * KSTR + kk * 2 + hh];
          sacc[kb2] = mfma32x2f(a, qreg[kk], sacc[kb2]);
        }
      }
    }

    if (!ks.full(t, r0, p.n)) mask_scores(sacc, ks.keep64(t, my_row, p.a, p.n, *fbuf(cur)), hh, -INFINITY);
    softmax_tile(sacc, oacc, m_run, l_run, p.scale_log2);

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
          const int kr = 16 * c + 4 * (g >> 1) + (li >> 2);
          const bf16x4 lo = lds_read_tr16(vt + kr * VSTR + dim);
          const bf16x4 hi = lds_read_tr16(vt + (kr + 8) * VSTR + dim);
          const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[db] = mfma32x16(a, pb, oacc[db]);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < BK / 2; ++c) {
        const int kb2 = c >> 4, rr = c & 15;
        const int kr = kb2 * 32 + 8 * (rr >> 2) + 4 * hh + (rr & 3);
        const float pb = sacc[kb2][rr];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const float a = vt[kr * VSTR + db * 32 + qn];
          oacc[db] = mfma32x2f(a, pb, oacc[db]);
        }
      }
    }

    store(cur ^ 1);
    __syncthreads();
  }

  store_rows<T>(p, oacc, m_run, l_run, b, h, my_row, hh);
}

// ---------------------------------------------------------------- bf16, 8 waves, ping-pong
//
// Same traversal and numerics.  The two waves that share a SIMD (waves w and
// w + 4 of the workgroup) alternate between a matrix phase C and a vector
// phase V, so one keeps the matrix core busy while the other runs the softmax:
//   C(t): S(t+1) = K(t+1) Q^T and O^T += V(t)^T P(t)^T      (32 MFMAs)
//   V(t): mask, running max, exponentials of S(t+1) -> P(t+1), row sums
// Every wave runs C(t), barrier, V(t), barrier; waves 4-7 pass one extra
// barrier first, so their C(t) runs beside the V(t) of waves 0-3.  In that
// shared interval both groups write their halves of K(t+2) and V(t+1) into
// LDS (group 0 from its V phase, group 1 from its C phase), over the buffers
// of K(t) and V(t-1), which every wave finished reading an interval earlier.
// Group 0 starts the global loads of its halves of K(t+3), V(t+2) after the
// first MFMAs of its C(t+1), where the issue overlaps the matrix core; group
// 1, whose C phase also holds its LDS stores, starts them in its V(t), an
// interval earlier (phase timers: its C phase bounded the shared interval).
// The separator masks of the tiles rotate through four slots: tile t's mask
// is read in V(t-1) while K(t+2)'s is written in the same interval.

template <int D>
__global__ __launch_bounds__(512) void fwd_pp_kernel(FwdParams p) {
  using LY = FwdLayout<bf16, D>;
  constexpr int NT = 512, BQ = 256;
  constexpr int KSTR = LY::KSTR, VSTR = LY::VSTR;
  constexpr int NKB = BK / 32;  // 32-key blocks per tile
  constexpr int NDB = D / 32;   // 32-dim blocks
  constexpr int KK = D / 16;    // 16-dim steps of the score product

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = wave >> 2;
  const TileWork tw = tile_work(blockIdx.x, p.B * p.Hq * p.n_qtiles, p.Hq, p.Hkv, p.n_qtiles);
  const int b = tw.b, h = tw.h;
  const int kvh = h / (p.Hq / p.Hkv);
  const int q0 = tw.qt * BQ;
  const int r0 = q0 + wave * 32;
  const int qn = lane & 31, hh = lane >> 5;
  const int my_row = r0 + qn;

  const bf16* qb = (const bf16*)p.q + b * p.sq[0] + h * p.sq[1];
  const bf16* kb = (const bf16*)p.k + b * p.sk[0] + kvh * p.sk[1];
  const bf16* vb = (const bf16*)p.v + b * p.sv[0] + kvh * p.sv[1];

  // ---- queries (B operand of the score product) in registers
  bf16x8 qreg[KK];
  {
    const bool ok = my_row < p.L;
    const bf16* qrow = qb + (int64_t)(ok ? my_row : 0) * p.sq[2];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qreg[kk] = __builtin_bit_cast(bf16x8, ok ? ld16(qrow + kk * 16 + hh * 8) : u32x4{0, 0, 0, 0});
  }

  using MV = RowMover<bf16, D, NT>;
  constexpr int PT = MV::PT;
  KeyStream<PT> ks;
  ks.init(q0, BQ, p.L, p.a, p.n, p.sep_before + (size_t)b * (p.L + 1), p.sep_idx + (size_t)b * p.L,
          p.is_sep + (size_t)b * p.L);
  const rsrc_t krs = make_rsrc(kb, p.k_span), vrs = make_rsrc(vb, p.v_span);
  const uint32_t krow = (uint32_t)(p.sk[2] * 2), vrow = (uint32_t)(p.sv[2] * 2);
  int rows[PT], key_k[PT], key_v[PT];
  MV::rows(rows);
  MV mk, mv;
  uint32_t flag = 0;

  auto kbuf = [&](int s) { return (bf16*)(smem + (s & 1) * LY::K_BYTES); };
  auto vbuf = [&](int s) { return (bf16*)(smem + 2 * LY::K_BYTES + (s & 1) * LY::V_BYTES); };
  auto fslot = [&](int t) { return (uint64_t*)(smem + 2 * LY::K_BYTES + 2 * LY::V_BYTES + (t & 3) * 8); };
  auto store_flag = [&](int t) {
    if (wave == 0) {
      const uint64_t bits = __ballot(flag != 0);
      if (lane == 0) *fslot(t) = bits;
    }
  };
  // Store site of interval t: K(t+2), V(t+1) into LDS; the loads of K(t+3),
  // V(t+2) start after the first MFMAs of the next matrix phase.
  auto store_site = [&](int t) {
    mk.template store<KSTR>(kbuf(t + 2));
    mv.template store<VSTR>(vbuf(t + 1));
    store_flag(t + 2);
  };
  auto fetch_site = [&](int t) {
    ks.keys(t + 3, rows, key_k);
    mk.load(krs, krow, key_k);
    mv.load(vrs, vrow, key_v);
    if (wave == 0) flag = ks.flag_byte(t + 3, lane);
    ks.issue_idx(t + 4, rows);
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
  auto matrix_phase = [&](const bf16* kt, const bf16* vt, int fetch_t) {
    const int g = lane >> 4, li = lane & 15;
    auto opnd = [&](int i) -> bf16x8 {
      if (i < NS) return *(const bf16x8*)(kt + ((i % NKB) * 32 + qn) * KSTR + (i / NKB) * 16 + hh * 8);
      // lane li of group g reads V[key_base + li/4][dim_base + 4*(li%4)]
      const int c = (i - NS) / NDB, db = (i - NS) % NDB;
      const int dim = db * 32 + 16 * (g & 1) + 4 * (li & 3);
      const int kr = 16 * c + 4 * (g >> 1) + (li >> 2);
      const bf16x4 lo = lds_read_tr16(vt + kr * VSTR + dim);
      const bf16x4 hi = lds_read_tr16(vt + (kr + 8) * VSTR + dim);
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
      if (i == 2 && fetch_t >= 0) fetch_site(fetch_t);  // beside the MFMAs, not in front of them
      if (i < NS) {
        sacc[i % NKB] = mfma32x16(op[i], qreg[i / NKB], sacc[i % NKB]);
      } else {
        const int j = i - NS;
        oacc[j % NDB] = mfma32x16(op[i], pb[j / NDB], oacc[j % NDB]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Vector phase: softmax of tile t's scores (in sacc) into pb.
  auto vector_phase = [&](int t) {
    if (!ks.full(t, r0, p.n)) mask_scores(sacc, ks.keep64(t, my_row, p.a, p.n, *fslot(t)), hh, -INFINITY);
    softmax_tile(sacc, oacc, m_run, l_run, p.scale_log2);
#pragma unroll
    for (int c = 0; c < BK / 16; ++c)
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) pb[c][sl] = (bf16)sacc[c >> 1][(c & 1) * 8 + sl];
  };

  // ---- prologue: K(0), V(0), K(1) in LDS, K(2) and V(1) in flight; P(0)
  ks.issue_idx(0, rows);
  ks.keys(0, rows, key_k);
  mk.load(krs, krow, key_k);
  mv.load(vrs, vrow, key_k);
  if (wave == 0) flag = ks.flag_byte(0, lane);
  ks.issue_idx(1, rows);
  mk.template store<KSTR>(kbuf(0));
  mv.template store<VSTR>(vbuf(0));
  store_flag(0);
  ks.keys(1, rows, key_v);
  mk.load(krs, krow, key_v);
  if (wave == 0) flag = ks.flag_byte(1, lane);
  ks.issue_idx(2, rows);
  mk.template store<KSTR>(kbuf(1));
  store_flag(1);
  ks.keys(2, rows, key_k);
  mk.load(krs, krow, key_k);
  mv.load(vrs, vrow, key_v);
  if (wave == 0) flag = ks.flag_byte(2, lane);
  ks.issue_idx(3, rows);
#pragma unroll
  for (int u = 0; u < PT; ++u) key_v[u] = key_k[u];
  __syncthreads();
  {
    const bf16* kt = kbuf(0);
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2) sacc[kb2] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) {
        const bf16x8 a = *(const bf16x8*)(kt + (kb2 * 32 + qn) * KSTR + kk * 16 + hh * 8);
        sacc[kb2] = mfma32x16(a, qreg[kk], sacc[kb2]);
      }
  }
  vector_phase(0);

  if (grp == 1) __syncthreads();  // group 1 runs one phase behind
  for (int t = 0; t < ks.n_tiles; ++t) {
    // ---- C(t)
    __builtin_amdgcn_s_setprio(1);
    matrix_phase(kbuf(t + 1), vbuf(t), grp == 0 ? t - 1 : -1);
    __builtin_amdgcn_s_setprio(0);
    if (grp == 1) store_site(t);
    __syncthreads();
    // ---- V(t)
    if (t + 1 < ks.n_tiles) vector_phase(t + 1);
    if (grp == 0) store_site(t);
    else fetch_site(t);
    __syncthreads();
  }
  if (grp == 0) __syncthreads();

  store_rows<bf16>(p, oacc, m_run, l_run, b, h, my_row, hh);
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
  using LY = FwdLayout<T, D>;
  const int smem = 2 * (LY::K_BYTES + LY::V_BYTES + 16);
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
