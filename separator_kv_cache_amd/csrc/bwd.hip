// Backward of attention under the SepLLM mask (anthology record LIT-748,
// "Key takeaways": the mask is trained through; the mask bullet defines it).
//
// With P the masked softmax and D_i = sum_d dO_i O_i:
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Two kernels, every output row written by one workgroup:
//  * dq_kernel: query-major, the forward's traversal (gathered anchors, then
//    the band).  Its prologue computes D for its rows and stores it.
//  * dkdv_kernel: key-major.  Keys are split into two compacted classes:
//    anchors (sinks j < a and separators), which every later row sees, and
//    plain tokens, which only rows within n see.  A workgroup owns 32*WAVES
//    keys of one class and walks the rows that can see them: [first key, L)
//    for anchors, [first key, last key + n) for plain keys, summing over the
//    q heads of its KV head.  Which workgroup takes which key tile is decided
//    when it starts, from a counter per XCD (the only atomics); the results do
//    not depend on it.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "traverse.h"

namespace {

constexpr int BK = KTILE;  // keys per tile (dq)
constexpr int RB = 64;   // rows per block (dkdv)

struct BwdParams {
  const bf16 *q, *k, *v, *o, *dout;
  const float* lse;
  bf16 *dq, *dk, *dv;
  float* dsum;  // D [B, Hq, L]
  uint32_t* queue;  // dkdv: the next key tile of each XCD's range (8 counters, 128 bytes apart)
  int64_t sq[3], sk[3], sv[3], so[3];
  uint32_t k_span, v_span;  // bytes of one (sequence, KV head) slice of K, V
  uint32_t q_span, o_span;  // bytes of one (sequence, q head) slice of Q (dQ), O (dO)
  const uint8_t* is_sep;
  const int32_t* sep_idx;
  const int32_t* sep_before;
  const int32_t* sep_cnt;
  const int32_t* plain_idx;
  const int32_t* plain_cnt;
  int B, Hq, Hkv, L, a, n;
  int n_qtiles;     // dq
  int n_key_tiles;  // dkdv: tiles per class
  float scale, scale_log2;
};

// ---------------------------------------------------------------- dq
//
// The forward's lockstep traversal (traverse.h): every wave loads its share
// of key tile t+1 into registers while tile t is computed from LDS.  Wave w
// owns query rows [q0 + 32w, q0 + 32w + 32); per tile it forms S^T = K Q^T
// and dP^T = V dO^T (one query per lane), dS^T = P^T (dP^T - D) with
// P = exp2(scale_log2 S - lse2), then dQ^T += K^T dS^T with K^T from
// transposing LDS reads.

// Row strides of tiles read both by 16-byte row reads (MFMA operands along a
// row) and by transposing reads: an odd number of 16-byte chunks keeps the
// row reads of 16 lanes on distinct banks (the stride at d = 64).
template <int D>
constexpr int dual_read_stride() { return D == 128 ? 152 : 88; }

// dQ's K and V tiles.  At d = 128 the rows are 160 elements apart, which
// keeps the four rows of a transposing read of K (dQ's A operand) in
// distinct banks, and chunk c of row r sits at chunk position
// c ^ ((r >> 2) & 3), which spreads the 16 rows of a row read (S and dP) over
// all banks too (the layout of dK/dV's Q/dO tiles below).  At d = 64 the
// stride is padded instead.
template <int D>
struct DqLayout {
  static constexpr bool SWZ = D == 128;
  static constexpr int STR = SWZ ? 160 : dual_read_stride<D>();
  __device__ static int tau(int r) { return SWZ ? (r >> 2) & 3 : 0; }
  static constexpr int K_BYTES = BK * STR * 2;
  static constexpr int BUF_BYTES = 2 * K_BYTES + 16;  // K, V, separator bits
};

template <int D, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void dq_kernel(BwdParams p) {
  using LY = DqLayout<D>;
  constexpr int NT = WAVES * 64, BQ = WAVES * 32, STR = LY::STR;
  constexpr int NKB = BK / 32, NDB = D / 32, NKK = D / 16;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const TileWork tw = tile_work(blockIdx.x, p.B * p.Hq * p.n_qtiles, p.Hq, p.Hkv, p.n_qtiles);
  const int b = tw.b, h = tw.h;
  const int kvh = h / (p.Hq / p.Hkv);
  const int q0 = tw.qt * BQ;
  const int r0 = q0 + wave * 32;
  const int qn = lane & 31, hh = lane >> 5;
  const int my_row = r0 + qn;
  const bool row_ok = my_row < p.L;

  const bf16* kb = p.k + b * p.sk[0] + kvh * p.sk[1];
  const bf16* vb = p.v + b * p.sv[0] + kvh * p.sv[1];

  // ---- prologue: Q, dO (B operands), LSE, D = rowsum(dO * O)
  bf16x8 qreg[NKK], doreg[NKK];
  float dpart = 0.f;
  {
    const int rr = row_ok ? my_row : 0;
    const bf16* qrow = p.q + b * p.sq[0] + h * p.sq[1] + (int64_t)rr * p.sq[2];
    const bf16* drow = p.dout + b * p.so[0] + h * p.so[1] + (int64_t)rr * p.so[2];
    const bf16* orow = p.o + b * p.so[0] + h * p.so[1] + (int64_t)rr * p.so[2];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int off = kk * 16 + hh * 8;
      u32x4 xq = row_ok ? ld16(qrow + off) : u32x4{0, 0, 0, 0};
      u32x4 xd = row_ok ? ld16(drow + off) : u32x4{0, 0, 0, 0};
      u32x4 xo = row_ok ? ld16(orow + off) : u32x4{0, 0, 0, 0};
      qreg[kk] = __builtin_bit_cast(bf16x8, xq);
      doreg[kk] = __builtin_bit_cast(bf16x8, xd);
      const bf16x8 ov = __builtin_bit_cast(bf16x8, xo);
#pragma unroll
      for (int s = 0; s < 8; ++s) dpart += bf2f(doreg[kk][s]) * bf2f(ov[s]);
    }
  }
  const float Dv = dpart + xor32(dpart);
  const size_t rowid = ((size_t)b * p.Hq + h) * p.L + (row_ok ? my_row : 0);
  const float lse2 = row_ok ? p.lse[rowid] * 1.4426950408889634f : 0.f;
  if (row_ok && hh == 0) p.dsum[rowid] = Dv;
  // the dK/dV kernel that follows takes its key tiles from these counters
  if (blockIdx.x == 0 && threadIdx.x < 8)
    __hip_atomic_store(p.queue + 32 * threadIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  using MV = RowMover<bf16, D, NT>;
  constexpr int PT = MV::PT;
  KeyStream<PT> ks;
  ks.init(q0, BQ, p.L, p.a, p.n, p.sep_before + (size_t)b * (p.L + 1), p.sep_idx + (size_t)b * p.L,
          p.is_sep + (size_t)b * p.L);
  const rsrc_t krs = make_rsrc(kb, p.k_span), vrs = make_rsrc(vb, p.v_span);
  const uint32_t krow = (uint32_t)(p.sk[2] * 2), vrow = (uint32_t)(p.sv[2] * 2);
  int rows[PT], key[PT];
  MV::rows(rows);
  MV mk, mv;
  uint32_t flag = 0;

  auto kbuf = [&](int s) { return (bf16*)(smem + s * LY::BUF_BYTES); };
  auto vbuf = [&](int s) { return (bf16*)(smem + s * LY::BUF_BYTES + LY::K_BYTES); };
  auto fbuf = [&](int s) { return (uint64_t*)(smem + s * LY::BUF_BYTES + 2 * LY::K_BYTES); };
  auto fetch = [&](int t) {
    ks.keys(t, rows, key);
    mk.load(krs, krow, key);
    mv.load(vrs, vrow, key);
    if (wave == 0) flag = ks.flag_byte(t, lane);
  };
  auto store = [&](int s) {
    mk.template store<STR, LY::SWZ>(kbuf(s));
    mv.template store<STR, LY::SWZ>(vbuf(s));
    if (wave == 0) {
      const uint64_t bits = __ballot(flag != 0);
      if (lane == 0) *fbuf(s) = bits;
    }
  };

  ks.issue_idx(0, rows);
  fetch(0);
  ks.issue_idx(1, rows);
  store(0);
  __syncthreads();

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16{};

  for (int t = 0; t < ks.n_tiles; ++t) {
    const int cur = t & 1;
    const bf16* kt = kbuf(cur);
    const bf16* vt = vbuf(cur);

    // S^T and dP^T as one stream of MFMAs (S, dP alternating) whose LDS
    // operand reads run PD MFMAs ahead; the next tile's loads are issued
    // after the first MFMAs, so their address work runs beside the matrix
    // core instead of in front of it.
    constexpr int NSD = 2 * NKK * NKB, PD = 4;
    // row x * 32 + qn, chunk c = 2 kk + hh at position 4 (c >> 2) + ((c & 3) ^ tau)
    const int ta = LY::tau(qn);
    auto opnd = [&](int i) -> bf16x8 {
      const int kk = i / (2 * NKB), x = (i >> 1) % NKB;
      const int pos = 4 * (kk >> 1) + ((2 * (kk & 1) + hh) ^ ta);
      return *(const bf16x8*)(((i & 1) ? vt : kt) + (x * 32 + qn) * STR + pos * 8);
    };
    f32x16 sacc[NKB], dpacc[NKB];
#pragma unroll
    for (int x = 0; x < NKB; ++x) { sacc[x] = f32x16{}; dpacc[x] = f32x16{}; }
    bf16x8 op[NSD];
#pragma unroll
    for (int i = 0; i < PD; ++i) op[i] = opnd(i);
#pragma unroll
    for (int i = 0; i < NSD; ++i) {
      if (i + PD < NSD) op[i + PD] = opnd(i + PD);
      if (i == 2) {
        fetch(t + 1);  // all-absent past the last tile
        ks.issue_idx(t + 2, rows);
      }
      const int kk = i / (2 * NKB), x = (i >> 1) % NKB;
      if (i & 1) dpacc[x] = mfma32x16(op[i], doreg[kk], dpacc[x]);
      else sacc[x] = mfma32x16(op[i], qreg[kk], sacc[x]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // dS^T = P^T (dP^T - D), kept in sacc; masked keys get P = exp2(-inf) = 0
    if (!ks.full(t, r0, p.n)) mask_scores(sacc, ks.keep64(t, my_row, p.a, p.n, *fbuf(cur)), hh, -INFINITY);
#pragma unroll
    for (int x = 0; x < NKB; ++x)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sacc[x][r] = fast_exp2(__builtin_fmaf(sacc[x][r], p.scale_log2, -lse2)) * (dpacc[x][r] - Dv);

    // dQ^T += K^T dS^T (K^T through LDS transposing reads): rows kr and
    // kr + 8 (tau (g >> 1) and (g >> 1) + 2), chunk 4 db + clo
    const int g = lane >> 4, li = lane & 15;
    const int clo = 2 * (g & 1) + ((li & 3) >> 1);
    const int kr0 = 4 * (g >> 1) + (li >> 2);
    const int tr_lo = kr0 * STR + (clo ^ LY::tau(kr0)) * 8 + 4 * (li & 1);
    const int tr_hi = (kr0 + 8) * STR + (clo ^ LY::tau(kr0 + 8)) * 8 + 4 * (li & 1);
#pragma unroll
    for (int c = 0; c < BK / 16; ++c) {
      bf16x8 bsv;
#pragma unroll
      for (int s = 0; s < 8; ++s) bsv[s] = (bf16)sacc[c >> 1][(c & 1) * 8 + s];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x4 lo = lds_read_tr16(kt + 16 * c * STR + 32 * db + tr_lo);
        const bf16x4 hi = lds_read_tr16(kt + 16 * c * STR + 32 * db + tr_hi);
        const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        dqacc[db] = mfma32x16(a, bsv, dqacc[db]);
      }
    }
    store(cur ^ 1);
    __syncthreads();
  }

  if (row_ok) {
    bf16* drow = p.dq + b * p.sq[0] + h * p.sq[1] + (int64_t)my_row * p.sq[2];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 w = {(bf16)(dqacc[db][4 * i + 0] * p.scale), (bf16)(dqacc[db][4 * i + 1] * p.scale),
                    (bf16)(dqacc[db][4 * i + 2] * p.scale), (bf16)(dqacc[db][4 * i + 3] * p.scale)};
        *(bf16x4*)(drow + db * 32 + 8 * i + 4 * hh) = w;
      }
  }
}

// ---------------------------------------------------------------- dk, dv
//
// Key-major: a workgroup of 8 waves owns KT = 128 keys of one class and walks
// the rows that see them in blocks of RB = 64 rows, for each q head of its KV
// head in turn (iteration j = row block * group + head).  Waves 2kg and
// 2kg + 1 own the same 32 keys (key group kg); the wave with hf = w % 2 forms
// S = Q K^T and dP = dO V^T for the rows [32 hf, 32 hf + 32) and from them P
// and dS, which the two waves exchange through LDS; each then accumulates
// dV^T += dO^T P and dK^T += Q^T dS over all 64 rows for the head dims
// [D/2 hf, D/2 hf + D/2).  No MFMA work is duplicated, and a wave keeps K, V
// of its keys for all dims but dK, dV for half of them, which fits two waves
// per SIMD.
//
// Every wave alternates a matrix phase M(j) (the MFMAs of S, dP for block
// j + 1 and of dV, dK for block j) and a vector phase V(j) (P and dS of block
// j from the scores M(j - 1) left in registers, written to LDS), with a
// workgroup barrier after each.  The two waves on a SIMD (w and w + 4) are in
// different halves of the workgroup, and the second half runs one phase
// behind the first, so at any time one wave of a SIMD issues only MFMAs (at
// raised priority) while the other issues only vector work.  Both waves of a
// key-group pair are in the same half, so their exchange sits between V(j)
// and M(j) of that half.
//
// Q/dO tiles (with lse and D of their rows) rotate through three LDS buffers:
// tile j is read from M(j - 1) of the first half to M(j) of the second.  Each
// half moves its own 32 rows of a tile (global -> registers -> LDS): the
// first half stores rows [0, 32) of tile j + 1 in its V(j), the second half
// rows [32, 64) of tile j + 2 in its V(j), which falls between the last read
// of the buffer's previous tile and the first read of the new one.  Each
// half issues the loads of its next rows from inside the following M phase,
// between its first MFMAs: there the address arithmetic and the load issue
// run beside the matrix core instead of in front of it (measured: issuing
// them at the head of either phase put several hundred cycles on the
// critical path of every interval).

// Q/dO tiles of dK/dV are read by rows (16 lanes, one 16-byte chunk of 16
// consecutive rows) and by transposing reads (32 lanes, 8 bytes of 4
// consecutive rows each, 64 bytes per row).  At d = 128 the row stride is
// 160 elements, which keeps the transposing reads' four rows in distinct
// banks, and chunk c of row r sits at chunk position c ^ ((r >> 2) & 3),
// which spreads the 16 rows of a row read over all banks as well.  The XOR
// only touches the low two bits of the chunk index, so a lane's addresses
// are two precomputed bases plus immediates.  At d = 64 the stride is padded
// instead.
template <int D>
struct DkvLayout {
  static constexpr bool SWZ = D == 128;
  static constexpr int STR = SWZ ? 160 : dual_read_stride<D>();  // Q/dO row stride (elements)
  __device__ static int tau(int r) { return SWZ ? (r >> 2) & 3 : 0; }
  static constexpr int T_BYTES = RB * STR * 2;                // one Q or dO tile
  static constexpr int BUF_BYTES = 2 * T_BYTES + 2 * RB * 4;  // Q, dO, lse2, D
  static constexpr int NBUF = 3;
  static constexpr int PSTR = RB + 8;                         // P/dS: row stride per key (elements)
  static constexpr int X_BYTES = 128 * PSTR * 2;              // P or dS of the 128 keys
  static constexpr int SMEM = NBUF * BUF_BYTES + 2 * X_BYTES;
  static_assert(SMEM <= 160 * 1024, "dK/dV tiles exceed the LDS of a workgroup");
};

// One key tile of the dK/dV pass: logical tile lam (below).
template <int D>
__device__ __forceinline__ void dkdv_tile(const BwdParams& p, int lam) {
  using LY = DkvLayout<D>;
  constexpr int KT = 128, STR = LY::STR, PSTR = LY::PSTR;
  constexpr int NKK = D / 16;          // 16-dim steps of S and dP
  constexpr int HD = D / 2;            // head dims whose dK, dV a wave accumulates
  constexpr int NDBH = HD / 32;        // 32-dim blocks of them
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int HT = 256;              // threads of a half
  constexpr int PT = (RB / 2) * CH / HT;  // chunks per thread of a half tile (Q and dO each)
  static_assert(PT * HT == (RB / 2) * CH, "half-tile chunks must divide the half workgroup");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kg = wave >> 1, hf = wave & 1, half = wave >> 2;
  const int ht = (int)threadIdx.x & (HT - 1);
  const int per = 2 * p.n_key_tiles;
  const int bk = lam / per, rem = lam % per;
  const int b = bk / p.Hkv, kvh = bk % p.Hkv;
  const bool anchors = rem < p.n_key_tiles;
  const int tile = anchors ? rem : rem - p.n_key_tiles;
  const int n_sink = min(p.a, p.L);
  const int count = anchors ? n_sink + p.sep_cnt[b] : p.plain_cnt[b];
  const int c0 = tile * KT;
  if (c0 >= count) return;  // uniform across the workgroup
  const int32_t* si = p.sep_idx + (size_t)b * p.L;
  const int32_t* pl = p.plain_idx + (size_t)b * p.L;
  auto key_at = [&](int c) -> int { return anchors ? (c < n_sink ? c : si[c - n_sink]) : pl[c]; };

  const int qn = lane & 31, hh = lane >> 5;
  const int my_c = c0 + kg * 32 + qn;
  const bool key_ok = my_c < count;
  const int my_key = key_ok ? key_at(my_c) : 0;
  const int j_first = key_at(c0), j_last = key_at(min(c0 + KT, count) - 1);
  const int row_end = anchors ? p.L : min(p.L, j_last + p.n);
  const int key_hi = !key_ok ? -1 : anchors ? p.L : min(p.L, my_key + p.n);  // rows [my_key, key_hi) see it

  // ---- this lane's key as B operands (K^T, V^T rows), all head dims
  bf16x8 kreg[NKK], vreg[NKK];
  {
    const bf16* krow = p.k + b * p.sk[0] + kvh * p.sk[1] + (int64_t)my_key * p.sk[2];
    const bf16* vrow = p.v + b * p.sv[0] + kvh * p.sv[1] + (int64_t)my_key * p.sv[2];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int off = kk * 16 + hh * 8;
      kreg[kk] = __builtin_bit_cast(bf16x8, key_ok ? ld16(krow + off) : u32x4{0, 0, 0, 0});
      vreg[kk] = __builtin_bit_cast(bf16x8, key_ok ? ld16(vrow + off) : u32x4{0, 0, 0, 0});
    }
  }

  const int group = p.Hq / p.Hkv;
  const int n_rb = (row_end - j_first + RB - 1) / RB;
  const int n_it = n_rb * group;
  // Anchor tiles walk their row blocks last to first.  They all end at row
  // L, so the anchor tiles of one (sequence, KV head), which run together on
  // one XCD, read the same rows at the same time and share them in L2;
  // walking up from their different first keys they would share none.
  // (The band tiles' ranges are staggered at both ends, so their order does
  // not change what they share.)
  const int rs_first = anchors ? j_first + RB * (n_rb - 1) : j_first;
  const int rs_step = anchors ? -RB : RB;
  // LDS: P and dS first, then the three tile buffers, so that every access is
  // a per-lane base plus an offset below 64 KiB
  char* xp = smem;              // P of the 128 keys, [key][row]
  char* xd = xp + LY::X_BYTES;  // dS
  // (unsigned offsets, so that constant parts fold into the LDS instructions)
  auto tbuf_off = [&](int j) -> uint32_t {  // j >= -1
    return 2u * LY::X_BYTES + ((uint32_t)(j + LY::NBUF) % (uint32_t)LY::NBUF) * (uint32_t)LY::BUF_BYTES;
  };
  // A lane's LDS address in tile buffer j: its own offset plus the buffer's,
  // made opaque so that the compiler adds the constant parts of each access
  // as instruction offsets instead of keeping one register per access.
  auto at_buf = [&](int j, uint32_t lane_off) -> char* {
    uint32_t o = tbuf_off(j) + lane_off;
    asm volatile("" : "+v"(o));
    return smem + o;
  };

  // ---- this half's 32 rows of a Q/dO tile: global -> registers -> LDS.
  // Thread x of the half moves chunk x % CH of rows 32 half + x / CH +
  // u * (HT / CH); rows past L load as zeros and get lse2 = +inf, so their P
  // is exactly 0.  fetch_half() is called for tiles 0, 1, 2, ... in order:
  // (row block, head) of the next call advance as counters.
  u32x4 qr[PT], dr[PT];
  float lse_r = 0.f, d_r = 0.f;
  bool lse_ok = false;
  int f_rs = rs_first, f_h = kvh * group;
  auto fetch_half = [&](int j) {
    // (uniform values; readfirstlane keeps the buffer resources in scalar
    // registers, else each load becomes a loop over distinct descriptors)
    const int rs = __builtin_amdgcn_readfirstlane(f_rs), h = __builtin_amdgcn_readfirstlane(f_h);
    const bool live = j < n_it;
    if (++f_h == (kvh + 1) * group) { f_h = kvh * group; f_rs += rs_step; }
    const rsrc_t qrs = make_rsrc(p.q + b * p.sq[0] + h * p.sq[1], p.q_span);
    const rsrc_t drs = make_rsrc(p.dout + b * p.so[0] + h * p.so[1], p.o_span);
    const uint32_t qrow = (uint32_t)(p.sq[2] * 2), orow = (uint32_t)(p.so[2] * 2);
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int i = rs + 32 * half + ht / CH + u * (HT / CH);
      const bool ok = live && i < p.L;
      const uint32_t c16 = (ht % CH) * 16;
      qr[u] = bld16(qrs, ok ? (uint32_t)i * qrow + c16 : BUF_OOB);
      dr[u] = bld16(drs, ok ? (uint32_t)i * orow + c16 : BUF_OOB);
    }
    if (ht < 32) {
      const size_t rowb = ((size_t)b * p.Hq + h) * p.L;
      const rsrc_t lrs = make_rsrc(p.lse + rowb, (uint32_t)p.L * 4u);
      const rsrc_t srs = make_rsrc(p.dsum + rowb, (uint32_t)p.L * 4u);
      const int i = rs + 32 * half + ht;
      lse_ok = live && i < p.L;
      const uint32_t off = lse_ok ? (uint32_t)i * 4u : BUF_OOB;
      lse_r = __builtin_bit_cast(float, bld4(lrs, off));
      d_r = __builtin_bit_cast(float, bld4(srs, off));
    }
  };
  // (row 32 half + ht / CH + u (HT / CH) has tau of ht / CH + u (HT / CH):
  // HT / CH is a multiple of 16 at d = 128)
  const uint32_t st_off = (uint32_t)((32 * half + ht / CH) * STR * 2 + ((ht % CH) ^ LY::tau(ht / CH)) * 16);
  auto store_half = [&](int j) {
    char* buf = at_buf(j, st_off);
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      st16(buf + u * (HT / CH) * STR * 2, qr[u]);
      st16(buf + LY::T_BYTES + u * (HT / CH) * STR * 2, dr[u]);
    }
    if (ht < 32) {
      float* ls = (float*)(smem + tbuf_off(j) + 2 * LY::T_BYTES);
      ls[32 * half + ht] = lse_ok ? lse_r * 1.4426950408889634f : INFINITY;
      ls[RB + 32 * half + ht] = lse_ok ? d_r : 0.f;
    }
  };

  f32x16 dkacc[NDBH], dvacc[NDBH];
#pragma unroll
  for (int db = 0; db < NDBH; ++db) { dkacc[db] = f32x16{}; dvacc[db] = f32x16{}; }
  f32x16 sacc, dpacc;  // S, dP of the next block, from M(j - 1) to V(j)
  const int g = lane >> 4, li = lane & 15;

  // ---- matrix phase M(j): with WITH_DKV, dV^T += dO^T P and dK^T += Q^T dS
  // over the 64 rows of block j for head dims [HD hf, HD hf + HD): A through
  // transposing reads of the tile, B = P, dS of this key group (lane l: key
  // l % 32, the 8 rows at position 16c + 8(l / 32)); then S, dP for rows
  // [32 hf, 32 hf + 32) of block j + 1 x this lane's key (lane = key; S and
  // dP alternate so that consecutive MFMAs are independent).  One stream of
  // MFMAs whose LDS operand reads run PD MFMAs ahead; the scores come last,
  // so their accumulators are not live beside those of the dV, dK part.  On
  // the last block the scores of the (absent) next block are formed from
  // whatever the buffer holds and never used.
  constexpr int NS = 2 * NKK, NB = (RB / 16) * NDBH * 2, PD = 4;
  const int r0 = 4 * (g >> 1) + (li >> 2);
  const int clo = 2 * (g & 1) + ((li & 3) >> 1);
  const uint32_t tr_lo = (uint32_t)(r0 * STR * 2 + HD * hf * 2 + ((clo ^ LY::tau(r0)) * 16) + 8 * (li & 1));
  const uint32_t tr_hi = (uint32_t)((r0 + 8) * STR * 2 + HD * hf * 2 + ((clo ^ LY::tau(r0 + 8)) * 16) + 8 * (li & 1));
  const int ta = LY::tau(32 * hf + qn);
  const uint32_t rd0 = (uint32_t)((32 * hf + qn) * STR * 2 + ((hh ^ ta) * 16));
  const uint32_t rd1 = (uint32_t)((32 * hf + qn) * STR * 2 + (((2 + hh) ^ ta) * 16));
  auto matrix_phase = [&](auto with_dkv, int j, int fetch_j) {
    constexpr bool DKV = decltype(with_dkv)::value;
    constexpr int N0 = DKV ? NB : 0, NM = N0 + NS;
    // dV, dK operands: row 4 (g >> 1) + (li >> 2) (+ 8 for the upper half,
    // + 16 c), column HD hf + 16 (g & 1) + 4 (li & 3) (+ 32 db) of tile j
    const char* abase_lo = at_buf(j, tr_lo);
    const char* abase_hi = at_buf(j, tr_hi);
    const char* pb = xp + ((kg * 32 + qn) * PSTR + 8 * hh) * 2;
    const char* sb = xd + ((kg * 32 + qn) * PSTR + 8 * hh) * 2;
    // S, dP operands: row 32 hf + qn of tile j + 1, chunk c = 2 (i >> 1) + hh
    // at position 4 (c >> 2) + ((c & 3) ^ tau): two bases, by bit 1 of c
    const char* base0 = at_buf(j + 1, rd0);
    const char* base1 = at_buf(j + 1, rd1);
    // MFMA i < N0: chunk i / (2 NDBH), block (i >> 1) % NDBH, dV (even) / dK
    // (odd); i >= N0: k = i - N0 is S (even) / dP (odd) of dims 16 (k >> 1)
    auto opnd = [&](int i) -> bf16x8 {
      if (i < N0) {
        const int c = i / (2 * NDBH), db = (i >> 1) % NDBH;
        const int off = ((i & 1) ? 0 : LY::T_BYTES) + (16 * c * STR + 32 * db) * 2;  // dO for dV, Q for dK
        const bf16x4 lo4 = lds_read_tr16(abase_lo + off);
        const bf16x4 hi4 = lds_read_tr16(abase_hi + off);
        return bf16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      }
      const int k = (i - N0) >> 1;
      return *(const bf16x8*)(((k & 1) ? base1 : base0) + (((i - N0) & 1) ? LY::T_BYTES : 0) + (k >> 1) * 64);
    };
    bf16x8 op[NM], bp[RB / 16], bs[RB / 16];
    auto prefetch = [&](int i) {
      op[i] = opnd(i);
      if (i < N0 && i % (2 * NDBH) == 0) {  // first MFMA of a row chunk: its P and dS
        const int c = i / (2 * NDBH);
        bp[c] = *(const bf16x8*)(pb + 16 * c * 2);
        bs[c] = *(const bf16x8*)(sb + 16 * c * 2);
      }
    };
#pragma unroll
    for (int i = 0; i < PD; ++i) prefetch(i);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + PD < NM) prefetch(i + PD);
      if (DKV && i == 2) fetch_half(fetch_j);  // address work and issue beside the MFMAs
      if (i == N0) {
        sacc = f32x16{};
        dpacc = f32x16{};
      }
      if (i < N0) {
        const int c = i / (2 * NDBH), db = (i >> 1) % NDBH;
        if (i & 1) dkacc[db] = mfma32x16(op[i], bs[c], dkacc[db]);
        else dvacc[db] = mfma32x16(op[i], bp[c], dvacc[db]);
      } else {
        const int k = i - N0;
        if (k & 1) dpacc = mfma32x16(op[i], vreg[k >> 1], dpacc);
        else sacc = mfma32x16(op[i], kreg[k >> 1], sacc);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- vector phase V(j): P = exp2(scale_log2 S - lse2) on the rows of
  // block j that see the key, dS = P (dP - D); register r holds local row
  // 32 hf + 8(r/4) + 4 hh + r%4.  P, dS go to LDS per key in the order the
  // row contraction consumes them: its B slot s of a lane with hh = l/32
  // must hold row 16c + 8(s/4) + 4 hh + s%4 (the row the transposing read
  // puts in A slot s), so within each 16-row chunk the rows are stored as
  // 0-3, 8-11, 4-7, 12-15 and a lane reads its 8 values at position
  // 16c + 8 hh with one 16-byte read.
  int v_rs = rs_first, v_h = 0;  // row block of the next vector_phase call (called for j = 0, 1, ...)
  auto vector_phase = [&](int j) {
    const char* buf = smem + tbuf_off(j);
    const int rs = v_rs;
    if (++v_h == group) { v_h = 0; v_rs += rs_step; }
    // lse2 and D of this lane's rows: four runs of 4 consecutive rows
    const float* ls = (const float*)(buf + 2 * LY::T_BYTES) + 32 * hf + 4 * hh;
    f32x4 l2[4], dd[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      l2[q4] = *(const f32x4*)(ls + 8 * q4);
      dd[q4] = *(const f32x4*)(ls + RB + 8 * q4);
    }
    // The key is seen by the local rows [lo, lo + width); element r of this
    // lane is local row lr0 + 8(r/4) + r%4.  Blocks where it sees all of this
    // lane's rows skip the test (a wave-uniform branch).
    const int lr0 = 32 * hf + 4 * hh;
    const int lo = my_key - rs - lr0;
    const uint32_t width = (uint32_t)max(key_hi - my_key, 0);
    char* pw = xp + ((kg * 32 + qn) * PSTR + 32 * hf + 8 * hh) * 2;
    char* dw = xd + ((kg * 32 + qn) * PSTR + 32 * hf + 8 * hh) * 2;
    auto pds = [&](bool masked) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 pv, dv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q4 + e;
          float pr = fast_exp2(__builtin_fmaf(sacc[r], p.scale_log2, -l2[q4][e]));
          if (masked) pr = (uint32_t)(8 * q4 + e - lo) < width ? pr : 0.f;
          pv[e] = (bf16)pr;
          dv[e] = (bf16)(pr * (dpacc[r] - dd[q4][e]));
        }
        const int pos = 16 * (q4 >> 1) + 4 * (q4 & 1);  // rows 8 q4 + 4 hh + 0..3 of this wave's 32
        *(bf16x4*)(pw + pos * 2) = pv;
        *(bf16x4*)(dw + pos * 2) = dv;
      }
    };
    if (__all(lo <= 0 && (uint32_t)(27 - lo) < width)) pds(false);
    else pds(true);
  };

  // ---- prologue: tile 0 and rows [32, 64) of tile 1 in LDS; the first half
  // holds its rows of tile 1, the second half its rows of tile 2 in flight
  fetch_half(0);
  store_half(0);
  fetch_half(1);
  if (half == 1) {
    store_half(1);
    fetch_half(2);
  }
  __syncthreads();
  matrix_phase(std::false_type{}, -1, 0);  // S, dP of block 0

  if (half == 1) __syncthreads();  // the second half runs one phase behind
  for (int j = 0; j < n_it; ++j) {
    store_half(j + 1 + half);
    vector_phase(j);
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);
    matrix_phase(std::true_type{}, j, j + 2 + half);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
  }
  if (half == 0) __syncthreads();

  if (key_ok) {
    bf16* dkrow = p.dk + b * p.sk[0] + kvh * p.sk[1] + (int64_t)my_key * p.sk[2] + HD * hf;
    bf16* dvrow = p.dv + b * p.sv[0] + kvh * p.sv[1] + (int64_t)my_key * p.sv[2] + HD * hf;
#pragma unroll
    for (int db = 0; db < NDBH; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dim = db * 32 + 8 * i + 4 * hh;
        bf16x4 wk = {(bf16)(dkacc[db][4 * i + 0] * p.scale), (bf16)(dkacc[db][4 * i + 1] * p.scale),
                     (bf16)(dkacc[db][4 * i + 2] * p.scale), (bf16)(dkacc[db][4 * i + 3] * p.scale)};
        bf16x4 wv = {(bf16)dvacc[db][4 * i + 0], (bf16)dvacc[db][4 * i + 1], (bf16)dvacc[db][4 * i + 2],
                     (bf16)dvacc[db][4 * i + 3]};
        *(bf16x4*)(dkrow + dim) = wk;
        *(bf16x4*)(dvrow + dim) = wv;
      }
  }
}

// Persistent: one workgroup per compute unit, each taking key tiles until
// none is left.  Logical tiles: B * Hkv * 2 * n_key_tiles, (sequence, KV
// head) major, anchor tiles (the longest row ranges, longest first) before
// plain ones; when their number divides by 8, XCD x owns the range
// [x N/8, (x+1) N/8), so the key tiles of one (sequence, KV head) run on one
// XCD and share its L2 (spreading a head over all XCDs, to share the
// Infinity Cache instead, measured slower with more L2 misses).  A workgroup
// takes the next tile of its XCD's range from that range's counter, then of
// the other ranges once its own is exhausted: every tile is taken once, and
// the compute units of an XCD run its tiles longest first, each starting the
// next one as it finishes (launching one workgroup per tile instead left the
// order in which compute units receive workgroups to the dispatcher, which
// does not follow which ones are free: about 9 % of the pass was idle time).
// The counters are zeroed by the dQ kernel, which runs first.
template <int D>
__global__ __launch_bounds__(512) void dkdv_kernel(BwdParams p) {
  const int N = p.B * p.Hkv * 2 * p.n_key_tiles;
  const int R = N % 8 == 0 ? 8 : 1;  // ranges
  const int len = N / R;
  const int x = R == 8 ? (int)__builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & 7 : 0;  // XCC_ID[3:0]
  __shared__ int pick;
  for (;;) {
    if (threadIdx.x == 0) {
      int job = -1;
      for (int r = 0; r < R && job < 0; ++r) {
        const int xr = (x + r) % R;
        const uint32_t k = __hip_atomic_fetch_add(p.queue + 32 * xr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (k < (uint32_t)len) job = xr * len + (int)k;
      }
      pick = job;
    }
    __syncthreads();
    const int lam = pick;
    __syncthreads();  // read by every wave before the next tile's pick
    if (lam < 0) break;
    dkdv_tile<D>(p, lam);
  }
}

template <int D, int WAVES>
int launch_dq(const BwdParams& p, hipStream_t st) {
  const int smem = 2 * DqLayout<D>::BUF_BYTES;
  auto kern = dq_kernel<D, WAVES>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return sepattn_hip_check(e, "dq smem attribute");
  hipLaunchKernelGGL(kern, dim3(p.B * p.Hq * p.n_qtiles), dim3(WAVES * 64), smem, st, p);
  return sepattn_hip_check(hipGetLastError(), "dq launch");
}

template <int D>
int launch_dkdv(const BwdParams& p, hipStream_t st) {
  const int smem = DkvLayout<D>::SMEM;
  auto kern = dkdv_kernel<D>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return sepattn_hip_check(e, "dkdv smem attribute");
  int dev = 0, cus = 0;
  SEPATTN_TRY(sepattn_hip_check(hipGetDevice(&dev), "hipGetDevice"));
  SEPATTN_TRY(sepattn_hip_check(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev),
                                "compute unit count"));
  const int tiles = p.B * p.Hkv * 2 * p.n_key_tiles;
  hipLaunchKernelGGL(kern, dim3(std::max(1, std::min(tiles, cus))), dim3(512), smem, st, p);
  return sepattn_hip_check(hipGetLastError(), "dkdv launch");
}

}  // namespace

// The workspace of sepattn_bwd_noalloc: D for up to SEPATTN_BWD_NOALLOC_MAX_ROWS
// rows and the dK/dV tile counters, a file-scope array that each device holds from the moment this
// library's code is loaded on it until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is a stand-in, not a
// device address): it looks the address up once per device and passes that.
static __device__ __align__(256) float scratch[SEPATTN_BWD_NOALLOC_MAX_ROWS + SEPATTN_BWD_QUEUE_BYTES / 4];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// The device address of `scratch` on the current device (looked up on the
// first call per device, with that device current).
static int scratch_address(float** out) {
  int dev = 0;
  SEPATTN_TRY(sepattn_hip_check(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices) return sepattn_fail(SEPATTN_ENOTSUP, "bwd_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    SEPATTN_TRY(sepattn_hip_check(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    g_scratch_ptr[dev] = (float*)ptr;
  }
  *out = g_scratch_ptr[dev];
  return SEPATTN_OK;
}

int sepattn_launch_bwd(const sepattn_shape* s, int dtype, const sepattn_mask* m, const void* q, const void* k,
                       const void* v, const void* o, const float* lse, const void* dout, float scale, void* dq,
                       void* dk, void* dv, float* dsum, hipStream_t st);

int sepattn_launch_bwd_noalloc(const sepattn_shape* s, int dtype, const sepattn_mask* m, const void* q,
                               const void* k, const void* v, const void* o, const float* lse, const void* dout,
                               float scale, void* dq, void* dk, void* dv, hipStream_t st) {
  float* ws = nullptr;
  SEPATTN_TRY(scratch_address(&ws));
  // D is written for every row, and the counters are cleared, by the dQ
  // kernel before the dK/dV kernel reads them, so nothing needs clearing
  // between calls
  return sepattn_launch_bwd(s, dtype, m, q, k, v, o, lse, dout, scale, dq, dk, dv, ws, st);
}

int sepattn_launch_bwd(const sepattn_shape* s, int dtype, const sepattn_mask* m, const void* q, const void* k,
                       const void* v, const void* o, const float* lse, const void* dout, float scale, void* dq,
                       void* dk, void* dv, float* dsum, hipStream_t st) {
  if (dtype != SEPATTN_BF16) return sepattn_fail(SEPATTN_ENOTSUP, "bwd: only bf16 is implemented");
  BwdParams p;
  p.q = (const bf16*)q; p.k = (const bf16*)k; p.v = (const bf16*)v; p.o = (const bf16*)o;
  p.dout = (const bf16*)dout; p.lse = lse;
  p.dq = (bf16*)dq; p.dk = (bf16*)dk; p.dv = (bf16*)dv; p.dsum = dsum;
  p.queue = (uint32_t*)((char*)dsum + sepattn_bwd_d_bytes(s));
  for (int i = 0; i < 3; ++i) {
    p.sq[i] = s->q_stride[i]; p.sk[i] = s->k_stride[i]; p.sv[i] = s->v_stride[i]; p.so[i] = s->o_stride[i];
  }
  p.is_sep = m->is_sep; p.sep_idx = m->sep_idx; p.sep_before = m->sep_before; p.sep_cnt = m->sep_cnt;
  p.plain_idx = m->plain_idx; p.plain_cnt = m->plain_cnt;
  p.B = s->B; p.Hq = s->Hq; p.Hkv = s->Hkv; p.L = s->L; p.a = m->a; p.n = m->n;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.k_span = (uint32_t)((((int64_t)s->L - 1) * s->k_stride[2] + s->d) * 2);
  p.v_span = (uint32_t)((((int64_t)s->L - 1) * s->v_stride[2] + s->d) * 2);
  p.q_span = (uint32_t)((((int64_t)s->L - 1) * s->q_stride[2] + s->d) * 2);
  p.o_span = (uint32_t)((((int64_t)s->L - 1) * s->o_stride[2] + s->d) * 2);
  const int rows = fwd_tile_rows(m->n);  // dQ query tile: as the forward's
  p.n_qtiles = (s->L + rows - 1) / rows;
  p.n_key_tiles = (s->L + 127) / 128;
  int rc;
  if (s->d == 128) rc = rows == 256 ? launch_dq<128, 8>(p, st) : launch_dq<128, 2>(p, st);
  else rc = rows == 256 ? launch_dq<64, 8>(p, st) : launch_dq<64, 2>(p, st);
  if (rc != SEPATTN_OK) return rc;
  return s->d == 128 ? launch_dkdv<128>(p, st) : launch_dkdv<64>(p, st);
}
