// Backward of attention under the SepLLM mask (anthology record LIT-748,
// "Key takeaways": the mask is trained through; the mask bullet defines it).
//
// With P the masked softmax and D_i = sum_d dO_i O_i:
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Two kernels, no atomics, every output row written by one workgroup:
//  * dq_kernel: query-major, the forward's traversal (gathered anchors, then
//    the band).  Its prologue computes D for its rows and stores it.
//  * dkdv_kernel: key-major.  Keys are split into two compacted classes:
//    anchors (sinks j < a and separators), which every later row sees, and
//    plain tokens, which only rows within n see.  A workgroup owns 32*WAVES
//    keys of one class and walks the rows that can see them: [first key, L)
//    for anchors, [first key, last key + n) for plain keys, summing over the
//    q heads of its KV head.
#include "common.h"
#include "traverse.h"

namespace {

constexpr int BK = KTILE;  // keys per tile (dq)
constexpr int RB = 32;   // rows per block (dkdv)

struct BwdParams {
  const bf16 *q, *k, *v, *o, *dout;
  const float* lse;
  bf16 *dq, *dk, *dv;
  float* dsum;  // D [B, Hq, L]
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

template <int D>
struct DqLayout {
  static constexpr int STR = D + 8;
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
    mk.template store<STR>(kbuf(s));
    mv.template store<STR>(vbuf(s));
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
    fetch(t + 1);  // all-absent past the last tile
    ks.issue_idx(t + 2, rows);
    const bf16* kt = kbuf(cur);
    const bf16* vt = vbuf(cur);

    f32x16 sacc[NKB], dpacc[NKB];
#pragma unroll
    for (int x = 0; x < NKB; ++x) { sacc[x] = f32x16{}; dpacc[x] = f32x16{}; }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int x = 0; x < NKB; ++x) {
        const bf16x8 ka = *(const bf16x8*)(kt + (x * 32 + qn) * STR + kk * 16 + hh * 8);
        sacc[x] = mfma32x16(ka, qreg[kk], sacc[x]);
        const bf16x8 va = *(const bf16x8*)(vt + (x * 32 + qn) * STR + kk * 16 + hh * 8);
        dpacc[x] = mfma32x16(va, doreg[kk], dpacc[x]);
      }
    }

    // dS^T = P^T (dP^T - D), kept in sacc; masked keys get P = exp2(-inf) = 0
    if (!ks.full(t, r0, p.n)) mask_scores(sacc, ks.keep64(t, my_row, p.a, p.n, *fbuf(cur)), hh, -INFINITY);
#pragma unroll
    for (int x = 0; x < NKB; ++x)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sacc[x][r] = fast_exp2(__builtin_fmaf(sacc[x][r], p.scale_log2, -lse2)) * (dpacc[x][r] - Dv);

    // dQ^T += K^T dS^T (K^T through LDS transposing reads)
    const int g = lane >> 4, li = lane & 15;
#pragma unroll
    for (int c = 0; c < BK / 16; ++c) {
      bf16x8 bsv;
#pragma unroll
      for (int s = 0; s < 8; ++s) bsv[s] = (bf16)sacc[c >> 1][(c & 1) * 8 + s];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int dim = db * 32 + 16 * (g & 1) + 4 * (li & 3);
        const int kr = 16 * c + 4 * (g >> 1) + (li >> 2);
        const bf16x4 lo = lds_read_tr16(kt + kr * STR + dim);
        const bf16x4 hi = lds_read_tr16(kt + (kr + 8) * STR + dim);
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
// Key-major: a workgroup of 4 waves owns KT = 128 keys of one class and walks
// the rows that see them in blocks of RB = 32 rows, for each q head of its KV
// head in turn (iteration it = row block * group + head).  Wave w holds its
// 32 keys' K and V rows as B operands and their dK^T, dV^T accumulators, so
// it runs alone on its SIMD (over 256 registers) and overlaps its matrix and
// vector work itself: step it forms S and dP of iteration it, then turns
// them into P and dS while the matrix core accumulates dV^T += dO^T P and
// dK^T += Q^T dS of iteration it - 1.  Q/dO row tiles are triple-buffered in
// LDS: step it reads tiles it and it - 1 and writes tile it + 1 (loaded into
// registers one step earlier) over tile it - 2.

template <int D>
struct DkvLayout {
  static constexpr int STR = D + 8;
  static constexpr int T_BYTES = RB * STR * 2;
  static constexpr int BUF_BYTES = 2 * T_BYTES + 2 * RB * 4;  // Q, dO, lse2, D
};

template <int D>
__global__ __launch_bounds__(256) void dkdv_kernel(BwdParams p) {
  using LY = DkvLayout<D>;
  constexpr int NT = 256, KT = 128, STR = LY::STR;
  constexpr int NDB = D / 32, NKK = D / 16;
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int PT = RB * CH / NT;       // chunks per thread per tile
  constexpr int QB = RB / 32;             // 32-row blocks per iteration
  constexpr int NS = 2 * NKK * QB;        // S and dP MFMAs per iteration
  constexpr int NC = (RB / 16) * NDB * 2;  // dV and dK MFMAs per iteration
  constexpr int NE = 16 * QB;             // P/dS elements per lane per iteration
  constexpr int EPM = NE / NC;            // ... per dV/dK MFMA
  static_assert(EPM * NC == NE, "P/dS elements must spread evenly over the dV/dK MFMAs");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // XCD-aware order (as tile_work): the key tiles of one (sequence, KV head)
  // run on one XCD, anchor tiles (the longest row ranges) first.
  const int per = 2 * p.n_key_tiles;
  const int N = p.B * p.Hkv * per;
  const int lam = (N % 8 == 0) ? ((int)blockIdx.x % 8) * (N / 8) + (int)blockIdx.x / 8 : (int)blockIdx.x;
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
  const int my_c = c0 + wave * 32 + qn;
  const bool key_ok = my_c < count;
  const int my_key = key_ok ? key_at(my_c) : 0;
  const int c_last = min(c0 + KT, count) - 1;
  const int j_first = key_at(c0), j_last = key_at(c_last);
  const int wc_last = min(c0 + wave * 32 + 31, count - 1);
  const bool wave_any = c0 + wave * 32 < count;
  const bool wave_all = c0 + wave * 32 + 31 < count;
  const int jw_lo = wave_any ? key_at(c0 + wave * 32) : 0;
  const int jw_hi = wave_any ? key_at(wc_last) : 0;
  const int row_end = anchors ? p.L : min(p.L, j_last + p.n);

  // ---- this wave's 32 keys as B operands (K^T, V^T rows per lane)
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

  // ---- Q/dO row tiles: global -> registers -> LDS.  Thread x moves chunk
  // x % CH of rows x / CH + u * (NT / CH); rows past L load as zeros and get
  // lse2 = +inf, so their P is exactly 0.
  // Byte offset of the LDS buffer of tile it (it >= 0; unsigned arithmetic
  // lets the compiler fold constant offsets into the LDS instructions).
  auto tbuf = [&](int it) -> uint32_t { return ((uint32_t)it % 3u) * (uint32_t)LY::BUF_BYTES; };
  // Staging registers of one tile on its way to LDS.
  struct Stage {
    u32x4 q[PT], d[PT];
    float lse, dsum;
  };
  auto fetch = [&](Stage& sg, int it) {
    const int rs = j_first + (it / group) * RB;
    const int h = kvh * group + it % group;
    const bool live = it < n_it;
    const rsrc_t qrs = make_rsrc(p.q + b * p.sq[0] + h * p.sq[1], p.q_span);
    const rsrc_t drs = make_rsrc(p.dout + b * p.so[0] + h * p.so[1], p.o_span);
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int i = rs + (int)threadIdx.x / CH + u * (NT / CH);
      const bool ok = live && i < p.L;
      const uint32_t c16 = ((int)threadIdx.x % CH) * 16;
      sg.q[u] = bld16(qrs, ok ? (uint32_t)i * (uint32_t)(p.sq[2] * 2) + c16 : BUF_OOB);
      sg.d[u] = bld16(drs, ok ? (uint32_t)i * (uint32_t)(p.so[2] * 2) + c16 : BUF_OOB);
    }
    if (threadIdx.x < RB) {
      const size_t rowb = ((size_t)b * p.Hq + h) * p.L;
      const rsrc_t lrs = make_rsrc(p.lse + rowb, (uint32_t)p.L * 4u);
      const rsrc_t srs = make_rsrc(p.dsum + rowb, (uint32_t)p.L * 4u);
      const int i = rs + (int)threadIdx.x;
      const uint32_t off = live && i < p.L ? (uint32_t)i * 4u : BUF_OOB;
      sg.lse = __builtin_bit_cast(float, bld4(lrs, off));
      sg.dsum = __builtin_bit_cast(float, bld4(srs, off));
    }
  };
  auto store = [&](const Stage& sg, int it) {
    char* buf = smem + tbuf(it);
    bf16* qs = (bf16*)buf;
    bf16* ds = (bf16*)(buf + LY::T_BYTES);
    float* ls = (float*)(buf + 2 * LY::T_BYTES);
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int r = (int)threadIdx.x / CH + u * (NT / CH), c = (int)threadIdx.x % CH;
      st16(qs + r * STR + c * 8, sg.q[u]);
      st16(ds + r * STR + c * 8, sg.d[u]);
    }
    if (threadIdx.x < RB) {
      const int rs = j_first + (it / group) * RB;
      const bool ok = rs + (int)threadIdx.x < p.L;
      ls[threadIdx.x] = ok ? sg.lse * 1.4426950408889634f : INFINITY;
      ls[RB + threadIdx.x] = ok ? sg.dsum : 0.f;
    }
  };

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) { dkacc[db] = f32x16{}; dvacc[db] = f32x16{}; }
  const int g = lane >> 4, li = lane & 15;

  // S = Q K^T and dP = dO V^T of iteration it: RB rows x this wave's 32 keys
  // (lane = key) into s[0..QB) (S) and s[QB..2QB) (dP); operand reads PD ahead.
  f32x16 s[2 * QB];
  auto sdp = [&](int it) {
    const char* base = smem + tbuf(it) + (qn * STR + hh * 8) * 2;
    // MFMA i: S (i even) or dP (i odd), so that consecutive MFMAs never
    // accumulate into the same registers; kk = i / (2 QB), qb = (i / 2) % QB
    auto opnd = [&](int i) -> bf16x8 {
      const int kk = i / (2 * QB), qb = (i / 2) % QB;
      const int off = ((i & 1) ? LY::T_BYTES : 0) + (qb * 32 * STR + kk * 16) * 2;  // Q for S, dO for dP
      return *(const bf16x8*)(base + off);
    };
    constexpr int PD = 4;
    bf16x8 op[NS];
#pragma unroll
    for (int i = 0; i < PD; ++i) op[i] = opnd(i);
#pragma unroll
    for (int x = 0; x < 2 * QB; ++x) s[x] = f32x16{};
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + PD < NS) op[i + PD] = opnd(i + PD);
      const int kk = i / (2 * QB), qb = (i / 2) % QB;
      if (i & 1) s[QB + qb] = mfma32x16(op[i], vreg[kk], s[QB + qb]);
      else s[qb] = mfma32x16(op[i], kreg[kk], s[qb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // P, dS of iteration it (element e of this lane's NE) from s and the rows'
  // lse2, D, as the B operands of the row contraction: chunk c holds rows
  // 16c .. 16c + 15, slot sl is register (c & 1) * 8 + sl of block c >> 1.
  // This lane's key is seen by the local rows [lo, hi) of the block (its
  // position, the end of the sequence and, for plain keys, the window), so
  // the mask is two compares per element and no branch.
  struct PdS {
    bf16x8 p[RB / 16], d[RB / 16];
  };
  const int key_hi = !key_ok ? -1 : anchors ? p.L : min(p.L, my_key + p.n);  // rows [my_key, key_hi)
  auto pds = [&](PdS& o, const float* ls, int lo, int hi, int e, bool masked) {
    const int qb = e / 16, r = e % 16;
    const int rl0 = qb * 32 + 8 * (r >> 2) + (r & 3);  // local row is rl0 + 4 * hh
    const int rl = rl0 + 4 * hh;
    float pr = fast_exp2(__builtin_fmaf(s[qb][r], p.scale_log2, -ls[rl]));
    if (masked) pr = (rl0 >= lo && rl0 < hi) ? pr : 0.f;
    const float dsv = pr * (s[QB + qb][r] - ls[RB + rl]);
    const int c = qb * 2 + (r >> 3), sl = r & 7;
    o.p[c][sl] = (bf16)pr;
    o.d[c][sl] = (bf16)dsv;
    if (sl & 1) {
      // Pin the finished pair here: without a use at this point the compiler
      // sinks the whole P/dS computation to the end of the step (its first
      // real use is the next step's MFMAs), out of reach of the interleave.
      const uint32_t pw = __builtin_bit_cast(u32x4, o.p[c])[sl >> 1];
      const uint32_t dw = __builtin_bit_cast(u32x4, o.d[c])[sl >> 1];
      asm volatile("" ::"v"(pw), "v"(dw));
    }
  };
  auto pds_range = [&](int it, int& lo, int& hi) {  // in units of rl0 (hh folded in)
    const int rs = j_first + (it / group) * RB;
    lo = my_key - rs - 4 * hh;
    hi = key_hi - rs - 4 * hh;
  };

  // dV^T += dO^T P and dK^T += Q^T dS for iteration it - 1 (transposing
  // reads of its tile, P/dS in prev), interleaved with the P/dS of iteration
  // it into cur (EPM elements per MFMA).  Past the last iteration the P/dS
  // are formed from stale registers and never used.
  auto dvdk_pds = [&](int it, const PdS& prev, PdS& cur) {
    const char* pbuf = smem + tbuf(it + 2);  // tile it - 1
    const float* ls = (const float*)(smem + tbuf(it) + 2 * LY::T_BYTES);
    int lo, hi;
    pds_range(it, lo, hi);
    // lane li of group g reads row 16c + 4(g/2) + li/4 (and that + 8) at
    // dims db*32 + 16(g%2) + 4(li%4): a per-lane base plus constant offsets
    const char* base = pbuf + ((4 * (g >> 1) + (li >> 2)) * STR + 16 * (g & 1) + 4 * (li & 3)) * 2;
    auto opnd = [&](int i) -> bf16x8 {
      const int c = i / (2 * NDB), db = (i / 2) % NDB;
      const int off = ((i & 1) ? 0 : LY::T_BYTES) + (16 * c * STR + db * 32) * 2;  // Q for dK, dO for dV
      const bf16x4 lo4 = lds_read_tr16(base + off);
      const bf16x4 hi4 = lds_read_tr16(base + off + 8 * STR * 2);
      return bf16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    };
    auto run = [&](bool masked) {
      constexpr int PD = 4;
      bf16x8 op[NC];
#pragma unroll
      for (int i = 0; i < PD; ++i) op[i] = opnd(i);
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        if (i + PD < NC) op[i + PD] = opnd(i + PD);
        const int c = i / (2 * NDB), db = (i / 2) % NDB;
        if (i & 1) dkacc[db] = mfma32x16(op[i], prev.d[c], dkacc[db]);
        else dvacc[db] = mfma32x16(op[i], prev.p[c], dvacc[db]);
#pragma unroll
        for (int e = 0; e < EPM; ++e) pds(cur, ls, lo, hi, i * EPM + e, masked);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    run(true);
  };

  // ---- prologue: tile 0 in LDS, tile 1 in registers; step 0 = S, dP and
  // P, dS of iteration 0
  PdS pa, pb2;
  Stage sg;
  fetch(sg, 0);
  store(sg, 0);
  fetch(sg, 1);
  __syncthreads();
  sdp(0);
  {
    const float* ls = (const float*)(smem + 2 * LY::T_BYTES);
    int lo, hi;
    pds_range(0, lo, hi);
#pragma unroll
    for (int e = 0; e < NE; ++e) pds(pa, ls, lo, hi, e, true);
  }
  store(sg, 1);
  fetch(sg, 2);
  __syncthreads();

  // ---- step it (1 <= it < n_it): S, dP of it; P, dS of it beside dV, dK of
  // it - 1; tile it + 1 into LDS and tile it + 2 into the staging registers.
  // Unrolled by two so the P/dS register sets alternate without copies.
  auto step = [&](int it, const PdS& prev, PdS& cur) {
    sdp(it);
    dvdk_pds(it, prev, cur);
    store(sg, it + 1);
    fetch(sg, it + 2);
    __syncthreads();
  };
  int it = 1;
  for (; it + 1 < n_it; it += 2) {
    step(it, pa, pb2);
    step(it + 1, pb2, pa);
  }
  // (the final dV, dK step also forms P, dS of a block past the end; unused)
  if (it < n_it) {
    step(it, pa, pb2);
    dvdk_pds(it + 1, pb2, pa);
  } else {
    dvdk_pds(it, pa, pb2);
  }

  if (key_ok) {
    bf16* dkrow = p.dk + b * p.sk[0] + kvh * p.sk[1] + (int64_t)my_key * p.sk[2];
    bf16* dvrow = p.dv + b * p.sv[0] + kvh * p.sv[1] + (int64_t)my_key * p.sv[2];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
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
  const int smem = 3 * DkvLayout<D>::BUF_BYTES;
  auto kern = dkdv_kernel<D>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return sepattn_hip_check(e, "dkdv smem attribute");
  hipLaunchKernelGGL(kern, dim3(p.B * p.Hkv * 2 * p.n_key_tiles), dim3(256), smem, st, p);
  return sepattn_hip_check(hipGetLastError(), "dkdv launch");
}

}  // namespace

int sepattn_launch_bwd(const sepattn_shape* s, int dtype, const sepattn_mask* m, const void* q, const void* k,
                       const void* v, const void* o, const float* lse, const void* dout, float scale, void* dq,
                       void* dk, void* dv, float* dsum, hipStream_t st) {
  if (dtype != SEPATTN_BF16) return sepattn_fail(SEPATTN_ENOTSUP, "bwd: only bf16 is implemented");
  BwdParams p;
  p.q = (const bf16*)q; p.k = (const bf16*)k; p.v = (const bf16*)v; p.o = (const bf16*)o;
  p.dout = (const bf16*)dout; p.lse = lse;
  p.dq = (bf16*)dq; p.dk = (bf16*)dk; p.dv = (bf16*)dv; p.dsum = dsum;
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
