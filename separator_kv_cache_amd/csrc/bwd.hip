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
constexpr int RB = 64;   // rows per block (dkdv)

struct BwdParams {
  const bf16 *q, *k, *v, *o, *dout;
  const float* lse;
  bf16 *dq, *dk, *dv;
  float* dsum;  // D [B, Hq, L]
  int64_t sq[3], sk[3], sv[3], so[3];
  uint32_t k_span, v_span;  // bytes of one (sequence, KV head) slice of K, V
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

template <int D>
struct DkvLayout {
  static constexpr int STR = D + 8;
  static constexpr int T_BYTES = RB * STR * 2;
  static constexpr int BUF_BYTES = 2 * T_BYTES + 2 * RB * 4;  // Q, dO, lse2, D
};

template <int D, int NT>
struct QdoLoader {
  static constexpr int CH = D / 8;
  static constexpr int PER = RB * CH / NT;
  u32x4 qr[PER], dr[PER];
  float lse2, dsum;
  __device__ __forceinline__ void load(const bf16* qb, const bf16* db, int64_t sql, int64_t sol,
                                       const float* lse_row, const float* d_row, int rs, int L) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int ch = threadIdx.x + u * NT;
      const int r = ch / CH, c = ch % CH;
      const int i = rs + r;
      if (i < L) {
        qr[u] = ld16(qb + (int64_t)i * sql + c * 8);
        dr[u] = ld16(db + (int64_t)i * sol + c * 8);
      } else {
        qr[u] = u32x4{0, 0, 0, 0};
        dr[u] = u32x4{0, 0, 0, 0};
      }
    }
    if (threadIdx.x < RB) {
      const int i = rs + threadIdx.x;
      lse2 = i < L ? lse_row[i] * 1.4426950408889634f : INFINITY;
      dsum = i < L ? d_row[i] : 0.f;
    }
  }
  __device__ __forceinline__ void store(char* buf) {
    bf16* qs = (bf16*)buf;
    bf16* ds = (bf16*)(buf + DkvLayout<D>::T_BYTES);
    float* ls = (float*)(buf + 2 * DkvLayout<D>::T_BYTES);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int ch = threadIdx.x + u * NT;
      const int r = ch / CH, c = ch % CH;
      st16(qs + r * DkvLayout<D>::STR + c * 8, qr[u]);
      st16(ds + r * DkvLayout<D>::STR + c * 8, dr[u]);
    }
    if (threadIdx.x < RB) {
      ls[threadIdx.x] = lse2;
      ls[RB + threadIdx.x] = dsum;
    }
  }
};

template <int D, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void dkdv_kernel(BwdParams p) {
  using LY = DkvLayout<D>;
  constexpr int NT = WAVES * 64, KT = WAVES * 32, STR = LY::STR;
  constexpr int NDB = D / 32, NKK = D / 16;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.x / p.Hkv, kvh = blockIdx.x % p.Hkv;
  const bool anchors = (int)blockIdx.y < p.n_key_tiles;
  const int tile = anchors ? blockIdx.y : blockIdx.y - p.n_key_tiles;
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
  QdoLoader<D, NT> ld;
  auto load_it = [&](int it) {
    const int rs = j_first + (it / group) * RB;
    const int h = kvh * group + it % group;
    const bf16* qb = p.q + b * p.sq[0] + h * p.sq[1];
    const bf16* dob = p.dout + b * p.so[0] + h * p.so[1];
    const size_t rowb = ((size_t)b * p.Hq + h) * p.L;
    ld.load(qb, dob, p.sq[2], p.so[2], p.lse + rowb, p.dsum + rowb, rs, p.L);
  };
  if (n_it > 0) {
    load_it(0);
    ld.store(smem);
  }
  __syncthreads();

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) { dkacc[db] = f32x16{}; dvacc[db] = f32x16{}; }

  for (int it = 0; it < n_it; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < n_it;
    if (more) load_it(it + 1);
    const char* buf = smem + cur * LY::BUF_BYTES;
    const bf16* qs = (const bf16*)buf;
    const bf16* ds = (const bf16*)(buf + LY::T_BYTES);
    const float* ls = (const float*)(buf + 2 * LY::T_BYTES);
    const int rs = j_first + (it / group) * RB;

    // S = Q K^T and dP = dO V^T for 64 rows x 32 keys: lane = key
    f32x16 sacc[2], dpacc[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) { sacc[qb] = f32x16{}; dpacc[qb] = f32x16{}; }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const bf16x8 qa = *(const bf16x8*)(qs + (qb * 32 + qn) * STR + kk * 16 + hh * 8);
        sacc[qb] = mfma32x16(qa, kreg[kk], sacc[qb]);
        const bf16x8 da = *(const bf16x8*)(ds + (qb * 32 + qn) * STR + kk * 16 + hh * 8);
        dpacc[qb] = mfma32x16(da, vreg[kk], dpacc[qb]);
      }
    }
    const bool full = wave_all && jw_hi <= rs && rs + RB - 1 < p.L &&
                      (anchors || rs + RB - 1 - jw_lo < p.n);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int rl = qb * 32 + 8 * i4 + 4 * hh;  // local row of register 4*i4
        const f32x4 l2 = *(const f32x4*)(ls + rl);
        const f32x4 dd = *(const f32x4*)(ls + RB + rl);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * i4 + e;
          float pr = fast_exp2(sacc[qb][r] * p.scale_log2 - l2[e]);
          if (!full) {
            const int i = rs + rl + e;
            bool keep = key_ok && my_key <= i && i < p.L;
            if (!anchors) keep = keep && i - my_key < p.n;
            pr = keep ? pr : 0.f;
          }
          sacc[qb][r] = pr;                           // P
          dpacc[qb][r] = pr * (dpacc[qb][r] - dd[e]);  // dS
        }
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS (row-contraction, transposing reads)
    const int g = lane >> 4, li = lane & 15;
#pragma unroll
    for (int c = 0; c < RB / 16; ++c) {
      bf16x8 pb, sb;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        pb[s] = (bf16)sacc[c >> 1][(c & 1) * 8 + s];
        sb[s] = (bf16)dpacc[c >> 1][(c & 1) * 8 + s];
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int dim = db * 32 + 16 * (g & 1) + 4 * (li & 3);
        const int row = 16 * c + 4 * (g >> 1) + (li >> 2);
        const bf16x4 dlo = lds_read_tr16(ds + row * STR + dim);
        const bf16x4 dhi = lds_read_tr16(ds + (row + 8) * STR + dim);
        const bf16x8 da = {dlo[0], dlo[1], dlo[2], dlo[3], dhi[0], dhi[1], dhi[2], dhi[3]};
        dvacc[db] = mfma32x16(da, pb, dvacc[db]);
        const bf16x4 qlo = lds_read_tr16(qs + row * STR + dim);
        const bf16x4 qhi = lds_read_tr16(qs + (row + 8) * STR + dim);
        const bf16x8 qa = {qlo[0], qlo[1], qlo[2], qlo[3], qhi[0], qhi[1], qhi[2], qhi[3]};
        dkacc[db] = mfma32x16(qa, sb, dkacc[db]);
      }
    }
    if (more) ld.store(smem + (cur ^ 1) * LY::BUF_BYTES);
    __syncthreads();
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
  constexpr int WAVES = 4;
  const int smem = 2 * DkvLayout<D>::BUF_BYTES;
  auto kern = dkdv_kernel<D, WAVES>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return sepattn_hip_check(e, "dkdv smem attribute");
  hipLaunchKernelGGL(kern, dim3(p.B * p.Hkv, 2 * p.n_key_tiles), dim3(WAVES * 64), smem, st, p);
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
  const int rows = fwd_tile_rows(m->n);  // dQ query tile: as the forward's
  p.n_qtiles = (s->L + rows - 1) / rows;
  p.n_key_tiles = (s->L + 127) / 128;
  int rc;
  if (s->d == 128) rc = rows == 256 ? launch_dq<128, 8>(p, st) : launch_dq<128, 2>(p, st);
  else rc = rows == 256 ? launch_dq<64, 8>(p, st) : launch_dq<64, 2>(p, st);
  if (rc != SEPATTN_OK) return rc;
  return s->d == 128 ? launch_dkdv<128>(p, st) : launch_dkdv<64>(p, st);
}
