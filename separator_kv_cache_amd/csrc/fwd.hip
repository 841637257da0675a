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
  static constexpr int BUF_BYTES = K_BYTES + V_BYTES;
};

template <int D>
struct FwdLayout<float, D> {
  static constexpr int KSTR = D + 4;
  static constexpr int VSTR = D + 4;
  static constexpr int K_BYTES = BK * KSTR * 4;
  static constexpr int V_BYTES = BK * VSTR * 4;
  static constexpr int BUF_BYTES = K_BYTES + V_BYTES;
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t sq[3], sk[3], sv[3], so[3];
  const uint8_t* is_sep;
  const int32_t* sep_idx;
  const int32_t* sep_before;
  int B, Hq, Hkv, L, a, n;
  int n_qtiles;
  float scale_log2;  // softmax scale * log2(e)
};

// Loads one 64-key tile (rows of K and V) of the workgroup into registers.
// Row r of the tile is key key_of(r) or absent (< 0: zeros).
template <typename T, int D, int NT>
struct TileLoader {
  static constexpr int CH_PER_ROW = D * (int)sizeof(T) / 16;  // 16-byte chunks per row
  static constexpr int NCH = BK * CH_PER_ROW;
  static constexpr int PER_THREAD = NCH / NT;
  static_assert(NCH % NT == 0, "tile chunks must divide the workgroup");
  u32x4 kr[PER_THREAD], vr[PER_THREAD];

  template <typename KeyOf>
  __device__ __forceinline__ void load(const T* kbase, const T* vbase, int64_t skl, int64_t svl,
                                       KeyOf key_of) {
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
      const int ch = threadIdx.x + u * NT;
      const int r = ch / CH_PER_ROW, c = ch % CH_PER_ROW;
      const int j = key_of(r);
      if (j >= 0) {
        kr[u] = ld16((const char*)(kbase + (int64_t)j * skl) + c * 16);
        vr[u] = ld16((const char*)(vbase + (int64_t)j * svl) + c * 16);
      } else {
        kr[u] = u32x4{0, 0, 0, 0};
        vr[u] = u32x4{0, 0, 0, 0};
      }
    }
  }
  template <int KSTR, int VSTR>
  __device__ __forceinline__ void store(T* ks, T* vs) {
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
      const int ch = threadIdx.x + u * NT;
      const int r = ch / CH_PER_ROW, c = ch % CH_PER_ROW;
      st16((char*)(ks + r * KSTR) + c * 16, kr[u]);
      st16((char*)(vs + r * VSTR) + c * 16, vr[u]);
    }
  }
};

template <typename T, int D, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void fwd_kernel(FwdParams p) {
  using LY = FwdLayout<T, D>;
  constexpr int NT = WAVES * 64;
  constexpr int BQ = WAVES * 32;
  constexpr bool BF = sizeof(T) == 2;
  constexpr int KSTR = LY::KSTR, VSTR = LY::VSTR;

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bh = blockIdx.x;
  const int b = bh / p.Hq, h = bh % p.Hq;
  const int kvh = h / (p.Hq / p.Hkv);
  const int qt = p.n_qtiles - 1 - (int)blockIdx.y;  // heaviest tiles first
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

  auto key_of = [&](int t, int r) -> int {
    if (t < n_gt) {
      const int c = t * BK + r;
      return c < tk.n_gather ? gather_key(c, tk.n_sink, si) : -1;
    }
    const int j = tk.band_lo + (t - n_gt) * BK + r;
    return j < tk.band_hi ? j : -1;
  };

  TileLoader<T, D, NT> ld;
  auto kbuf = [&](int s) { return (T*)(smem + s * LY::BUF_BYTES); };
  auto vbuf = [&](int s) { return (T*)(smem + s * LY::BUF_BYTES + LY::K_BYTES); };

  // ---- prologue: tile 0
  if (n_tiles > 0) {
    ld.load(kb, vb, p.sk[2], p.sv[2], [&](int r) { return key_of(0, r); });
    ld.template store<KSTR, VSTR>(kbuf(0), vbuf(0));
  }
  __syncthreads();

  constexpr int NKB = BK / 32;  // 32-key blocks per tile
  constexpr int NDB = D / 32;   // 32-dim blocks
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  for (int t = 0; t < n_tiles; ++t) {
    const int cur = t & 1;
    const bool more = t + 1 < n_tiles;
    if (more) ld.load(kb, vb, p.sk[2], p.sv[2], [&](int r) { return key_of(t + 1, r); });
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
    bool full;
    int k0 = 0;
    if (t < n_gt) {
      full = (t + 1) * BK <= tk.n_gather;
    } else {
      k0 = tk.band_lo + (t - n_gt) * BK;
      full = (k0 + BK <= tk.band_hi) && (k0 + BK - 1 <= r0) && (r0 + 31 - k0 < p.n);
    }
    if (!full) {
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kl = kb2 * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          bool keep;
          if (t < n_gt) keep = t * BK + kl < tk.n_gather;
          else {
            const int j = k0 + kl;
            keep = j < tk.band_hi && band_keep(my_row, j, p.a, p.n, fs);
          }
          if (!keep) sacc[kb2][r] = -INFINITY;
        }
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
    for (int kb2 = 0; kb2 < NKB; ++kb2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(__builtin_fmaf(sacc[kb2][r], p.scale_log2, -m_use));
        sacc[kb2][r] = e;
        l_run += e;
      }
    }

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

    if (more) ld.template store<KSTR, VSTR>(kbuf(cur ^ 1), vbuf(cur ^ 1));
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

template <typename T, int D, int WAVES>
int launch_fwd(const FwdParams& p, hipStream_t st) {
  constexpr int BQ = WAVES * 32;
  const int smem = 2 * FwdLayout<T, D>::BUF_BYTES;
  auto kern = fwd_kernel<T, D, WAVES>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return sepattn_hip_check(e, "fwd smem attribute");
  dim3 grid(p.B * p.Hq, (p.L + BQ - 1) / BQ);
  hipLaunchKernelGGL(kern, grid, dim3(WAVES * 64), smem, st, p);
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
  p.is_sep = m->is_sep; p.sep_idx = m->sep_idx; p.sep_before = m->sep_before;
  p.B = s->B; p.Hq = s->Hq; p.Hkv = s->Hkv; p.L = s->L; p.a = m->a; p.n = m->n;
  p.scale_log2 = scale * 1.4426950408889634f;
  const int rows = fwd_tile_rows(m->n);
  p.n_qtiles = (s->L + rows - 1) / rows;
  const bool big = rows == 256;
  if (dtype == SEPATTN_BF16) {
    if (s->d == 128) return big ? launch_fwd<bf16, 128, 8>(p, st) : launch_fwd<bf16, 128, 2>(p, st);
    return big ? launch_fwd<bf16, 64, 8>(p, st) : launch_fwd<bf16, 64, 2>(p, st);
  }
  if (s->d == 128) return big ? launch_fwd<float, 128, 8>(p, st) : launch_fwd<float, 128, 2>(p, st);
  return big ? launch_fwd<float, 64, 8>(p, st) : launch_fwd<float, 64, 2>(p, st);
}
