// C ABI entry points: argument validation, error reporting and dispatch to
// the kernel launchers.  Validation runs before any HIP call, so argument
// errors are reported (and testable) without a GPU.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <vector>

#include "common.h"
#include "traverse.h"

// kernel launchers (mask.hip, fwd.hip, bwd.hip, cache.hip)
int sepattn_launch_build_mask_fixed(int delta, const sepattn_mask* m, hipStream_t st);
int sepattn_launch_build_mask(const int32_t* tok, const int32_t* ids, int n_ids, const sepattn_mask* m,
                              hipStream_t st);
int sepattn_launch_mask_bits(const sepattn_mask* m, uint32_t* bits, hipStream_t st);
int sepattn_launch_tile_desc(const sepattn_mask* m, int tile_rows, int32_t* desc, hipStream_t st);
int sepattn_launch_fwd(const sepattn_shape* s, int dtype, const sepattn_mask* m, const void* q,
                       const void* k, const void* v, float scale, void* o, float* lse, hipStream_t st);
int sepattn_launch_bwd(const sepattn_shape* s, int dtype, const sepattn_mask* m, const void* q,
                       const void* k, const void* v, const void* o, const float* lse, const void* dout,
                       float scale, void* dq, void* dk, void* dv, float* dsum, hipStream_t st);
int sepattn_launch_bwd_noalloc(const sepattn_shape* s, int dtype, const sepattn_mask* m, const void* q,
                               const void* k, const void* v, const void* o, const float* lse, const void* dout,
                               float scale, void* dq, void* dk, void* dv, hipStream_t st);
int sepcache_launch_reset(const sepcache* c, hipStream_t st);
int sepcache_launch_update(const sepcache* c, const void* k_new, const void* v_new, const uint8_t* is_sep,
                           int do_append, int do_evict, hipStream_t st);
size_t sepcache_decode_ws_bytes(const sepcache* c, int Hq);
int sepcache_launch_decode(const sepcache* c, int Hq, const void* q, float scale, int shift, void* o,
                           void* ws, hipStream_t st);
int sepcache_launch_export(const sepcache* c, int32_t* pos, int32_t* len, hipStream_t st);
int sepcache_launch_prefill(const sepcache* c, const void* k, const void* v, const int64_t* ks, const int64_t* vs,
                            const sepattn_mask* m, hipStream_t st);
int sepcache_launch_step(const sepcache* c, const void* k_new, const void* v_new, const uint8_t* is_sep, int Hq,
                         const void* q, float scale, int shift, void* o, void* ws, hipStream_t st);

static thread_local char g_err[512] = "";

int sepattn_fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int sepattn_hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return SEPATTN_OK;
  return sepattn_fail(SEPATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int sepattn_check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return sepattn_hip_check(e, "hipGetDevice");
  static thread_local int cached_dev = -1, cached_ok = 0;
  if (dev == cached_dev) return cached_ok ? SEPATTN_OK : sepattn_fail(SEPATTN_ENOTSUP, "device is not gfx950");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return sepattn_hip_check(e, "hipGetDeviceProperties");
  cached_dev = dev;
  cached_ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (!cached_ok) return sepattn_fail(SEPATTN_ENOTSUP, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  return SEPATTN_OK;
}

extern "C" {

const char* sepattn_last_error(void) { return g_err; }
int sepattn_version(void) { return 10000; }

// ------------------------------------------------------------------ mask

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t sepattn_mask_bytes(int B, int L) {
  if (B <= 0 || L <= 0) return 0;
  const size_t b = B, l = L;
  return align256(b * l) + align256(4 * b * l) + align256(4 * b * (l + 1)) + align256(4 * b) +
         align256(4 * b * l) + align256(4 * b) + align256(8 * b);
}

int sepattn_mask_carve(sepattn_mask* m, int B, int L, int a, int n, void* buffer, size_t bytes) {
  g_err[0] = 0;
  if (!m || !buffer) return sepattn_fail(SEPATTN_EINVAL, "mask_carve: null pointer");
  if (B <= 0 || L <= 0) return sepattn_fail(SEPATTN_EINVAL, "mask_carve: B=%d L=%d must be positive", B, L);
  if (a < 0 || n < 1) return sepattn_fail(SEPATTN_EINVAL, "mask_carve: need a >= 0 and n >= 1 (a=%d n=%d)", a, n);
  if (bytes < sepattn_mask_bytes(B, L))
    return sepattn_fail(SEPATTN_ESPACE, "mask_carve: %zu bytes < %zu needed", bytes, sepattn_mask_bytes(B, L));
  char* p = (char*)buffer;
  const size_t b = B, l = L;
  m->B = B; m->L = L; m->a = a; m->n = n;
  m->is_sep = (uint8_t*)p; p += align256(b * l);
  m->sep_idx = (int32_t*)p; p += align256(4 * b * l);
  m->sep_before = (int32_t*)p; p += align256(4 * b * (l + 1));
  m->sep_cnt = (int32_t*)p; p += align256(4 * b);
  m->plain_idx = (int32_t*)p; p += align256(4 * b * l);
  m->plain_cnt = (int32_t*)p; p += align256(4 * b);
  m->kept = (int64_t*)p;
  return SEPATTN_OK;
}

static int check_mask(const sepattn_mask* m, const char* who) {
  if (!m) return sepattn_fail(SEPATTN_EINVAL, "%s: null mask", who);
  if (m->B <= 0 || m->L <= 0) return sepattn_fail(SEPATTN_EINVAL, "%s: mask B=%d L=%d", who, m->B, m->L);
  if (m->a < 0 || m->n < 1) return sepattn_fail(SEPATTN_EINVAL, "%s: need a >= 0, n >= 1 (a=%d n=%d)", who, m->a, m->n);
  if (!m->is_sep || !m->sep_idx || !m->sep_before || !m->sep_cnt || !m->plain_idx || !m->plain_cnt || !m->kept)
    return sepattn_fail(SEPATTN_EINVAL, "%s: null mask array", who);
  return SEPATTN_OK;
}

int sepattn_build_mask(const int32_t* tok, const int32_t* sep_ids, int n_sep, const sepattn_mask* m,
                       void* stream) {
  g_err[0] = 0;
  SEPATTN_TRY(check_mask(m, "build_mask"));
  if (!tok || !sep_ids) return sepattn_fail(SEPATTN_EINVAL, "build_mask: null tokens or separator ids");
  if (n_sep < 1 || n_sep > SEPATTN_MAX_SEP_IDS)
    return sepattn_fail(SEPATTN_EINVAL, "build_mask: n_sep=%d not in [1, %d]", n_sep, SEPATTN_MAX_SEP_IDS);
  SEPATTN_TRY(sepattn_check_device());
  return sepattn_launch_build_mask(tok, sep_ids, n_sep, m, (hipStream_t)stream);
}

int sepattn_build_mask_fixed(int delta, const sepattn_mask* m, void* stream) {
  g_err[0] = 0;
  SEPATTN_TRY(check_mask(m, "build_mask_fixed"));
  if (delta < 1) return sepattn_fail(SEPATTN_EINVAL, "build_mask_fixed: delta=%d < 1", delta);
  SEPATTN_TRY(sepattn_check_device());
  return sepattn_launch_build_mask_fixed(delta, m, (hipStream_t)stream);
}

int sepattn_mask_bits(const sepattn_mask* m, uint32_t* bits, void* stream) {
  g_err[0] = 0;
  SEPATTN_TRY(check_mask(m, "mask_bits"));
  if (!bits) return sepattn_fail(SEPATTN_EINVAL, "mask_bits: null output");
  if (m->L > 65536) return sepattn_fail(SEPATTN_EINVAL, "mask_bits: L=%d > 65536", m->L);
  SEPATTN_TRY(sepattn_check_device());
  return sepattn_launch_mask_bits(m, bits, (hipStream_t)stream);
}

int sepattn_fwd_tile_rows(int n) { return n < 1 ? -1 : fwd_tile_rows(n); }

int sepattn_tile_desc(const sepattn_mask* m, int tile_rows, int32_t* desc, void* stream) {
  g_err[0] = 0;
  SEPATTN_TRY(check_mask(m, "tile_desc"));
  if (!desc) return sepattn_fail(SEPATTN_EINVAL, "tile_desc: null output");
  if (tile_rows < 1) return sepattn_fail(SEPATTN_EINVAL, "tile_desc: tile_rows=%d < 1", tile_rows);
  SEPATTN_TRY(sepattn_check_device());
  return sepattn_launch_tile_desc(m, tile_rows, desc, (hipStream_t)stream);
}

// ------------------------------------------------------------------ attention

static int check_shape(const sepattn_shape* s, int dtype, const sepattn_mask* m, const char* who) {
  if (!s) return sepattn_fail(SEPATTN_EINVAL, "%s: null shape", who);
  SEPATTN_TRY(check_mask(m, who));
  if (s->B <= 0 || s->Hq <= 0 || s->Hkv <= 0 || s->L <= 0)
    return sepattn_fail(SEPATTN_EINVAL, "%s: B=%d Hq=%d Hkv=%d L=%d must be positive", who, s->B, s->Hq, s->Hkv, s->L);
  if (s->Hq % s->Hkv != 0)
    return sepattn_fail(SEPATTN_EINVAL, "%s: Hq=%d is not a multiple of Hkv=%d", who, s->Hq, s->Hkv);
  if (s->d != 64 && s->d != 128) return sepattn_fail(SEPATTN_ENOTSUP, "%s: head dim %d (64 or 128)", who, s->d);
  if (dtype != SEPATTN_F32 && dtype != SEPATTN_BF16) return sepattn_fail(SEPATTN_ENOTSUP, "%s: dtype %d", who, dtype);
  if (m->B != s->B || m->L != s->L)
    return sepattn_fail(SEPATTN_EINVAL, "%s: mask is for B=%d L=%d, shape has B=%d L=%d", who, m->B, m->L, s->B, s->L);
  if ((int64_t)s->B * s->Hq * (((int64_t)s->L + 63) / 64) > ((int64_t)1 << 31))
    return sepattn_fail(SEPATTN_EINVAL, "%s: problem too large", who);
  const int64_t* st[4] = {s->q_stride, s->k_stride, s->v_stride, s->o_stride};
  const int esz = dtype == SEPATTN_BF16 ? 2 : 4;
  for (int t = 0; t < 4; ++t)
    for (int i = 0; i < 3; ++i) {
      if (st[t][i] < 0) return sepattn_fail(SEPATTN_EINVAL, "%s: negative stride", who);
      if ((st[t][i] * esz) % 16 != 0)
        return sepattn_fail(SEPATTN_EINVAL, "%s: strides must be multiples of 16 bytes", who);
    }
  for (int t = 0; t < 4; ++t) {
    const int64_t span = (((int64_t)s->L - 1) * st[t][2] + s->d) * esz;
    if (span >= ((int64_t)1 << 31))
      return sepattn_fail(SEPATTN_ENOTSUP, "%s: a (sequence, head) slice spans %lld bytes (limit 2 GiB)", who,
                          (long long)span);
  }
  return SEPATTN_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// True when no two rows (b, h, l) of a [B, H, L, d] tensor with these
// element strides (batch, head, token) and a contiguous last dimension share
// an element: ordered by stride, every dimension of extent above one must
// step past everything the smaller ones span.  Outputs must satisfy it, or
// workgroups writing different rows would write the same memory.
static bool rows_disjoint(const int64_t st[3], int B, int H, int L, int d) {
  const int64_t ext[3] = {B, H, L};
  int idx[3], k = 0;
  for (int i = 0; i < 3; ++i)
    if (ext[i] > 1) idx[k++] = i;
  for (int i = 1; i < k; ++i)  // insertion sort by stride
    for (int j = i; j > 0 && st[idx[j]] < st[idx[j - 1]]; --j) {
      const int t = idx[j];
      idx[j] = idx[j - 1];
      idx[j - 1] = t;
    }
  int64_t span = d;  // elements one row covers, then everything below the next dimension
  for (int i = 0; i < k; ++i) {
    if (st[idx[i]] < span) return false;
    span += (ext[idx[i]] - 1) * st[idx[i]];
  }
  return true;
}

int sepattn_fwd(const sepattn_shape* s, int dtype, const sepattn_mask* m, const void* q, const void* k,
                const void* v, float scale, void* o, float* lse, void* stream) {
  g_err[0] = 0;
  SEPATTN_TRY(check_shape(s, dtype, m, "fwd"));
  if (!q || !k || !v || !o) return sepattn_fail(SEPATTN_EINVAL, "fwd: null tensor");
  if (!rows_disjoint(s->o_stride, s->B, s->Hq, s->L, s->d))
    return sepattn_fail(SEPATTN_EINVAL, "fwd: o_stride makes output rows overlap");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return sepattn_fail(SEPATTN_EINVAL, "fwd: tensors must be 16-byte aligned");
  if (!std::isfinite(scale)) return sepattn_fail(SEPATTN_EINVAL, "fwd: scale is not finite");
  SEPATTN_TRY(sepattn_check_device());
  return sepattn_launch_fwd(s, dtype, m, q, k, v, scale, o, lse, (hipStream_t)stream);
}

size_t sepattn_bwd_workspace_size(const sepattn_shape* s) {
  if (!s || s->B <= 0 || s->Hq <= 0 || s->L <= 0) return 0;
  return sepattn_bwd_d_bytes(s) + SEPATTN_BWD_QUEUE_BYTES;
}

int sepattn_bwd(const sepattn_shape* s, int dtype, const sepattn_mask* m, const void* q, const void* k,
                const void* v, const void* o, const float* lse, const void* dout, float scale, void* dq,
                void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  SEPATTN_TRY(check_shape(s, dtype, m, "bwd"));
  if (dtype != SEPATTN_BF16) return sepattn_fail(SEPATTN_ENOTSUP, "bwd: only bf16 is implemented");
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace)
    return sepattn_fail(SEPATTN_EINVAL, "bwd: null tensor or workspace");
  // dQ, dK and dV are written with the strides of Q, K and V
  if (!rows_disjoint(s->q_stride, s->B, s->Hq, s->L, s->d) || !rows_disjoint(s->k_stride, s->B, s->Hkv, s->L, s->d) ||
      !rows_disjoint(s->v_stride, s->B, s->Hkv, s->L, s->d))
    return sepattn_fail(SEPATTN_EINVAL, "bwd: q/k/v strides (also those of dq/dk/dv) make output rows overlap");
  const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv, workspace};
  for (const void* pp : ptrs)
    if (!aligned16(pp)) return sepattn_fail(SEPATTN_EINVAL, "bwd: tensors must be 16-byte aligned");
  if (workspace_bytes < sepattn_bwd_workspace_size(s))
    return sepattn_fail(SEPATTN_ESPACE, "bwd: workspace %zu bytes < %zu", workspace_bytes,
                        sepattn_bwd_workspace_size(s));
  if (!std::isfinite(scale)) return sepattn_fail(SEPATTN_EINVAL, "bwd: scale is not finite");
  SEPATTN_TRY(sepattn_check_device());
  return sepattn_launch_bwd(s, dtype, m, q, k, v, o, lse, dout, scale, dq, dk, dv, (float*)workspace,
                            (hipStream_t)stream);
}

int sepattn_bwd_noalloc(const sepattn_shape* s, int dtype, const sepattn_mask* m, const void* q, const void* k,
                        const void* v, const void* o, const float* lse, const void* dout, float scale, void* dq,
                        void* dk, void* dv, void* stream) {
  g_err[0] = 0;
  SEPATTN_TRY(check_shape(s, dtype, m, "bwd_noalloc"));
  if (dtype != SEPATTN_BF16) return sepattn_fail(SEPATTN_ENOTSUP, "bwd_noalloc: only bf16 is implemented");
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
    return sepattn_fail(SEPATTN_EINVAL, "bwd_noalloc: null tensor");
  const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* pp : ptrs)
    if (!aligned16(pp)) return sepattn_fail(SEPATTN_EINVAL, "bwd_noalloc: tensors must be 16-byte aligned");
  if (!rows_disjoint(s->q_stride, s->B, s->Hq, s->L, s->d) || !rows_disjoint(s->k_stride, s->B, s->Hkv, s->L, s->d) ||
      !rows_disjoint(s->v_stride, s->B, s->Hkv, s->L, s->d))
    return sepattn_fail(SEPATTN_EINVAL, "bwd_noalloc: q/k/v strides (also those of dq/dk/dv) make output rows overlap");
  const int64_t rows = (int64_t)s->B * s->Hq * s->L;
  if (rows > SEPATTN_BWD_NOALLOC_MAX_ROWS)
    return sepattn_fail(SEPATTN_ESPACE, "bwd_noalloc: B*Hq*L = %lld rows exceed the static workspace's %d",
                        (long long)rows, SEPATTN_BWD_NOALLOC_MAX_ROWS);
  if (!std::isfinite(scale)) return sepattn_fail(SEPATTN_EINVAL, "bwd_noalloc: scale is not finite");
  SEPATTN_TRY(sepattn_check_device());
  return sepattn_launch_bwd_noalloc(s, dtype, m, q, k, v, o, lse, dout, scale, dq, dk, dv, (hipStream_t)stream);
}

// ------------------------------------------------------------------ SepCache

int sepcache_slots(int a, int s, int n, int c) {
  if (a < 0 || s < 0 || n < 1 || c < 0 || (c > 0 && (int64_t)c < (int64_t)a + s + n)) return -1;
  const int64_t cap = c > 0 ? (int64_t)c : (int64_t)a + s + n;
  return cap + 1 > 65536 ? -1 : (int)(cap + 1);
}

int sepcache_k_rows(int slots) { return slots < 1 || slots > 65536 ? -1 : sepcache_k_rows_of(slots); }

static int check_cache(const sepcache* c, const char* who) {
  if (!c) return sepattn_fail(SEPATTN_EINVAL, "%s: null cache", who);
  if (c->B <= 0 || c->Hkv <= 0) return sepattn_fail(SEPATTN_EINVAL, "%s: B=%d Hkv=%d", who, c->B, c->Hkv);
  if (c->d != 64 && c->d != 128) return sepattn_fail(SEPATTN_ENOTSUP, "%s: head dim %d (64 or 128)", who, c->d);
  if (c->a < 0 || c->s < 0 || c->n < 1)
    return sepattn_fail(SEPATTN_EINVAL, "%s: need a >= 0, s >= 0, n >= 1 (a=%d s=%d n=%d)", who, c->a, c->s, c->n);
  if (c->c < 0 || (c->c > 0 && (int64_t)c->c < (int64_t)c->a + c->s + c->n))
    return sepattn_fail(SEPATTN_EINVAL, "%s: capacity c=%d below a + s + n = %d", who, c->c, c->a + c->s + c->n);
  if (sepcache_slots(c->a, c->s, c->n, c->c) < 0) return sepattn_fail(SEPATTN_EINVAL, "%s: cache too large", who);
  if (!c->k || !c->v || !c->slot_pos || !c->slot_sep || !c->state)
    return sepattn_fail(SEPATTN_EINVAL, "%s: null cache array", who);
  if (!aligned16(c->k) || !aligned16(c->v)) return sepattn_fail(SEPATTN_EINVAL, "%s: K/V not 16-byte aligned", who);
  if (!(c->theta > 1.f) || !std::isfinite(c->theta)) return sepattn_fail(SEPATTN_EINVAL, "%s: theta=%g", who, c->theta);
  return SEPATTN_OK;
}

int sepcache_reset(const sepcache* c, void* stream) {
  g_err[0] = 0;
  SEPATTN_TRY(check_cache(c, "reset"));
  SEPATTN_TRY(sepattn_check_device());
  return sepcache_launch_reset(c, (hipStream_t)stream);
}

static int update(const sepcache* c, const void* k_new, const void* v_new, const uint8_t* is_sep, int app,
                  int ev, void* stream, const char* who) {
  g_err[0] = 0;
  SEPATTN_TRY(check_cache(c, who));
  if (app && (!k_new || !v_new || !is_sep)) return sepattn_fail(SEPATTN_EINVAL, "%s: null input", who);
  if (app && (!aligned16(k_new) || !aligned16(v_new)))
    return sepattn_fail(SEPATTN_EINVAL, "%s: K/V rows not 16-byte aligned", who);
  SEPATTN_TRY(sepattn_check_device());
  return sepcache_launch_update(c, k_new, v_new, is_sep, app, ev, (hipStream_t)stream);
}

int sepcache_append(const sepcache* c, const void* k_new, const void* v_new, const uint8_t* is_sep, void* stream) {
  return update(c, k_new, v_new, is_sep, 1, 0, stream, "append");
}
int sepcache_evict(const sepcache* c, void* stream) { return update(c, nullptr, nullptr, nullptr, 0, 1, stream, "evict"); }
int sepcache_push(const sepcache* c, const void* k_new, const void* v_new, const uint8_t* is_sep, void* stream) {
  return update(c, k_new, v_new, is_sep, 1, 1, stream, "push");
}

size_t sepcache_decode_workspace_size(const sepcache* c, int Hq) {
  if (!c || c->B <= 0 || c->Hkv <= 0 || Hq <= 0 || Hq % c->Hkv != 0 || (c->d != 64 && c->d != 128) ||
      sepcache_slots(c->a, c->s, c->n, c->c) < 0)
    return 0;
  return sepcache_decode_ws_bytes(c, Hq);
}

static int check_attend(const sepcache* c, int Hq, const void* q, float scale, void* o, const char* who) {
  SEPATTN_TRY(check_cache(c, who));
  if (Hq <= 0 || Hq % c->Hkv != 0)
    return sepattn_fail(SEPATTN_EINVAL, "%s: Hq=%d is not a positive multiple of Hkv=%d", who, Hq, c->Hkv);
  const int G = Hq / c->Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return sepattn_fail(SEPATTN_ENOTSUP, "%s: %d q heads per KV head (1, 2, 4 or 8)", who, G);
  if (!q || !o) return sepattn_fail(SEPATTN_EINVAL, "%s: null q or o", who);
  if (!aligned16(q) || !aligned16(o)) return sepattn_fail(SEPATTN_EINVAL, "%s: q/o not 16-byte aligned", who);
  if (!std::isfinite(scale)) return sepattn_fail(SEPATTN_EINVAL, "%s: scale is not finite", who);
  return SEPATTN_OK;
}

static int check_ws(const sepcache* c, int Hq, const void* ws, size_t bytes, const char* who) {
  const size_t need = sepcache_decode_ws_bytes(c, Hq);
  if (need == 0) return SEPATTN_OK;  // the single-kernel path uses none
  if (!ws || bytes < need) return sepattn_fail(SEPATTN_ESPACE, "%s: workspace %zu bytes < %zu", who, bytes, need);
  if (!aligned16(ws)) return sepattn_fail(SEPATTN_EINVAL, "%s: workspace not 16-byte aligned", who);
  return SEPATTN_OK;
}

int sepcache_decode(const sepcache* c, int Hq, const void* q, float scale, int shift, void* o, void* workspace,
                    size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  SEPATTN_TRY(check_attend(c, Hq, q, scale, o, "decode"));
  SEPATTN_TRY(check_ws(c, Hq, workspace, workspace_bytes, "decode"));
  SEPATTN_TRY(sepattn_check_device());
  return sepcache_launch_decode(c, Hq, q, scale, shift, o, workspace, (hipStream_t)stream);
}

int sepcache_step(const sepcache* c, const void* k_new, const void* v_new, const uint8_t* is_sep, int Hq,
                  const void* q, float scale, int shift, void* o, void* workspace, size_t workspace_bytes,
                  void* stream) {
  g_err[0] = 0;
  SEPATTN_TRY(check_attend(c, Hq, q, scale, o, "step"));
  if (!k_new || !v_new || !is_sep) return sepattn_fail(SEPATTN_EINVAL, "step: null input");
  if (!aligned16(k_new) || !aligned16(v_new)) return sepattn_fail(SEPATTN_EINVAL, "step: K/V rows not 16-byte aligned");
  SEPATTN_TRY(check_ws(c, Hq, workspace, workspace_bytes, "step"));
  SEPATTN_TRY(sepattn_check_device());
  return sepcache_launch_step(c, k_new, v_new, is_sep, Hq, q, scale, shift, o, workspace, (hipStream_t)stream);
}

int sepcache_prefill(const sepcache* c, const void* k, const void* v, const int64_t* k_stride,
                     const int64_t* v_stride, const sepattn_mask* m, void* stream) {
  g_err[0] = 0;
  SEPATTN_TRY(check_cache(c, "prefill"));
  SEPATTN_TRY(check_mask(m, "prefill"));
  if (m->B != c->B) return sepattn_fail(SEPATTN_EINVAL, "prefill: mask B=%d, cache B=%d", m->B, c->B);
  if (m->a != c->a) return sepattn_fail(SEPATTN_EINVAL, "prefill: mask a=%d, cache a=%d", m->a, c->a);
  if (!k || !v || !k_stride || !v_stride) return sepattn_fail(SEPATTN_EINVAL, "prefill: null K/V or strides");
  if (!aligned16(k) || !aligned16(v)) return sepattn_fail(SEPATTN_EINVAL, "prefill: K/V not 16-byte aligned");
  for (int i = 0; i < 3; ++i)
    if (k_stride[i] < 0 || v_stride[i] < 0 || k_stride[i] % 8 != 0 || v_stride[i] % 8 != 0)
      return sepattn_fail(SEPATTN_EINVAL, "prefill: strides must be non-negative multiples of 8 elements");
  SEPATTN_TRY(sepattn_check_device());
  return sepcache_launch_prefill(c, k, v, k_stride, v_stride, m, (hipStream_t)stream);
}

int sepcache_export_order(const sepcache* c, int32_t* pos, int32_t* len, void* stream) {
  g_err[0] = 0;
  SEPATTN_TRY(check_cache(c, "export_order"));
  if (!pos || !len) return sepattn_fail(SEPATTN_EINVAL, "export_order: null output");
  SEPATTN_TRY(sepattn_check_device());
  return sepcache_launch_export(c, pos, len, (hipStream_t)stream);
}

}  // extern "C"
