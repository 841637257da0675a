/* Host-side driver for the sanitizer build of the C ABI: every call below is
 * one the library must refuse (or that needs a GPU, which the build host does
 * not have), so only argument validation and error reporting run, under
 * AddressSanitizer and UndefinedBehaviorSanitizer.  Exit status 0 when every
 * return code is the expected one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sepattn.h"

static int fails = 0;
#define EXPECT(call, want)                                                                  \
  do {                                                                                      \
    int _rc = (call);                                                                       \
    if (_rc != (want)) {                                                                    \
      fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, _rc, \
              (want), sepattn_last_error());                                                \
      ++fails;                                                                              \
    }                                                                                       \
  } while (0)

static void shape(sepattn_shape* s, int B, int Hq, int Hkv, int L, int d) {
  memset(s, 0, sizeof *s);
  s->B = B; s->Hq = Hq; s->Hkv = Hkv; s->L = L; s->d = d;
  int64_t* st[4] = {s->q_stride, s->k_stride, s->v_stride, s->o_stride};
  for (int t = 0; t < 4; ++t) {
    const int H = (t == 0 || t == 3) ? Hq : Hkv;
    st[t][0] = (int64_t)H * L * d; st[t][1] = (int64_t)L * d; st[t][2] = d;
  }
}

int main(void) {
  static unsigned char host_buf[1 << 20] __attribute__((aligned(256)));
  void* p = (void*)(uintptr_t)4096;  /* never dereferenced: every call below fails validation */
  sepattn_mask m, m2;
  const size_t mb = sepattn_mask_bytes(1, 64);
  EXPECT(sepattn_mask_carve(&m, 1, 64, 4, 8, host_buf, mb), SEPATTN_OK);
  EXPECT(sepattn_mask_carve(&m2, 0, 64, 4, 8, host_buf, mb), SEPATTN_EINVAL);
  EXPECT(sepattn_mask_carve(&m2, 1, 64, 4, 0, host_buf, mb), SEPATTN_EINVAL);
  EXPECT(sepattn_mask_carve(&m2, 2, 100, 1, 3, host_buf, 64), SEPATTN_ESPACE);
  EXPECT(sepattn_mask_carve(NULL, 1, 64, 4, 8, host_buf, mb), SEPATTN_EINVAL);
  if (sepattn_mask_bytes(0, 10) != 0 || sepattn_mask_bytes(-3, -3) != 0) ++fails;
  const int32_t ids[2] = {5, 7};
  EXPECT(sepattn_build_mask(NULL, ids, 2, &m, NULL), SEPATTN_EINVAL);
  EXPECT(sepattn_build_mask((const int32_t*)p, ids, 0, &m, NULL), SEPATTN_EINVAL);
  EXPECT(sepattn_build_mask((const int32_t*)p, ids, SEPATTN_MAX_SEP_IDS + 1, &m, NULL), SEPATTN_EINVAL);
  EXPECT(sepattn_build_mask_fixed(0, &m, NULL), SEPATTN_EINVAL);
  EXPECT(sepattn_mask_bits(&m, NULL, NULL), SEPATTN_EINVAL);
  EXPECT(sepattn_tile_desc(&m, 0, (int32_t*)p, NULL), SEPATTN_EINVAL);
  EXPECT(sepattn_tile_desc(NULL, 64, (int32_t*)p, NULL), SEPATTN_EINVAL);
  if (sepattn_fwd_tile_rows(0) != -1 || sepattn_fwd_tile_rows(256) != 64 || sepattn_fwd_tile_rows(257) != 256) ++fails;

  sepattn_shape s;
  shape(&s, 1, 3, 2, 64, 64);
  EXPECT(sepattn_fwd(&s, SEPATTN_BF16, &m, p, p, p, 0.1f, p, NULL, NULL), SEPATTN_EINVAL);
  shape(&s, 1, 4, 2, 64, 96);
  EXPECT(sepattn_fwd(&s, SEPATTN_BF16, &m, p, p, p, 0.1f, p, NULL, NULL), SEPATTN_ENOTSUP);
  shape(&s, 1, 4, 2, 64, 64);
  EXPECT(sepattn_fwd(&s, 7, &m, p, p, p, 0.1f, p, NULL, NULL), SEPATTN_ENOTSUP);
  EXPECT(sepattn_fwd(&s, SEPATTN_BF16, &m, NULL, p, p, 0.1f, p, NULL, NULL), SEPATTN_EINVAL);
  EXPECT(sepattn_fwd(&s, SEPATTN_BF16, &m, (void*)(uintptr_t)4098, p, p, 0.1f, p, NULL, NULL), SEPATTN_EINVAL);
  EXPECT(sepattn_fwd(&s, SEPATTN_BF16, &m, p, p, p, __builtin_inff(), p, NULL, NULL), SEPATTN_EINVAL);
  s.o_stride[1] = 0;
  EXPECT(sepattn_fwd(&s, SEPATTN_BF16, &m, p, p, p, 0.1f, p, NULL, NULL), SEPATTN_EINVAL);
  shape(&s, 1, 4, 2, 64, 64);
  s.q_stride[2] = 3;
  EXPECT(sepattn_fwd(&s, SEPATTN_BF16, &m, p, p, p, 0.1f, p, NULL, NULL), SEPATTN_EINVAL);
  shape(&s, 1, 4, 2, 64, 64);
  s.q_stride[2] = (int64_t)1 << 40;  /* a slice beyond 2 GiB */
  EXPECT(sepattn_fwd(&s, SEPATTN_BF16, &m, p, p, p, 0.1f, p, NULL, NULL), SEPATTN_ENOTSUP);
  shape(&s, 1, 4, 2, 64, 64);
  const size_t ws = sepattn_bwd_workspace_size(&s);
  EXPECT(sepattn_bwd(&s, SEPATTN_BF16, &m, p, p, p, p, (const float*)p, p, 0.1f, p, p, p, p, ws - 1, NULL),
         SEPATTN_ESPACE);
  EXPECT(sepattn_bwd(&s, SEPATTN_F32, &m, p, p, p, p, (const float*)p, p, 0.1f, p, p, p, p, ws, NULL),
         SEPATTN_ENOTSUP);
  s.k_stride[1] = 0;
  EXPECT(sepattn_bwd(&s, SEPATTN_BF16, &m, p, p, p, p, (const float*)p, p, 0.1f, p, p, p, p, ws, NULL),
         SEPATTN_EINVAL);
  sepattn_mask mbig;
  EXPECT(sepattn_mask_carve(&mbig, 1, 2048, 4, 8, host_buf, sepattn_mask_bytes(1, 2048)), SEPATTN_OK);
  shape(&s, 1, 4096, 1, 2048, 64);
  EXPECT(sepattn_bwd_noalloc(&s, SEPATTN_BF16, &mbig, p, p, p, p, (const float*)p, p, 0.1f, p, p, p, NULL),
         SEPATTN_ESPACE);

  if (sepcache_slots(4, 64, 256, 0) != 325 || sepcache_slots(4, 64, 256, 800) != 801 ||
      sepcache_slots(4, 64, 256, 300) != -1 || sepcache_slots(4, 64, 0, 0) != -1 ||
      sepcache_slots(0, 0, 70000, 0) != -1)
    ++fails;
  if (sepcache_k_rows(325) != 336 || sepcache_k_rows(0) != -1 || sepcache_k_rows(65537) != -1) ++fails;
  sepcache c;
  memset(&c, 0, sizeof c);
  c.B = 2; c.Hkv = 2; c.d = 64; c.a = 4; c.s = 8; c.n = 0;
  EXPECT(sepcache_reset(&c, NULL), SEPATTN_EINVAL);
  c.n = 16; c.d = 80;
  EXPECT(sepcache_reset(&c, NULL), SEPATTN_ENOTSUP);
  c.d = 64;
  EXPECT(sepcache_reset(&c, NULL), SEPATTN_EINVAL);
  c.k = c.v = p; c.slot_pos = (int32_t*)p; c.slot_sep = (uint8_t*)p; c.state = (int32_t*)p;
  EXPECT(sepcache_decode(&c, 4, p, 0.1f, 1, p, p, 1000000, NULL), SEPATTN_EINVAL); /* theta 0 */
  c.theta = 10000.f;
  EXPECT(sepcache_decode(&c, 3, p, 0.1f, 1, p, p, 1000000, NULL), SEPATTN_EINVAL);
  EXPECT(sepcache_decode(&c, 32, p, 0.1f, 1, p, p, 1000000, NULL), SEPATTN_ENOTSUP);
  c.s = 2000;
  const size_t need = sepcache_decode_workspace_size(&c, 4);
  if (need == 0) ++fails;
  EXPECT(sepcache_decode(&c, 4, p, 0.1f, 1, p, p, need - 1, NULL), SEPATTN_ESPACE);
  c.s = 8; c.c = 20;
  EXPECT(sepcache_reset(&c, NULL), SEPATTN_EINVAL);
  c.c = 0;
  EXPECT(sepcache_step(&c, NULL, p, (const uint8_t*)p, 4, p, 0.1f, 1, p, NULL, 0, NULL), SEPATTN_EINVAL);
  const int64_t st3[3] = {0, 0, 64}, bad[3] = {0, 0, 65};
  EXPECT(sepcache_prefill(&c, p, p, st3, st3, NULL, NULL), SEPATTN_EINVAL);
  sepattn_mask mk;
  EXPECT(sepattn_mask_carve(&mk, 2, 10, 3, 3, host_buf, sepattn_mask_bytes(2, 10)), SEPATTN_OK);
  EXPECT(sepcache_prefill(&c, p, p, st3, st3, &mk, NULL), SEPATTN_EINVAL);  /* a = 3 vs 4 */
  mk.a = 4;
  EXPECT(sepcache_prefill(&c, p, p, bad, st3, &mk, NULL), SEPATTN_EINVAL);
  EXPECT(sepcache_export_order(&c, NULL, NULL, NULL), SEPATTN_EINVAL);
  if (strlen(sepattn_last_error()) == 0) ++fails;
  printf("%s: %d unexpected return codes\n", fails ? "FAIL" : "ok", fails);
  return fails ? 1 : 0;
}
