#include "common.h"
int sepcache_launch_reset(const sepcache*, hipStream_t) { return sepattn_fail(SEPATTN_ENOTSUP, "not built yet"); }
int sepcache_launch_update(const sepcache*, const void*, const void*, const uint8_t*, int, int, hipStream_t) {
  return sepattn_fail(SEPATTN_ENOTSUP, "not built yet");
}
size_t sepcache_decode_ws_bytes(const sepcache*, int) { return 0; }
int sepcache_launch_decode(const sepcache*, int, const void*, float, int, void*, void*, hipStream_t) {
  return sepattn_fail(SEPATTN_ENOTSUP, "not built yet");
}
int sepcache_launch_export(const sepcache*, int32_t*, int32_t*, hipStream_t) {
  return sepattn_fail(SEPATTN_ENOTSUP, "not built yet");
}
