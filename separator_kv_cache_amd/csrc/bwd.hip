#include "common.h"
int sepattn_launch_bwd(const sepattn_shape*, int, const sepattn_mask*, const void*, const void*, const void*,
                       const void*, const float*, const void*, float, void*, void*, void*, float*, hipStream_t) {
  return sepattn_fail(SEPATTN_ENOTSUP, "bwd: not built yet");
}
