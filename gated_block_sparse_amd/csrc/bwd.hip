// Backward of the prefill forward -- placeholder until the kernels land.
#include "sas_internal.h"

namespace sas {

size_t bwd_ws_bytes(const sas_dims&, int) { return 0; }

sas_status launch_bwd(const sas_dims&, const void*, const void*, const void*, const void*,
                      const void*, const float*, int, const int32_t*, const float*, float, void*,
                      void*, void*, float*, void*, hipStream_t) {
  return fail(SAS_ERR_UNSUPPORTED, "backward is not built yet");
}

}  // namespace sas
