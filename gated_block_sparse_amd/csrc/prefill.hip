// Prefill / training forward (bf16 MFMA) -- placeholder until the kernel lands.
#include "sas_internal.h"

namespace sas {

size_t prefill_ws_bytes(const sas_dims&, int) { return 0; }

sas_status launch_prefill_fwd(const sas_dims&, const void*, const void*, const void*, int,
                              const int32_t*, const float*, float, void*, float*, void*,
                              hipStream_t) {
  return fail(SAS_ERR_UNSUPPORTED, "prefill forward is not built yet");
}

size_t bwd_ws_bytes(const sas_dims&, int) { return 0; }

sas_status launch_bwd(const sas_dims&, const void*, const void*, const void*, const void*,
                      const void*, const float*, int, const int32_t*, const float*, float, void*,
                      void*, void*, float*, void*, hipStream_t) {
  return fail(SAS_ERR_UNSUPPORTED, "backward is not built yet");
}

}  // namespace sas
