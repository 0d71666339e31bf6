// Paged causal prefill (MFMA) — not built yet: every shape reports unsupported.
#include "pa_internal.h"

namespace pa {

bool prefill_supported(pa_dtype, int, int) { return false; }

hipError_t launch_paged_prefill(const Cache&, void*, pa_dtype, const void*, const int32_t*, int32_t,
                                const int32_t*, const int32_t*, int32_t, int32_t, int32_t, float,
                                hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace pa
