// Prefill-chunk attention (MFMA) — not built yet: every row goes through the decode path.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace pkv {

bool prefill_supported(int, int, bool) { return false; }

hipError_t launch_prefill(const PrefillArgs&, int64_t, int, int, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace pkv
