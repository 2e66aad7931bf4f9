// Prefill instantiations: fp32 I/O with fp32 matrix-core operands (one state wave).
#include "prefill_dispatch.h"

namespace gdr {
hipError_t prefill_f32_any(const PrefillArgs<float>& a, int64_t nstate, int64_t DK, int mode,
                           int nsw, hipStream_t s) {
  (void)nsw;
  switch (DK) {
    case 16: return launch_prefill_mode<float, float, 16, 1>(a, nstate, mode, s);
    case 32: return launch_prefill_mode<float, float, 32, 1>(a, nstate, mode, s);
    case 64: return launch_prefill_mode<float, float, 64, 1>(a, nstate, mode, s);
    default: return launch_prefill_mode<float, float, 128, 1>(a, nstate, mode, s);
  }
}
}  // namespace gdr
