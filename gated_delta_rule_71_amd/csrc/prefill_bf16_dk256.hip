// Prefill instantiations: bf16 I/O, bf16 matrix-core operands, dk = 256 (the all-modes kernel;
// only the scalar- and no-decay layouts fit in LDS at this width).
#include "prefill_dispatch.h"

namespace gdr {
hipError_t prefill_bf16_dk256(const PrefillArgs<bf16_t>& a, int64_t nstate, int mode, int nsw,
                              hipStream_t s) {
  return launch_prefill_dk<bf16_t, __bf16, 256>(a, nstate, mode, nsw, s);
}
}  // namespace gdr
