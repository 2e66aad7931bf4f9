// Prefill instantiations: bf16 I/O, bf16 matrix-core operands, dk = 32.
#include "prefill_dispatch.h"

namespace gdr {
hipError_t prefill_bf16_dk32(const PrefillArgs<bf16_t>& a, int64_t nstate, int mode, int nsw,
                              hipStream_t s) {
  return launch_prefill_dk<bf16_t, __bf16, 32>(a, nstate, mode, nsw, s);
}
}  // namespace gdr
