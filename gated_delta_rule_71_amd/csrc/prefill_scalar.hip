// Launches of the pipelined scalar-decay prefill (bf16, dk in {32, 64, 128}, 16 or 32 columns).
#include "prefill_scalar.h"

namespace gdr {

template <int DK, int NSW>
static hipError_t launch_scalar_inst(const PrefillArgs<bf16_t>& a, int64_t nstate, hipStream_t s) {
  const int64_t blocks = nstate * a.nsl;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_scalar_kernel<DK, NSW>), dim3((unsigned)blocks), dim3(256 + 64 * NSW),
                     0, s, a);
  return hipGetLastError();
}

// Buffer addressing uses 32-bit byte offsets within one batch element's tokens.
bool prefill_scalar_ok(int64_t T, int64_t H, int64_t DK, int64_t DV, int b_kind) {
  const int64_t span = T * H * (DK > DV ? DK : DV) * 2;
  return (DK == 32 || DK == 64 || DK == 128) && DV % 16 == 0 && b_kind != kChannel &&
         span < (int64_t(1) << 31);
}

hipError_t prefill_scalar_launch(PrefillArgs<bf16_t> a, int64_t nstate, int64_t DK,
                                 hipStream_t s) {
  const int nsw = a.DV % 32 == 0 ? 2 : 1;
  a.nsl = static_cast<int>(a.DV / (16 * nsw));
  switch (DK * 10 + nsw) {
    case 322: return launch_scalar_inst<32, 2>(a, nstate, s);
    case 321: return launch_scalar_inst<32, 1>(a, nstate, s);
    case 642: return launch_scalar_inst<64, 2>(a, nstate, s);
    case 641: return launch_scalar_inst<64, 1>(a, nstate, s);
    case 1282: return launch_scalar_inst<128, 2>(a, nstate, s);
    case 1281: return launch_scalar_inst<128, 1>(a, nstate, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdr
