// Launch helpers for the prefill kernel: one instantiation set per (I/O type, dk),
// compiled in separate translation units so that the build runs in parallel.
#pragma once
#include "prefill_kernel.h"

namespace gdr {

template <typename IO, typename OT, int DK, int NSW, int MODE>
hipError_t launch_prefill_inst(const PrefillArgs<IO>& a, int64_t nstate, hipStream_t s) {
  if constexpr (!PrefillLayout<OT, DK, NSW, MODE>::fits) {
    return hipErrorInvalidValue;
  } else {
    const int64_t blocks = nstate * a.nsl;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_kernel<IO, OT, DK, NSW, MODE>), dim3((unsigned)blocks), dim3(256),
                       0, s, a);
    return hipGetLastError();
  }
}

template <typename IO, typename OT, int DK, int NSW>
hipError_t launch_prefill_mode(const PrefillArgs<IO>& a, int64_t nstate, int mode, hipStream_t s) {
  switch (mode) {
    case 0: return launch_prefill_inst<IO, OT, DK, NSW, 0>(a, nstate, s);
    case 1: return launch_prefill_inst<IO, OT, DK, NSW, 1>(a, nstate, s);
    default: return launch_prefill_inst<IO, OT, DK, NSW, 2>(a, nstate, s);
  }
}

// nsw in {1, 2, 4}: state waves (16 value columns each) per workgroup.
template <typename IO, typename OT, int DK>
hipError_t launch_prefill_dk(const PrefillArgs<IO>& a, int64_t nstate, int mode, int nsw,
                             hipStream_t s) {
  switch (nsw) {
    case 4: return launch_prefill_mode<IO, OT, DK, 4>(a, nstate, mode, s);
    case 2: return launch_prefill_mode<IO, OT, DK, 2>(a, nstate, mode, s);
    default: return launch_prefill_mode<IO, OT, DK, 1>(a, nstate, mode, s);
  }
}

template <typename OT, int DK>
constexpr bool prefill_fits(int mode, int nsw) {
  return mode == 0   ? (nsw == 4   ? PrefillLayout<OT, DK, 4, 0>::fits
                        : nsw == 2 ? PrefillLayout<OT, DK, 2, 0>::fits
                                   : PrefillLayout<OT, DK, 1, 0>::fits)
         : mode == 1 ? (nsw == 4   ? PrefillLayout<OT, DK, 4, 1>::fits
                        : nsw == 2 ? PrefillLayout<OT, DK, 2, 1>::fits
                                   : PrefillLayout<OT, DK, 1, 1>::fits)
                     : (nsw == 4   ? PrefillLayout<OT, DK, 4, 2>::fits
                        : nsw == 2 ? PrefillLayout<OT, DK, 2, 2>::fits
                                   : PrefillLayout<OT, DK, 1, 2>::fits);
}

hipError_t prefill_bf16_dk16(const PrefillArgs<bf16_t>&, int64_t, int, int, hipStream_t);
hipError_t prefill_bf16_dk32(const PrefillArgs<bf16_t>&, int64_t, int, int, hipStream_t);
hipError_t prefill_bf16_dk64(const PrefillArgs<bf16_t>&, int64_t, int, int, hipStream_t);
hipError_t prefill_bf16_dk128(const PrefillArgs<bf16_t>&, int64_t, int, int, hipStream_t);
hipError_t prefill_bf16_dk256(const PrefillArgs<bf16_t>&, int64_t, int, int, hipStream_t);
hipError_t prefill_f32_any(const PrefillArgs<float>&, int64_t, int64_t, int, int, hipStream_t);

}  // namespace gdr
