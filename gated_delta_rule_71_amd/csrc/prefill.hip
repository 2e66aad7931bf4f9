// Host entry for the chunkwise prefill: picks the kernel variant for a problem.
#include "prefill_dispatch.h"

namespace gdr {

bool prefill_wy_ok(int64_t DK, int64_t DV, int b_kind);
size_t prefill_wy_workspace_bytes(int64_t nstate, int64_t T, int64_t DK, int64_t DV);
hipError_t prefill_wy_launch(const PrefillArgs<bf16_t>& p, int64_t nstate, int64_t DK,
                             void* workspace, hipEvent_t mark, hipStream_t s);
bool prefill_wyc_ok(int64_t DK, int64_t DV);
size_t prefill_wyc_workspace_bytes(int64_t nstate, int64_t T, int64_t DK, int64_t DV, bool two);
hipError_t prefill_wyc_launch(const PrefillArgs<bf16_t>& p, int64_t nstate, int64_t DK, bool two,
                              void* workspace, hipEvent_t mark, hipStream_t s);
bool prefill_seg_ok(int64_t DK, int64_t DV, int alpha_kind, int b_kind, int w_kind, bool decay_first);
size_t prefill_seg_workspace_bytes(int64_t nstate, int64_t T);
hipError_t prefill_seg_launch(const PrefillArgs<bf16_t>& pa, int64_t nstate, bool two, void* workspace,
                              hipEvent_t mark, hipStream_t s);
template <typename IO>
hipError_t prefill_recur(const PrefillArgs<IO>& a, int64_t nstate, int64_t DK, bool decay_first,
                         hipStream_t s);

namespace {

// MODE 0: scalar (or no) decay; 1: per-channel decay applied before the erase;
// 2: per-channel decay applied after the erase (the unified equation's order).
int prefill_mode(int alpha_kind, bool decay_first) {
  if (alpha_kind != kChannel) return 0;
  return decay_first ? 1 : 2;
}

template <typename OT>
bool fits_dk(int64_t DK, int mode, int nsw) {
  switch (DK) {
    case 16: return prefill_fits<OT, 16>(mode, nsw);
    case 32: return prefill_fits<OT, 32>(mode, nsw);
    case 64: return prefill_fits<OT, 64>(mode, nsw);
    case 128: return prefill_fits<OT, 128>(mode, nsw);
    case 256: return prefill_fits<OT, 256>(mode, nsw);
    default: return false;
  }
}

// State waves per workgroup for bf16: the widest slice (2 or 1 x 16 columns) that divides dv
// and fits in LDS.
int choose_nsw_bf16(int64_t DK, int64_t DV, int mode) {
  for (int nsw = 2; nsw >= 1; nsw /= 2)
    if (DV % (16 * nsw) == 0 && fits_dk<__bf16>(DK, mode, nsw)) return nsw;
  return 0;
}

// The optional phase marker of a single-kernel problem goes before its one launch.
hipError_t record_mark(hipEvent_t mark, hipStream_t stream) {
  return mark != nullptr ? hipEventRecord(mark, stream) : hipSuccess;
}

}  // namespace

size_t prefill_workspace_bytes(int io_dtype, int64_t nstate, int64_t T, int64_t DK, int64_t DV,
                               int alpha_kind, int b_kind, int w_kind, bool decay_first) {
  if (io_dtype != 0) return 0;
  if (prefill_seg_ok(DK, DV, alpha_kind, b_kind, w_kind, decay_first || alpha_kind != kChannel))
    return prefill_seg_workspace_bytes(nstate, T);
  if (alpha_kind != kChannel)
    return prefill_wy_ok(DK, DV, b_kind) ? prefill_wy_workspace_bytes(nstate, T, DK, DV) : 0;
  return prefill_wyc_ok(DK, DV) ? prefill_wyc_workspace_bytes(nstate, T, DK, DV, !decay_first) : 0;
}

// Every validated shape runs: the chunkwise kernels where their LDS layout fits, else the token
// recurrence (dk >= 64 only; dk 16 and 32 always fit).
bool prefill_supported(int io_dtype, int64_t DK, int64_t DV, int alpha_kind, bool decay_first) {
  if (DV % 16 != 0) return false;
  return DK == 16 || DK == 32 || DK == 64 || DK == 128 || DK == 256;
}

// Whether the chunkwise all-modes kernel fits this problem (else the token recurrence runs).
bool chunk_kernel_fits(int io_dtype, int64_t DK, int64_t DV, int mode) {
  if (io_dtype == 0) return choose_nsw_bf16(DK, DV, mode) > 0;
  return fits_dk<float>(DK, mode, 1);
}

template <typename IO>
hipError_t launch_prefill(const IO* q, const IO* k, const IO* v, const IO* la, const IO* bg,
                          const IO* wg, const float* S0, IO* o, float* S_T, int64_t B, int64_t T,
                          int64_t H, int64_t Hk, int64_t DK, int64_t DV, int alpha_kind,
                          int b_kind, int w_kind, bool decay_first, void* workspace,
                          hipEvent_t mark, hipStream_t stream) {
  const int mode = prefill_mode(alpha_kind, decay_first);
  PrefillArgs<IO> a{q, k, v, la, bg, wg, S0, o, S_T, T, H, DV, alpha_kind, b_kind, w_kind, 1, Hk};
  const int64_t nstate = B * H;
  if constexpr (sizeof(IO) == 2) {
    // the fused segment kernel for d_k = d_v = 128 and the gates it is built for (a scalar decay
    // commutes with the erase, so it takes the decay-first form)
    if (prefill_seg_ok(DK, DV, alpha_kind, b_kind, w_kind, decay_first || alpha_kind != kChannel))
      return prefill_seg_launch(a, nstate, mode == 2, workspace, mark, stream);
    if (mode == 0) {
      if (prefill_wy_ok(DK, DV, b_kind)) return prefill_wy_launch(a, nstate, DK, workspace, mark, stream);
    } else if (prefill_wyc_ok(DK, DV)) {
      return prefill_wyc_launch(a, nstate, DK, mode == 2, workspace, mark, stream);
    }
    const int nsw = choose_nsw_bf16(DK, DV, mode);
    if (const hipError_t e = record_mark(mark, stream); e != hipSuccess) return e;
    if (nsw == 0) return prefill_recur(a, nstate, DK, decay_first, stream);
    a.nsl = static_cast<int>(DV / (16 * nsw));
    switch (DK) {
      case 16: return prefill_bf16_dk16(a, nstate, mode, nsw, stream);
      case 32: return prefill_bf16_dk32(a, nstate, mode, nsw, stream);
      case 64: return prefill_bf16_dk64(a, nstate, mode, nsw, stream);
      case 128: return prefill_bf16_dk128(a, nstate, mode, nsw, stream);
      default: return prefill_bf16_dk256(a, nstate, mode, nsw, stream);
    }
  } else {
    if (const hipError_t e = record_mark(mark, stream); e != hipSuccess) return e;
    if (!fits_dk<float>(DK, mode, 1)) return prefill_recur(a, nstate, DK, decay_first, stream);
    a.nsl = static_cast<int>(DV / 16);
    return prefill_f32_any(a, nstate, DK, mode, 1, stream);
  }
}

template hipError_t launch_prefill<bf16_t>(const bf16_t*, const bf16_t*, const bf16_t*,
                                           const bf16_t*, const bf16_t*, const bf16_t*,
                                           const float*, bf16_t*, float*, int64_t, int64_t,
                                           int64_t, int64_t, int64_t, int64_t, int, int, int,
                                           bool, void*,
                                           hipEvent_t, hipStream_t);
template hipError_t launch_prefill<float>(const float*, const float*, const float*, const float*,
                                          const float*, const float*, const float*, float*, float*,
                                          int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int,
                                          int, int, bool, void*, hipEvent_t, hipStream_t);

}  // namespace gdr
