// Host side of the two-kernel scalar-decay prefill: workspace carving and launches.
#include "prefill_wy.h"

namespace gdr {

namespace {
size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
}  // namespace

// bf16 I/O, scalar or no decay, no per-channel erase gate, dk in {32, 64, 128}, dv a multiple
// of 16 up to 256.
bool prefill_wy_ok(int64_t DK, int64_t DV, int b_kind) {
  return (DK == 32 || DK == 64 || DK == 128) && DV % 16 == 0 && DV > 0 && DV <= 256 &&
         b_kind != kChannel;
}

// Per 64-token chunk: W (64 x dk), U (64 x dv), -M (64 x 64), all bf16, and kWyE floats of
// exponentials; each array 256-byte aligned.
size_t prefill_wy_workspace_bytes(int64_t nstate, int64_t T, int64_t DK, int64_t DV) {
  const size_t chunks = static_cast<size_t>(nstate) * static_cast<size_t>((T + 63) / 64);
  return align256(chunks * 64 * DK * 2) + align256(chunks * 64 * DV * 2) +
         align256(chunks * 64 * 64 * 2) + align256(chunks * kWyE * 4);
}

namespace {
template <int DK, bool ERASE>
hipError_t launch_dk(WyArgs a, int64_t nstate, hipEvent_t mark, hipStream_t s) {
  const int64_t nprep = nstate * a.nch;
  if (nprep > 0) {
    if (a.DV <= 128)
      hipLaunchKernelGGL((wy_prep_kernel<DK, 128, ERASE>), dim3((unsigned)nprep), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((wy_prep_kernel<DK, 256, ERASE>), dim3((unsigned)nprep), dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (mark != nullptr) {
    const hipError_t e = hipEventRecord(mark, s);
    if (e != hipSuccess) return e;
  }
  // two state waves of 16 columns each (one LDS copy of a chunk feeds both), else one
  if (a.DV % 32 == 0) {
    a.nsl = static_cast<int>(a.DV / 32);
    hipLaunchKernelGGL((wy_state_kernel<DK, 1, 2, ERASE>), dim3((unsigned)(nstate * a.nsl)), dim3(256), 0, s, a);
  } else {
    a.nsl = static_cast<int>(a.DV / 16);
    hipLaunchKernelGGL((wy_state_kernel<DK, 1, 1, ERASE>), dim3((unsigned)(nstate * a.nsl)), dim3(192), 0, s, a);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t prefill_wy_launch(const PrefillArgs<bf16_t>& p, int64_t nstate, int64_t DK,
                             void* workspace, hipEvent_t mark, hipStream_t s) {
  WyArgs a{};
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.la = p.la;
  a.bg = p.bg;
  a.wg = p.wg;
  a.S0 = p.S0;
  a.o = p.o;
  a.S_T = p.S_T;
  a.T = p.T;
  a.H = p.H;
  a.DV = p.DV;
  a.Hk = p.Hk;
  a.nch = (p.T + 63) / 64;
  a.alpha_kind = p.alpha_kind;
  a.b_kind = p.b_kind;
  a.w_kind = p.w_kind;
  const size_t chunks = static_cast<size_t>(nstate) * static_cast<size_t>(a.nch);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  a.W = reinterpret_cast<__bf16*>(ws);
  ws += align256(chunks * 64 * DK * 2);
  a.U = reinterpret_cast<__bf16*>(ws);
  ws += align256(chunks * 64 * p.DV * 2);
  a.M = reinterpret_cast<__bf16*>(ws);
  ws += align256(chunks * 64 * 64 * 2);
  a.E = reinterpret_cast<float*>(ws);
  const bool erase = p.b_kind != kNone;  // without an erase gate: W = 0, U = X
  switch (DK) {
    case 32: return erase ? launch_dk<32, true>(a, nstate, mark, s) : launch_dk<32, false>(a, nstate, mark, s);
    case 64: return erase ? launch_dk<64, true>(a, nstate, mark, s) : launch_dk<64, false>(a, nstate, mark, s);
    default: return erase ? launch_dk<128, true>(a, nstate, mark, s) : launch_dk<128, false>(a, nstate, mark, s);
  }
}

}  // namespace gdr
