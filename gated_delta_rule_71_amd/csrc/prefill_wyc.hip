// Host side of the two-kernel per-channel-decay prefill: workspace carving and launches.
#include "prefill_wyc.h"

namespace gdr {

namespace {
size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct WycSizes {
  size_t W, Qp, Pn, Kb, Mn, Y, Z, Xt, Egn, flag;
  size_t total() const { return W + Qp + Pn + Kb + Mn + Y + Z + Xt + Egn + flag; }
};

WycSizes wyc_sizes(int64_t nstate, int64_t T, int64_t DK, int64_t DV, bool two) {
  const size_t ch = static_cast<size_t>(nstate) * static_cast<size_t>((T + 63) / 64);
  WycSizes s;
  s.W = align256(ch * 64 * DK * 2);
  s.Qp = s.W;
  s.Pn = align256(ch * DK * 64 * 2);
  s.Kb = two ? s.Pn : 0;
  s.Mn = align256(ch * 64 * 64 * 2);
  s.Y = align256(ch * 64 * DV * 2);
  s.Z = two ? s.Y : 0;
  s.Xt = two ? s.Y : 0;
  s.Egn = align256(ch * DK * 4);
  s.flag = align256(ch * 4);
  return s;
}

template <int DK, int MODE>
hipError_t launch_mode(WycArgs a, int64_t nstate, hipEvent_t mark, hipStream_t s) {
  const int64_t nprep = nstate * a.nch;
  if (nprep > 0) {
    if (a.DV <= 128)
      hipLaunchKernelGGL((wyc_prep_kernel<DK, 128, MODE>), dim3((unsigned)nprep), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((wyc_prep_kernel<DK, 256, MODE>), dim3((unsigned)nprep), dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (mark != nullptr) {
    const hipError_t e = hipEventRecord(mark, s);
    if (e != hipSuccess) return e;
  }
  // 32-column slices when that still gives a workgroup per compute unit, else 16 columns
  if (a.DV % 32 == 0 && nstate * (a.DV / 32) >= 256) {
    a.nsl = static_cast<int>(a.DV / 32);
    hipLaunchKernelGGL((wyc_state_kernel<DK, 2, MODE>), dim3((unsigned)(nstate * a.nsl)), dim3(192), 0, s, a);
  } else {
    a.nsl = static_cast<int>(a.DV / 16);
    hipLaunchKernelGGL((wyc_state_kernel<DK, 1, MODE>), dim3((unsigned)(nstate * a.nsl)), dim3(192), 0, s, a);
  }
  return hipGetLastError();
}
}  // namespace

// bf16 I/O, per-channel decay, dk in {32, 64, 128}, dv a multiple of 16 up to 256.
bool prefill_wyc_ok(int64_t DK, int64_t DV) {
  return (DK == 32 || DK == 64 || DK == 128) && DV % 16 == 0 && DV > 0 && DV <= 256;
}

size_t prefill_wyc_workspace_bytes(int64_t nstate, int64_t T, int64_t DK, int64_t DV, bool two) {
  return wyc_sizes(nstate, T, DK, DV, two).total();
}

hipError_t prefill_wyc_launch(const PrefillArgs<bf16_t>& p, int64_t nstate, int64_t DK, bool two,
                              void* workspace, hipEvent_t mark, hipStream_t s) {
  WycArgs a{};
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
  a.b_kind = p.b_kind;
  a.w_kind = p.w_kind;
  const WycSizes z = wyc_sizes(nstate, p.T, DK, p.DV, two);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  a.W = reinterpret_cast<__bf16*>(ws);
  ws += z.W;
  a.Qp = reinterpret_cast<__bf16*>(ws);
  ws += z.Qp;
  a.Pn = reinterpret_cast<__bf16*>(ws);
  ws += z.Pn;
  a.Kb = reinterpret_cast<__bf16*>(ws);
  ws += z.Kb;
  a.Mn = reinterpret_cast<__bf16*>(ws);
  ws += z.Mn;
  a.Y = reinterpret_cast<__bf16*>(ws);
  ws += z.Y;
  a.Z = reinterpret_cast<__bf16*>(ws);
  ws += z.Z;
  a.Xt = reinterpret_cast<__bf16*>(ws);
  ws += z.Xt;
  a.Egn = reinterpret_cast<float*>(ws);
  ws += z.Egn;
  a.flag = reinterpret_cast<int*>(ws);
  switch (DK) {
    case 32: return two ? launch_mode<32, 2>(a, nstate, mark, s) : launch_mode<32, 1>(a, nstate, mark, s);
    case 64: return two ? launch_mode<64, 2>(a, nstate, mark, s) : launch_mode<64, 1>(a, nstate, mark, s);
    default: return two ? launch_mode<128, 2>(a, nstate, mark, s) : launch_mode<128, 1>(a, nstate, mark, s);
  }
}

}  // namespace gdr
