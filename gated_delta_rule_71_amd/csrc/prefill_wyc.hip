// Host side of the two-kernel per-channel-decay prefill: workspace carving and launches.
#include "prefill_wyc.h"

namespace gdr {

namespace {
size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct WycSizes {
  size_t Qd, Ad, Dt, Zd, Egn, flag;
  size_t total() const { return Qd + Ad + Dt + Zd + Egn + flag; }
};

// per chunk: Q' (64 x dk), A' (dk x dk), D^T (dv x dk), Z' (64 x dv) in bf16, dk + 4 floats, a flag
WycSizes wyc_sizes(int64_t nstate, int64_t T, int64_t DK, int64_t DV) {
  const size_t ch = static_cast<size_t>(nstate) * static_cast<size_t>((T + 63) / 64);
  WycSizes s;
  s.Qd = align256(ch * 64 * DK * 2);
  s.Ad = align256(ch * DK * DK * 2);
  s.Dt = align256(ch * DV * DK * 2);
  s.Zd = align256(ch * 64 * DV * 2);
  s.Egn = align256(ch * (DK + 4) * 4);
  s.flag = align256(ch * 4);
  return s;
}

// SPLIT = 2: two state waves per 16 columns, each with half of the channels (d_k >= 64, up to 32
// columns a workgroup by LDS)
template <int DK, int NSW, bool AZ>
void launch_state(WycArgs a, int64_t nstate, hipStream_t s) {
  a.nsl = static_cast<int>(a.DV / (16 * NSW));
  constexpr int SPLIT = (DK >= 64 && NSW <= 2) ? 2 : 1;
  hipLaunchKernelGGL((wyc_state_kernel<DK, NSW, SPLIT, AZ>), dim3((unsigned)(nstate * a.nsl)),
                     dim3(64 * (2 + NSW * SPLIT)), 0, s, a);
}

// MODE 0: no erase gate (either order), 1: decay then erase, 2: erase then decay
template <int DK, int MODE>
hipError_t launch_mode(WycArgs a, int64_t nstate, hipEvent_t mark, hipStream_t s) {
  constexpr bool AZ = MODE == 0;
  const int64_t nprep = nstate * a.nch;
  if (nprep > 0) {
    if constexpr (AZ) {
      if (a.DV <= 128)
        hipLaunchKernelGGL((wyg_prep_kernel<DK, 128>), dim3((unsigned)nprep), dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((wyg_prep_kernel<DK, 256>), dim3((unsigned)nprep), dim3(256), 0, s, a);
    } else {
      if (a.DV <= 128)
        hipLaunchKernelGGL((wyc_prep_kernel<DK, 128, MODE>), dim3((unsigned)nprep), dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((wyc_prep_kernel<DK, 256, MODE>), dim3((unsigned)nprep), dim3(512), 0, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (mark != nullptr) {
    const hipError_t e = hipEventRecord(mark, s);
    if (e != hipSuccess) return e;
  }
  // the widest value slice (64, 32 or 16 columns: one state wave per 16) that still gives a
  // workgroup per compute unit, else the narrowest (the most workgroups)
  const int64_t DV = a.DV;
  if (DV % 64 == 0 && nstate * (DV / 64) >= 256)
    launch_state<DK, 4, AZ>(a, nstate, s);
  else if (DV % 32 == 0 && nstate * (DV / 32) >= 256)
    launch_state<DK, 2, AZ>(a, nstate, s);
  else
    launch_state<DK, 1, AZ>(a, nstate, s);
  return hipGetLastError();
}
}  // namespace

// bf16 I/O, per-channel decay, dk in {32, 64, 128}, dv a multiple of 16 up to 256.
bool prefill_wyc_ok(int64_t DK, int64_t DV) {
  return (DK == 32 || DK == 64 || DK == 128) && DV % 16 == 0 && DV > 0 && DV <= 256;
}

size_t prefill_wyc_workspace_bytes(int64_t nstate, int64_t T, int64_t DK, int64_t DV, bool two) {
  (void)two;
  return wyc_sizes(nstate, T, DK, DV).total();
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
  a.alpha_kind = kChannel;
  const WycSizes z = wyc_sizes(nstate, p.T, DK, p.DV);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  a.Qd = reinterpret_cast<__bf16*>(ws);
  ws += z.Qd;
  a.Ad = reinterpret_cast<__bf16*>(ws);
  ws += z.Ad;
  a.Dt = reinterpret_cast<__bf16*>(ws);
  ws += z.Dt;
  a.Zd = reinterpret_cast<__bf16*>(ws);
  ws += z.Zd;
  a.Egn = reinterpret_cast<float*>(ws);
  ws += z.Egn;
  a.flag = reinterpret_cast<int*>(ws);
  // without an erase gate both orders are the same recurrence, and A' = 0
  const int mode = p.b_kind == kNone ? 0 : two ? 2 : 1;
  switch (DK) {
    case 32: return mode == 0 ? launch_mode<32, 0>(a, nstate, mark, s)
                    : mode == 2 ? launch_mode<32, 2>(a, nstate, mark, s) : launch_mode<32, 1>(a, nstate, mark, s);
    case 64: return mode == 0 ? launch_mode<64, 0>(a, nstate, mark, s)
                    : mode == 2 ? launch_mode<64, 2>(a, nstate, mark, s) : launch_mode<64, 1>(a, nstate, mark, s);
    default: return mode == 0 ? launch_mode<128, 0>(a, nstate, mark, s)
                    : mode == 2 ? launch_mode<128, 2>(a, nstate, mark, s) : launch_mode<128, 1>(a, nstate, mark, s);
  }
}

}  // namespace gdr
