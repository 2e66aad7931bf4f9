// Launches of the fused segment prefill (prefill_seg.h): bf16, d_k = d_v = 128.
#include "prefill_seg.h"

namespace gdr {

namespace {

constexpr int64_t kSegTargetGroups = 256;  // one workgroup per CU (the kernel takes most of a CU's LDS)

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

struct SegPlan {
  int64_t nch, nseg, L;
};

// Segments per state: enough workgroups to fill the chip, at least one chunk each.
SegPlan seg_plan(int64_t nstate, int64_t T) {
  SegPlan p;
  p.nch = (T + kSegC - 1) / kSegC;
  if (nstate <= 0 || p.nch == 0) {
    p.nseg = 1;
    p.L = p.nch > 0 ? p.nch : 1;
    return p;
  }
  int64_t want = (kSegTargetGroups + nstate - 1) / nstate;
  if (want > p.nch) want = p.nch;
  if (want < 1) want = 1;
  p.L = (p.nch + want - 1) / want;
  p.nseg = (p.nch + p.L - 1) / p.L;
  return p;
}

}  // namespace

// Gate combinations with an instantiation: the Gated DeltaNet-2 gates (per-channel decay, erase
// and write gates), the KDA gates (per-channel decay, one scalar beta as erase and write gate),
// either order, and the Gated DeltaNet gates (scalar decay, scalar beta; a scalar decay commutes
// with the erase, so it takes the decay-first form).  Any other combination takes the two-kernel
// path.
bool prefill_seg_ok(int64_t DK, int64_t DV, int alpha_kind, int b_kind, int w_kind, bool decay_first) {
  (void)decay_first;  // both orders are built
  if (DK != 128 || DV != 128) return false;
  const bool gdn2 = alpha_kind == kChannel && b_kind == kChannel && w_kind == kChannel;
  const bool kda = alpha_kind == kChannel && b_kind == kScalar && w_kind == kScalar;
  const bool gdn = alpha_kind == kScalar && b_kind == kScalar && w_kind == kScalar;
  return gdn2 || kda || gdn;
}

// Workspace of a segmented call (none for a single segment per state): Q~ and the read-out of N of
// every chunk, and per segment N, Phi, the state leaving segment 0 (fp32) and the entering states
// (bf16).
size_t prefill_seg_workspace_bytes(int64_t nstate, int64_t T) {
  const SegPlan p = seg_plan(nstate, T);
  if (p.nseg <= 1) return 0;
  const size_t per = static_cast<size_t>(nstate * p.nseg) * 128 * 128;
  return 2 * align256(static_cast<size_t>(nstate * p.nch) * kSegC * 128 * 2) + 3 * align256(per * 4) +
         align256(per * 2);
}

hipError_t prefill_seg_launch(const PrefillArgs<bf16_t>& pa, int64_t nstate, bool two, void* workspace,
                              hipEvent_t mark, hipStream_t s) {
  const SegPlan p = seg_plan(nstate, pa.T);
  SegArgs a{};
  a.q = pa.q;
  a.k = pa.k;
  a.v = pa.v;
  a.la = pa.la;
  a.bg = pa.bg;
  a.wg = pa.wg;
  a.S0 = pa.S0;
  a.o = pa.o;
  a.S_T = pa.S_T;
  a.T = pa.T;
  a.H = pa.H;
  a.Hk = pa.Hk;
  a.nch = p.nch;
  a.nseg = p.nseg;
  a.L = p.L;
  a.alpha_kind = pa.alpha_kind;
  a.b_kind = pa.b_kind;
  a.w_kind = pa.w_kind;
  if (p.nseg > 1) {
    unsigned char* w = static_cast<unsigned char*>(workspace);
    const size_t per = static_cast<size_t>(nstate * p.nseg) * 128 * 128;
    a.Qt = reinterpret_cast<__bf16*>(w);
    w += align256(static_cast<size_t>(nstate * p.nch) * kSegC * 128 * 2);
    a.On = reinterpret_cast<__bf16*>(w);
    w += align256(static_cast<size_t>(nstate * p.nch) * kSegC * 128 * 2);
    a.Nseg = reinterpret_cast<float*>(w);
    w += align256(per * 4);
    a.Pseg = reinterpret_cast<float*>(w);
    w += align256(per * 4);
    a.Eseg = reinterpret_cast<float*>(w);
    w += align256(per * 4);
    a.Ebf = reinterpret_cast<__bf16*>(w);
  }
  if (nstate == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(nstate * p.nseg)), block(kSegThreads);
  const bool bch = a.b_kind == kChannel;
  if (a.alpha_kind == kScalar)
    hipLaunchKernelGGL((seg_kernel<1, kScalar, kScalar, kScalar>), grid, block, 0, s, a);
  else if (two && bch)
    hipLaunchKernelGGL((seg_kernel<2, kChannel, kChannel, kChannel>), grid, block, 0, s, a);
  else if (two)
    hipLaunchKernelGGL((seg_kernel<2, kChannel, kScalar, kScalar>), grid, block, 0, s, a);
  else if (bch)
    hipLaunchKernelGGL((seg_kernel<1, kChannel, kChannel, kChannel>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((seg_kernel<1, kChannel, kScalar, kScalar>), grid, block, 0, s, a);
  if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (mark != nullptr)
    if (const hipError_t e = hipEventRecord(mark, s); e != hipSuccess) return e;
  if (p.nseg > 1) {
    // (16 columns per workgroup while that still leaves CUs free, else 32)
    if (nstate * 8 <= kSegTargetGroups)
      hipLaunchKernelGGL((seg_chain_kernel<1>), dim3(static_cast<unsigned>(nstate * 8)), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((seg_chain_kernel<2>), dim3(static_cast<unsigned>(nstate * 4)), dim3(256), 0, s, a);
    if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    const int64_t ngrp = (p.L + kFixGroup - 1) / kFixGroup;
    hipLaunchKernelGGL(seg_fix_kernel, dim3(static_cast<unsigned>(nstate * (p.nseg - 1) * ngrp)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace gdr
