// Host side of the backward pass: workspace carving and the launches.
#include "backward_ch.h"

namespace gdr {

namespace {
size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace, per 64-token chunk of every state: the chunk map (as for the per-channel forward),
// four checkpoints and Q'^T dO (bf16 dk x dv each).  Partial gradients, when the chunk-local
// adjoint's sums are completed afterwards: dq and dk per value head and column half (grouped
// heads or d_v > 128), and with d_v > 128 per half also db (per channel or scalar), d log alpha
// and a scalar dw.
struct BwdSizes {
  size_t Qd, Ad, Dt, Zd, Egn, flag, ck;
  size_t pqk;  // one partial dq (or dk): value-head rows x dk, bf16
  size_t pg;   // one partial per-token gate gradient (dk wide for a per-channel b): bf16
  int nh;      // column halves
  bool partial_qk;
  size_t total() const {
    return Qd + Ad + Dt + Zd + Egn + flag + 5 * ck + (partial_qk ? 2 * nh * pqk : 0) +
           (nh > 1 ? 3 * nh * pg : 0);
  }
};

BwdSizes bwd_sizes(int64_t B, int64_t H, int64_t Hk, int64_t T, int64_t DK, int64_t DV) {
  const size_t ch = static_cast<size_t>(B * H) * static_cast<size_t>((T + 63) / 64);
  const size_t rows = static_cast<size_t>(B * T * H);
  BwdSizes s;
  s.Qd = align256(ch * 64 * DK * 2);
  s.Ad = align256(ch * DK * DK * 2);
  s.Dt = align256(ch * DV * DK * 2);
  s.Zd = align256(ch * 64 * DV * 2);
  s.Egn = align256(ch * (DK + 4) * 4);
  s.flag = align256(ch * 4);
  s.ck = align256(ch * DK * DV * 2);
  s.nh = DV > 128 ? 2 : 1;
  s.partial_qk = s.nh > 1 || Hk < H;
  s.pqk = align256(rows * DK * 2);
  s.pg = align256(rows * DK * 2);
  return s;
}

// the chains over 32 value columns a workgroup where d_v allows and that still gives at least 128
// workgroups (the chunk's A' then serves two slices), else 16 (twice the A' reads, but twice the
// chains side by side: with few states the chip is otherwise mostly idle)
template <int DK, bool REV>
void launch_chain(const BwdArgs& a, int64_t nstate, hipStream_t s) {
  if (a.DV % 32 == 0 && nstate * (a.DV / 32) >= 128)
    hipLaunchKernelGGL((bwd_chain_kernel<DK, REV, 2>), dim3((unsigned)(nstate * (a.DV / 32))),
                       dim3(64 * (2 + 2 * DK / 32)), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_chain_kernel<DK, REV, 1>), dim3((unsigned)(nstate * (a.DV / 16))),
                       dim3(64 * (2 + DK / 32)), 0, s, a);
}

// Both chains: side by side in one launch when together they still fit one workgroup per CU
// (each chain alone would leave half the chip idle), else one after the other.
constexpr int64_t kChipCUs = 256;  // MI355X compute units

template <int DK>
void launch_chains(const BwdArgs& a, int64_t nstate, hipStream_t s) {
  const int64_t n16 = nstate * (a.DV / 16);  // 16-column workgroups per chain
  if (2 * n16 <= kChipCUs) {
    hipLaunchKernelGGL((bwd_chains_kernel<DK, 1>), dim3((unsigned)(2 * n16)), dim3(64 * (2 + DK / 32)), 0, s, a);
    return;
  }
  launch_chain<DK, false>(a, nstate, s);
  launch_chain<DK, true>(a, nstate, s);
}

// Per-channel decay (dk = 128, dv 64 or 128): the chunk maps in the order MODE (2: erase first,
// 1: decay first), the chains, then the chunk-local adjoint by matrix products for every chunk
// whose gates stay in range and token by token for the others.
template <int MODE>
hipError_t launch_channel(WycArgs f, const BwdArgs& a, int64_t nstate, hipStream_t s) {
  const int64_t nblk = nstate * a.nch;
  hipLaunchKernelGGL((wyc_prep_kernel<128, 128, MODE>), dim3((unsigned)nblk), dim3(512), 0, s, f);
  hipLaunchKernelGGL((bwd_db_kernel<128, 128>), dim3((unsigned)nblk), dim3(256), 0, s, a);
  launch_chains<128>(a, nstate, s);
  hipLaunchKernelGGL((bwd_chl_kernel<MODE>), dim3((unsigned)nblk), dim3(512), 0, s, a);
  hipLaunchKernelGGL((bwd_chl_token_kernel<MODE>), dim3((unsigned)nblk), dim3((unsigned)(64 * (a.DV / 16))), 0, s, a);
  return hipGetLastError();
}

// halves: the chunk-local adjoint's argument sets, one per 128 value columns
template <int DK>
hipError_t launch_dk(WycArgs f, const BwdArgs& a, const BwdArgs* halves, int nh, int64_t nstate,
                     hipStream_t s) {
  const int64_t nblk = nstate * a.nch;
  if (a.DV <= 128) {
    hipLaunchKernelGGL((wyc_prep_kernel<DK, 128, 1>), dim3((unsigned)nblk), dim3(512), 0, s, f);
    hipLaunchKernelGGL((bwd_db_kernel<DK, 128>), dim3((unsigned)nblk), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((wyc_prep_kernel<DK, 256, 1>), dim3((unsigned)nblk), dim3(512), 0, s, f);
    hipLaunchKernelGGL((bwd_db_kernel<DK, 256>), dim3((unsigned)nblk), dim3(256), 0, s, a);
  }
  launch_chains<DK>(a, nstate, s);
  for (int h = 0; h < nh; ++h)
    hipLaunchKernelGGL((bwd_local_kernel<DK>), dim3((unsigned)nblk), dim3(512), 0, s, halves[h]);
  return hipGetLastError();
}

void sum_parts(const bf16_t* s0, const bf16_t* s1, bf16_t* dst, int64_t rows, int64_t G, int64_t width,
               hipStream_t s) {
  const int64_t n = rows * width;
  if (n > 0)
    hipLaunchKernelGGL(bwd_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, s0, s1, dst,
                       rows, G, width);
}
}  // namespace

// bf16 I/O; a scalar decay or none with dk in {32, 64, 128} and dv a multiple of 16 up to 256,
// or a per-channel decay with dk = 128 and dv 64 or 128.
bool backward_supported(int io_dtype_bf16, int64_t DK, int64_t DV, int alpha_kind) {
  if (!io_dtype_bf16) return false;
  if (alpha_kind == kChannel) return DK == 128 && (DV == 64 || DV == 128);
  return (DK == 32 || DK == 64 || DK == 128) && DV % 16 == 0 && DV > 0 && DV <= 256;
}

size_t backward_workspace_bytes(int64_t B, int64_t H, int64_t Hk, int64_t T, int64_t DK, int64_t DV) {
  return bwd_sizes(B, H, Hk, T, DK, DV).total();
}

hipError_t launch_backward(const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* la,
                           const bf16_t* bg, const bf16_t* wg, const float* S0, const bf16_t* dO,
                           const float* dST, bf16_t* dq, bf16_t* dk, bf16_t* dv, bf16_t* dla,
                           bf16_t* db, bf16_t* dw, float* dS0, int64_t B, int64_t T, int64_t H,
                           int64_t Hk, int64_t DK, int64_t DV, int alpha_kind, int b_kind, int w_kind,
                           bool decay_first, void* workspace, hipStream_t s) {
  const int64_t nstate = B * H;
  if (nstate == 0) return hipSuccess;
  if (T == 0) {
    const int64_t n = nstate * DK * DV;
    if (dS0 != nullptr)
      hipLaunchKernelGGL(bwd_pass_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dST, dS0, n);
    return hipGetLastError();
  }
  const BwdSizes z = bwd_sizes(B, H, Hk, T, DK, DV);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  WycArgs f{};
  f.q = q;
  f.k = k;
  f.v = v;
  f.la = la;
  f.bg = bg;
  f.wg = wg;
  f.T = T;
  f.H = H;
  f.DV = DV;
  f.Hk = Hk;
  f.nch = (T + 63) / 64;
  f.b_kind = b_kind;
  f.w_kind = w_kind;
  f.alpha_kind = alpha_kind;
  f.Qd = reinterpret_cast<__bf16*>(ws);
  ws += z.Qd;
  f.Ad = reinterpret_cast<__bf16*>(ws);
  ws += z.Ad;
  f.Dt = reinterpret_cast<__bf16*>(ws);
  ws += z.Dt;
  f.Zd = reinterpret_cast<__bf16*>(ws);
  ws += z.Zd;
  f.Egn = reinterpret_cast<float*>(ws);
  ws += z.Egn;
  f.flag = reinterpret_cast<int*>(ws);
  ws += z.flag;
  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.la = la;
  a.bg = bg;
  a.wg = wg;
  a.dO = dO;
  a.S0 = S0;
  a.dST = dST;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dla = dla;
  a.db = db;
  a.dw = dw;
  a.dS0 = dS0;
  a.Qd = f.Qd;
  a.Ad = f.Ad;
  a.Dt = f.Dt;
  a.Egn = f.Egn;
  a.cflag = f.flag;  // (the chunk maps' flags are not read after the chains)
  a.SR = reinterpret_cast<__bf16*>(ws);
  a.ST = reinterpret_cast<__bf16*>(ws + z.ck);
  a.GR = reinterpret_cast<__bf16*>(ws + 2 * z.ck);
  a.GT = reinterpret_cast<__bf16*>(ws + 3 * z.ck);
  a.Dbt = reinterpret_cast<__bf16*>(ws + 4 * z.ck);
  ws += 5 * z.ck;
  a.T = T;
  a.H = H;
  a.DV = DV;
  a.nch = f.nch;
  a.alpha_kind = alpha_kind;
  a.b_kind = b_kind;
  a.w_kind = w_kind;
  a.Hk = Hk;
  a.c0 = 0;
  a.DVh = static_cast<int>(DV < 128 ? DV : 128);

  // the chunk-local adjoint per column half, its summed outputs redirected to partial buffers
  const int nh = z.nh;
  BwdArgs halves[2] = {a, a};
  bf16_t* pq[2] = {nullptr, nullptr};
  bf16_t* pk[2] = {nullptr, nullptr};
  bf16_t* pla[2] = {nullptr, nullptr};
  bf16_t* pb[2] = {nullptr, nullptr};
  bf16_t* pw[2] = {nullptr, nullptr};
  for (int h = 0; h < nh; ++h) {
    halves[h].c0 = 128 * h;
    halves[h].DVh = static_cast<int>(DV - 128 * h < 128 ? DV - 128 * h : 128);
    if (z.partial_qk) {
      pq[h] = reinterpret_cast<bf16_t*>(ws);
      pk[h] = reinterpret_cast<bf16_t*>(ws + z.pqk);
      ws += 2 * z.pqk;
      halves[h].dq = pq[h];
      halves[h].dk = pk[h];
    }
  }
  if (nh > 1) {
    for (int h = 0; h < nh; ++h) {
      pla[h] = reinterpret_cast<bf16_t*>(ws);
      pb[h] = reinterpret_cast<bf16_t*>(ws + z.pg);
      pw[h] = reinterpret_cast<bf16_t*>(ws + 2 * z.pg);
      ws += 3 * z.pg;
      halves[h].dla = pla[h];
      halves[h].db = pb[h];
      if (w_kind == kScalar) halves[h].dw = pw[h];  // (a per-channel dw is per column: direct)
    }
  }
  hipError_t e;
  if (alpha_kind == kChannel) {
    // (d_v <= 128: one column half; the chunk-local kernels take every value column)
    e = decay_first ? launch_channel<1>(f, halves[0], nstate, s) : launch_channel<2>(f, halves[0], nstate, s);
  } else {
    switch (DK) {
      case 32: e = launch_dk<32>(f, a, halves, nh, nstate, s); break;
      case 64: e = launch_dk<64>(f, a, halves, nh, nstate, s); break;
      default: e = launch_dk<128>(f, a, halves, nh, nstate, s); break;
    }
  }
  if (e != hipSuccess) return e;
  const int64_t rows = B * T * H;
  if (z.partial_qk) {
    sum_parts(pq[0], pq[1], dq, B * T * Hk, H / Hk, DK, s);
    sum_parts(pk[0], pk[1], dk, B * T * Hk, H / Hk, DK, s);
  }
  if (nh > 1) {
    if (alpha_kind == kScalar) sum_parts(pla[0], pla[1], dla, rows, 1, 1, s);
    if (b_kind != kNone) sum_parts(pb[0], pb[1], db, rows, 1, b_kind == kChannel ? DK : 1, s);
    if (w_kind == kScalar) sum_parts(pw[0], pw[1], dw, rows, 1, 1, s);
  }
  return hipGetLastError();
}

}  // namespace gdr
