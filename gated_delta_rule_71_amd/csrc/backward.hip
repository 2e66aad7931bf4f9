// Host side of the backward pass: workspace carving and the four launches.
#include "backward.h"

namespace gdr {

namespace {
size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct BwdSizes {
  size_t Qd, Ad, Dt, Zd, Egn, flag, ck, grp;
  size_t total() const { return Qd + Ad + Dt + Zd + Egn + flag + 5 * ck + 2 * grp; }
};

// grouped: value-head rows B T H when q / k have fewer heads (dq and dk per value head), else 0
BwdSizes bwd_sizes(int64_t nstate, int64_t T, int64_t DK, int64_t DV, int64_t grouped = 0) {
  const size_t ch = static_cast<size_t>(nstate) * static_cast<size_t>((T + 63) / 64);
  BwdSizes s;
  s.Qd = align256(ch * 64 * DK * 2);
  s.Ad = align256(ch * DK * DK * 2);
  s.Dt = align256(ch * DV * DK * 2);
  s.Zd = align256(ch * 64 * DV * 2);
  s.Egn = align256(ch * (DK + 4) * 4);
  s.flag = align256(ch * 4);
  s.ck = align256(ch * DK * DV * 2);
  s.grp = align256(static_cast<size_t>(grouped) * DK * 2);
  return s;
}

// the chains over 32 value columns a workgroup where d_v allows (the chunk's A' then serves two
// slices), else 16
template <int DK, bool REV>
void launch_chain(const BwdArgs& a, int64_t nstate, hipStream_t s) {
  if (a.DV % 32 == 0)
    hipLaunchKernelGGL((bwd_chain_kernel<DK, REV, 2>), dim3((unsigned)(nstate * (a.DV / 32))),
                       dim3(64 * (2 + 2 * DK / 32)), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_chain_kernel<DK, REV, 1>), dim3((unsigned)(nstate * (a.DV / 16))),
                       dim3(64 * (2 + DK / 32)), 0, s, a);
}

template <int DK>
hipError_t launch_dk(WycArgs f, BwdArgs a, int64_t nstate, hipStream_t s) {
  const int64_t nblk = nstate * a.nch;
  hipLaunchKernelGGL((wyc_prep_kernel<DK, 128, 1>), dim3((unsigned)nblk), dim3(512), 0, s, f);
  hipLaunchKernelGGL((bwd_db_kernel<DK>), dim3((unsigned)nblk), dim3(256), 0, s, a);
  launch_chain<DK, false>(a, nstate, s);
  launch_chain<DK, true>(a, nstate, s);
  hipLaunchKernelGGL((bwd_local_kernel<DK>), dim3((unsigned)nblk), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t group_sum(const bf16_t* src, bf16_t* dst, int64_t rows, int64_t G, int64_t DK, hipStream_t s) {
  const int64_t items = rows * (DK / 8);
  if (items > 0)
    hipLaunchKernelGGL(bwd_group_sum_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, src, dst,
                       rows, G, DK);
  return hipGetLastError();
}
}  // namespace

// bf16 I/O, a scalar decay or none, dk in {32, 64, 128}, dv a multiple of 16 up to 128.
bool backward_supported(int io_dtype_bf16, int64_t DK, int64_t DV, int alpha_kind) {
  return io_dtype_bf16 && (DK == 32 || DK == 64 || DK == 128) && DV % 16 == 0 && DV > 0 && DV <= 128 &&
         alpha_kind != kChannel;
}

size_t backward_workspace_bytes(int64_t B, int64_t H, int64_t Hk, int64_t T, int64_t DK, int64_t DV) {
  return bwd_sizes(B * H, T, DK, DV, Hk < H ? B * T * H : 0).total();
}

hipError_t launch_backward(const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* la,
                           const bf16_t* bg, const bf16_t* wg, const float* S0, const bf16_t* dO,
                           const float* dST, bf16_t* dq, bf16_t* dk, bf16_t* dv, bf16_t* dla,
                           bf16_t* db, bf16_t* dw, float* dS0, int64_t B, int64_t T, int64_t H,
                           int64_t Hk, int64_t DK, int64_t DV, int alpha_kind, int b_kind, int w_kind,
                           void* workspace, hipStream_t s) {
  const int64_t nstate = B * H;
  const bool grouped = Hk < H;
  const BwdSizes z = bwd_sizes(nstate, T, DK, DV, grouped ? B * T * H : 0);
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
  a.SR = reinterpret_cast<__bf16*>(ws);
  a.ST = reinterpret_cast<__bf16*>(ws + z.ck);
  a.GR = reinterpret_cast<__bf16*>(ws + 2 * z.ck);
  a.GT = reinterpret_cast<__bf16*>(ws + 3 * z.ck);
  a.Dbt = reinterpret_cast<__bf16*>(ws + 4 * z.ck);
  bf16_t* gq = reinterpret_cast<bf16_t*>(ws + 5 * z.ck);
  bf16_t* gk = reinterpret_cast<bf16_t*>(ws + 5 * z.ck + z.grp);
  a.Hk = Hk;
  if (grouped) {  // per value head first
    a.dq = gq;
    a.dk = gk;
  }
  a.T = T;
  a.H = H;
  a.DV = DV;
  a.nch = f.nch;
  a.alpha_kind = alpha_kind;
  a.b_kind = b_kind;
  a.w_kind = w_kind;
  if (nstate == 0 || T == 0) return hipSuccess;
  hipError_t e;
  switch (DK) {
    case 32: e = launch_dk<32>(f, a, nstate, s); break;
    case 64: e = launch_dk<64>(f, a, nstate, s); break;
    default: e = launch_dk<128>(f, a, nstate, s); break;
  }
  if (e != hipSuccess || !grouped) return e;
  e = group_sum(gq, dq, B * T * Hk, H / Hk, DK, s);
  if (e != hipSuccess) return e;
  return group_sum(gk, dk, B * T * Hk, H / Hk, DK, s);
}

}  // namespace gdr
