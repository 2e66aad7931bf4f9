// Single-token decode step of the gated delta rule on gfx950.
//
// Per (batch, head) the state S (dk x dv fp32) is read once and written once.
// With c = b . k, x = w . v and alpha = exp(log alpha):
//
//   erase then decay ("Recurrent Memory: Write, Erase, Decay, Read", section 05):
//     r = c S,  y = (q . alpha) S
//     S' = alpha . S - (alpha . k)^T r + k^T x
//     o  = y - ((q . alpha) . k) r + (q . k) x          (= q S')
//   decay then erase:
//     r = (c . alpha) S,  y = (q . alpha) S
//     S' = alpha . S - k^T r + k^T x
//     o  = y - (q . k) r + (q . k) x
//
// Both reductions over dk (r and y) come from the same registers, so S crosses
// HBM exactly twice.  Columns of S are independent (the transition multiplies
// S from the left), so a workgroup owns a block of NCB columns of one state:
// each thread holds 4 consecutive columns (one float4) of DK / RPP rows.
#include "gdr_common.h"

namespace gdr {

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <typename IO>
struct DecodeArgs {
  const IO* q;
  const IO* k;
  const IO* v;
  const IO* la;
  const IO* bg;
  const IO* wg;
  float* S;
  IO* o;
  int64_t H;
  int64_t DV;
  int alpha_kind, b_kind, w_kind;
  int ncb_per_state;  // DV / NCB
  int64_t Hk;         // q / k heads (H is a multiple): value head h reads q / k head h / (H / Hk)
};

template <int NCB, int DK>
struct DecodeShape {
  static constexpr int TPR = NCB / 4;                                   // threads per row
  static constexpr int RPP = (256 / TPR) < DK ? (256 / TPR) : DK;       // rows per pass
  static constexpr int NT = TPR * RPP;                                  // threads per block
  static constexpr int NPASS = DK / RPP;
  static constexpr int NW = (NT + 63) / 64;                             // waves
};

template <typename IO, int DK, int NCB, bool DECAY_FIRST>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs<IO> a) {
  using Sh = DecodeShape<NCB, DK>;
  constexpr int TPR = Sh::TPR, RPP = Sh::RPP, NT = Sh::NT, NPASS = Sh::NPASS, NW = Sh::NW;
  static_assert(TPR <= 64 && 64 % TPR == 0, "a row's threads must sit in one wave");

  __shared__ float sh_al[DK], sh_cp[DK], sh_kp[DK], sh_k[DK], sh_qa[DK];
  __shared__ float sh_x[NCB];
  __shared__ float sh_red[NW][2][NCB];
  __shared__ float sh_dot[NW][2];
  __shared__ float sh_r[NCB], sh_y[NCB];

  const int tid = threadIdx.x;
  const int cq = tid % TPR;  // which float4 of the column block
  const int rr = tid / TPR;  // which row inside a pass
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t blk = blockIdx.x;
  const int64_t bh = blk / a.ncb_per_state;  // token row of a [B, 1, H] layout == b*H + h
  const int64_t col0 = (blk % a.ncb_per_state) * NCB;
  float* Sp = a.S + bh * DK * a.DV + col0;

  // 1) issue the state loads first: they are the only long-latency traffic.  Loads are
  // ordinary cached loads; the write-back below is nontemporal, since the updated state is not
  // read again in this step (measured on MI355X: nontemporal stores with ordinary loads beat
  // nontemporal accesses in both directions).
  f32x4v s[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p)
    s[p] = *reinterpret_cast<const f32x4v*>(Sp + (int64_t)(p * RPP + rr) * a.DV + cq * 4);

  // 2) per-channel vectors of this token
  float dot_qk = 0.f, dot_gamma = 0.f;
  const int64_t bqk = (bh / a.H) * a.Hk + (bh % a.H) / (a.H / a.Hk);  // this state's q / k row
  for (int d = tid; d < DK; d += NT) {
    const int64_t i = bh * DK + d;
    const float qd = ld(a.q, bqk * DK + d), kd = ld(a.k, bqk * DK + d);
    const float lad = a.alpha_kind == kNone ? 0.f : ld(a.la, a.alpha_kind == kScalar ? bh : i);
    const float bd = a.b_kind == kNone ? 0.f : ld(a.bg, a.b_kind == kScalar ? bh : i);
    const float al = __expf(lad);
    const float c = bd * kd;
    sh_al[d] = al;
    sh_k[d] = kd;
    sh_qa[d] = qd * al;
    if (DECAY_FIRST) {
      sh_cp[d] = c * al;
      sh_kp[d] = kd;
      dot_gamma += qd * kd;
    } else {
      sh_cp[d] = c;
      sh_kp[d] = al * kd;
      dot_gamma += qd * al * kd;
    }
    dot_qk += qd * kd;
  }
  for (int n = tid; n < NCB; n += NT) {
    const int64_t i = bh * a.DV + col0 + n;
    const float wn = a.w_kind == kNone ? 1.f : ld(a.wg, a.w_kind == kScalar ? bh : i);
    sh_x[n] = wn * ld(a.v, i);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    dot_qk += __shfl_xor(dot_qk, off);
    dot_gamma += __shfl_xor(dot_gamma, off);
  }
  if (lane == 0) {
    sh_dot[wave][0] = dot_qk;
    sh_dot[wave][1] = dot_gamma;
  }
  lds_barrier();

  // 3) both dk-reductions from the same registers
  float r[4] = {0.f, 0.f, 0.f, 0.f}, y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int d = p * RPP + rr;
    const float cp = sh_cp[d], qa = sh_qa[d];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[j] += cp * s[p][j];
      y[j] += qa * s[p][j];
    }
  }
  // rows that share a column live in the same wave at lane strides of TPR
#pragma unroll
  for (int off = TPR; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[j] += __shfl_xor(r[j], off);
      y[j] += __shfl_xor(y[j], off);
    }
  }
  if (lane < TPR) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sh_red[wave][0][cq * 4 + j] = r[j];
      sh_red[wave][1][cq * 4 + j] = y[j];
    }
  }
  lds_barrier();
  for (int n = tid; n < NCB; n += NT) {
    float rs = 0.f, ys = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      rs += sh_red[w][0][n];
      ys += sh_red[w][1][n];
    }
    sh_r[n] = rs;
    sh_y[n] = ys;
  }
  lds_barrier();

  // 4) update in registers, write S back once
  float rv[4], xv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    rv[j] = sh_r[cq * 4 + j];
    xv[j] = sh_x[cq * 4 + j];
  }
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int d = p * RPP + rr;
    const float al = sh_al[d], kp = sh_kp[d], kd = sh_k[d];
    f32x4v o4;
#pragma unroll
    for (int j = 0; j < 4; ++j) o4[j] = al * s[p][j] - kp * rv[j] + kd * xv[j];
    __builtin_nontemporal_store(o4, reinterpret_cast<f32x4v*>(Sp + (int64_t)d * a.DV + cq * 4));
  }

  // 5) read-out
  if (tid < NCB) {
    float qk = 0.f, gamma = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      qk += sh_dot[w][0];
      gamma += sh_dot[w][1];
    }
    const int n = tid;
    st(a.o, bh * a.DV + col0 + n, sh_y[n] - gamma * sh_r[n] + qk * sh_x[n]);
  }
}

template <typename IO, int DK, int NCB>
static hipError_t launch_decode_ncb(const DecodeArgs<IO>& a, int64_t n_states, bool decay_first,
                                    hipStream_t stream) {
  using Sh = DecodeShape<NCB, DK>;
  const int64_t blocks = n_states * a.ncb_per_state;
  if (blocks == 0) return hipSuccess;
  if (decay_first)
    hipLaunchKernelGGL((decode_kernel<IO, DK, NCB, true>), dim3((unsigned)blocks), dim3(Sh::NT), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<IO, DK, NCB, false>), dim3((unsigned)blocks), dim3(Sh::NT), 0,
                       stream, a);
  return hipGetLastError();
}

template <typename IO, int DK>
static hipError_t launch_decode_dk(DecodeArgs<IO> a, int64_t n_states, bool decay_first,
                                   hipStream_t stream) {
  // (the widest block that still fits the registers: fewer, larger workgroups measured faster,
  // 170 us against 181 us per step with 64 columns for 8,192 states of 128 x 128)
  if (DK <= 128 && a.DV % 128 == 0) {
    a.ncb_per_state = (int)(a.DV / 128);
    return launch_decode_ncb<IO, DK, 128>(a, n_states, decay_first, stream);
  }
  if (a.DV % 64 == 0) {
    a.ncb_per_state = (int)(a.DV / 64);
    return launch_decode_ncb<IO, DK, 64>(a, n_states, decay_first, stream);
  }
  if (a.DV % 32 == 0) {
    a.ncb_per_state = (int)(a.DV / 32);
    return launch_decode_ncb<IO, DK, 32>(a, n_states, decay_first, stream);
  }
  a.ncb_per_state = (int)(a.DV / 16);
  return launch_decode_ncb<IO, DK, 16>(a, n_states, decay_first, stream);
}

// Host launcher; arguments are validated by the caller (gdr_api.hip).
template <typename IO>
hipError_t launch_decode(const IO* q, const IO* k, const IO* v, const IO* la, const IO* bg,
                         const IO* wg, float* S, IO* o, int64_t B, int64_t H, int64_t Hk,
                         int64_t DK, int64_t DV, int alpha_kind, int b_kind, int w_kind,
                         bool decay_first, hipStream_t stream) {
  DecodeArgs<IO> a{q, k, v, la, bg, wg, S, o, H, DV, alpha_kind, b_kind, w_kind, 1, Hk};
  const int64_t n = B * H;
  switch (DK) {
    case 16: return launch_decode_dk<IO, 16>(a, n, decay_first, stream);
    case 32: return launch_decode_dk<IO, 32>(a, n, decay_first, stream);
    case 64: return launch_decode_dk<IO, 64>(a, n, decay_first, stream);
    case 128: return launch_decode_dk<IO, 128>(a, n, decay_first, stream);
    case 256: return launch_decode_dk<IO, 256>(a, n, decay_first, stream);
    default: return hipErrorInvalidValue;
  }
}

template hipError_t launch_decode<bf16_t>(const bf16_t*, const bf16_t*, const bf16_t*,
                                          const bf16_t*, const bf16_t*, const bf16_t*, float*,
                                          bf16_t*, int64_t, int64_t, int64_t, int64_t, int64_t, int,
                                          int, int, bool, hipStream_t);
template hipError_t launch_decode<float>(const float*, const float*, const float*, const float*,
                                         const float*, const float*, float*, float*, int64_t,
                                         int64_t, int64_t, int64_t, int64_t, int, int, int, bool,
                                         hipStream_t);

}  // namespace gdr
