// Prefill by the token recurrence itself, for the problems the chunkwise kernels do not fit in
// LDS: the all-fp32 mode at dk = 128 and 256 (and at dk = 64 with the decay after the erase),
// and bf16 at dk = 256 with a per-channel decay after the erase.
//
// One wave per (batch, head) and block of 16 value columns walks the tokens in order and keeps
// its 16 columns of S in registers from S0 to S_T.  Per token, with c = b . k, x = w . v and
// alpha = exp(log alpha) ("Recurrent Memory: Write, Erase, Decay, Read", section 05 for the
// unified update, section 01 for the read; the read sees the token's own write):
//
//   erase then decay:  r = c S,            y = (q . alpha) S
//                      S' = alpha . S - (alpha . k)^T r + k^T x
//                      o  = y - ((q . alpha) . k) r + (q . k) x
//   decay then erase:  r = (c . alpha) S,  y = (q . alpha) S
//                      S' = alpha . S - k^T r + k^T x
//                      o  = y - (q . k) r + (q . k) x
//
// (o = q S' in both cases, expanded so that both dk-reductions read the state before the update.)
// Columns of S are independent (the transition multiplies S from the left), so the column blocks
// run in separate waves with no exchange.  Lane l holds rows R (l / 4) .. R (l / 4) + R - 1 of
// the block (R = dk / 16) and its columns 4 (l % 4) .. 4 (l % 4) + 3;
// each lane reads its rows of q, k, log alpha and b as contiguous runs, and the reductions over
// dk are the lane's own rows followed by four shuffles across lanes of equal l % 4.
#include "gdr_common.h"
#include "prefill_dispatch.h"

namespace gdr {

namespace {

template <typename IO, int N>
struct Run;  // N consecutive elements of an IO array as floats
template <int N>
struct Run<bf16_t, N> {
  __device__ __forceinline__ static void load(const bf16_t* p, float* out) {
    static_assert(N % 4 == 0, "runs of 4 bf16");
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(p + i);
      out[i] = bf16_to_f32(u.x & 0xffffu);
      out[i + 1] = bf16_to_f32(u.x >> 16);
      out[i + 2] = bf16_to_f32(u.y & 0xffffu);
      out[i + 3] = bf16_to_f32(u.y >> 16);
    }
  }
};
template <int N>
struct Run<float, N> {
  __device__ __forceinline__ static void load(const float* p, float* out) {
    static_assert(N % 4 == 0, "runs of 4 floats");
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const float4 u = *reinterpret_cast<const float4*>(p + i);
      out[i] = u.x;
      out[i + 1] = u.y;
      out[i + 2] = u.z;
      out[i + 3] = u.w;
    }
  }
};

// Per-token inputs of one lane: its R rows of q, k, log alpha and b, its 4 columns of v and w.
template <typename IO, int R>
struct TokenIn {
  float q[R], k[R], la[R], b[R], v[4], w[4];
  float las, bs, ws;  // scalar gates
};

}  // namespace

template <typename IO, int DK, bool DECAY_FIRST>
__global__ __launch_bounds__(64) void recur_kernel(PrefillArgs<IO> a) {
  constexpr int R = DK / 16;  // rows per lane
  const int lane = threadIdx.x;
  const int rg = lane >> 2, cq = lane & 3;
  const int d0 = rg * R;  // first row of this lane
  const int64_t nsl = a.DV / 16;
  const int64_t bh = blockIdx.x / nsl;
  const int64_t col0 = (blockIdx.x % nsl) * 16 + 4 * cq;  // first column of this lane
  const int64_t H = a.H, DV = a.DV, T = a.T;
  const int64_t bi = bh / H, hi = bh % H;
  const int64_t Hk = a.Hk, hk = hi / (H / Hk);

  float s[R][4];
  if (a.S0 != nullptr) {
    const float* S0 = a.S0 + bh * DK * DV;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float4 u = *reinterpret_cast<const float4*>(S0 + (d0 + i) * DV + col0);
      s[i][0] = u.x;
      s[i][1] = u.y;
      s[i][2] = u.z;
      s[i][3] = u.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i) s[i][0] = s[i][1] = s[i][2] = s[i][3] = 0.f;
  }

  auto fetch = [&](int64_t t, TokenIn<IO, R>& in) {
    const int64_t row = (bi * T + t) * H + hi, qrow = (bi * T + t) * Hk + hk;
    Run<IO, R>::load(a.q + qrow * DK + d0, in.q);
    Run<IO, R>::load(a.k + qrow * DK + d0, in.k);
    if (a.alpha_kind == kChannel) Run<IO, R>::load(a.la + row * DK + d0, in.la);
    if (a.b_kind == kChannel) Run<IO, R>::load(a.bg + row * DK + d0, in.b);
    Run<IO, 4>::load(a.v + row * DV + col0, in.v);
    if (a.w_kind == kChannel) Run<IO, 4>::load(a.wg + row * DV + col0, in.w);
    in.las = a.alpha_kind == kScalar ? ld(a.la, row) : 0.f;
    in.bs = a.b_kind == kScalar ? ld(a.bg, row) : 0.f;
    in.ws = a.w_kind == kScalar ? ld(a.wg, row) : 1.f;
  };

  TokenIn<IO, R> cur, nxt;
  if (T > 0) fetch(0, cur);
  for (int64_t t = 0; t < T; ++t) {
    if (t + 1 < T) fetch(t + 1, nxt);  // the next token's loads stay in flight over this one
    float al[R], cp[R], kp[R], qa[R];
    float dqk = 0.f, dg = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float lad = a.alpha_kind == kChannel ? cur.la[i] : cur.las;
      const float bd = a.b_kind == kChannel ? cur.b[i] : cur.bs;
      al[i] = a.alpha_kind == kNone ? 1.f : __expf(lad);
      const float c = a.b_kind == kNone ? 0.f : bd * cur.k[i];
      qa[i] = cur.q[i] * al[i];
      dqk += cur.q[i] * cur.k[i];
      if (DECAY_FIRST) {
        cp[i] = c * al[i];
        kp[i] = cur.k[i];
      } else {
        cp[i] = c;
        kp[i] = al[i] * cur.k[i];
      }
      dg += cur.q[i] * kp[i];  // q . (alpha . k); q . k with the decay first
    }
    float r[4] = {0.f, 0.f, 0.f, 0.f}, y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        r[j] += cp[i] * s[i][j];
        y[j] += qa[i] * s[i][j];
      }
    // sum over the 16 row groups: lanes of equal cq
#pragma unroll
    for (int off = 4; off < 64; off <<= 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        r[j] += __shfl_xor(r[j], off);
        y[j] += __shfl_xor(y[j], off);
      }
      dqk += __shfl_xor(dqk, off);
      dg += __shfl_xor(dg, off);
    }
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = cur.v[j] * (a.w_kind == kChannel ? cur.w[j] : cur.ws);
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) s[i][j] = al[i] * s[i][j] - kp[i] * r[j] + cur.k[i] * x[j];
    if (rg == 0) {
      const int64_t orow = (bi * T + t) * H + hi;
#pragma unroll
      for (int j = 0; j < 4; ++j) st(a.o, orow * DV + col0 + j, y[j] - dg * r[j] + dqk * x[j]);
    }
    if (t + 1 < T) cur = nxt;
  }
  if (a.S_T != nullptr) {
    float* ST = a.S_T + bh * DK * DV;
#pragma unroll
    for (int i = 0; i < R; ++i)
      *reinterpret_cast<float4*>(ST + (d0 + i) * DV + col0) = make_float4(s[i][0], s[i][1], s[i][2], s[i][3]);
  }
}

template <typename IO, int DK>
static hipError_t launch_recur_dk(const PrefillArgs<IO>& a, int64_t nstate, bool decay_first,
                                  hipStream_t s) {
  const int64_t blocks = nstate * (a.DV / 16);
  if (blocks == 0) return hipSuccess;
  if (decay_first)
    hipLaunchKernelGGL((recur_kernel<IO, DK, true>), dim3((unsigned)blocks), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((recur_kernel<IO, DK, false>), dim3((unsigned)blocks), dim3(64), 0, s, a);
  return hipGetLastError();
}

// dk in {64, 128, 256}: a lane's rows are runs of at least four elements.
template <typename IO>
hipError_t prefill_recur(const PrefillArgs<IO>& a, int64_t nstate, int64_t DK, bool decay_first,
                         hipStream_t s) {
  switch (DK) {
    case 64: return launch_recur_dk<IO, 64>(a, nstate, decay_first, s);
    case 128: return launch_recur_dk<IO, 128>(a, nstate, decay_first, s);
    case 256: return launch_recur_dk<IO, 256>(a, nstate, decay_first, s);
    default: return hipErrorInvalidValue;
  }
}

template hipError_t prefill_recur<bf16_t>(const PrefillArgs<bf16_t>&, int64_t, int64_t, bool, hipStream_t);
template hipError_t prefill_recur<float>(const PrefillArgs<float>&, int64_t, int64_t, bool, hipStream_t);

}  // namespace gdr
