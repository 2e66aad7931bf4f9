// Prefill by the token recurrence itself, for the problems the chunkwise kernels do not fit in
// LDS: the all-fp32 mode at dk = 128 and 256 (and at dk = 64 with the decay after the erase),
// and bf16 at dk = 256 with a per-channel decay after the erase.
//
// One wave per (batch, head) and block of 16 value columns walks the tokens in order and keeps
// its 16 columns of S in registers from S0 to S_T.  The tokens' inputs arrive in LDS by
// direct-to-LDS loads, a block of 8 tokens ahead of their use, so that the walk waits on the
// memory latency once per block instead of once per token.  Per token, with c = b . k, x = w . v and
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

// One token's inputs in LDS: the rows of q and k and of per-channel log alpha and b (dk elements
// each), then the 16 value columns of v and of a per-channel w of this wave's block.
template <typename IO, int DK>
struct RecurSlot {
  static constexpr int EL = sizeof(IO), ROWB = DK * EL;
  static constexpr int oQ = 0, oK = ROWB, oLA = 2 * ROWB, oB = 3 * ROWB, oV = 4 * ROWB, oW = oV + 64;
  static constexpr int bytes = oW + 64;
};

// Direct-to-LDS load of 16 bytes per active lane: bytes 16 i .. 16 i + 15 past `off` of the buffer
// `r` (zeros past its end) into LDS at m0 + 16 i for lane i.  Issued from an asm statement, so the
// compiler inserts no wait for it; the kernel waits for its loads itself.  m0 and r are uniform.
typedef int recur_i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ recur_i32x4 recur_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  recur_i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p)));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p >> 32) & 0xffffu));  // stride 0
  r.z = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r.w = 0x00020000;
  return r;
}
__device__ __forceinline__ uint32_t recur_m0(unsigned char* lds) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)lds)));
}
__device__ __forceinline__ void recur_dma16(recur_i32x4 r, uint32_t m0, uint32_t off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(off), "s"(r)
               : "memory", "m0");
}

template <typename IO, int DK, bool DECAY_FIRST>
__global__ __launch_bounds__(64) void recur_kernel(PrefillArgs<IO> a) {
  using SL = RecurSlot<IO, DK>;
  constexpr int R = DK / 16;  // rows per lane
  constexpr int TB = 8;       // tokens per block: block b + 1 loads while block b is computed
  constexpr int EL = SL::EL;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * TB * SL::bytes];
  const int lane = threadIdx.x;
  const int rg = lane >> 2, cq = lane & 3;
  const int d0 = rg * R;  // first row of this lane
  const int64_t nsl = a.DV / 16;
  const int64_t bh = blockIdx.x / nsl;
  const int64_t cb0 = (blockIdx.x % nsl) * 16;  // first column of this wave's block
  const int64_t col0 = cb0 + 4 * cq;            // first column of this lane
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

  // per input: this state's token-0 element, the row stride and the bytes to the end of its last
  // row; each block of tokens addresses its loads from its own first token (64-bit base, 32-bit
  // offsets under 8 row strides)
  struct In {
    const unsigned char* p;
    int64_t stride;
    int64_t end;
  };
  auto in_of = [&](const IO* x, int64_t heads, int64_t head, int64_t width, int64_t first) {
    const int64_t stride = heads * width * EL;
    return In{reinterpret_cast<const unsigned char*>(x + (bi * T * heads + head) * width + first), stride,
              (T - 1) * stride + (width - first) * EL};
  };
  const In inQ = in_of(a.q, Hk, hk, DK, 0), inK = in_of(a.k, Hk, hk, DK, 0);
  const In inV = in_of(a.v, H, hi, DV, cb0);
  // (per-channel gates only: a scalar gate's element is not 16-byte aligned; those come through
  // registers below)
  const In inA = in_of(a.alpha_kind == kChannel ? a.la : a.q, a.alpha_kind == kChannel ? H : Hk,
                       a.alpha_kind == kChannel ? hi : hk, DK, 0);
  const In inB = in_of(a.b_kind == kChannel ? a.bg : a.q, a.b_kind == kChannel ? H : Hk,
                       a.b_kind == kChannel ? hi : hk, DK, 0);
  const In inW = in_of(a.w_kind == kChannel ? a.wg : a.v, H, hi, DV, cb0);
  // block b's loads into its buffer, token u of the block into slot u: whole rows of q and k (and
  // of per-channel gates), the block's 16 columns of v (and of a per-channel w)
  auto dma_block = [&](int64_t b) {
    unsigned char* buf = smem + (b & 1) * TB * SL::bytes;
    const int64_t t0 = b * TB;
    const int nt = static_cast<int>(T - t0 < TB ? T - t0 : TB);
    auto rows = [&](const In& in, int dst, int nbytes) {
      const int64_t left = in.end - t0 * in.stride;
      const recur_i32x4 r = recur_rsrc(in.p + t0 * in.stride, static_cast<uint32_t>(left < 0x7fffffff ? left : 0x7fffffff));
      for (int u = 0; u < nt; ++u) {
        const uint32_t m0 = recur_m0(buf + u * SL::bytes + dst);
        if (lane * 16 < nbytes) recur_dma16(r, m0, static_cast<uint32_t>(u * in.stride + lane * 16));
      }
    };
    rows(inQ, SL::oQ, SL::ROWB);
    rows(inK, SL::oK, SL::ROWB);
    if (a.alpha_kind == kChannel) rows(inA, SL::oLA, SL::ROWB);
    if (a.b_kind == kChannel) rows(inB, SL::oB, SL::ROWB);
    rows(inV, SL::oV, 16 * EL);
    if (a.w_kind == kChannel) rows(inW, SL::oW, 16 * EL);
  };
  // scalar gates of block b: lane u < 8 holds token u's (log alpha, b, w), loaded a block ahead
  auto scalars_of = [&](int64_t b, float& la_, float& b_, float& w_) {
    const int64_t t = b * TB + lane;
    la_ = 0.f;
    b_ = 0.f;
    w_ = 1.f;
    if (lane < TB && t < T) {
      const int64_t row = (bi * T + t) * H + hi;
      if (a.alpha_kind == kScalar) la_ = ld(a.la, row);
      if (a.b_kind == kScalar) b_ = ld(a.bg, row);
      if (a.w_kind == kScalar) w_ = ld(a.wg, row);
    }
  };

  const int64_t nblk = (T + TB - 1) / TB;
  float nla = 0.f, nb = 0.f, nw = 1.f;  // the next block's scalar gates
  if (nblk > 0) {
    dma_block(0);
    scalars_of(0, nla, nb, nw);
  }
  for (int64_t b = 0; b < nblk; ++b) {
    // block b's loads (issued one block ago) are in LDS; every store of block b - 1 is done
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    const float cla = nla, cbs = nb, cws = nw;
    // block b + 1 into the other buffer, whose last reads (block b - 1) have returned
    if (b + 1 < nblk) {
      dma_block(b + 1);
      scalars_of(b + 1, nla, nb, nw);
    }
    const unsigned char* buf = smem + (b & 1) * TB * SL::bytes;
    const int nt = static_cast<int>(T - b * TB < TB ? T - b * TB : TB);
    for (int u = 0; u < nt; ++u) {
      const int64_t t = b * TB + u;
      const unsigned char* slot = buf + u * SL::bytes;
      TokenIn<IO, R> cur;
      Run<IO, R>::load(reinterpret_cast<const IO*>(slot + SL::oQ) + d0, cur.q);
      Run<IO, R>::load(reinterpret_cast<const IO*>(slot + SL::oK) + d0, cur.k);
      if (a.alpha_kind == kChannel) Run<IO, R>::load(reinterpret_cast<const IO*>(slot + SL::oLA) + d0, cur.la);
      if (a.b_kind == kChannel) Run<IO, R>::load(reinterpret_cast<const IO*>(slot + SL::oB) + d0, cur.b);
      Run<IO, 4>::load(reinterpret_cast<const IO*>(slot + SL::oV) + 4 * cq, cur.v);
      if (a.w_kind == kChannel) Run<IO, 4>::load(reinterpret_cast<const IO*>(slot + SL::oW) + 4 * cq, cur.w);
      cur.las = __shfl(cla, u);
      cur.bs = __shfl(cbs, u);
      cur.ws = __shfl(cws, u);

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
      // sum over the 16 row groups (lanes of equal cq): inside each row of 16 lanes by DPP row
      // rotations (8, then 4), then across the four rows by two lane exchanges
      auto row_sum4 = [](float v) {
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));
        return v;
      };
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        r[j] = row_sum4(r[j]);
        y[j] = row_sum4(y[j]);
      }
      dqk = row_sum4(dqk);
      dg = row_sum4(dg);
#pragma unroll
      for (int off = 16; off < 64; off <<= 1) {
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
    }
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
