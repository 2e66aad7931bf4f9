// Gradients of a prefill by the adjoint of the token recurrence itself, in fp32, for the problems
// the chunkwise backward does not cover: the all-fp32 mode, dk = 16 and 256, and a per-channel
// decay at widths other than dk = 128 with dv 64 or 128.  Exact for any gate values.
//
// Per token ("Recurrent Memory: Write, Erase, Decay, Read", section 05 for the unified update,
// section 01 for the read, which sees the token's own write), with c = b . k, x = w . v and
// a = exp(log alpha), from the state S before the token:
//   erase then decay:  r = c S,  E = S - k^T r,  S_t = Diag(a) E + k^T x,  o = q S_t
//   decay then erase:  D = Diag(a) S,  r = c D,  S_t = D - k^T r + k^T x,  o = q S_t
// Given G, the gradient of S_t from the tokens after it, and do, its adjoint is (Gt = G + q^T do):
//   erase then decay:  dq = do S_t^T,  dx = k Gt,  dE = Diag(a) Gt,  dr = -k dE,
//                      dk = Gt x^T - dE r^T + b . dc,  da = rowsum(Gt . E),  dc = dr S^T,
//                      G_prev = dE + c^T dr
//   decay then erase:  dq = do S_t^T,  dx = k Gt,  dr = -dx,  dk = Gt (x - r)^T + b . dc,
//                      dD = Gt + c^T dr,  dc = dr D^T,  da = rowsum(dD . S),  G_prev = Diag(a) dD
// and dv = w . dx, dw = v . dx, db = k . dc, d log alpha = a . da (a scalar gate sums its
// channels).  Scalar gates: b, w or a is one value for every channel.
//
// Layout.  One workgroup of 4 waves per (batch, head) and block of up to 64 value columns; wave w
// holds columns 16 w .. 16 w + 15 of S and of G, lane l rows R (l / 4) .. R (l / 4) + R - 1
// (R = dk / 16) and columns 4 (l % 4) .. 4 (l % 4) + 3 of them.  Sums over dk are the lane's own
// rows and four exchanges across lanes of equal l % 4; sums over the value columns are the lane's
// own four, two exchanges inside the quad, and the waves' partial rows added through LDS.
//
// Order.  A first pass walks the tokens forward from S0 and stores the state before every 8th
// token (the checkpoints).  The second walks the blocks of 8 tokens backward: for each token, last
// first, it recomputes the state before it from the block's checkpoint, or from the state before
// the block's fifth token (formed once per block), and applies the adjoint above.  Each token's column sums of the four row gradients (dq, dk, d log alpha, db) and the
// scalar gates' sums are written per column block; a last kernel adds the blocks (and, with grouped
// heads, the value heads of each q / k head) in a fixed order, so results do not depend on timing.
#include "gdr_common.h"

namespace gdr {

struct TokBwdArgs {
  const void *q, *k, *v, *la, *bg, *wg, *dO;
  const float* S0;
  const float* dST;
  void *dv, *dw;  // per column outputs: written here
  float* dS0;
  float* ck;  // [bh][nb][DK][DV] state before tokens 0, 8, 16, ...
  float* P;   // [ncb][rows][4][DK] per column block: dq, dk, d log alpha, db of every token
  float* Ps;  // [ncb][rows][4] per column block: the scalar gates' sums (alpha, b, w)
  int64_t T, H, Hk, DV, nb, ncb, rows;  // rows = B T H
  int alpha_kind, b_kind, w_kind;
};

namespace {

constexpr int kTokB = 8;     // tokens per block (checkpoint interval)
constexpr int kTokMid = 4;   // the block's second restart point, kept in registers
constexpr int kTokCols = 64;  // value columns per workgroup
constexpr int kTokThreads = 256;
constexpr int kTokWaves = kTokThreads / 64;

template <int DK>
struct TokLds {
  // one block of inputs as fp32: q, k, a = exp(log alpha), b per channel (scalar gates
  // broadcast), and this workgroup's columns of v, w and do
  static constexpr int iQ = 0, iK = iQ + kTokB * DK, iA = iK + kTokB * DK, iB = iA + kTokB * DK;
  static constexpr int iV = iB + kTokB * DK, iW = iV + kTokB * kTokCols, iD = iW + kTokB * kTokCols;
  static constexpr int iEnd = iD + kTokB * kTokCols;
  // per token, two buffers: each wave's partial rows [waves][4][DK] and scalars [waves][4]
  static constexpr int rRow = iEnd, rSc = rRow + 2 * kTokWaves * 4 * DK;
  static constexpr int floats = rSc + 2 * kTokWaves * 4;
};

template <int M>
__device__ __forceinline__ float dpp_ror(float x) {  // rotate right by M within each 16-lane row
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + M, 0xf, 0xf, false));
}
template <int PERM>
__device__ __forceinline__ float dpp_quad(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), PERM, 0xf, 0xf, false));
}
// sum over the 16 lanes of equal lane % 4 (lanes 4 g + lane % 4, g = 0 .. 15)
__device__ __forceinline__ float sum_rows(float x) {
  x += dpp_ror<4>(x);
  x += dpp_ror<8>(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
__device__ __forceinline__ float quad_xor2(float x) { return dpp_quad<0x4e>(x); }  // lanes ^ 2
__device__ __forceinline__ float quad_xor1(float x) { return dpp_quad<0xb1>(x); }  // lanes ^ 1

template <typename IO>
__device__ __forceinline__ void store4(void* base, int64_t i, const float* f) {
  IO* p = static_cast<IO*>(base);
#pragma unroll
  for (int c = 0; c < 4; ++c) st<IO>(p, i + c, f[c]);
}

// One forward token (tt inside the block in LDS) on this lane's rows and columns of S, the state
// before the token on entry.
template <int DK, bool DF>
__device__ __forceinline__ void tok_forward(float (&s)[DK / 16][4], const float* L, int tt, int d0, int lc0) {
  using LY = TokLds<DK>;
  constexpr int R = DK / 16;
  const float* kk = L + LY::iK + tt * DK + d0;
  const float* ka = L + LY::iA + tt * DK + d0;
  const float* kb = L + LY::iB + tt * DK + d0;
  const float* kv = L + LY::iV + tt * kTokCols + lc0;
  const float* kw = L + LY::iW + tt * kTokCols + lc0;
  float x[4], r[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) x[c] = kw[c] * kv[c];
#pragma unroll
  for (int c = 0; c < 4; ++c) r[c] = 0.f;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const float ci = kb[i] * kk[i] * (DF ? ka[i] : 1.f);
#pragma unroll
    for (int c = 0; c < 4; ++c) r[c] = fmaf(ci, s[i][c], r[c]);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) r[c] = sum_rows(r[c]);
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const float ki = kk[i], ai = ka[i];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (DF)
        s[i][c] = fmaf(ki, x[c] - r[c], ai * s[i][c]);
      else
        s[i][c] = fmaf(ki, x[c], ai * fmaf(-ki, r[c], s[i][c]));
    }
  }
}

}  // namespace

template <typename IO, int DK, bool DF>
__global__ __launch_bounds__(kTokThreads) void bwd_tok_kernel(TokBwdArgs a) {
  constexpr int R = DK / 16;
  constexpr bool CK_REG = R <= 8;  // the block's checkpoint kept in registers (else reread)
  using LY = TokLds<DK>;
  __shared__ __attribute__((aligned(16))) float L[LY::floats];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rg = lane >> 2, cq = lane & 3, d0 = rg * R;
  const int64_t ncb = a.ncb, bh = blockIdx.x / ncb, cb = blockIdx.x % ncb;
  const int64_t H = a.H, Hk = a.Hk, T = a.T, DV = a.DV, nb = a.nb;
  const int64_t bi = bh / H, hi = bh % H, hk = hi / (H / Hk);
  const int64_t cbase = cb * kTokCols;
  const int ncols = static_cast<int>(DV - cbase < kTokCols ? DV - cbase : kTokCols);
  const bool active = wave < ncols / 16;  // (uniform per wave)
  const int lc0 = 16 * wave + 4 * cq;     // first column of this lane inside the block
  const int64_t col0 = cbase + lc0;
  const IO* q = static_cast<const IO*>(a.q);
  const IO* kx = static_cast<const IO*>(a.k);
  const IO* v = static_cast<const IO*>(a.v);
  const IO* la = static_cast<const IO*>(a.la);
  const IO* bg = static_cast<const IO*>(a.bg);
  const IO* wg = static_cast<const IO*>(a.wg);
  const IO* dO = static_cast<const IO*>(a.dO);
  const int AK = a.alpha_kind, BK = a.b_kind, WK = a.w_kind;

  // inputs of tokens t0 .. t0 + n - 1 into LDS as fp32 (gates broadcast to every channel)
  auto load_block = [&](int64_t t0, int n) {
    for (int e = tid; e < n * DK; e += kTokThreads) {
      const int tt = e / DK, i = e % DK;
      const int64_t row = (bi * T + t0 + tt) * H + hi;  // value-head row
      const int64_t qrow = (bi * T + t0 + tt) * Hk + hk;
      L[LY::iQ + e] = ld<IO>(q, qrow * DK + i);
      L[LY::iK + e] = ld<IO>(kx, qrow * DK + i);
      L[LY::iA + e] = AK == kNone ? 1.f : expf(ld<IO>(la, AK == kChannel ? row * DK + i : row));
      L[LY::iB + e] = BK == kNone ? 0.f : ld<IO>(bg, BK == kChannel ? row * DK + i : row);
    }
    for (int e = tid; e < n * kTokCols; e += kTokThreads) {
      const int tt = e / kTokCols, c = e % kTokCols;
      if (c >= ncols) continue;
      const int64_t row = (bi * T + t0 + tt) * H + hi;
      L[LY::iV + e] = ld<IO>(v, row * DV + cbase + c);
      L[LY::iD + e] = ld<IO>(dO, row * DV + cbase + c);
      L[LY::iW + e] = WK == kNone ? 1.f : ld<IO>(wg, WK == kChannel ? row * DV + cbase + c : row);
    }
  };

  float s[R][4], g[R][4];
  if (active) {
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        s[i][c] = a.S0 ? a.S0[(bh * DK + d0 + i) * DV + col0 + c] : 0.f;
  }

  // ---- forward: the checkpoints ----
  for (int64_t j = 0; j < nb; ++j) {
    const int64_t t0 = j * kTokB;
    const int n = static_cast<int>(T - t0 < kTokB ? T - t0 : kTokB);
    if (active) {
      float* ck = a.ck + ((bh * nb + j) * DK + d0) * DV + col0;
#pragma unroll
      for (int i = 0; i < R; ++i)
        *reinterpret_cast<float4*>(ck + i * DV) = make_float4(s[i][0], s[i][1], s[i][2], s[i][3]);
    }
    __syncthreads();  // the previous block's LDS inputs are no longer read
    load_block(t0, n);
    __syncthreads();
    if (active)
      for (int tt = 0; tt < n; ++tt) tok_forward<DK, DF>(s, L, tt, d0, lc0);
  }
  __syncthreads();  // (the checkpoint stores complete before they are read back below)

  // ---- backward over the blocks, last first ----
  if (active) {
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        g[i][c] = a.dST ? a.dST[(bh * DK + d0 + i) * DV + col0 + c] : 0.f;
  }
  float ckr[CK_REG ? R : 1][4];
  float mid[R][4];
  int par = 0;
  for (int64_t j = nb - 1; j >= 0; --j) {
    const int64_t t0 = j * kTokB;
    const int n = static_cast<int>(T - t0 < kTokB ? T - t0 : kTokB);
    const float* ckp = a.ck + ((bh * nb + j) * DK + d0) * DV + col0;
    if (CK_REG && active) {
#pragma unroll
      for (int i = 0; i < (CK_REG ? R : 1); ++i) {
        const float4 u = *reinterpret_cast<const float4*>(ckp + i * DV);
        ckr[i][0] = u.x;
        ckr[i][1] = u.y;
        ckr[i][2] = u.z;
        ckr[i][3] = u.w;
      }
    }
    __syncthreads();
    load_block(t0, n);
    __syncthreads();
    // the state before token kTokMid of the block, from the checkpoint: tokens kTokMid .. n - 1
    // restart from it, tokens 0 .. kTokMid - 1 from the checkpoint (16 forward steps a block
    // instead of 28)
    if (active && n > kTokMid) {
      if constexpr (CK_REG) {
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
          for (int c = 0; c < 4; ++c) mid[i][c] = ckr[i][c];
      } else {
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const float4 u = *reinterpret_cast<const float4*>(ckp + i * DV);
          mid[i][0] = u.x;
          mid[i][1] = u.y;
          mid[i][2] = u.z;
          mid[i][3] = u.w;
        }
      }
      for (int u = 0; u < kTokMid; ++u) tok_forward<DK, DF>(mid, L, u, d0, lc0);
    }
    for (int tt = n - 1; tt >= 0; --tt, par ^= 1) {
      float* red = L + LY::rRow + par * (kTokWaves * 4 * DK);
      float* sred = L + LY::rSc + par * (kTokWaves * 4);
      if (active) {
        // the state before token tt
        const int u0 = tt >= kTokMid ? kTokMid : 0;
        if (tt >= kTokMid) {
#pragma unroll
          for (int i = 0; i < R; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) s[i][c] = mid[i][c];
        } else if constexpr (CK_REG) {
#pragma unroll
          for (int i = 0; i < R; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) s[i][c] = ckr[i][c];
        } else {
#pragma unroll
          for (int i = 0; i < R; ++i) {
            const float4 u = *reinterpret_cast<const float4*>(ckp + i * DV);
            s[i][0] = u.x;
            s[i][1] = u.y;
            s[i][2] = u.z;
            s[i][3] = u.w;
          }
        }
        for (int u = u0; u < tt; ++u) tok_forward<DK, DF>(s, L, u, d0, lc0);

        const float* kq = L + LY::iQ + tt * DK + d0;
        const float* kk = L + LY::iK + tt * DK + d0;
        const float* ka = L + LY::iA + tt * DK + d0;
        const float* kb = L + LY::iB + tt * DK + d0;
        float x[4], vv[4], ww[4], dd[4], r[4], dx[4], dr[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          vv[c] = L[LY::iV + tt * kTokCols + lc0 + c];
          ww[c] = L[LY::iW + tt * kTokCols + lc0 + c];
          dd[c] = L[LY::iD + tt * kTokCols + lc0 + c];
          x[c] = ww[c] * vv[c];
          r[c] = 0.f;
        }
        // r = c S (erase first) or c D (decay first)
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const float ci = kb[i] * kk[i] * (DF ? ka[i] : 1.f);
#pragma unroll
          for (int c = 0; c < 4; ++c) r[c] = fmaf(ci, s[i][c], r[c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) r[c] = sum_rows(r[c]);
        // dq (from S_t), then Gt = G + q^T do and dx = k Gt
        float pq[R], pk[R], pa[R], pc[R];
#pragma unroll
        for (int c = 0; c < 4; ++c) dx[c] = 0.f;
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const float ki = kk[i], ai = ka[i], qi = kq[i];
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float st_ = DF ? fmaf(ki, x[c] - r[c], ai * s[i][c]) : fmaf(ki, x[c], ai * fmaf(-ki, r[c], s[i][c]));
            acc = fmaf(dd[c], st_, acc);
            g[i][c] = fmaf(qi, dd[c], g[i][c]);
            dx[c] = fmaf(ki, g[i][c], dx[c]);
          }
          pq[i] = acc;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) dx[c] = sum_rows(dx[c]);
        if constexpr (DF) {
#pragma unroll
          for (int c = 0; c < 4; ++c) dr[c] = -dx[c];
#pragma unroll
          for (int i = 0; i < R; ++i) {
            const float ai = ka[i], ci = kb[i] * kk[i];
            float dk_ = 0.f, dc_ = 0.f, da_ = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              dk_ = fmaf(g[i][c], x[c] - r[c], dk_);
              dc_ = fmaf(dr[c], ai * s[i][c], dc_);
              const float dD = fmaf(ci, dr[c], g[i][c]);
              da_ = fmaf(dD, s[i][c], da_);
              g[i][c] = ai * dD;
            }
            pk[i] = fmaf(kb[i], dc_, dk_);
            pa[i] = ai * da_;
            pc[i] = kk[i] * dc_;
          }
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) dr[c] = 0.f;
          float dkw[R], da[R];
#pragma unroll
          for (int i = 0; i < R; ++i) {
            const float ki = kk[i], ai = ka[i];
            float w_ = 0.f, e_ = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              w_ = fmaf(g[i][c], x[c], w_);
              e_ = fmaf(g[i][c], fmaf(-ki, r[c], s[i][c]), e_);
              g[i][c] *= ai;  // dE
              dr[c] = fmaf(-ki, g[i][c], dr[c]);
            }
            dkw[i] = w_;
            da[i] = e_;
          }
#pragma unroll
          for (int c = 0; c < 4; ++c) dr[c] = sum_rows(dr[c]);
#pragma unroll
          for (int i = 0; i < R; ++i) {
            const float ki = kk[i], ai = ka[i], ci = kb[i] * ki;
            float ke = 0.f, dc_ = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              ke = fmaf(g[i][c], r[c], ke);
              dc_ = fmaf(dr[c], s[i][c], dc_);
              g[i][c] = fmaf(ci, dr[c], g[i][c]);
            }
            pk[i] = fmaf(kb[i], dc_, dkw[i] - ke);
            pa[i] = ai * da[i];
            pc[i] = ki * dc_;
          }
        }
        // per column outputs: dv = w . dx, a per-channel dw = v . dx (lanes of row group 0)
        if (rg == 0) {
          const int64_t row = (bi * T + t0 + tt) * H + hi;
          float o4[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) o4[c] = ww[c] * dx[c];
          store4<IO>(a.dv, row * DV + col0, o4);
          if (WK == kChannel) {
#pragma unroll
            for (int c = 0; c < 4; ++c) o4[c] = vv[c] * dx[c];
            store4<IO>(a.dw, row * DV + col0, o4);
          }
        }
        // the quad's four columns: lane cq keeps quantity cq (0 dq, 1 dk, 2 d log alpha, 3 db)
        const bool hi2 = (cq & 2) != 0, hi1 = (cq & 1) != 0;
        float h0[R], h1[R], own[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const float send0 = hi2 ? pq[i] : pa[i], send1 = hi2 ? pk[i] : pc[i];
          h0[i] = (hi2 ? pa[i] : pq[i]) + quad_xor2(send0);
          h1[i] = (hi2 ? pc[i] : pk[i]) + quad_xor2(send1);
        }
#pragma unroll
        for (int i = 0; i < R; ++i) own[i] = (hi1 ? h1[i] : h0[i]) + quad_xor1(hi1 ? h0[i] : h1[i]);
        float* dst = red + (wave * 4 + cq) * DK + d0;
#pragma unroll
        for (int i = 0; i < R; ++i) dst[i] = own[i];
        // scalar gates: a's and b's sums over the wave's rows, w's over its columns
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < R; ++i) tot += own[i];
        tot = sum_rows(tot);
        float sw = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) sw = fmaf(vv[c], dx[c], sw);
        sw += quad_xor2(sw);
        sw += quad_xor1(sw);
        if (lane == 2) sred[wave * 4 + 0] = tot;
        if (lane == 3) sred[wave * 4 + 1] = tot;
        if (lane == 0) sred[wave * 4 + 2] = sw;
      }
      __syncthreads();
      // the waves' partials in order, to this column block's slot
      {
        const int nw = ncols / 16;
        const int64_t row = (bi * T + t0 + tt) * H + hi;
        const int64_t rows = a.rows;
        float* P = a.P + (cb * rows + row) * 4 * DK;
        for (int e = tid; e < 4 * DK; e += kTokThreads) {
          float acc = 0.f;
          for (int w = 0; w < nw; ++w) acc += red[w * 4 * DK + e];
          P[e] = acc;
        }
        if (tid < 3) {
          float acc = 0.f;
          for (int w = 0; w < nw; ++w) acc += sred[w * 4 + tid];
          a.Ps[(cb * rows + row) * 4 + tid] = acc;
        }
      }
    }
  }
  if (active && a.dS0) {
#pragma unroll
    for (int i = 0; i < R; ++i)
      *reinterpret_cast<float4*>(a.dS0 + (bh * DK + d0 + i) * DV + col0) =
          make_float4(g[i][0], g[i][1], g[i][2], g[i][3]);
  }
}

// The row gradients from the column blocks' partials: one thread per (value-head row, channel).
// dq and dk of a q / k head sum its G = H / Hk value heads (rows h0 .. h0 + G - 1 of one token).
template <typename IO>
__global__ __launch_bounds__(256) void bwd_tok_finish_kernel(TokBwdArgs a, void* dq, void* dk, void* dla,
                                                             void* db, void* dw, int64_t rows, int DK) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= rows * DK) return;
  const int64_t row = e / DK;
  const int i = static_cast<int>(e % DK);
  const int64_t H = a.H, G = a.H / a.Hk, ncb = a.ncb;
  auto part = [&](int64_t r, int qn) {
    float acc = 0.f;
    for (int64_t cb = 0; cb < ncb; ++cb) acc += a.P[((cb * rows + r) * 4 + qn) * DK + i];
    return acc;
  };
  auto spart = [&](int qn) {
    float acc = 0.f;
    for (int64_t cb = 0; cb < ncb; ++cb) acc += a.Ps[(cb * rows + row) * 4 + qn];
    return acc;
  };
  if (a.alpha_kind == kChannel) st<IO>(static_cast<IO*>(dla), row * DK + i, part(row, 2));
  if (a.b_kind == kChannel) st<IO>(static_cast<IO*>(db), row * DK + i, part(row, 3));
  if (i == 0) {
    if (a.alpha_kind == kScalar) st<IO>(static_cast<IO*>(dla), row, spart(0));
    if (a.b_kind == kScalar) st<IO>(static_cast<IO*>(db), row, spart(1));
    if (a.w_kind == kScalar) st<IO>(static_cast<IO*>(dw), row, spart(2));
  }
  const int64_t h = row % H;
  if (h % G == 0) {
    float sq = 0.f, sk = 0.f;
    for (int64_t gi = 0; gi < G; ++gi) {
      sq += part(row + gi, 0);
      sk += part(row + gi, 1);
    }
    const int64_t qrow = (row / H) * a.Hk + h / G;
    st<IO>(static_cast<IO*>(dq), qrow * DK + i, sq);
    st<IO>(static_cast<IO*>(dk), qrow * DK + i, sk);
  }
}

namespace {
size_t al256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct TokSizes {
  size_t ck, P, Ps;
};
TokSizes tok_sizes(int64_t B, int64_t H, int64_t T, int64_t DK, int64_t DV) {
  const int64_t nb = (T + kTokB - 1) / kTokB, ncb = (DV + kTokCols - 1) / kTokCols;
  const size_t rows = static_cast<size_t>(B * T * H);
  return {al256(static_cast<size_t>(B * H * nb) * DK * DV * 4), al256(ncb * rows * 4 * DK * 4),
          al256(ncb * rows * 4 * 4)};
}

template <typename IO, int DK>
void launch_tok_dk(const TokBwdArgs& a, bool decay_first, int64_t nstate, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(nstate * a.ncb));
  if (decay_first)
    hipLaunchKernelGGL((bwd_tok_kernel<IO, DK, true>), grid, dim3(kTokThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_tok_kernel<IO, DK, false>), grid, dim3(kTokThreads), 0, s, a);
}

template <typename IO>
void launch_tok(const TokBwdArgs& a, int64_t DK, bool decay_first, int64_t nstate, hipStream_t s) {
  switch (DK) {
    case 16: launch_tok_dk<IO, 16>(a, decay_first, nstate, s); break;
    case 32: launch_tok_dk<IO, 32>(a, decay_first, nstate, s); break;
    case 64: launch_tok_dk<IO, 64>(a, decay_first, nstate, s); break;
    case 128: launch_tok_dk<IO, 128>(a, decay_first, nstate, s); break;
    default: launch_tok_dk<IO, 256>(a, decay_first, nstate, s); break;
  }
}
}  // namespace

size_t backward_tok_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t DK, int64_t DV) {
  const TokSizes z = tok_sizes(B, H, T, DK, DV);
  return z.ck + z.P + z.Ps;
}

// io_bf16: the I/O type of every tensor but the states (fp32 either way)
hipError_t launch_backward_tok(bool io_bf16, const void* q, const void* k, const void* v, const void* la,
                               const void* bg, const void* wg, const float* S0, const void* dO,
                               const float* dST, void* dq, void* dk, void* dv, void* dla, void* db,
                               void* dw, float* dS0, int64_t B, int64_t T, int64_t H, int64_t Hk,
                               int64_t DK, int64_t DV, int alpha_kind, int b_kind, int w_kind,
                               bool decay_first, void* workspace, hipStream_t s) {
  const int64_t nstate = B * H;
  if (nstate == 0) return hipSuccess;
  const TokSizes z = tok_sizes(B, H, T, DK, DV);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  TokBwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.la = la;
  a.bg = bg;
  a.wg = wg;
  a.dO = dO;
  a.S0 = S0;
  a.dST = dST;
  a.dv = dv;
  a.dw = dw;
  a.dS0 = dS0;
  a.ck = reinterpret_cast<float*>(ws);
  a.P = reinterpret_cast<float*>(ws + z.ck);
  a.Ps = reinterpret_cast<float*>(ws + z.ck + z.P);
  a.T = T;
  a.H = H;
  a.Hk = Hk;
  a.DV = DV;
  a.nb = (T + kTokB - 1) / kTokB;
  a.ncb = (DV + kTokCols - 1) / kTokCols;
  a.rows = B * T * H;
  a.alpha_kind = alpha_kind;
  a.b_kind = b_kind;
  a.w_kind = w_kind;
  if (io_bf16)
    launch_tok<bf16_t>(a, DK, decay_first, nstate, s);
  else
    launch_tok<float>(a, DK, decay_first, nstate, s);
  const int64_t rows = B * T * H;
  if (rows > 0) {
    const dim3 grid(static_cast<unsigned>((rows * DK + 255) / 256));
    if (io_bf16)
      hipLaunchKernelGGL(bwd_tok_finish_kernel<bf16_t>, grid, dim3(256), 0, s, a, dq, dk, dla, db, dw, rows, static_cast<int>(DK));
    else
      hipLaunchKernelGGL(bwd_tok_finish_kernel<float>, grid, dim3(256), 0, s, a, dq, dk, dla, db, dw, rows, static_cast<int>(DK));
  }
  return hipGetLastError();
}

}  // namespace gdr
