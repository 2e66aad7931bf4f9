// Chunkwise prefill with a per-channel decay, as two kernels: a chunk-local kernel over every
// chunk of every state at once, and a state kernel that walks the chunks of each state in order
// and does only the work that depends on S.
//
// Chunk form (derived by unrolling the recurrence over a chunk: "Recurrent Memory: Write,
// Erase, Decay, Read", section 03 for the linear erase that reassociates over a chunk and
// section 04 for the decay as prefix sums G_t of log alpha; the Gated DeltaNet-2 abstract for a
// channel-wise decay absorbed into separate erase factors).  With c = b . k, X = w . v and
// per-channel prefix sums G_t (G_0 = 0):
//
//   decay after the erase (the unified equation's order; MODE 2), two key families:
//     Chat_t = c_t e^{G_{t-1}}, Phat_i = k_i e^{-G_{i-1}}, Khat_i = k_i e^{-G_i}, Qhat_t = q_t e^{G_t}
//     L_P = strict_tril(Chat Phat^T), L_K = strict_tril(Chat Khat^T),
//     M_QK = tril(Qhat Khat^T), M_QP = tril(Qhat Phat^T), T = (I + L_P)^{-1}
//     R = W S + Y with W = T Chat, Y = T L_K X              (R_t = c_t S_{t-1}: the erase reads)
//     O = Qhat S + Z - M_QP R with Z = M_QK X
//     S' = e^{G_n} . S + Kbar^T X - Pbar^T R, Kbar_i = k_i e^{G_n - G_i}, Pbar_i = k_i e^{G_n - G_{i-1}}
//   decay before the erase (MODE 1), rank one per token:
//     Chat_t = c_t e^{G_t}, L = strict_tril(Chat Khat^T), M = tril(Qhat Khat^T), T = (I + L)^{-1}
//     R = W S + Y with W = T Chat, Y = -T X;   O = Qhat S - M R;   S' = e^{G_n} . S - Kbar^T R
//
// The Gram products use the same factors split around G_ref = G_31 (e^{G_t - G_ref} on row
// operands, e^{G_ref - G_i} on column operands) so that every factor stays inside the fp32
// range; W, Qhat, Pbar and Kbar themselves only carry e^{non-positive} factors.
//
// Substituting R into the read-out and the update turns each chunk into an affine map of the
// state it starts from (R is never formed in the state kernel):
//   S' = e^{G_n} . S + A' S + D,   O = Q' S + Z',
//   A' = -Pbar^T W,  D = Kbar^T X - Pbar^T Y,  Q' = Qhat - M_QP W,  Z' = Z - M_QP Y
// (MODE 1: Pbar -> Kbar, M_QP -> M and no Kbar^T X, Z terms).  The chunk-local kernel forms these
// four matrices; the state kernel then does two products per chunk.  A chunk whose prefix sums
// span more than kWycSpanLimit nats (or are not finite) is flagged, and the chunk-local kernel
// forms its four matrices by running the recurrence over the chunk token by token in fp32 from
// the identity (A) and from zero (D) instead: exact for any gate values.
#pragma once
#include <type_traits>
#include "gdr_common.h"
#include "mfma.h"
#include "prefill_kernel.h"
#include "prefill_wy.h"

namespace gdr {

struct WycArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* la;
  const bf16_t* bg;
  const bf16_t* wg;
  const float* S0;
  bf16_t* o;
  float* S_T;
  // workspace, per chunk index cix = state * nch + chunk: the affine chunk map, each matrix as
  // 16 x 16 tiles of 512 bytes (tiled16 below), so that an MFMA output tile is one contiguous store
  __bf16* Qd;  // [cix][64][dk]  Q'
  __bf16* Ad;  // [cix][dk][dk]  A'
  __bf16* Dt;  // [cix][dv][dk]  D^T
  __bf16* Zd;  // [cix][64][dv]  Z'
  float* Egn;  // [cix][dk + 4]  e^{G_n}, then the flag (as int) and 3 unused
  int* flag;   // [cix]          1: exact token path
  int64_t T, H, DV, nch;
  int b_kind, w_kind;
  int alpha_kind;  // kChannel; kScalar (one log alpha per token, broadcast over the channels) and
                   // kNone (alpha = 1) in the chunk-local kernel with an erase gate only
  int nsl;     // value slices per state (state kernel)
  int64_t Hk;  // q / k heads (H is a multiple): value head h reads q / k head h / (H / Hk)
};

constexpr float kWycSpanLimit = 76.f;

// Element (r, c) of a matrix with ncols columns (a multiple of 16) stored as 16 x 16 tiles of 512
// bytes: row-major inside a tile, tiles row-major.
__host__ __device__ constexpr inline int64_t tiled16(int64_t r, int64_t c, int64_t ncols) {
  return ((r >> 4) * (ncols >> 4) + (c >> 4)) * 256 + (r & 15) * 16 + (c & 15);
}

// ------------------------------------------------------------------ chunk-local kernel

template <int DK, int DVP, int MODE, int NSEGX>
struct WycPrepLayoutN {
  static constexpr bool TWO = MODE == 2;
  static constexpr int C = 64;
  static constexpr int LDT = DK + 8;
  static constexpr int LDX = DVP + 8;
  static constexpr int LDD = C + 8;
  static constexpr int LDA = 48 + 8;
  static constexpr int LDI = 24;
  static constexpr int LDL = 20;
  static constexpr int NCG = DK / 8;
  static constexpr int NSEG = NSEGX;  // token segments of the prefix sums (threads NSEG * NCG)
  static constexpr int TPS = C / NSEG;
  static constexpr int oQ = 0;                              // split Qhat  [64][LDT]
  static constexpr int oC = oQ + C * LDT * 2;               // split Chat  [64][LDT]
  static constexpr int oK = oC + C * LDT * 2;               // split Khat  [64][LDT]
  static constexpr int oP = oK + C * LDT * 2;               // split Phat  [64][LDT] (MODE 2)
  static constexpr int oX = oP + (TWO ? C * LDT * 2 : 0);   // X rows [64][LDX]
  static constexpr int oA = oX + C * LDX * 2;               // -L_P off-diagonal blocks (packed)
  static constexpr int oM = oA + 48 * LDA * 2;              // -M_QP / -M [64][LDD]
  static constexpr int oLK = oM + C * LDD * 2;              // L_K [64][LDD] (MODE 2)
  static constexpr int oMQK = oLK + (TWO ? C * LDD * 2 : 0);  // M_QK [64][LDD] (MODE 2)
  static constexpr int oT = oMQK + (TWO ? C * LDD * 2 : 0);   // T [64][LDD]
  static constexpr int oI = oT + C * LDD * 2;               // T_ii [4][16][LDI]
  static constexpr int oLD = oI + 4 * 16 * LDI * 2;         // fp32 L_ii column-major
  static constexpr int oSEG = oLD + 4 * 16 * LDL * 4;       // fp32 segment sums [NSEG][DK]
  static constexpr int oF = oSEG + NSEG * DK * 4;           // fp32 G_ref, e^{G_ref}, e^{G_n - G_ref} [DK] each; flag
  static constexpr int total = oF + (3 * DK + 4) * 4;
  static constexpr bool fits = total <= kLdsLimit;
  static_assert(oF % 16 == 0, "the per-channel factors are read as float4");
};
// 512 threads; the prefix sums over as many token segments as there are threads for (NT / NCG,
// at most 64) when their LDS fits, else half as many
template <int DK, int DVP, int MODE>
struct WycPrepLayoutSel {
  static constexpr int NT = 512;
  static constexpr int NS1 = (NT / (DK / 8)) < 64 ? (NT / (DK / 8)) : 64;
  using type = typename std::conditional<WycPrepLayoutN<DK, DVP, MODE, NS1>::fits, WycPrepLayoutN<DK, DVP, MODE, NS1>,
                                         WycPrepLayoutN<DK, DVP, MODE, NS1 / 2>>::type;
};
template <int DK, int DVP, int MODE>
using WycPrepLayout = typename WycPrepLayoutSel<DK, DVP, MODE>::type;

// The affine map of a flagged chunk from the recurrence itself, token by token in fp32.  Two
// adjacent lanes share a column, 64 channels each (the dot products are the pair's two partial
// sums): lane pairs 0 .. 127 carry column j of the transition product A (started from the
// identity; its outputs q_t A_t are row t of Q'), lane pairs 128 .. 255 carry value column
// v (and v + 128) of the state D started from zero (outputs q_t D_t: Z').  Every lane pair reads
// the same raw row at once.  Rows past the last token are zero (alpha = 1, no erase, no write),
// so all 64 rows run.
template <int DK, int LDT, int LDX, bool TWO>
__device__ __forceinline__ void wyc_exact_chunk(const WycArgs& a, int64_t cix, const __bf16* rQ,
                                                const __bf16* rK, const __bf16* rC, const __bf16* rL,
                                                const __bf16* tX, const float* fEgn, int tid) {
  constexpr int C = 64, DH = DK / 2;
  const int64_t DV = a.DV;
  const int hf = tid & 1, pr = tid >> 1, d0 = hf * DH;  // this lane's channels d0 .. d0 + DH - 1
  // one column s through the chunk; col_x < 0: no write (the transition); y_t = q_t s_t to element
  // (t, ycol) of yout (tiled, ypitch columns), by the even lane
  auto run = [&](float (&s)[DH], int col_x, __bf16* yout, int ycol, int64_t ypitch) {
    for (int t = 0; t < C; ++t) {
      float r = 0.f;  // c_t s (after the decay in MODE 1)
#pragma unroll
      for (int p = 0; p < DH / 8; ++p) {
        float c8[8];
        load8f(reinterpret_cast<const bf16_t*>(rC + t * LDT + d0 + 8 * p), c8);
        if (!TWO) {
          float l8[8];
          load8f(reinterpret_cast<const bf16_t*>(rL + t * DK + d0 + 8 * p), l8);
#pragma unroll
          for (int e = 0; e < 8; ++e) s[8 * p + e] *= __expf(l8[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) r += c8[e] * s[8 * p + e];
      }
      r += __shfl_xor(r, 1);
      const float x = col_x >= 0 ? static_cast<float>(tX[t * LDX + col_x]) : 0.f;
      float y = 0.f;
#pragma unroll
      for (int p = 0; p < DH / 8; ++p) {
        float k8[8], q8[8], l8[8];
        load8f(reinterpret_cast<const bf16_t*>(rK + t * LDT + d0 + 8 * p), k8);
        load8f(reinterpret_cast<const bf16_t*>(rQ + t * LDT + d0 + 8 * p), q8);
        if (TWO) load8f(reinterpret_cast<const bf16_t*>(rL + t * DK + d0 + 8 * p), l8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float sv = s[8 * p + e] - k8[e] * r;
          if (TWO) sv *= __expf(l8[e]);
          sv += k8[e] * x;
          s[8 * p + e] = sv;
          y += q8[e] * sv;
        }
      }
      y += __shfl_xor(y, 1);
      if (hf == 0) yout[tiled16(t, ycol, ypitch)] = static_cast<__bf16>(y);
    }
  };
  if (pr < 128) {
    const int j = pr;
    if (j < DK) {
      float s[DH];
#pragma unroll
      for (int i = 0; i < DH; ++i) s[i] = d0 + i == j ? 1.f : 0.f;
      run(s, -1, a.Qd + cix * C * DK, j, DK);
      // A' = A - diag(e^{G_n}), column j
      const float egn_j = fEgn[j];
      __bf16* Ao = a.Ad + cix * DK * DK;
#pragma unroll
      for (int i = 0; i < DH; ++i)
        Ao[tiled16(d0 + i, j, DK)] = static_cast<__bf16>(s[i] - (d0 + i == j ? egn_j : 0.f));
    }
  } else {
    for (int v = pr - 128; v < DV; v += 128) {
      float s[DH];
#pragma unroll
      for (int i = 0; i < DH; ++i) s[i] = 0.f;
      run(s, v, a.Zd + cix * C * DV, v, DV);
      __bf16* Do = a.Dt + cix * DV * DK;  // row v of D^T, this lane's channels
#pragma unroll
      for (int p = 0; p < DH / 8; ++p) {
        bf16x8 d8;
#pragma unroll
        for (int e = 0; e < 8; ++e) d8[e] = static_cast<__bf16>(s[8 * p + e]);
        *reinterpret_cast<bf16x8*>(Do + tiled16(v, d0 + 8 * p, DK)) = d8;
      }
    }
  }
}

template <int DK, int DVP, int MODE>
__global__ __launch_bounds__(512) void wyc_prep_kernel(WycArgs a) {
  using L = WycPrepLayout<DK, DVP, MODE>;
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  static_assert(L::fits, "LDS layout exceeds the gfx950 workgroup limit");
  static_assert(DK % 32 == 0, "dk must be a multiple of 32");
  constexpr bool TWO = L::TWO;
  constexpr int C = L::C, LDT = L::LDT, LDX = L::LDX, LDD = L::LDD, LDA = L::LDA, LDI = L::LDI,
                LDL = L::LDL;
  constexpr int NCG = L::NCG, NSEG = L::NSEG, TPS = L::TPS, NKB = DK / 32, NTD = DK / 16;
  constexpr int NT = 512, NW = NT / 64;  // threads, waves

  __shared__ __attribute__((aligned(32))) unsigned char smem[L::total];
  __bf16* tQ = reinterpret_cast<__bf16*>(smem + L::oQ);
  __bf16* tC = reinterpret_cast<__bf16*>(smem + L::oC);
  __bf16* tK = reinterpret_cast<__bf16*>(smem + L::oK);
  __bf16* tP = reinterpret_cast<__bf16*>(smem + L::oP);
  __bf16* tX = reinterpret_cast<__bf16*>(smem + L::oX);
  __bf16* gA = reinterpret_cast<__bf16*>(smem + L::oA);
  __bf16* gM = reinterpret_cast<__bf16*>(smem + L::oM);
  __bf16* gLK = reinterpret_cast<__bf16*>(smem + L::oLK);
  __bf16* gMQK = reinterpret_cast<__bf16*>(smem + L::oMQK);
  __bf16* tT = reinterpret_cast<__bf16*>(smem + L::oT);
  __bf16* dInv = reinterpret_cast<__bf16*>(smem + L::oI);
  float* Ld = reinterpret_cast<float*>(smem + L::oLD);
  float* segtot = reinterpret_cast<float*>(smem + L::oSEG);
  float* fRef = reinterpret_cast<float*>(smem + L::oF);
  float* fEref = fRef + DK;
  float* fEgr = fRef + 2 * DK;  // e^{G_n - G_ref}
  int* sFlag = reinterpret_cast<int*>(fRef + 3 * DK);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int64_t nch = a.nch, DV = a.DV, H = a.H;
  const int64_t bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int64_t bi = bh / H, hi = bh % H;
  const int64_t t0 = c * C;
  const int64_t rr = (bi * a.T + t0) * H + hi;
  const int64_t left = a.T - t0;
  const int64_t cix = bh * nch + c;
  const int ts = tid / NCG, d0 = (tid % NCG) * 8;
  const bool act = ts < NSEG;

  // ---- loads: every load first; out-of-range rows and absent gate kinds read zero ----
  const uint32_t oob = 0x80000000u;
  const uint32_t hdk = static_cast<uint32_t>(H * DK * 2), hdv = static_cast<uint32_t>(H * DV * 2);
  const uint32_t h1 = static_cast<uint32_t>(H * 2);
  const uint32_t hqk = static_cast<uint32_t>(a.Hk * DK * 2);      // token stride of q and k
  const int64_t rqk = (bi * a.T + t0) * a.Hk + hi / (H / a.Hk);  // their row of the first token
  const auto rq = make_rsrc(a.q + rqk * DK, wy_range(left, a.Hk, DK));
  const auto rk = make_rsrc(a.k + rqk * DK, wy_range(left, a.Hk, DK));
  const auto rla = make_rsrc(a.alpha_kind == kChannel ? a.la + rr * DK : a.q, a.alpha_kind == kChannel ? wy_range(left, H, DK) : 0u);
  const auto rlas = make_rsrc(a.alpha_kind == kScalar ? a.la + rr : a.q, a.alpha_kind == kScalar ? wy_range(left, H, 1) : 0u);
  const auto rbc = make_rsrc(a.b_kind == kChannel ? a.bg + rr * DK : a.q, a.b_kind == kChannel ? wy_range(left, H, DK) : 0u);
  const auto rbs = make_rsrc(a.b_kind == kScalar ? a.bg + rr : a.q, a.b_kind == kScalar ? wy_range(left, H, 1) : 0u);
  const auto rv = make_rsrc(a.v + rr * DV, wy_range(left, H, DV));
  const auto rwc = make_rsrc(a.w_kind == kChannel ? a.wg + rr * DV : a.v, a.w_kind == kChannel ? wy_range(left, H, DV) : 0u);
  const auto rws = make_rsrc(a.w_kind == kScalar ? a.wg + rr : a.v, a.w_kind == kScalar ? wy_range(left, H, 1) : 0u);
  uint4 pq[TPS], pk[TPS], pb[TPS], pl[TPS];
  uint16_t pbs[TPS];
#pragma unroll
  for (int u = 0; u < TPS; ++u) {
    const uint32_t t = ts * TPS + u;
    const uint32_t off = act ? t * hdk + d0 * 2 : oob;
    const uint32_t qo = act ? t * hqk + d0 * 2 : oob;
    pq[u] = buf_load16(rq, qo);
    pk[u] = buf_load16(rk, qo);
    pb[u] = buf_load16(rbc, off);
    pl[u] = buf_load16(rla, off);
    pbs[u] = buf_load_u16(rbs, act ? t * h1 : oob);
    if (a.alpha_kind == kScalar) {  // one log alpha per token on every channel
      const uint32_t h = buf_load_u16(rlas, act ? t * h1 : oob);
      const uint32_t w2 = h | (h << 16);
      pl[u] = make_uint4(w2, w2, w2, w2);
    }
  }
  constexpr int XPT = C * (DVP / 8) / NT;
  const int nxg = static_cast<int>(DV / 8);
  uint4 pv[XPT], pw[XPT];
  uint16_t pws[XPT];
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int item = tid + NT * j;
    const bool in = item < C * nxg;
    const uint32_t t = in ? item / nxg : 0, xg = in ? item % nxg : 0;
    pv[j] = buf_load16(rv, in ? t * hdv + xg * 16 : oob);
    pw[j] = buf_load16(rwc, in ? t * hdv + xg * 16 : oob);
    pws[j] = buf_load_u16(rws, in ? t * h1 : oob);
  }

  // ---- gate prefix sums: per-thread runs over TPS tokens, then a scan over segments ----
  float la8[TPS][8], G8[TPS][8];
  if (act) {
    float run[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < TPS; ++u) {
      load8f(reinterpret_cast<const bf16_t*>(&pl[u]), la8[u]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        run[j] += la8[u][j];
        G8[u][j] = run[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) segtot[ts * DK + d0 + j] = run[j];
  }
  // X rows (x = w . v) meanwhile
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int item = tid + NT * j;
    if (item < C * nxg) {
      const int t = item / nxg, xg = item % nxg;
      float x[8];
      load8f(reinterpret_cast<const bf16_t*>(&pv[j]), x);
      if (a.w_kind == kChannel) {
        float w8[8];
        load8f(reinterpret_cast<const bf16_t*>(&pw[j]), w8);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= w8[e];
      } else if (a.w_kind == kScalar) {
        const float ws = bf16_to_f32(pws[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= ws;
      }
      bf16x8 xb;
#pragma unroll
      for (int e = 0; e < 8; ++e) xb[e] = static_cast<__bf16>(x[e]);
      *reinterpret_cast<bf16x8*>(tX + t * LDX + xg * 8) = xb;
    }
  }
  if (tid == 0) sFlag[0] = 0;
  lds_barrier();
  float egn_own = 0.f;  // e^{G_n} of channel tid
  if (tid < DK) {
    float run = 0.f;
    for (int s = 0; s < NSEG; ++s) {
      const float tv = segtot[s * DK + tid];
      segtot[s * DK + tid] = run;
      run += tv;
    }
    const float ref = segtot[(NSEG / 2) * DK + tid];  // G_31
    fRef[tid] = ref;
    fEref[tid] = __expf(ref);
    fEgr[tid] = __expf(run - ref);
    egn_own = __expf(run);
    a.Egn[cix * (DK + 4) + tid] = egn_own;
    if (!(fabsf(ref) <= kWycSpanLimit && fabsf(run - ref) <= kWycSpanLimit)) sFlag[0] = 1;  // NaN, inf too
  }
  GDR_PMARK(0);
  lds_barrier();
  const bool robust = sFlag[0] != 0;
  if (tid < 4) {
    reinterpret_cast<int*>(a.Egn + cix * (DK + 4) + DK)[tid] = tid == 0 && robust ? 1 : 0;
    if (tid == 0) a.flag[cix] = robust ? 1 : 0;
  }
  if (robust) {
    if (tid < DK) fEgr[tid] = egn_own;  // (e^{G_n - G_ref} is not needed here: e^{G_n} in its place)
    // raw rows into LDS: q, k, c = b . k and log alpha (bf16) beside the x rows
    __bf16* rQ = tQ;
    __bf16* rK = tK;
    __bf16* rC = tC;
    __bf16* rL = gA;  // [64][DK], inside the (here unused) Gram and inverse arrays
    static_assert(L::oI - L::oA >= C * DK * 2, "log alpha rows need the Gram and inverse arrays");
    if (act) {
#pragma unroll
      for (int u = 0; u < TPS; ++u) {
        const int t = ts * TPS + u;
        float k[8], cc[8];
        load8f(reinterpret_cast<const bf16_t*>(&pk[u]), k);
        if (a.b_kind == kChannel) {
          load8f(reinterpret_cast<const bf16_t*>(&pb[u]), cc);
#pragma unroll
          for (int j = 0; j < 8; ++j) cc[j] *= k[j];
        } else {
          const float bs = a.b_kind == kScalar ? bf16_to_f32(pbs[u]) : 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) cc[j] = bs * k[j];
        }
        bf16x8 cb;
#pragma unroll
        for (int j = 0; j < 8; ++j) cb[j] = static_cast<__bf16>(cc[j]);
        *reinterpret_cast<uint4*>(rQ + t * LDT + d0) = pq[u];
        *reinterpret_cast<uint4*>(rK + t * LDT + d0) = pk[u];
        *reinterpret_cast<bf16x8*>(rC + t * LDT + d0) = cb;
        *reinterpret_cast<uint4*>(rL + t * DK + d0) = pl[u];
      }
    }
    lds_barrier();
    wyc_exact_chunk<DK, LDT, LDX, TWO>(a, cix, rQ, rK, rC, rL, tX, fEgr, tid);
    return;
  }

  // ---- operands: split Gram operands into LDS; Qhat, -Pbar^T, Kbar^T out to the workspace ----
  if (act) {
    float off[8], ref[8], eref[8], egr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      off[j] = segtot[ts * DK + d0 + j];
      ref[j] = fRef[d0 + j];
      eref[j] = fEref[d0 + j];
      egr[j] = fEgr[d0 + j];
    }
#pragma unroll
    for (int u = 0; u < TPS; ++u) {
      const int t = ts * TPS + u;
      float q[8], k[8], cc[8];
      load8f(reinterpret_cast<const bf16_t*>(&pq[u]), q);
      load8f(reinterpret_cast<const bf16_t*>(&pk[u]), k);
      if (a.b_kind == kChannel) {
        load8f(reinterpret_cast<const bf16_t*>(&pb[u]), cc);
#pragma unroll
        for (int j = 0; j < 8; ++j) cc[j] *= k[j];
      } else {
        const float bs = a.b_kind == kScalar ? bf16_to_f32(pbs[u]) : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) cc[j] = bs * k[j];
      }
      bf16x8 oq, oc, ok, op;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float G = G8[u][j] + off[j];
        const float eq = __expf(G - ref[j]);          // e^{G_t - G_ref}
        const float er = __builtin_amdgcn_rcpf(eq);   // e^{G_ref - G_t}
        oq[j] = static_cast<__bf16>(q[j] * eq);
        ok[j] = static_cast<__bf16>(k[j] * er);
        if (TWO) {
          const float ep = __expf(G - la8[u][j] - ref[j]);  // e^{G_{t-1} - G_ref}
          const float epr = __builtin_amdgcn_rcpf(ep);
          oc[j] = static_cast<__bf16>(cc[j] * ep);
          op[j] = static_cast<__bf16>(k[j] * epr);
        } else {
          oc[j] = static_cast<__bf16>(cc[j] * eq);
        }
      }
      *reinterpret_cast<bf16x8*>(tQ + t * LDT + d0) = oq;
      *reinterpret_cast<bf16x8*>(tC + t * LDT + d0) = oc;
      *reinterpret_cast<bf16x8*>(tK + t * LDT + d0) = ok;
      if (TWO) *reinterpret_cast<bf16x8*>(tP + t * LDT + d0) = op;
    }
  }
  // tiles above the diagonal of -M, L_K and M_QK are never written by the Gram phase but are
  // read as zero by the products below (the three arrays are contiguous)
  for (int i = tid; i < (L::oT - L::oM) / 4; i += NT) reinterpret_cast<uint32_t*>(gM)[i] = 0u;
  GDR_PMARK(1);
  lds_barrier();

  // ---- Gram tiles: 20 jobs = 2 row operands x 10 tile pairs, job wave + NW jj ----
  {
    constexpr int JPW = (20 + NW - 1) / NW;
    F8 fa[2][NKB], fb[2][NKB], fc[2][NKB];
    auto job_of = [&](int jj, int& grp, int& ta, int& tb) {
      const int job = wave + NW * jj;
      grp = job / 10;
      const int tix = job % 10;
      ta = tix >= 6 ? 3 : tix >= 3 ? 2 : tix >= 1 ? 1 : 0;
      tb = tix - ta * (ta + 1) / 2;
    };
    auto load_job = [&](int jj, int bsel) {
      int grp, ta, tb;
      job_of(jj, grp, ta, tb);
      const __bf16* ar = (grp == 0 ? tC : tQ) + (16 * ta + l16) * LDT;
      const __bf16* br = ((TWO && grp == 0) ? tP : tK) + (16 * tb + l16) * LDT;
      const __bf16* cr = (grp == 0 ? tK : tP) + (16 * tb + l16) * LDT;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        fa[bsel][kb] = lds_load8(ar + 32 * kb + 8 * g);
        fb[bsel][kb] = lds_load8(br + 32 * kb + 8 * g);
        if (TWO) fc[bsel][kb] = lds_load8(cr + 32 * kb + 8 * g);
      }
    };
    // which: 0 = L_P (strict; off-diagonal -> gA as -L, diagonal -> Ld), 1 = -M_QP (or -M),
    // 2 = L_K (strict), 3 = M_QK (inclusive)
    auto store_tile = [&](int which, int ta, int tb, const f32x4& acc) {
      const int r0 = 16 * ta + 4 * g, cc = 16 * tb + l16;
      if (ta > tb) {
        __bf16* dst = (which == 0 ? gA + (r0 - 16) * LDA : which == 1 ? gM + r0 * LDD
                       : which == 2 ? gLK + r0 * LDD : gMQK + r0 * LDD) + cc;
        const int pitch = which == 0 ? LDA : LDD;
        const float sgn = which <= 1 ? -1.f : 1.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i * pitch] = static_cast<__bf16>(acc[i] * sgn);
        return;
      }
      const bool strict = which == 0 || which == 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + i;
        const float val = (strict ? (cc < r) : (cc <= r)) ? acc[i] : 0.f;
        if (which == 0)
          Ld[(ta * 16 + (cc & 15)) * LDL + (r & 15)] = val;
        else if (which == 1)
          gM[r * LDD + cc] = static_cast<__bf16>(-val);
        else if (which == 2)
          gLK[r * LDD + cc] = static_cast<__bf16>(val);
        else
          gMQK[r * LDD + cc] = static_cast<__bf16>(val);
      }
    };
    load_job(0, 0);
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      if (wave + NW * jj >= 20) break;  // (uniform)
      const int cur = jj & 1;
      if (jj + 1 < JPW && wave + NW * (jj + 1) < 20) load_job(jj + 1, cur ^ 1);
      int grp, ta, tb;
      job_of(jj, grp, ta, tb);
      f32x4 acc1 = zero4(), acc2 = zero4();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        acc1 = MM::mma8(fa[cur][kb], fb[cur][kb], acc1);
        if (TWO) acc2 = MM::mma8(fa[cur][kb], fc[cur][kb], acc2);
      }
      if (TWO) {
        store_tile(grp == 0 ? 0 : 3, ta, tb, acc1);
        store_tile(grp == 0 ? 2 : 1, ta, tb, acc2);
      } else {
        store_tile(grp == 0 ? 0 : 1, ta, tb, acc1);
      }
    }
  }
  GDR_PMARK(2);
  lds_barrier();

  // ---- diagonal inverses (waves 0-1) ----
  if (wave < 2 && lane < 32) wy_diag_inverses<LDL, LDI>(Ld, dInv, wave, lane, l16);
  GDR_PMARK(3);
  lds_barrier();

  // ---- T = (I + L_P)^{-1}: wave j < 4 solves column block j on the identity ----
  if (wave < 4) {
    const int j = wave;
    bf16x4 af[6], tf[4];
#pragma unroll
    for (int i = 0, n = 0; i < 4; ++i) {
      tf[i] = lds_load4(dInv + (16 * i + l16) * LDI + 4 * g);
#pragma unroll
      for (int m = 0; m < i; ++m, ++n) af[n] = lds_load4(gA + (16 * i - 16 + l16) * LDA + 16 * m + 4 * g);
    }
    f32x4 R[4];
#pragma unroll
    for (int i = 0, n = 0; i < 4; ++i) {
      f32x4 acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = (i == j && 4 * g + e == l16) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m, ++n)
        if (m >= j) acc = MM::mma4(af[n], acc_frag4<__bf16>(R[m]), acc);
      R[i] = i < j ? zero4() : MM::mma4(tf[i], acc_frag4<__bf16>(acc), zero4());
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) tT[(16 * i + 4 * g + e) * LDD + 16 * j + l16] = static_cast<__bf16>(R[i][e]);
  }
  GDR_PMARK(4);
  lds_barrier();

  // ---- the affine chunk map ----
  // B fragments of T^T (and of L_K^T, M_QK^T, -M^T) are pair fragments of the rows of T (L_K,
  // M_QK, -M); every column tile below is one wave's, kept in registers from product to product.
  auto row_frags = [&](const __bf16* m, F8* f) {  // 6 fragments: lower-triangular 64 x 64
#pragma unroll
    for (int ta = 0, n = 0; ta < 4; ++ta) {
      f[n++] = lds_pair_frag_k<C>(m + (16 * ta + l16) * LDD, 0, g);
      if (ta >= 2) f[n++] = lds_pair_frag_k<C>(m + (16 * ta + l16) * LDD, 32, g);
    }
  };
  // column tile of a token-major LDS array as A (or B) fragments: 8 tokens (tile-pair order) of
  // column col per lane (two transposing reads per 32-token block: source lane
  // (a, m) = (l16 & 3, l16 >> 2) of group g points at token 32 ks + 16 h + 4 g + m, columns
  // col - l16 + 4 a ..)
  auto col_frags = [&](const __bf16* base, int pitch, int col, F8* f) {
    const int c0 = col - l16 + 4 * (l16 & 3), m_ = l16 >> 2;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x4 v = lds_read_tr4(reinterpret_cast<const unsigned char*>(
            base + (32 * ks + 16 * h + 4 * g + m_) * pitch + c0));
#pragma unroll
        for (int e = 0; e < 4; ++e) f[ks][4 * h + e] = v[e];
      }
  };

  // D^T tiles of (lower-triangular 64 x 64 B-side matrix) x (A-side 64 x 16 tile): out[ta] lane
  // holds D[token 16 ta + l16][column 4 g + i]
  auto tr_product = [&](const F8* af, const F8* bf, f32x4* out, bool acc) {
#pragma unroll
    for (int ta = 0, n = 0; ta < 4; ++ta) {
      out[ta] = MM::mma8(af[0], bf[n++], acc ? out[ta] : zero4());
      if (ta >= 2) out[ta] = MM::mma8(af[1], bf[n++], out[ta]);
    }
  };
  // upright tiles of (lower-triangular 64 x 64 A-side matrix) x (64 x 16 B-side tile), as the
  // two pair fragments (tokens as k) of the product: lane holds tokens 32 ks + 4 g + (e & 3) +
  // 16 (e >> 2) of column l16, times sgn (a factor of that column)
  auto up_frags = [&](const F8* af, const F8* bf, float sgn, F8* out) {
    f32x4 D[4];
#pragma unroll
    for (int ta = 0, n = 0; ta < 4; ++ta) {
      D[ta] = MM::mma8(af[n++], bf[0], zero4());
      if (ta >= 2) D[ta] = MM::mma8(af[n++], bf[1], D[ta]);
    }
#pragma unroll
    for (int ta = 0; ta < 4; ++ta)
#pragma unroll
      for (int i = 0; i < 4; ++i) D[ta][i] *= sgn;
    out[0] = acc_pair_frag<__bf16>(D[0], D[1]);
    out[1] = acc_pair_frag<__bf16>(D[2], D[3]);
  };
  auto store4 = [&](__bf16* dst, const f32x4& v) {
    bf16x4 ob;
#pragma unroll
    for (int i = 0; i < 4; ++i) ob[i] = static_cast<__bf16>(v[i]);
    *reinterpret_cast<bf16x4*>(dst) = ob;
  };
  {
    // (1) this wave's W column tiles (W = T Chat, the split Chat times e^{G_ref} per channel) as
    //     pair fragments, and Q' = Qhat - M W from them: lane holds Q'[16 ta + l16][16 ct + 4 g + i]
    //     (Qhat = split Q times e^{G_ref})
    // (2) this wave's value column tiles X and Y = T L_K X (MODE 1: -T X) as pair fragments, and
    //     Z' = M_QK X - M Y: lane holds Z'[16 ta + l16][16 cv + 4 g + i]
    // (3) channel tile by channel tile, Phat (MODE 1: Khat) and Khat with channels as rows, then
    //     A' = -Pbar^T W:          lane holds A'[16 tl + l16][16 ct + 4 g + i]
    //     D = Kbar^T X - Pbar^T Y: lane holds D[16 tl + 4 g + i][16 cv + l16], i.e. row 16 cv + l16
    //                              of D^T, four consecutive channels
    constexpr int WPW = (NTD + NW - 1) / NW;        // W tiles per wave (at most)
    constexpr int VPW = (DVP / 16 + NW - 1) / NW;   // value tiles per wave (at most)
    const int nct_u = static_cast<int>(DV / 16);
    F8 wf[WPW][2], xf[VPW][2], yf[VPW][2];
    {
      F8 tfr[6], mnf[6];
      row_frags(tT, tfr);
      row_frags(gM, mnf);
      __bf16* Qo = a.Qd + cix * C * DK;
#pragma unroll
      for (int w = 0; w < WPW; ++w) {
        const int ct = wave + NW * w;
        if (ct < NTD) {
          const int col = 16 * ct + l16;
          F8 cf[2];
          col_frags(tC, LDT, col, cf);
          up_frags(tfr, cf, fEref[col], wf[w]);
          f32x4 Qt[4];
          tr_product(wf[w], mnf, Qt, false);
          const float4 er = *reinterpret_cast<const float4*>(fEref + 16 * ct + 4 * g);
#pragma unroll
          for (int ta = 0; ta < 4; ++ta) {
            const bf16x4 q4 = *reinterpret_cast<const bf16x4*>(tQ + (16 * ta + l16) * LDT + 16 * ct + 4 * g);
            Qt[ta][0] += static_cast<float>(q4[0]) * er.x;
            Qt[ta][1] += static_cast<float>(q4[1]) * er.y;
            Qt[ta][2] += static_cast<float>(q4[2]) * er.z;
            Qt[ta][3] += static_cast<float>(q4[3]) * er.w;
            store4(Qo + tiled16(16 * ta + l16, 16 * ct + 4 * g, DK), Qt[ta]);
          }
        }
      }
      GDR_PMARK(6);
      F8 lkf[6], mqf[6];
      if (TWO) {
        row_frags(gLK, lkf);
        row_frags(gMQK, mqf);
      }
      __bf16* Zo = a.Zd + cix * C * DV;
#pragma unroll
      for (int w = 0; w < VPW; ++w) {
        const int cv = wave + NW * w;
        if (cv < nct_u) {
          col_frags(tX, LDX, 16 * cv + l16, xf[w]);
          if (TWO) {
            F8 lf[2];
            up_frags(lkf, xf[w], 1.f, lf);
            up_frags(tfr, lf, 1.f, yf[w]);
          } else {
            up_frags(tfr, xf[w], -1.f, yf[w]);
          }
          f32x4 Zt[4];
          tr_product(yf[w], mnf, Zt, false);
          if (TWO) tr_product(xf[w], mqf, Zt, true);
#pragma unroll
          for (int ta = 0; ta < 4; ++ta) store4(Zo + tiled16(16 * ta + l16, 16 * cv + 4 * g, DV), Zt[ta]);
        }
      }
    }
    GDR_PMARK(7);
    __bf16* Ao = a.Ad + cix * DK * DK;
    __bf16* Do = a.Dt + cix * DV * DK;
    const __bf16* pn_src = TWO ? tP : tK;
#pragma unroll 2
    for (int tl = 0; tl < NTD; ++tl) {
      // the split rows as they are; their per-channel factor e^{G_n - G_ref} scales the rows of
      // A' and D afterwards (lane: channel 16 tl + l16 of A', 16 tl + 4 g + i of D)
      F8 pf[2], kf[2];
      col_frags(pn_src, LDT, 16 * tl + l16, pf);
      if (TWO) col_frags(tK, LDT, 16 * tl + l16, kf);
      f32x4 acc[WPW + VPW];
      const float fa = -fEgr[16 * tl + l16];
      const float4 fd = *reinterpret_cast<const float4*>(fEgr + 16 * tl + 4 * g);
#pragma unroll
      for (int w = 0; w < WPW; ++w) {
        acc[w] = MM::mma8(wf[w][0], pf[0], zero4());
        acc[w] = MM::mma8(wf[w][1], pf[1], acc[w]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[w][i] *= fa;
      }
#pragma unroll
      for (int w = 0; w < VPW; ++w) {
        f32x4& d = acc[WPW + w];
        d = MM::mma8(pf[0], yf[w][0], zero4());
        d = MM::mma8(pf[1], yf[w][1], d);
        if (TWO) {  // Khat^T X - Phat^T Y
          f32x4 dk = MM::mma8(kf[0], xf[w][0], zero4());
          dk = MM::mma8(kf[1], xf[w][1], dk);
#pragma unroll
          for (int i = 0; i < 4; ++i) d[i] = dk[i] - d[i];
        } else {  // -Khat^T Y
#pragma unroll
          for (int i = 0; i < 4; ++i) d[i] = -d[i];
        }
        d[0] *= fd.x;
        d[1] *= fd.y;
        d[2] *= fd.z;
        d[3] *= fd.w;
      }
#pragma unroll
      for (int w = 0; w < WPW; ++w) {
        const int ct = wave + NW * w;
        if (ct < NTD) store4(Ao + tiled16(16 * tl + l16, 16 * ct + 4 * g, DK), acc[w]);
      }
#pragma unroll
      for (int w = 0; w < VPW; ++w) {
        const int cv = wave + NW * w;
        if (cv < nct_u) store4(Do + tiled16(16 * cv + l16, 16 * tl + 4 * g, DK), acc[WPW + w]);
      }
    }
  }
  GDR_PMARK(5);
}

// ------------------------------------------------------------------ no erase gate

// Per-channel decay without an erase gate (b = 0: gated linear attention): T = I, W = Y = 0 and
// A' = 0, so the chunk map is Q' = Qhat, D = Kbar^T X and Z' = M X with M = tril(Qhat Khat^T)
// (either order of the missing erase and the decay gives the same recurrence).  One Gram product
// per chunk and no solve.  A chunk whose prefix sums span too far for the split Gram forms D and
// Z' token by token instead (Q' = q e^{G_t} never overflows and is formed the same way for every
// chunk).  256 threads.
template <int DK, int DVP>
struct WygPrepLayout {
  static constexpr int C = 64;
  static constexpr int LDT = DK + 8;
  static constexpr int LDX = DVP + 8;
  static constexpr int LDD = C + 8;
  static constexpr int NCG = DK / 8;
  static constexpr int NSEG = (256 / NCG) < C ? (256 / NCG) : C;
  static constexpr int TPS = C / NSEG;
  static constexpr int oQ = 0;                     // split Qhat [64][LDT] (flagged: q rows)
  static constexpr int oK = oQ + C * LDT * 2;      // split Khat [64][LDT] (flagged: k rows)
  static constexpr int oX = oK + C * LDT * 2;      // X rows [64][LDX]
  static constexpr int oM = oX + C * LDX * 2;      // M [64][LDD] (flagged: log alpha rows [64][DK], with the next)
  static constexpr int oSEG = oM + C * LDD * 2;    // fp32 segment sums [NSEG][DK]
  static constexpr int oF = oSEG + NSEG * DK * 4;  // fp32 G_ref, e^{G_ref}, e^{G_n - G_ref} [DK] each; flag
  static constexpr int total = oF + (3 * DK + 4) * 4;
  static constexpr bool fits = total <= kLdsLimit;
  static_assert(oF - oM >= C * DK * 2, "log alpha rows of a flagged chunk need the M and segment arrays");
};

template <int DK, int DVP>
__global__ __launch_bounds__(256) void wyg_prep_kernel(WycArgs a) {
  using L = WygPrepLayout<DK, DVP>;
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  static_assert(L::fits, "LDS layout exceeds the gfx950 workgroup limit");
  static_assert(DK % 32 == 0, "dk must be a multiple of 32");
  constexpr int C = L::C, LDT = L::LDT, LDX = L::LDX, LDD = L::LDD;
  constexpr int NCG = L::NCG, NSEG = L::NSEG, TPS = L::TPS, NKB = DK / 32, NTD = DK / 16;

  __shared__ __attribute__((aligned(32))) unsigned char smem[L::total];
  __bf16* tQ = reinterpret_cast<__bf16*>(smem + L::oQ);
  __bf16* tK = reinterpret_cast<__bf16*>(smem + L::oK);
  __bf16* tX = reinterpret_cast<__bf16*>(smem + L::oX);
  __bf16* gM = reinterpret_cast<__bf16*>(smem + L::oM);
  float* segtot = reinterpret_cast<float*>(smem + L::oSEG);
  float* fRef = reinterpret_cast<float*>(smem + L::oF);
  float* fEref = fRef + DK;
  float* fEgr = fRef + 2 * DK;  // e^{G_n - G_ref}
  int* sFlag = reinterpret_cast<int*>(fRef + 3 * DK);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int64_t nch = a.nch, DV = a.DV, H = a.H;
  const int64_t bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int64_t bi = bh / H, hi = bh % H;
  const int64_t t0 = c * C;
  const int64_t rr = (bi * a.T + t0) * H + hi;
  const int64_t left = a.T - t0;
  const int64_t cix = bh * nch + c;
  const int ts = tid / NCG, d0 = (tid % NCG) * 8;
  const bool act = ts < NSEG;

  // ---- loads: every load first; out-of-range rows and absent gate kinds read zero ----
  const uint32_t oob = 0x80000000u;
  const uint32_t hdk = static_cast<uint32_t>(H * DK * 2), hdv = static_cast<uint32_t>(H * DV * 2);
  const uint32_t h1 = static_cast<uint32_t>(H * 2);
  const uint32_t hqk = static_cast<uint32_t>(a.Hk * DK * 2);
  const int64_t rqk = (bi * a.T + t0) * a.Hk + hi / (H / a.Hk);
  const auto rq = make_rsrc(a.q + rqk * DK, wy_range(left, a.Hk, DK));
  const auto rk = make_rsrc(a.k + rqk * DK, wy_range(left, a.Hk, DK));
  const auto rla = make_rsrc(a.la + rr * DK, wy_range(left, H, DK));
  const auto rv = make_rsrc(a.v + rr * DV, wy_range(left, H, DV));
  const auto rwc = make_rsrc(a.w_kind == kChannel ? a.wg + rr * DV : a.v, a.w_kind == kChannel ? wy_range(left, H, DV) : 0u);
  const auto rws = make_rsrc(a.w_kind == kScalar ? a.wg + rr : a.v, a.w_kind == kScalar ? wy_range(left, H, 1) : 0u);
  uint4 pq[TPS], pk[TPS], pl[TPS];
#pragma unroll
  for (int u = 0; u < TPS; ++u) {
    const uint32_t t = ts * TPS + u;
    pq[u] = buf_load16(rq, act ? t * hqk + d0 * 2 : oob);
    pk[u] = buf_load16(rk, act ? t * hqk + d0 * 2 : oob);
    pl[u] = buf_load16(rla, act ? t * hdk + d0 * 2 : oob);
  }
  constexpr int XPT = C * (DVP / 8) / 256;
  const int nxg = static_cast<int>(DV / 8);
  uint4 pv[XPT], pw[XPT];
  uint16_t pws[XPT];
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int item = tid + 256 * j;
    const bool in = item < C * nxg;
    const uint32_t t = in ? item / nxg : 0, xg = in ? item % nxg : 0;
    pv[j] = buf_load16(rv, in ? t * hdv + xg * 16 : oob);
    pw[j] = buf_load16(rwc, in ? t * hdv + xg * 16 : oob);
    pws[j] = buf_load_u16(rws, in ? t * h1 : oob);
  }

  // ---- gate prefix sums; X rows ----
  float G8[TPS][8];
  if (act) {
    float run[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < TPS; ++u) {
      float la8[8];
      load8f(reinterpret_cast<const bf16_t*>(&pl[u]), la8);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        run[j] += la8[j];
        G8[u][j] = run[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) segtot[ts * DK + d0 + j] = run[j];
  }
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int item = tid + 256 * j;
    if (item < C * nxg) {
      const int t = item / nxg, xg = item % nxg;
      float x[8];
      load8f(reinterpret_cast<const bf16_t*>(&pv[j]), x);
      if (a.w_kind == kChannel) {
        float w8[8];
        load8f(reinterpret_cast<const bf16_t*>(&pw[j]), w8);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= w8[e];
      } else if (a.w_kind == kScalar) {
        const float ws = bf16_to_f32(pws[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= ws;
      }
      bf16x8 xb;
#pragma unroll
      for (int e = 0; e < 8; ++e) xb[e] = static_cast<__bf16>(x[e]);
      *reinterpret_cast<bf16x8*>(tX + t * LDX + xg * 8) = xb;
    }
  }
  if (tid == 0) sFlag[0] = 0;
  lds_barrier();
  if (tid < DK) {
    float run = 0.f;
    for (int s = 0; s < NSEG; ++s) {
      const float tv = segtot[s * DK + tid];
      segtot[s * DK + tid] = run;
      run += tv;
    }
    const float ref = segtot[(NSEG / 2) * DK + tid];  // G_31
    fRef[tid] = ref;
    fEref[tid] = __expf(ref);
    fEgr[tid] = __expf(run - ref);
    a.Egn[cix * (DK + 4) + tid] = __expf(run);
    if (!(fabsf(ref) <= kWycSpanLimit && fabsf(run - ref) <= kWycSpanLimit)) sFlag[0] = 1;  // NaN, inf too
  }
  lds_barrier();
  const bool robust = sFlag[0] != 0;
  if (tid < 4) {
    reinterpret_cast<int*>(a.Egn + cix * (DK + 4) + DK)[tid] = tid == 0 && robust ? 1 : 0;
    if (tid == 0) a.flag[cix] = robust ? 1 : 0;
  }

  // ---- operands: Q' = q e^{G_t} straight out (tiled); split Qhat, Khat into LDS (flagged: raw
  // q, k and log alpha rows) ----
  if (act) {
    float off[8], ref[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      off[j] = segtot[ts * DK + d0 + j];
      ref[j] = fRef[d0 + j];
    }
#pragma unroll
    for (int u = 0; u < TPS; ++u) {
      const int t = ts * TPS + u;
      float q[8], k[8];
      load8f(reinterpret_cast<const bf16_t*>(&pq[u]), q);
      load8f(reinterpret_cast<const bf16_t*>(&pk[u]), k);
      bf16x8 oq, ok, oqp;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float G = G8[u][j] + off[j];
        oqp[j] = static_cast<__bf16>(q[j] * __expf(G));  // q e^{G_t}
        if (!robust) {
          const float eq = __expf(G - ref[j]);  // e^{G_t - G_ref}
          oq[j] = static_cast<__bf16>(q[j] * eq);
          ok[j] = static_cast<__bf16>(k[j] * __builtin_amdgcn_rcpf(eq));
        }
      }
      *reinterpret_cast<bf16x8*>(a.Qd + cix * C * DK + tiled16(t, d0, DK)) = oqp;
      if (robust) {
        *reinterpret_cast<uint4*>(tQ + t * LDT + d0) = pq[u];
        *reinterpret_cast<uint4*>(tK + t * LDT + d0) = pk[u];
      } else {
        *reinterpret_cast<bf16x8*>(tQ + t * LDT + d0) = oq;
        *reinterpret_cast<bf16x8*>(tK + t * LDT + d0) = ok;
      }
    }
  }
  // tiles above the diagonal of M are never written by the Gram phase but are read as zero
  if (!robust)
    for (int i = tid; i < C * LDD / 8; i += 256) reinterpret_cast<uint4*>(gM)[i] = make_uint4(0, 0, 0, 0);
  lds_barrier();  // (the raw log alpha rows of a flagged chunk overwrite the segment sums)
  if (robust) {
    __bf16* rL = gM;  // [64][DK] over the M and segment arrays
    if (act) {
#pragma unroll
      for (int u = 0; u < TPS; ++u) *reinterpret_cast<uint4*>(rL + (ts * TPS + u) * DK + d0) = pl[u];
    }
    lds_barrier();
    // D and Z' from the recurrence without erase, token by token in fp32: lane pairs of 64
    // channels each carry value column v of the state from zero
    constexpr int DH = DK / 2;
    const int hf = tid & 1, pr = tid >> 1, c0 = hf * DH;
    for (int v = pr; v < DV; v += 128) {
      float sv[DH];
#pragma unroll
      for (int i = 0; i < DH; ++i) sv[i] = 0.f;
      for (int t = 0; t < C; ++t) {
        const float x = static_cast<float>(tX[t * LDX + v]);
        float y = 0.f;
#pragma unroll
        for (int p = 0; p < DH / 8; ++p) {
          float k8[8], q8[8], l8[8];
          load8f(reinterpret_cast<const bf16_t*>(tK + t * LDT + c0 + 8 * p), k8);
          load8f(reinterpret_cast<const bf16_t*>(tQ + t * LDT + c0 + 8 * p), q8);
          load8f(reinterpret_cast<const bf16_t*>(rL + t * DK + c0 + 8 * p), l8);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float s_ = sv[8 * p + e] * __expf(l8[e]) + k8[e] * x;
            sv[8 * p + e] = s_;
            y += q8[e] * s_;
          }
        }
        y += __shfl_xor(y, 1);
        if (hf == 0) a.Zd[cix * C * DV + tiled16(t, v, DV)] = static_cast<__bf16>(y);
      }
      __bf16* Do = a.Dt + cix * DV * DK;
#pragma unroll
      for (int p = 0; p < DH / 8; ++p) {
        bf16x8 d8;
#pragma unroll
        for (int e = 0; e < 8; ++e) d8[e] = static_cast<__bf16>(sv[8 * p + e]);
        *reinterpret_cast<bf16x8*>(Do + tiled16(v, c0 + 8 * p, DK)) = d8;
      }
    }
    return;
  }

  // ---- M = tril(Qhat Khat^T): 10 tile pairs over the 4 waves ----
  for (int job = wave; job < 10; job += 4) {
    const int ta = job >= 6 ? 3 : job >= 3 ? 2 : job >= 1 ? 1 : 0, tb = job - ta * (ta + 1) / 2;
    const __bf16* ar = tQ + (16 * ta + l16) * LDT;
    const __bf16* br = tK + (16 * tb + l16) * LDT;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) acc = MM::mma8(lds_load8(ar + 32 * kb + 8 * g), lds_load8(br + 32 * kb + 8 * g), acc);
    const int r0 = 16 * ta + 4 * g, cc = 16 * tb + l16;
#pragma unroll
    for (int i = 0; i < 4; ++i) gM[(r0 + i) * LDD + cc] = static_cast<__bf16>(cc <= r0 + i ? acc[i] : 0.f);
  }
  lds_barrier();

  // ---- products per value column tile: Z' = M X (lane: Z'[16 ta + l16][16 cv + 4 g + i]) and
  // D = Kbar^T X = e^{G_n - G_ref} . (Khat^T X) (lane: D[16 tl + 4 g + i][16 cv + l16]) ----
  auto col_frags = [&](const __bf16* base, int pitch, int col, F8* f) {
    const int cx = col - l16 + 4 * (l16 & 3), m_ = l16 >> 2;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x4 v = lds_read_tr4(reinterpret_cast<const unsigned char*>(base + (32 * ks + 16 * h + 4 * g + m_) * pitch + cx));
#pragma unroll
        for (int e = 0; e < 4; ++e) f[ks][4 * h + e] = v[e];
      }
  };
  F8 mf[6];
#pragma unroll
  for (int ta = 0, n = 0; ta < 4; ++ta) {
    mf[n++] = lds_pair_frag_k<C>(gM + (16 * ta + l16) * LDD, 0, g);
    if (ta >= 2) mf[n++] = lds_pair_frag_k<C>(gM + (16 * ta + l16) * LDD, 32, g);
  }
  auto store4 = [&](__bf16* dst, const f32x4& v) {
    bf16x4 ob;
#pragma unroll
    for (int i = 0; i < 4; ++i) ob[i] = static_cast<__bf16>(v[i]);
    *reinterpret_cast<bf16x4*>(dst) = ob;
  };
  const int nct_u = static_cast<int>(DV / 16);
  __bf16* Zo = a.Zd + cix * C * DV;
  __bf16* Do = a.Dt + cix * DV * DK;
  for (int cv = wave; cv < nct_u; cv += 4) {
    F8 xf[2];
    col_frags(tX, LDX, 16 * cv + l16, xf);
#pragma unroll
    for (int ta = 0, n = 0; ta < 4; ++ta) {
      f32x4 z = MM::mma8(xf[0], mf[n++], zero4());
      if (ta >= 2) z = MM::mma8(xf[1], mf[n++], z);
      store4(Zo + tiled16(16 * ta + l16, 16 * cv + 4 * g, DV), z);
    }
#pragma unroll 2
    for (int tl = 0; tl < NTD; ++tl) {
      F8 kf[2];
      col_frags(tK, LDT, 16 * tl + l16, kf);
      f32x4 d = MM::mma8(kf[0], xf[0], zero4());
      d = MM::mma8(kf[1], xf[1], d);
      const float4 fd = *reinterpret_cast<const float4*>(fEgr + 16 * tl + 4 * g);
      d[0] *= fd.x;
      d[1] *= fd.y;
      d[2] *= fd.z;
      d[3] *= fd.w;
      store4(Do + tiled16(16 * cv + l16, 16 * tl + 4 * g, DK), d);
    }
  }
}

// ------------------------------------------------------------------ state kernel

// Direct-to-LDS copies of a tiled16 matrix into the swizzled row-major LDS form of DmaPlan
// (prefill_wy.h): LDS piece s holds piece (s mod NCHR) ^ key of row s / NCHR, fetched from its tile
// (tile rows `trs` bytes apart).  A lane's offsets repeat every P instructions (the key's row
// period, 16 or 32 rows, over the rows an instruction covers), shifted by whole tile rows.
template <int NCHR, bool PERM, int NPIECE>
struct TiledPlan {
  static_assert(NPIECE % 64 == 0, "whole instructions only");
  static constexpr int NI = NPIECE / 64;
  static constexpr int RPI = 64 / NCHR;  // rows per instruction
  static constexpr int PERIOD = NCHR == 16 ? (PERM ? 8 : 4) : NCHR == 8 ? (PERM ? 4 : 2) : NCHR == 4 ? (PERM ? 2 : 1) : 1;
  static constexpr int P = PERIOD < NI ? PERIOD : NI;
  uint32_t off[8];  // (a fixed bound: see DmaPlan)
  static_assert(P <= 8, "period above the fixed bound");
  __device__ __forceinline__ void init(uint32_t trs, int lane) {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int s = 64 * i + lane, row = s / NCHR, piece = (s % NCHR) ^ swz_key<NCHR, PERM>(row);
      off[i] = static_cast<uint32_t>(row >> 4) * trs + static_cast<uint32_t>(piece >> 1) * 512u +
               static_cast<uint32_t>(row & 15) * 32u + static_cast<uint32_t>(piece & 1) * 16u;
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, unsigned char* lds, uint32_t trs) const {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(lds + 1024 * i), 16, off[i % P],
          static_cast<int>(static_cast<uint32_t>(RPI * (i - i % P) / 16) * trs), 0, 0);
  }
};

// One chunk buffer: the chunk's affine map, rows in the swizzled form above (AZ: A' = 0, no slots).
template <int DK, int DVS, int NXW, bool AZ = false>
struct WycStateLayout {
  static constexpr int C = 64;
  static constexpr int NCQ = DK / 8;   // 16-byte pieces per row of dk channels
  static constexpr int NCU = DVS / 8;  // pieces per row of a value slice
  static constexpr int AS = DK * DK * 2;          // one A' slot [dk][dk], rows read in perm_row order
  // a chunk buffer (two of them)
  static constexpr int oQ = 0;                    // Q' [64][dk]
  static constexpr int oD = oQ + C * DK * 2;      // D^T slice [DVS][dk]
  static constexpr int oZ = oD + DVS * DK * 2;    // Z' slice [64][DVS]
  static constexpr int oE = oZ + C * DVS * 2;     // e^{G_n} [dk] fp32 (+ flag)
  static constexpr int BUF = oE + ((DK + 4) * 4 + 255) / 256 * 256;
  static constexpr int XW = DK / 64 * 1024;       // one wave's bf16 S half (its pair fragments, 16 bytes a lane)
  static constexpr int REST = 2 * BUF + C * DVS * 2 + 2 * NXW * XW;
  static constexpr int NA = AZ ? 0 : 3 * AS + REST <= kLdsLimit ? 3 : 2;  // A' slots
  static constexpr int oB = NA * AS;              // the two chunk buffers
  static constexpr int oO = oB + 2 * BUF;         // O rows of one chunk [64][DVS]
  static constexpr int oX = oO + C * DVS * 2;     // bf16 S halves exchanged: [2][NXW waves][XW]
  static constexpr int total = oX + 2 * NXW * XW;
  static constexpr bool fits = total <= kLdsLimit;
};

// s_waitcnt immediate that waits until at most n vector memory operations are outstanding
constexpr int wait_vmcnt(int n) { return 0x0F70 | (n & 0xF) | (((n >> 4) & 3) << 14); }

// Workgroup = 2 loader waves and NSW x SPLIT state waves for one state and a slice of DVS = 16 NSW
// value columns; state wave j holds columns 16 (j / SPLIT) .. + 15 of the slice and, with SPLIT = 2,
// only half of S's channels (rows): the S update needs all of bf16(S), so the two waves of a
// column group swap their bf16 halves through LDS once per chunk (written at the end of a
// chunk's products, read at the start of the next one's: barriers A and B lie between), and each
// takes half of O's token rows.  Chunk c's map sits in LDS
// buffer c mod 2, filled by direct-to-LDS loads that loader wave c mod 2 issues a whole chunk
// ahead.  Two barriers per chunk c:
//   up to A: the state waves compute, from S_b = bf16(S),
//              O = Q' S_b (+ Z' later),   S <- e^{G_n} . S + D + A' S_b;
//            loader wave c mod 2 copies the O rows of chunk c-1 from the O buffer to HBM;
//   A to B:  the state waves write O + Z' into the O buffer; loader wave c mod 2 refills buffer
//            c mod 2 with chunk c+2 and the other waits for its loads of chunk c+1.
// The state waves issue no global stores in the loop, and the loader wave that reads the O buffer
// has no loads in flight when it does.
// AZ (no erase gate: A' = 0): no A' copies or products, S <- e^{G_n} . S + D.
// (one workgroup per compute unit by its LDS: the scheduler may spend registers on latency)
template <int DK, int NSW, int SPLIT, bool AZ>
__global__ __launch_bounds__(64 * (2 + NSW * SPLIT)) __attribute__((amdgpu_waves_per_eu(1, 1))) void wyc_state_kernel(WycArgs a) {
  constexpr int DVS = 16 * NSW;
  using L = WycStateLayout<DK, DVS, SPLIT == 2 ? NSW * 2 : 0, AZ>;
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  static_assert(L::fits, "LDS layout exceeds the gfx950 workgroup limit");
  static_assert(DK % 32 == 0, "dk must be a multiple of 32");
  static_assert(SPLIT == 1 || (SPLIT == 2 && DK >= 64), "rows split in halves of whole k-steps");
  constexpr int C = L::C, NCQ = L::NCQ, NCU = L::NCU;
  constexpr int NTD = DK / 16, NKB = DK / 32;
  constexpr int NTH = NTD / SPLIT, NKH = NKB / SPLIT, NTA = 4 / SPLIT;  // this wave's tiles, k-steps, O tiles

  __shared__ __attribute__((aligned(1024))) unsigned char smem[L::total];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const bool loader = wave < 2;
  const int sw = loader ? 0 : wave - 2;         // state wave index
  const int cb = 16 * (sw / SPLIT);             // its first column in the slice
  const int rh = sw % SPLIT;                    // its half of the channels (rows): tiles rh NTH ..

  const int64_t nb = gridDim.x, bid = blockIdx.x;
  const int64_t p = (nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
  const int64_t bh = p / a.nsl;
  const int sl = static_cast<int>(p % a.nsl);
  const int64_t bi = bh / a.H, hi = bh % a.H;
  const int64_t DV = a.DV, H = a.H, T = a.T, nch = a.nch;
  const int64_t col0 = static_cast<int64_t>(sl) * DVS;
  const uint32_t hdv = static_cast<uint32_t>(H * DV * 2);

  auto buf = [&](int64_t c) -> unsigned char* { return smem + L::oB + (c & 1) * L::BUF; };
  auto aslot = [&](int64_t c) -> unsigned char* { return smem + (AZ ? 0 : (c % L::NA) * L::AS); };
  __bf16* oO = reinterpret_cast<__bf16*>(smem + L::oO);

  // ---------------- loader waves ----------------
  TiledPlan<NCQ, true, DK * NCQ> plA;
  TiledPlan<NCQ, false, C * NCQ> plQ;
  TiledPlan<NCQ, false, DVS * NCQ> plD;
  TiledPlan<NCU, false, C * NCU> plZ;
  const uint32_t tq = DK / 16 * 512, tu = static_cast<uint32_t>(DV / 16 * 512);  // tile row strides
  {
    const int dl = tid & 63;
    plA.init(tq, dl);
    plQ.init(tq, dl);
    plD.init(tq, dl);
    plZ.init(tu, dl);
  }
  // a chunk's copies in two parts: dma_b (A', half the bytes, into its own slot) and dma_a (the
  // rest, into the chunk buffer); see the pipeline below
  auto dma_b = [&](int64_t c) {
    const int64_t cix = bh * nch + c;
    plA.issue(make_rsrc(a.Ad + cix * DK * DK, DK * DK * 2), aslot(c), tq);
  };
  auto dma_a = [&](int64_t c) {
    unsigned char* B = buf(c);
    const int64_t cix = bh * nch + c;
    plQ.issue(make_rsrc(a.Qd + cix * C * DK, C * DK * 2), B + L::oQ, tq);
    // the slice's rows of D^T are whole tile rows; its columns of Z' start at tile column col0 / 16
    plD.issue(make_rsrc(a.Dt + cix * DV * DK + col0 * DK, DVS * DK * 2), B + L::oD, tq);
    plZ.issue(make_rsrc(a.Zd + cix * C * DV + col0 * 16, static_cast<uint32_t>((C * DV - col0 * 16) * 2)),
              B + L::oZ, tu);
    if (lane < (DK + 4) / 4) lds_dma16(make_rsrc(a.Egn + cix * (DK + 4), (DK + 4) * 4), B + L::oE, lane * 16);
  };
  // O rows of chunk c from the O buffer to HBM, 16 bytes per store; rows past the last token are
  // dropped by the range
  auto store_o = [&](int64_t c) {
    const int64_t t0 = c * C;
    const int64_t rr = (bi * T + t0) * H + hi;
    const int64_t bytes = ((T - t0 - 1) * H + 1) * DV * 2 - col0 * 2;
    const auto ro = make_rsrc(a.o + rr * DV + col0, static_cast<uint32_t>(bytes < 0x7fffffff ? bytes : 0x7fffffff));
#pragma unroll
    for (int j = 0; j < C * NCU / 64; ++j) {
      const int item = lane + 64 * j, t = item / NCU, part = item % NCU;
      buf_store16(ro, t * hdv + part * 16, *reinterpret_cast<const uint4*>(oO + t * DVS + part * 8));
    }
  };

  // ---------------- state waves ----------------
  // S[u] (u = tl - rh NTH): accumulator row 4 g + i holds channel perm_row(tl, 4 g + i) of column
  // cb + l16, so that the pair fragment of tiles 2 kb, 2 kb + 1 carries channels 32 kb + 8 g ..
  // 32 kb + 8 g + 7 (k-steps rh NKH .. are this wave's own)
  f32x4 S[NTH];
#pragma unroll
  for (int u = 0; u < NTH; ++u) {
    S[u] = zero4();
    if (!loader && a.S0 != nullptr) {
      const int64_t sb = bh * DK * DV + col0 + cb + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) S[u][i] = a.S0[sb + (int64_t)perm_row(rh * NTH + u, 4 * g + i) * DV];
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // this wave's bf16 S half into exchange slot `slot` (SPLIT = 2), as its pair fragments
  F8 sown[NKH];
  auto make_own = [&]() {
#pragma unroll
    for (int h = 0; h < NKH; ++h) sown[h] = acc_pair_frag<__bf16>(S[2 * h], S[2 * h + 1]);
  };
  auto put_own = [&](int slot) {
    if constexpr (SPLIT == 2) {
      unsigned char* X = smem + L::oX + (slot * NSW * 2 + sw) * L::XW;
#pragma unroll
      for (int h = 0; h < NKH; ++h) *reinterpret_cast<F8*>(X + h * 1024 + lane * 16) = sown[h];
    }
  };
  if (!loader) {
    make_own();
    put_own(0);
  }

  // Operands (one 16-byte read each): A' rows perm_row(tl, l16) (S's channel order) and Q' rows
  // 16 ta + l16, channels 32 kb + 8 g ..;  D^T row cb + l16 and e^{G_n} at this lane's channels;
  // Z' row 16 ta + l16, columns cb + 4 g ..
  f32x4 Ot[NTA];
  bf16x4 zv[NTA];
  auto compute = [&](int64_t c) {
    const unsigned char* B = buf(c);
    const unsigned char* A = aslot(c);
    // fragments of k-step kb in ring slot kb mod 3, read two k-steps ahead of their products
    constexpr int NR = NKB < 3 ? NKB : 3;
    F8 fa[NR][NTH], fq[NR][NTA];
    auto read_k = [&](int kb, int r) {
      if constexpr (!AZ)
#pragma unroll
        for (int u = 0; u < NTH; ++u) fa[r][u] = lds_piece<NCQ, true>(A, perm_row(rh * NTH + u, l16), 4 * kb + g);
#pragma unroll
      for (int t = 0; t < NTA; ++t) fq[r][t] = lds_piece<NCQ, false>(B + L::oQ, 16 * (rh * NTA + t) + l16, 4 * kb + g);
    };
    read_k(0, 0);
    if (NKB > 1) read_k(1, 1);
    // bf16(S) for every k-step: this wave's own, and the other half from its partner
    F8 sf[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (kb / NKH == rh) {
        sf[kb] = sown[kb % NKH];
      } else if constexpr (SPLIT == 2) {
        const unsigned char* X = smem + L::oX + ((int)(c & 1) * NSW * 2 + (sw ^ 1)) * L::XW;
        sf[kb] = *reinterpret_cast<const F8*>(X + (kb % NKH) * 1024 + lane * 16);
      }
    }
    const float* E = reinterpret_cast<const float*>(B + L::oE);
    float4 e4[NTH];
    bf16x4 d4[NTH];
#pragma unroll
    for (int u = 0; u < NTH; ++u) {
      const int tl = rh * NTH + u;
      e4[u] = *reinterpret_cast<const float4*>(E + perm_row(tl, 4 * g));
      d4[u] = *reinterpret_cast<const bf16x4*>(swz_addr<NCQ, false>(B + L::oD, cb + l16, 4 * (tl >> 1) + g) + 8 * (tl & 1));
    }
#pragma unroll
    for (int u = 0; u < NTH; ++u) {
      S[u][0] = S[u][0] * e4[u].x + static_cast<float>(d4[u][0]);
      S[u][1] = S[u][1] * e4[u].y + static_cast<float>(d4[u][1]);
      S[u][2] = S[u][2] * e4[u].z + static_cast<float>(d4[u][2]);
      S[u][3] = S[u][3] * e4[u].w + static_cast<float>(d4[u][3]);
    }
#pragma unroll
    for (int t = 0; t < NTA; ++t) Ot[t] = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (kb + 2 < NKB) read_k(kb + 2, (kb + 2) % NR);
      __builtin_amdgcn_sched_barrier(0);  // the reads stay ahead of this k-step's products
      if constexpr (!AZ)
#pragma unroll
        for (int u = 0; u < NTH; ++u) S[u] = MM::mma8(fa[kb % NR][u], sf[kb], S[u]);
#pragma unroll
      for (int t = 0; t < NTA; ++t) Ot[t] = MM::mma8(sf[kb], fq[kb % NR][t], Ot[t]);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int col = cb + 4 * g;
#pragma unroll
    for (int t = 0; t < NTA; ++t)
      zv[t] = *reinterpret_cast<const bf16x4*>(swz_addr<NCU, false>(B + L::oZ, 16 * (rh * NTA + t) + l16, col >> 3) + 8 * ((col >> 2) & 1));
    // the next chunk's bf16(S), this wave's half, for both waves of the pair
    make_own();
    put_own(static_cast<int>((c + 1) & 1));
  };
  // Ot[t] lane (g, l16) holds O[16 ta + l16][cb + 4 g + i], ta = rh NTA + t
  auto write_o = [&]() {
#pragma unroll
    for (int t = 0; t < NTA; ++t) {
      bf16x4 ob;
#pragma unroll
      for (int i = 0; i < 4; ++i) ob[i] = static_cast<__bf16>(Ot[t][i] + static_cast<float>(zv[t][i]));
      *reinterpret_cast<bf16x4*>(oO + (16 * (rh * NTA + t) + l16) * DVS + cb + 4 * g) = ob;
    }
  };

  // ---------------- pipeline ----------------
  // Loader wave 0 issues every A' copy (dma_b), NA - 1 chunks ahead, while the state waves
  // compute (the slot of chunk c + NA - 1 held chunk c - 1, used before barrier A of chunk c - 1),
  // and between barriers A and B of chunk c waits until chunk c+1's copy is in.  Loader wave 1
  // issues the rest of chunk c+2 (dma_a) between barriers A and B of chunk c (its buffer is free
  // from A), and while chunk c computes waits for its copies of chunk c+1 and then copies the O
  // rows of chunk c-1 out.  Vector memory loads complete in order, so a wait for "at most n in
  // flight" covers every load older than the last n.
  constexpr int NIA = decltype(plA)::NI;
  if (nch > 0) {
    if (wave == 0) {
      dma_a(0);
      if constexpr (!AZ)
        for (int k = 0; k < L::NA - 1 && k < nch; ++k) dma_b(k);
    }
    if (wave == 1 && nch > 1) dma_a(1);
    if (loader) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }
  lds_barrier();
  for (int64_t ch = 0; ch < nch; ++ch) {
    // opaque per chunk: keeps lane-dependent LDS addresses from being hoisted out of the loop
    asm volatile("" : "+v"(lane), "+v"(g), "+v"(l16));
    GDR_MARK(0);
    const bool ahead = !AZ && ch + L::NA - 1 < nch;  // wave 0 issues A' of chunk ch + NA - 1 now
    if (!loader) {
      compute(ch);
    } else if (wave == 0) {
      if (ahead) dma_b(ch + L::NA - 1);
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // its copies of chunk ch+1 (and older stores)
      if (ch > 0) store_o(ch - 1);
    }
    GDR_MARK(1);
    lds_barrier_keep_vm();  // A: buffer ch mod 2, A' slot ch mod NA and the O buffer are free
    GDR_MARK(2);
    if (!loader) {
      write_o();
    } else if (wave == 0) {
      // A' of chunk ch+1 in; only the A' copies issued after it may still be in flight
      if (ahead && L::NA == 3)
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(NIA));
      else
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    } else {
      if (ch + 2 < nch) dma_a(ch + 2);
    }
    GDR_MARK(3);
    lds_barrier_keep_vm();  // B: chunk ch+1 is in, O of chunk ch in the O buffer
    GDR_MARK(4);
  }
  if (wave == 1 && nch > 0) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    store_o(nch - 1);
  }

  if (!loader && a.S_T != nullptr) {
    const int64_t sb = bh * DK * DV + col0 + cb + l16;
#pragma unroll
    for (int u = 0; u < NTH; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.S_T[sb + (int64_t)perm_row(rh * NTH + u, 4 * g + i) * DV] = S[u][i];
  }
}

}  // namespace gdr
