// Chunkwise prefill for a scalar (or no) decay with a scalar (or no) erase gate, as two kernels:
// a chunk-local kernel that runs on every chunk of every state at once, and a state kernel that
// walks the chunks of each state in order and does only the work that depends on S.
//
// Chunk form (rank one per token; "Recurrent Memory: Write, Erase, Decay, Read", section 03 for
// the linear erase that reassociates over a chunk, section 04 for the decay as prefix sums G_t of
// log alpha).  With A[t,i] = beta_t (k_t . k_i) e^{G_t - G_i} for i < t, T = (I + A)^{-1},
// M[t,i] = (q_t . k_i) e^{G_t - G_i} for i <= t and X = w . v:
//     W = T diag(beta_t e^{G_t}) K,   U = T X                        (chunk-local: wy_prep_kernel)
//     R = W S - U,   O = diag(e^{G_t}) Q S - M R,
//     S' = e^{G_n} S - K^T diag(e^{G_n - G_t}) R                      (per state: wy_state_kernel)
// R stacks the erase reads r_t (the negated "new values" of the delta rule).  The pairwise mask
// e^{G_t - G_i} <= 1 makes every factor safe for any gate values.
//
// The chunk-local kernel writes W and U (bf16), -M (bf16) and G (fp32) to a workspace; the
// state kernel streams them back, so the serial chain per chunk holds only S-dependent MFMAs.
#pragma once
#include "gdr_common.h"
#include "mfma.h"
#include "prefill_kernel.h"
#include "prefill_scalar.h"

// Phase markers: no-ops unless a profiling build defines them.
#ifndef GDR_PMARK
#define GDR_PMARK(id) ((void)0)
#endif
#ifndef GDR_MARK
#define GDR_MARK(id) ((void)0)
#endif

namespace gdr {

struct WyArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* la;
  const bf16_t* bg;
  const bf16_t* wg;
  const float* S0;
  bf16_t* o;
  float* S_T;
  __bf16* W;  // [B*H][nch][64][dk]
  __bf16* U;  // [B*H][nch][64][dv]
  __bf16* M;  // [B*H][nch][64][64], holds -M (zero above the diagonal)
  float* G;   // [B*H][nch][64]
  int64_t T, H, DV, nch;
  int alpha_kind, b_kind, w_kind;
  int nsl;  // value slices per state (state kernel)
};

// Byte range of `width`-element rows from a chunk's first token to the last token of its state.
__device__ __forceinline__ uint32_t wy_range(int64_t left, int64_t H, int64_t width) {
  const int64_t bytes = ((left - 1) * H + 1) * width * 2;
  return static_cast<uint32_t>(bytes < 0x7fffffff ? bytes : 0x7fffffff);
}

// Inverses of the four 16x16 unit-lower-triangular diagonal blocks of (I + A), from their strict
// lower parts in Ld (fp32, column-major [4][16][LDL]).  Runs on lanes 0-31 of waves 0 and 1:
// lane (block, j) solves column j by a column sweep (once x_m is final, every later x_i drops
// L[i][m] x_m; column m+1 is read while column m is applied).
template <int LDL, int LDI>
__device__ __forceinline__ void wy_diag_inverses(const float* Ld, __bf16* dInv, int wave, int lane,
                                                 int l16) {
  const int blk = (lane < 16) ? (wave == 0 ? 0 : 1) : (wave == 0 ? 3 : 2);
  const int j = l16;
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
  float4 col[2][4];
  auto load_col = [&](int m, float4* cv) {
    const float* p = Ld + (blk * 16 + m) * LDL;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      if (4 * q4 + 3 > m) cv[q4] = *reinterpret_cast<const float4*>(p + 4 * q4);
  };
  load_col(0, col[0]);
#pragma unroll
  for (int m = 0; m < 15; ++m) {
    if (m + 1 < 15) load_col(m + 1, col[(m + 1) & 1]);
    const float* cv = reinterpret_cast<const float*>(col[m & 1]);
#pragma unroll
    for (int i = m + 1; i < 16; ++i) x[i] -= cv[i] * x[m];
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) dInv[(blk * 16 + i) * LDI + j] = static_cast<__bf16>(x[i]);
}

// ------------------------------------------------------------------ chunk-local kernel

template <int DK, int DVP>
struct WyPrepLayout {
  static constexpr int C = 64;
  static constexpr int LDT = DK + 8;   // q, k rows
  static constexpr int LDX = DVP + 8;  // x rows
  static constexpr int LDD = C + 8;    // M rows
  static constexpr int LDA = 48 + 8;   // packed off-diagonal blocks of -A: rows 16..63, cols 0..47
  static constexpr int LDI = 24;
  static constexpr int LDL = 20;
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + C * LDT * 2;
  static constexpr int oX = oK + C * LDT * 2;
  static constexpr int oA = oX + C * LDX * 2;
  static constexpr int oM = oA + 48 * LDA * 2;
  static constexpr int oI = oM + C * LDD * 2;
  static constexpr int oLD = oI + 4 * 16 * LDI * 2;
  static constexpr int oS = oLD + 4 * 16 * LDL * 4;  // fp32: G, e^G, -, beta (64 each)
  static constexpr int total = oS + 4 * C * 4;
  static constexpr bool fits = total <= kLdsLimit;
};

// One workgroup per (state, chunk).  Phases (barriers between): inputs into LDS and gate prefix
// sums; Gram tiles (waves 0-1: A, waves 2-3: M); diagonal inverses (waves 0-1) while waves 2-3
// write -M out; blocked forward substitution for the 16-column tiles of W and U, each wave
// owning whole column tiles (R_i = T_ii (B_i - sum_{m<i} A_im R_m), B the scaled k or x tile).
template <int DK, int DVP>
__global__ __launch_bounds__(256) void wy_prep_kernel(WyArgs a) {
  using L = WyPrepLayout<DK, DVP>;
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  static_assert(L::fits, "LDS layout exceeds the gfx950 workgroup limit");
  static_assert(DK % 32 == 0, "dk must be a multiple of 32");
  constexpr int C = L::C, LDT = L::LDT, LDX = L::LDX, LDD = L::LDD, LDA = L::LDA, LDI = L::LDI,
                LDL = L::LDL;
  constexpr int NCG = DK / 8, IPT = C * NCG / 256;

  __shared__ __attribute__((aligned(32))) unsigned char smem[L::total];
  __bf16* tQ = reinterpret_cast<__bf16*>(smem + L::oQ);
  __bf16* tK = reinterpret_cast<__bf16*>(smem + L::oK);
  __bf16* tX = reinterpret_cast<__bf16*>(smem + L::oX);
  __bf16* gA = reinterpret_cast<__bf16*>(smem + L::oA);
  __bf16* gM = reinterpret_cast<__bf16*>(smem + L::oM);
  __bf16* dInv = reinterpret_cast<__bf16*>(smem + L::oI);
  float* Ld = reinterpret_cast<float*>(smem + L::oLD);
  float* sc = reinterpret_cast<float*>(smem + L::oS);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int64_t nch = a.nch, DV = a.DV, H = a.H;
  const int64_t bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int64_t bi = bh / H, hi = bh % H;
  const int64_t t0 = c * C;
  const int64_t rr = (bi * a.T + t0) * H + hi;  // row of the chunk's first token
  const int64_t left = a.T - t0;
  const int64_t cix = bh * nch + c;             // chunk index in the workspace

  // inputs: rows past the last token read as zero (identity padding)
  const auto rq = make_rsrc(a.q + rr * DK, wy_range(left, H, DK));
  const auto rk = make_rsrc(a.k + rr * DK, wy_range(left, H, DK));
  const auto rv = make_rsrc(a.v + rr * DV, wy_range(left, H, DV));
  const uint32_t hdk = static_cast<uint32_t>(H * DK * 2), hdv = static_cast<uint32_t>(H * DV * 2);
  const uint32_t h1 = static_cast<uint32_t>(H * 2);

  // every global load is issued before the first use: out-of-range items get an offset past
  // the buffer range (zero) and absent gate kinds an empty range
  constexpr int XPT = C * (DVP / 8) / 256;  // x items per thread at the widest dv
  const int nxg = static_cast<int>(DV / 8);
  const uint32_t oob = 0x80000000u;
  const auto rwc = make_rsrc(a.w_kind == kChannel ? a.wg + rr * DV : a.v,
                             a.w_kind == kChannel ? wy_range(left, H, DV) : 0u);
  const auto rws = make_rsrc(a.w_kind == kScalar ? a.wg + rr : a.v,
                             a.w_kind == kScalar ? wy_range(left, H, 1) : 0u);
  const auto rla = make_rsrc(a.alpha_kind != kNone ? a.la + rr : a.q,
                             a.alpha_kind != kNone ? wy_range(left, H, 1) : 0u);
  const auto rb = make_rsrc(a.b_kind != kNone ? a.bg + rr : a.q,
                            a.b_kind != kNone ? wy_range(left, H, 1) : 0u);
  uint4 qv[IPT], kv[IPT], vv[XPT], wv[XPT];
  uint16_t wsv[XPT];
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int item = tid + 256 * j;
    const uint32_t t = item / NCG, cg = item % NCG;
    qv[j] = buf_load16(rq, t * hdk + cg * 16);
    kv[j] = buf_load16(rk, t * hdk + cg * 16);
  }
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int item = tid + 256 * j;
    const bool in = item < C * nxg;
    const uint32_t t = in ? item / nxg : 0, xg = in ? item % nxg : 0;
    vv[j] = buf_load16(rv, in ? t * hdv + xg * 16 : oob);
    wv[j] = buf_load16(rwc, in ? t * hdv + xg * 16 : oob);
    wsv[j] = buf_load_u16(rws, in ? t * h1 : oob);
  }
  const uint16_t lav = buf_load_u16(rla, lane * h1), bev = buf_load_u16(rb, lane * h1);

  // M tiles above the diagonal are never written and must read as zero
  for (int i = tid; i < C * LDD / 2; i += 256) reinterpret_cast<uint32_t*>(gM)[i] = 0u;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int item = tid + 256 * j;
    const uint32_t t = item / NCG, cg = item % NCG;
    *reinterpret_cast<uint4*>(tQ + t * LDT + cg * 8) = qv[j];
    *reinterpret_cast<uint4*>(tK + t * LDT + cg * 8) = kv[j];
  }
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int item = tid + 256 * j;
    if (item < C * nxg) {
      const int t = item / nxg, xg = item % nxg;
      float x[8];
      load8f(reinterpret_cast<const bf16_t*>(&vv[j]), x);
      if (a.w_kind == kChannel) {
        float w8[8];
        load8f(reinterpret_cast<const bf16_t*>(&wv[j]), w8);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= w8[e];
      } else if (a.w_kind == kScalar) {
        const float ws = bf16_to_f32(wsv[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= ws;
      }
      bf16x8 xb;
#pragma unroll
      for (int e = 0; e < 8; ++e) xb[e] = static_cast<__bf16>(x[e]);
      *reinterpret_cast<bf16x8*>(tX + t * LDX + xg * 8) = xb;
    }
  }
  if (wave == 0) {
    // per-token scalars: G_t (inclusive prefix of log alpha), e^{G_t}, beta_t
    float x = bf16_to_f32(lav);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    sc[lane] = x;
    sc[C + lane] = __expf(x);
    sc[3 * C + lane] = bf16_to_f32(bev);
    a.G[cix * C + lane] = x;
  }
  GDR_PMARK(0);
  lds_barrier();

  // Gram tiles: waves 0-1 A (solve, with the fp32 diagonal blocks to Ld), waves 2-3 M
  {
    const int prod = wave >> 1;
    const __bf16* rows = prod == 0 ? tK : tQ;
    if (wave & 1)
      scalar_gram_pair<DK, 1, 2, LDT, LDD, LDA, LDL>(rows, tK, prod, g, l16, sc, gA, gM, Ld);
    else
      scalar_gram_pair<DK, 0, 3, LDT, LDD, LDA, LDL>(rows, tK, prod, g, l16, sc, gA, gM, Ld);
  }
  GDR_PMARK(1);
  lds_barrier();

  if (wave < 2) {
    if (lane < 32) wy_diag_inverses<LDL, LDI>(Ld, dInv, wave, lane, l16);
  } else {
    // -M out: 64 rows of 128 bytes, 16 bytes per item
    __bf16* Mo = a.M + cix * C * C;
    for (int item = tid - 128; item < C * 8; item += 128) {
      const int r = item >> 3, part = item & 7;
      *reinterpret_cast<uint4*>(Mo + r * C + part * 8) =
          *reinterpret_cast<const uint4*>(gM + r * LDD + part * 8);
    }
  }
  GDR_PMARK(2);
  lds_barrier();

  // T = (I + A)^{-1}: wave j solves column block j by blocked forward substitution on the
  // identity (T_jj, then T_ij = -T_ii sum_{j<=m<i} A_im T_mj), as bf16 into the M array,
  // which has been written out above and has T's shape
  {
    __bf16* tT = gM;
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
  lds_barrier();

  // W = T diag(beta e^G) K and U = T X, one 16-column tile at a time (no chain: T is known).
  // B fragments gather 8 tokens of one column (tile-pair order); the result overwrites the
  // same columns (each wave owns whole column tiles), to be written out coalesced below.
  {
    const __bf16* tT = gM;
    F8 tf[6];
#pragma unroll
    for (int ta = 0, n = 0; ta < 4; ++ta) {
      tf[n++] = lds_pair_frag_k<C>(tT + (16 * ta + l16) * LDD, 0, g);
      if (ta >= 2) tf[n++] = lds_pair_frag_k<C>(tT + (16 * ta + l16) * LDD, 32, g);
    }
    float sw[2][8];  // beta_t e^{G_t} of the tokens of this lane's B fragments
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = 32 * ks + 4 * g + (e & 3) + (e >> 2) * 16;
        sw[ks][e] = sc[3 * C + t] * sc[C + t];
      }
    auto gemm_tile = [&](__bf16* base, int pitch, int col, bool scale) {
      F8 bf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = 32 * ks + 4 * g + (e & 3) + (e >> 2) * 16;
          const float x = static_cast<float>(base[t * pitch + col]);
          bf[ks][e] = static_cast<__bf16>(scale ? x * sw[ks][e] : x);
        }
      f32x4 D[4];
#pragma unroll
      for (int ta = 0, n = 0; ta < 4; ++ta) {
        D[ta] = MM::mma8(tf[n++], bf[0], zero4());
        if (ta >= 2) D[ta] = MM::mma8(tf[n++], bf[1], D[ta]);
      }
#pragma unroll
      for (int ta = 0; ta < 4; ++ta)
#pragma unroll
        for (int e = 0; e < 4; ++e) base[(16 * ta + 4 * g + e) * pitch + col] = static_cast<__bf16>(D[ta][e]);
    };
    // tile loops without a per-tile guard where the counts divide evenly over the four waves,
    // so that the loads of every tile of a wave are issued together
    if constexpr (DK / 16 % 4 == 0) {
#pragma unroll
      for (int r = 0; r < DK / 64; ++r) gemm_tile(tK, LDT, 16 * (wave + 4 * r) + l16, true);
    } else {
#pragma unroll
      for (int r = 0; r < (DK / 16 + 3) / 4; ++r) {
        const int ct = wave + 4 * r;
        if (ct < DK / 16) gemm_tile(tK, LDT, 16 * ct + l16, true);
      }
    }
    const int nct_u = static_cast<int>(DV / 16);
    if (nct_u == DVP / 16) {
#pragma unroll
      for (int r = 0; r < DVP / 64; ++r) gemm_tile(tX, LDX, 16 * (wave + 4 * r) + l16, false);
    } else {
#pragma unroll
      for (int r = 0; r < DVP / 64; ++r) {
        const int ct = wave + 4 * r;
        if (ct < nct_u) gemm_tile(tX, LDX, 16 * ct + l16, false);
      }
    }
  }
  GDR_PMARK(3);
  lds_barrier();

  // W and U out, 16 bytes per item
  {
    __bf16* Wo = a.W + cix * C * DK;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int item = tid + 256 * j;
      const int t = item / NCG, cg = item % NCG;
      *reinterpret_cast<uint4*>(Wo + t * DK + cg * 8) = *reinterpret_cast<const uint4*>(tK + t * LDT + cg * 8);
    }
    __bf16* Uo = a.U + cix * C * DV;
    const int nxg = static_cast<int>(DV / 8);
    for (int item = tid; item < C * nxg; item += 256) {
      const int t = item / nxg, xg = item % nxg;
      *reinterpret_cast<uint4*>(Uo + t * DV + xg * 8) = *reinterpret_cast<const uint4*>(tX + t * LDX + xg * 8);
    }
  }
}

// ------------------------------------------------------------------ state kernel

template <int DK, int NCT>
struct WyStateLayout {
  static constexpr int C = 64;
  static constexpr int DVS = 16 * NCT;
  static constexpr int LDT = DK + 8;  // q and W rows
  static constexpr int LDD = C + 8;   // k^T rows, -M rows, U^T rows
  static constexpr int oQ = 0;
  static constexpr int oW = oQ + C * LDT * 2;
  static constexpr int oKT = oW + C * LDT * 2;
  static constexpr int oM = oKT + DK * LDD * 2;
  static constexpr int oU = oM + C * LDD * 2;
  static constexpr int oS = oU + DVS * LDD * 2;  // fp32: e^{G_t}, e^{G_n - G_t} (64 each), e^{G_n}
  static constexpr int BUF = oS + (2 * C + 4) * 4;
  static constexpr int total = 2 * BUF;
  static constexpr bool fits = total <= kLdsLimit;
};

// Workgroup = 2 loader waves and one state wave, for one state and a slice of DVS = 16 NCT value
// columns; the state wave holds that slice of S in its accumulators as NCT column tiles, so every
// A fragment read from LDS feeds NCT products.  Per chunk c (one barrier): the loaders write chunk
// c+1 into one LDS buffer from registers and issue the loads of chunk c+2, while the state wave
// consumes chunk c from the other buffer:
//     O = diag(e^{G_t}) Q S,  V = W S,  R = V - U,
//     S <- e^{G_n} S - K^T diag(e^{G_n - G_t}) R,  O -= M R,  O out.
template <int DK, int NCT>
__global__ __launch_bounds__(192) void wy_state_kernel(WyArgs a) {
  using L = WyStateLayout<DK, NCT>;
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  static_assert(L::fits, "LDS layout exceeds the gfx950 workgroup limit");
  static_assert(DK % 32 == 0, "dk must be a multiple of 32");
  constexpr int C = L::C, DVS = L::DVS, LDT = L::LDT, LDD = L::LDD;
  constexpr int NTD = DK / 16, NKB = DK / 32;
  constexpr int NLT = 128;  // loader threads (waves 0 and 1)
  constexpr int NCG = DK / 8, IPT = C * NCG / NLT;
  constexpr int NXG = DVS / 8, XPT = (C * NXG + NLT - 1) / NLT;
  constexpr int MPT = C * C / 8 / NLT;  // 16-byte items of -M per loader thread

  __shared__ __attribute__((aligned(32))) unsigned char smem[L::total];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const bool loader = wave < 2;

  const int64_t nb = gridDim.x, bid = blockIdx.x;
  const int64_t p = (nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
  const int64_t bh = p / a.nsl;
  const int sl = static_cast<int>(p % a.nsl);
  const int64_t bi = bh / a.H, hi = bh % a.H;
  const int64_t DV = a.DV, H = a.H, T = a.T, nch = a.nch;
  const int64_t col0 = static_cast<int64_t>(sl) * DVS;
  const uint32_t hdk = static_cast<uint32_t>(H * DK * 2), hdv = static_cast<uint32_t>(H * DV * 2);

  auto buf = [&](int64_t c) -> unsigned char* { return smem + (c & 1) * L::BUF; };

  // ---------------- loader registers ----------------
  uint4 pq[IPT], pk[IPT], pw[IPT], pm[MPT], pu[XPT];
  float pg = 0.f;
  auto prefetch = [&](int64_t c) {
    const int64_t t0 = c * C;
    const int64_t rr = (bi * T + t0) * H + hi;
    const int64_t cix = bh * nch + c;
    const auto rq = make_rsrc(a.q + rr * DK, wy_range(T - t0, H, DK));
    const auto rk = make_rsrc(a.k + rr * DK, wy_range(T - t0, H, DK));
    const auto rw = make_rsrc(a.W + cix * C * DK, C * DK * 2);
    const auto rm = make_rsrc(a.M + cix * C * C, C * C * 2);
    const auto ru = make_rsrc(a.U + cix * C * DV + col0, static_cast<uint32_t>((C * DV - col0) * 2));
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const uint32_t t = (tid / NCG) * IPT + j, cg = tid % NCG;
      pq[j] = buf_load16(rq, t * hdk + cg * 16);
      pk[j] = buf_load16(rk, t * hdk + cg * 16);
      pw[j] = buf_load16(rw, (t * DK + cg * 8) * 2);
    }
#pragma unroll
    for (int j = 0; j < MPT; ++j) pm[j] = buf_load16(rm, (tid + NLT * j) * 16);
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int item = tid + NLT * j;
      const uint32_t t = item / NXG, xg = item % NXG;
      pu[j] = buf_load16(ru, item < C * NXG ? (t * DV + xg * 8) * 2 : 0x80000000u);
    }
    if (wave == 0) {
      const auto rg = make_rsrc(a.G + cix * C, C * 4);
      pg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, lane * 4, 0, 0));
    }
  };

  auto store = [&](int64_t c) {
    unsigned char* B = buf(c);
    __bf16* tQ = reinterpret_cast<__bf16*>(B + L::oQ);
    __bf16* tW = reinterpret_cast<__bf16*>(B + L::oW);
    __bf16* kT = reinterpret_cast<__bf16*>(B + L::oKT);
    __bf16* gM = reinterpret_cast<__bf16*>(B + L::oM);
    __bf16* uT = reinterpret_cast<__bf16*>(B + L::oU);
    float* sc = reinterpret_cast<float*>(B + L::oS);
    const int cg = tid % NCG, tb = (tid / NCG) * IPT;
    uint16_t kh[8][IPT];
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      *reinterpret_cast<uint4*>(tQ + (tb + j) * LDT + cg * 8) = pq[j];
      *reinterpret_cast<uint4*>(tW + (tb + j) * LDT + cg * 8) = pw[j];
      const uint32_t w4[4] = {pk[j].x, pk[j].y, pk[j].z, pk[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kh[2 * e][j] = static_cast<uint16_t>(w4[e] & 0xffffu);
        kh[2 * e + 1][j] = static_cast<uint16_t>(w4[e] >> 16);
      }
    }
    uint16_t* kTu = reinterpret_cast<uint16_t*>(kT);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = cg * 8 + e;
      if constexpr (IPT >= 4) {
#pragma unroll
        for (int q4 = 0; q4 < IPT / 4; ++q4)
          *reinterpret_cast<uint2*>(kTu + row * LDD + swz((row >> 3) & 15, tb + 4 * q4)) =
              make_uint2(kh[e][4 * q4] | (uint32_t(kh[e][4 * q4 + 1]) << 16),
                         kh[e][4 * q4 + 2] | (uint32_t(kh[e][4 * q4 + 3]) << 16));
      } else {
        *reinterpret_cast<uint32_t*>(kTu + row * LDD + swz((row >> 3) & 15, tb)) =
            kh[e][0] | (uint32_t(kh[e][1]) << 16);
      }
    }
#pragma unroll
    for (int j = 0; j < MPT; ++j) {
      const int item = tid + NLT * j, r = item >> 3, part = item & 7;
      *reinterpret_cast<uint4*>(gM + r * LDD + part * 8) = pm[j];
    }
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int item = tid + NLT * j;
      if (item < C * NXG) {
        const int t = item / NXG, xg = item % NXG;
        const uint32_t w4[4] = {pu[j].x, pu[j].y, pu[j].z, pu[j].w};
        uint16_t* uTu = reinterpret_cast<uint16_t*>(uT);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uTu[(xg * 8 + 2 * e) * LDD + swz(2 * xg, t)] = static_cast<uint16_t>(w4[e] & 0xffffu);
          uTu[(xg * 8 + 2 * e + 1) * LDD + swz(2 * xg, t)] = static_cast<uint16_t>(w4[e] >> 16);
        }
      }
    }
    if (wave == 0) {
      const float gn = __shfl(pg, 63);
      sc[lane] = __expf(pg);
      sc[C + lane] = __expf(gn - pg);
      if (lane == 0) sc[2 * C] = __expf(gn);
    }
  };

  // ---------------- chain and output waves ----------------
  // S[ct][tl]: column tile ct (local columns 16 ct + l16), rows 16 tl + 4 g + i
  f32x4 S[NCT][NTD];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int tl = 0; tl < NTD; ++tl) {
      S[ct][tl] = zero4();
      if (!loader && a.S0 != nullptr) {
        const int64_t sb = bh * DK * DV + col0 + 16 * ct + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) S[ct][tl][i] = a.S0[sb + (int64_t)(16 * tl + 4 * g + i) * DV];
      }
    }

  // S <- e^{G_n} S + K^T rs   (rs = -R e^{G_n - G_t} as two tile-pair fragments per column tile)
  auto state_update = [&](const unsigned char* B, const F8 (*rs)[2]) {
    const __bf16* kT = reinterpret_cast<const __bf16*>(B + L::oKT);
    const float egn = reinterpret_cast<const float*>(B + L::oS)[2 * C];
    F8 kf[4][2];  // ring: tiles tl+1..tl+3 are in flight while tile tl multiplies
    auto load_kt = [&](int tl, F8* o) {
      const int row = 16 * tl + l16, key = (row >> 3) & 15;
      const __bf16* kr = kT + row * LDD;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x4 lo = lds_load4(kr + swz(key, 32 * kb + 4 * g));
        const bf16x4 hi = lds_load4(kr + swz(key, 32 * kb + 16 + 4 * g));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[kb][e] = lo[e];
          o[kb][4 + e] = hi[e];
        }
      }
    };
#pragma unroll
    for (int tl = 0; tl < 3 && tl < NTD; ++tl) load_kt(tl, kf[tl]);
#pragma unroll
    for (int tl = 0; tl < NTD; ++tl) {
      if (tl + 3 < NTD) load_kt(tl + 3, kf[(tl + 3) & 3]);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[ct][tl][i] *= egn;
        S[ct][tl] = MM::mma8(kf[tl & 3][0], rs[ct][0], S[ct][tl]);
        S[ct][tl] = MM::mma8(kf[tl & 3][1], rs[ct][1], S[ct][tl]);
      }
    }
  };

  // D[ct] = A S[ct] for A (64 x dk, row-major in LDS) as four 16-row tiles; all A fragments are
  // read first, and each feeds the NCT column tiles
  // Ot[ct][ta] = (Q S[ct])^T tiles (S as the A operand, the same fragments as B, so a lane holds
  // four consecutive columns of one row of Q S) and V[ct][ta] = W S[ct] tiles, as one stream of
  // eight 16-row tiles (Q then W) with three tiles in flight ahead of the one multiplying
  auto qs_ws = [&](const __bf16* tQ, const __bf16* tW, f32x4 (*Ot)[4], f32x4 (*V)[4]) {
    F8 sf[NCT][NKB];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sf[ct][kb] = acc_pair_frag<__bf16>(S[ct][2 * kb], S[ct][2 * kb + 1]);
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) {
        Ot[ct][ta] = zero4();
        V[ct][ta] = zero4();
      }
    }
    F8 af[4][NKB];
    auto load_a = [&](int j, F8* o) {
      const __bf16* rows = (j < 4 ? tQ : tW) + (16 * (j & 3) + l16) * LDT;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) o[kb] = lds_pair_frag_k<DK>(rows, 32 * kb, g);
    };
#pragma unroll
    for (int j = 0; j < 3; ++j) load_a(j, af[j]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j + 3 < 8) load_a(j + 3, af[(j + 3) & 3]);
      const int ta = j & 3;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          if (j < 4)
            Ot[ct][ta] = MM::mma8(sf[ct][kb], af[j & 3][kb], Ot[ct][ta]);
          else
            V[ct][ta] = MM::mma8(af[j & 3][kb], sf[ct][kb], V[ct][ta]);
        }
    }
  };

  auto state_chunk = [&](int64_t c) {
    [[maybe_unused]] const int64_t ch = c;  // for the phase markers
    const unsigned char* B = buf(c);
    const __bf16* uT = reinterpret_cast<const __bf16*>(B + L::oU);
    const __bf16* gM = reinterpret_cast<const __bf16*>(B + L::oM);
    const float* sc = reinterpret_cast<const float*>(B + L::oS);
    // O^T tiles: Ot[ct][ta] lane (g, l16) holds O[16 ta + l16][16 ct + 4 g + i]
    f32x4 Ot[NCT][4], V[NCT][4];
    qs_ws(reinterpret_cast<const __bf16*>(B + L::oQ), reinterpret_cast<const __bf16*>(B + L::oW), Ot, V);
    GDR_MARK(3);
    F8 rf[NCT][2], rs[NCT][2];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int n = 16 * ct + l16;
      f32x4 R[4], Rs[4];
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) {
        const bf16x4 u4 = *reinterpret_cast<const bf16x4*>(uT + n * LDD + swz(2 * (n >> 3), 16 * ta + 4 * g));
        const float4 d4 = *reinterpret_cast<const float4*>(sc + C + 16 * ta + 4 * g);
        const float d[4] = {d4.x, d4.y, d4.z, d4.w};
        const float e = sc[16 * ta + l16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          R[ta][i] = V[ct][ta][i] - static_cast<float>(u4[i]);
          Rs[ta][i] = -R[ta][i] * d[i];
          Ot[ct][ta][i] *= e;
        }
      }
      rf[ct][0] = acc_pair_frag<__bf16>(R[0], R[1]);
      rf[ct][1] = acc_pair_frag<__bf16>(R[2], R[3]);
      rs[ct][0] = acc_pair_frag<__bf16>(Rs[0], Rs[1]);
      rs[ct][1] = acc_pair_frag<__bf16>(Rs[2], Rs[3]);
    }
    F8 mf[6];
#pragma unroll
    for (int ta = 0, n = 0; ta < 4; ++ta) {
      mf[n++] = lds_pair_frag_k<C>(gM + (16 * ta + l16) * LDD, 0, g);
      if (ta >= 2) mf[n++] = lds_pair_frag_k<C>(gM + (16 * ta + l16) * LDD, 32, g);
    }
    state_update(B, rs);
    GDR_MARK(4);
    // O^T += R^T (-M)^T (gM holds -M), then O out, four columns of one token per 8-byte store;
    // rows past the last token are dropped by the range
    const int64_t t0 = c * C;
    const int64_t rr = (bi * T + t0) * H + hi;
    const int64_t bytes = ((T - t0 - 1) * H + 1) * DV * 2 - col0 * 2;
    const auto ro = make_rsrc(a.o + rr * DV + col0, static_cast<uint32_t>(bytes < 0x7fffffff ? bytes : 0x7fffffff));
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int ta = 0, n = 0; ta < 4; ++ta) {
        Ot[ct][ta] = MM::mma8(rf[ct][0], mf[n++], Ot[ct][ta]);
        if (ta >= 2) Ot[ct][ta] = MM::mma8(rf[ct][1], mf[n++], Ot[ct][ta]);
        bf16x4 ob;
#pragma unroll
        for (int i = 0; i < 4; ++i) ob[i] = static_cast<__bf16>(Ot[ct][ta][i]);
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ob), ro,
                                              (16 * ta + l16) * hdv + (16 * ct + 4 * g) * 2, 0, 0);
      }
  };

  // ---------------- pipeline ----------------
  // The loaders fetch and write chunk c+1 within iteration c: their registers are not live
  // across the loop, which leaves the state wave's accumulators in ordinary VGPRs.
  if (loader && nch > 0) {
    prefetch(0);
    store(0);
  }
  lds_barrier();
  for (int64_t ch = 0; ch < nch; ++ch) {
    // opaque per chunk: keeps lane-dependent LDS addresses from being hoisted out of the loop
    asm volatile("" : "+v"(lane), "+v"(g), "+v"(l16));
    GDR_MARK(0);
    if (loader) {
      if (ch + 1 < nch) {
        prefetch(ch + 1);
        store(ch + 1);
      }
      GDR_MARK(3);
    } else {
      state_chunk(ch);
    }
    GDR_MARK(1);
    lds_barrier();
    GDR_MARK(2);
  }

  if (!loader && a.S_T != nullptr) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int64_t sb = bh * DK * DV + col0 + 16 * ct + l16;
#pragma unroll
      for (int tl = 0; tl < NTD; ++tl)
#pragma unroll
        for (int i = 0; i < 4; ++i) a.S_T[sb + (int64_t)(16 * tl + 4 * g + i) * DV] = S[ct][tl][i];
    }
  }
}

}  // namespace gdr
