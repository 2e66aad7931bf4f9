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
// The chunk-local kernel writes W, U and -M (bf16) and e^{G_t}, e^{G_n - G_t}, e^{G_n} (fp32) to
// a workspace; the state kernel copies them, with the q and k rows, into LDS by direct-to-LDS
// loads, so its serial chain per chunk holds only S-dependent MFMAs.
#pragma once
#include "gdr_common.h"
#include "mfma.h"
#include "prefill_kernel.h"

// Phase markers: no-ops unless a profiling build defines them.
#ifndef GDR_PMARK
#define GDR_PMARK(id) ((void)0)
#endif
#ifndef GDR_MARK
#define GDR_MARK(id) ((void)0)
#endif

namespace gdr {

// Gram tiles of one key wave: row blocks RA and RB (16 rows each) of `rows` (k or q) against
// the 16-row column blocks of k at or below them.  prod 0: A = beta_t k_t . k_i e^{G_t - G_i}
// for i < t (off-diagonal blocks to gA as -A, diagonal blocks to Ld in fp32); prod 1:
// M = q_t . k_i e^{G_t - G_i} for i <= t, stored as -M.  All fragments are read before the
// first MFMA.
template <int DK, int RA, int RB, int LDT, int LDD, int LDA, int LDL>
__device__ __forceinline__ void scalar_gram_pair(const __bf16* rows, const __bf16* tK, int prod,
                                                 int g, int l16, const float* sc, __bf16* gA,
                                                 __bf16* gM, float* Ld) {
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  constexpr int C = 64, NKB = DK / 32, NT = RA + RB + 2;
  auto tile_a = [](int j) { return j <= RA ? RA : RB; };
  auto tile_b = [](int j) { return j <= RA ? j : j - RA - 1; };
  // Tiles are computed transposed (k block as the A operand) so that each lane ends up with four
  // consecutive columns of one output row: one 8-byte store.  The diagonal tiles of A are
  // computed upright and stored column-major in fp32 for the inverse.
  auto diag_a = [&](int j) { return prod == 0 && tile_a(j) == tile_b(j); };
  auto epilogue = [&](int j, const f32x4& acc) {
    const int ta = tile_a(j), tb = tile_b(j);
    if (diag_a(j)) {
      const int cc = 16 * tb + l16;
      const float gc = sc[cc];
      const float4 gr4 = *reinterpret_cast<const float4*>(sc + 16 * ta + 4 * g);
      const float4 br4 = *reinterpret_cast<const float4*>(sc + 3 * C + 16 * ta + 4 * g);
      const float gr[4] = {gr4.x, gr4.y, gr4.z, gr4.w}, br[4] = {br4.x, br4.y, br4.z, br4.w};
      float4 o;
      float* ov = reinterpret_cast<float*>(&o);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * ta + 4 * g + i;
        ov[i] = cc < r ? acc[i] * __expf(fminf(gr[i] - gc, 0.f)) * br[i] : 0.f;
      }
      *reinterpret_cast<float4*>(Ld + (ta * 16 + l16) * LDL + 4 * g) = o;  // column l16, rows 4g..
      return;
    }
    const int r = 16 * ta + l16, cc0 = 16 * tb + 4 * g;
    const float gr = sc[r], br = prod == 0 ? sc[3 * C + r] : 1.f;
    const float4 gc4 = *reinterpret_cast<const float4*>(sc + cc0);
    const float gc[4] = {gc4.x, gc4.y, gc4.z, gc4.w};
    bf16x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cc = cc0 + i;
      const bool keep = prod == 0 ? (cc < r) : (cc <= r);
      o[i] = static_cast<__bf16>(keep ? -acc[i] * __expf(fminf(gr - gc[i], 0.f)) * br : 0.f);
    }
    // one 8-byte store: the pitches are multiples of four elements and the arrays 16-byte aligned
    __bf16* dst = prod == 1 ? gM + r * LDD + cc0 : gA + (r - 16) * LDA + cc0;
    *reinterpret_cast<bf16x4*>(dst) = o;
  };
  F8 rf[NKB], cb[2][NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    rf[kb] = lds_load8(rows + (16 * RA + l16) * LDT + 32 * kb + 8 * g);
    cb[0][kb] = lds_load8(tK + l16 * LDT + 32 * kb + 8 * g);
  }
  f32x4 acc[2];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (j == RA + 1) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) rf[kb] = lds_load8(rows + (16 * RB + l16) * LDT + 32 * kb + 8 * g);
    }
    if (j + 1 < NT) {
      const int nb = tile_b(j + 1);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        cb[(j + 1) & 1][kb] = lds_load8(tK + (16 * nb + l16) * LDT + 32 * kb + 8 * g);
    }
    acc[j & 1] = zero4();
    if (diag_a(j)) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) acc[j & 1] = MM::mma8(rf[kb], cb[j & 1][kb], acc[j & 1]);
    } else {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) acc[j & 1] = MM::mma8(cb[j & 1][kb], rf[kb], acc[j & 1]);
    }
    if (j > 0) epilogue(j - 1, acc[(j - 1) & 1]);
  }
  epilogue(NT - 1, acc[(NT - 1) & 1]);
}

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
  float* E;   // [B*H][nch][kWyE]: e^{G_t} and e^{G_n - G_t} for the 64 tokens, e^{G_n}, 3 zeros
  int64_t T, H, DV, nch;
  int alpha_kind, b_kind, w_kind;
  int nsl;     // value slices per state (state kernel)
  int64_t Hk;  // q / k heads (H is a multiple): value head h reads q / k head h / (H / Hk)
};

constexpr int kWyE = 132;  // floats per chunk in WyArgs::E (33 pieces of 16 bytes)

// Byte range of `width`-element rows from a chunk's first token to the last token of its state.
__device__ __forceinline__ uint32_t wy_range(int64_t left, int64_t H, int64_t width) {
  const int64_t bytes = ((left - 1) * H + 1) * width * 2;
  return static_cast<uint32_t>(bytes < 0x7fffffff ? bytes : 0x7fffffff);
}

// Transposing 8-byte LDS read (gfx950): within each group of 16 lanes, lane 4 a + b receives
// element b of the 8-byte vectors that lanes a, a + 4, a + 8 and a + 12 of the group point at.
__device__ __forceinline__ bf16x4 lds_read_tr4(const unsigned char* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<unsigned char*>(p)));
  return __builtin_bit_cast(bf16x4, r);
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
  static constexpr int oS = oLD + 4 * 16 * LDL * 4;  // fp32: G, e^G, e^{G_n - G}, beta (64 each)
  static constexpr int total = oS + 4 * C * 4;
  static constexpr bool fits = total <= kLdsLimit;
};

// One workgroup per (state, chunk).  Phases (barriers between): inputs into LDS and gate prefix
// sums; Gram tiles (waves 0-1: A, waves 2-3: M); diagonal inverses (waves 0-1) while waves 2-3
// write -M out; T = (I + A)^{-1} by blocked forward substitution on the identity; W = T B_k and
// U = T X, each wave owning whole 16-column tiles (B_k the k tile scaled by beta_t e^{G_t}).
//
// Without an erase gate (ERASE false: b = 0, linear attention with a scalar or no decay) the
// Gram A vanishes, T = I, W = 0 and U = X: only M, U and the exponentials are formed.
template <int DK, int DVP, bool ERASE>
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
  const int64_t rqk = (bi * a.T + t0) * a.Hk + hi / (H / a.Hk);  // q / k row of the first token
  const auto rq = make_rsrc(a.q + rqk * DK, wy_range(left, a.Hk, DK));
  const auto rk = make_rsrc(a.k + rqk * DK, wy_range(left, a.Hk, DK));
  const auto rv = make_rsrc(a.v + rr * DV, wy_range(left, H, DV));
  const uint32_t hdk = static_cast<uint32_t>(a.Hk * DK * 2), hdv = static_cast<uint32_t>(H * DV * 2);
  const uint32_t h1 = static_cast<uint32_t>(H * 2);

  // every global load is issued before the first use: out-of-range items get an offset past
  // the buffer range (zero) and absent gate kinds an empty range
  constexpr int XPT = C * (DVP / 8) / 256;  // x items per thread at the widest dv
  const int nxg = static_cast<int>(DV / 8);
  // item / nxg for item < 2048 and nxg <= 32, without a division: with M = ceil(2^16 / nxg),
  // (item M) >> 16 is exact because item (M - 2^16 / nxg) / 2^16 < 1 / 32 <= 1 / nxg
  const uint32_t xdm = (65536u + static_cast<uint32_t>(nxg) - 1u) / static_cast<uint32_t>(nxg);
  auto xdiv = [&](uint32_t item) { return (item * xdm) >> 16; };
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
    const uint32_t t = in ? xdiv(item) : 0, xg = in ? item - t * nxg : 0;
    vv[j] = buf_load16(rv, in ? t * hdv + xg * 16 : oob);
    wv[j] = buf_load16(rwc, in ? t * hdv + xg * 16 : oob);
    wsv[j] = buf_load_u16(rws, in ? t * h1 : oob);
  }
  const uint16_t lav = buf_load_u16(rla, lane * h1), bev = buf_load_u16(rb, lane * h1);

  // M tiles above the diagonal are never written and must read as zero
  for (int i = tid; i < C * LDD / 8; i += 256) reinterpret_cast<uint4*>(gM)[i] = make_uint4(0, 0, 0, 0);
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
      const int t = static_cast<int>(xdiv(item)), xg = item - t * nxg;
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
    const float gn = __shfl(x, 63);
    const float ex = __expf(x);
    sc[lane] = x;
    sc[C + lane] = ex;
    sc[2 * C + lane] = __expf(gn - x);
    sc[3 * C + lane] = bf16_to_f32(bev);
    a.E[cix * kWyE + lane] = ex;
    a.E[cix * kWyE + C + lane] = sc[2 * C + lane];
    if (lane < kWyE - 2 * C) a.E[cix * kWyE + 2 * C + lane] = lane == 0 ? __expf(gn) : 0.f;
  }
  GDR_PMARK(0);
  lds_barrier();

  // Gram tiles: waves 0-1 A (solve, with the fp32 diagonal blocks to Ld), waves 2-3 M
  if (ERASE || wave >= 2) {
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
    if (ERASE && lane < 32) wy_diag_inverses<LDL, LDI>(Ld, dInv, wave, lane, l16);
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
  if constexpr (ERASE) {
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

  // W = T diag(beta e^G) K and U = T X, one 16-column tile at a time (no chain: T is known), as
  // transposed tiles W^T = (diag(beta e^G) K)^T T^T, each wave owning whole column tiles.  The A
  // fragments (8 tokens of one column, tile-pair order) come from two transposing reads of the
  // token-major rows per k-block (source lane (a, m) = (l16 & 3, l16 >> 2) of group g points at
  // token 32 ks + 16 h + 4 g + m, columns 16 ct + 4 a ..); each lane then holds four consecutive
  // columns of one token and overwrites them in place with one 8-byte write per token tile, to be
  // written out coalesced below.
  if constexpr (ERASE) {
    const __bf16* tT = gM;
    F8 tf[6];
#pragma unroll
    for (int ta = 0, n = 0; ta < 4; ++ta) {
      tf[n++] = lds_pair_frag_k<C>(tT + (16 * ta + l16) * LDD, 0, g);
      if (ta >= 2) tf[n++] = lds_pair_frag_k<C>(tT + (16 * ta + l16) * LDD, 32, g);
    }
    float sw[2][8];  // beta_t e^{G_t} of the tokens of this lane's fragments
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = 32 * ks + 4 * g + (e & 3) + (e >> 2) * 16;
        sw[ks][e] = sc[3 * C + t] * sc[C + t];
      }
    const int a_ = l16 & 3, m_ = l16 >> 2;
    auto gemm_tile = [&](__bf16* base, int pitch, int ct, bool scale) {
      F8 af[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x4 v = lds_read_tr4(reinterpret_cast<const unsigned char*>(
              base + (32 * ks + 16 * h + 4 * g + m_) * pitch + 16 * ct + 4 * a_));
#pragma unroll
          for (int e = 0; e < 4; ++e)
            af[ks][4 * h + e] = scale ? static_cast<__bf16>(static_cast<float>(v[e]) * sw[ks][4 * h + e]) : v[e];
        }
      f32x4 D[4];  // D[ta] lane (g, l16): columns 16 ct + 4 g + i of token 16 ta + l16
#pragma unroll
      for (int ta = 0, n = 0; ta < 4; ++ta) {
        D[ta] = MM::mma8(af[0], tf[n++], zero4());
        if (ta >= 2) D[ta] = MM::mma8(af[1], tf[n++], D[ta]);
      }
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) {
        bf16x4 ob;
#pragma unroll
        for (int i = 0; i < 4; ++i) ob[i] = static_cast<__bf16>(D[ta][i]);
        *reinterpret_cast<bf16x4*>(base + (16 * ta + l16) * pitch + 16 * ct + 4 * g) = ob;
      }
    };
    // tile loops without a per-tile guard where the counts divide evenly over the four waves,
    // so that the loads of every tile of a wave are issued together
    if constexpr (DK / 16 % 4 == 0) {
#pragma unroll
      for (int r = 0; r < DK / 64; ++r) gemm_tile(tK, LDT, wave + 4 * r, true);
    } else {
#pragma unroll
      for (int r = 0; r < (DK / 16 + 3) / 4; ++r) {
        const int ct = wave + 4 * r;
        if (ct < DK / 16) gemm_tile(tK, LDT, ct, true);
      }
    }
    const int nct_u = static_cast<int>(DV / 16);
    if (nct_u == DVP / 16) {
#pragma unroll
      for (int r = 0; r < DVP / 64; ++r) gemm_tile(tX, LDX, wave + 4 * r, false);
    } else {
#pragma unroll
      for (int r = 0; r < DVP / 64; ++r) {
        const int ct = wave + 4 * r;
        if (ct < nct_u) gemm_tile(tX, LDX, ct, false);
      }
    }
  }
  GDR_PMARK(3);
  lds_barrier();

  // W and U out (without the erase, U = X), 16 bytes per item
  {
    __bf16* Wo = a.W + cix * C * DK;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int item = tid + 256 * j;
      const int t = item / NCG, cg = item % NCG;
      if (ERASE) *reinterpret_cast<uint4*>(Wo + t * DK + cg * 8) = *reinterpret_cast<const uint4*>(tK + t * LDT + cg * 8);
    }
    __bf16* Uo = a.U + cix * C * DV;
    for (int item = tid; item < C * nxg; item += 256) {
      const int t = static_cast<int>(xdiv(item)), xg = item - t * nxg;
      *reinterpret_cast<uint4*>(Uo + t * DV + xg * 8) = *reinterpret_cast<const uint4*>(tX + t * LDX + xg * 8);
    }
  }
}

// ------------------------------------------------------------------ state kernel

// One 16-byte direct-to-LDS load per lane: lane L's piece lands at lds + 16 L (the LDS address
// must be the same for the whole wave); pieces outside the buffer range arrive as zeros.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off,
                                           0, 0, 0);
}

// Row-major bf16 arrays of NCHR 16-byte pieces per row live in LDS without padding, the pieces
// of each row permuted by XOR with a key of the row.  A fragment read touches 16 rows at once:
// either 16 consecutive rows (NAT: row bits 0-3 vary) or the rows of perm_row below (PERM: bits
// 0, 1, 3 and 4 vary); the key takes those bits so that the 16 pieces read land in 16 distinct
// bank groups (rows of 256, 128 or 64 bytes).
template <int NCHR, bool PERM>
__host__ __device__ constexpr inline int swz_key(int row) {
  if constexpr (NCHR == 16) return PERM ? ((row & 3) | ((row >> 1) & 12)) : (row & 15);
  else if constexpr (NCHR == 8) return PERM ? (((row >> 1) & 1) | ((row >> 2) & 6)) : ((row >> 1) & 7);
  else if constexpr (NCHR == 4) return PERM ? ((row >> 3) & 3) : ((row >> 2) & 3);
  else return PERM ? ((row >> 3) & 1) : ((row >> 3) & 1);
}

// Row m of 16-row tile `tile` when the tile's accumulator rows 4 g + i are to hold rows whose
// pair-fragment k slots (tiles 2 kb and 2 kb + 1, rows 4 g + i) are the 8 consecutive rows
// 32 kb + 8 g .. 32 kb + 8 g + 7: one 16-byte read then gives a lane its whole fragment.
__device__ __forceinline__ int perm_row(int tile, int m) {
  return 32 * (tile >> 1) + 4 * (tile & 1) + 8 * (m >> 2) + (m & 3);
}

// A row-major global array (row stride `stride` bytes) is copied into that form 64 pieces per
// instruction: LDS piece s holds piece (s mod NCHR) ^ key of row s / NCHR.  dma_offsets gives a
// lane's source offsets (the same for every chunk, so they are computed once); dma_rows issues
// the copies.
template <int NCHR, bool PERM, int NPIECE>
__device__ __forceinline__ void dma_offsets(uint32_t stride, int lane, uint32_t* off) {
  static_assert(NPIECE % 64 == 0, "whole instructions only");
#pragma unroll
  for (int i = 0; i < NPIECE / 64; ++i) {
    const int s = 64 * i + lane, row = s / NCHR, piece = (s % NCHR) ^ swz_key<NCHR, PERM>(row);
    off[i] = static_cast<uint32_t>(row) * stride + static_cast<uint32_t>(piece) * 16u;
  }
}
template <int NPIECE>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t r, unsigned char* lds, const uint32_t* off) {
#pragma unroll
  for (int i = 0; i < NPIECE / 64; ++i) lds_dma16(r, lds + 1024 * i, off[i]);
}

// The same copies with fewer lane registers: instruction i covers rows (64 / NCHR) i .., and a
// lane's piece pattern repeats every P instructions (P = 1, 2 or 4 for these keys), so a lane keeps
// P offsets and instruction i adds the uniform row offset of i - i mod P as the scalar offset.
// (instruction i covers rows R = (64 / NCHR) i + lane / NCHR; the key reads row bits 0-3 (NAT,
// NCHR 16), 0, 1, 3, 4 (PERM, 16), 1-3 (NAT, 8), 1, 3, 4 (PERM, 8), 2, 3 (NAT, 4), 3, 4 (PERM, 4)
// or 3 (2), so the bits of R above lane / NCHR that it reads fix the period)
template <int NCHR, bool PERM, int NPIECE>
struct DmaPlan {
  static_assert(NPIECE % 64 == 0, "whole instructions only");
  static constexpr int NI = NPIECE / 64;
  // (instruction i covers rows (64 / NCHR) i + lane / NCHR; the key reads row bits 0-3 (NAT,
  // NCHR 16), 0, 1, 3, 4 (PERM, 16), 1-3 (NAT, 8), 1, 3, 4 (PERM, 8), 2, 3 (NAT, 4), 3, 4 (PERM, 4)
  // or 3 (2), so the row bits above lane / NCHR that it reads fix the period)
  static constexpr int PERIOD = NCHR == 16 ? (PERM ? 8 : 4) : NCHR == 8 ? (PERM ? 4 : 2) : NCHR == 4 ? (PERM ? 2 : 1) : 1;
  static constexpr int P = PERIOD < NI ? PERIOD : NI;
  // (a fixed bound: a bound that depends on the template arguments here keeps the host pass of
  // hipcc from emitting the launch stubs of kernels that hold a plan)
  uint32_t off[8];
  static_assert(P <= 8, "period above the fixed bound");
  __device__ __forceinline__ void init(uint32_t stride, int lane) {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int s = 64 * i + lane, row = s / NCHR, piece = (s % NCHR) ^ swz_key<NCHR, PERM>(row);
      off[i] = static_cast<uint32_t>(row) * stride + static_cast<uint32_t>(piece) * 16u;
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, unsigned char* lds, uint32_t stride) const {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(lds + 1024 * i), 16, off[i % P],
          static_cast<int>(static_cast<uint32_t>((64 / NCHR) * (i - i % P)) * stride), 0, 0);
  }
};

// Byte address of piece `piece` of row `row` of such an array.
template <int NCHR, bool PERM>
__device__ __forceinline__ const unsigned char* swz_addr(const unsigned char* base, int row, int piece) {
  return base + row * NCHR * 16 + ((piece ^ swz_key<NCHR, PERM>(row)) << 4);
}

// The 16-byte piece `piece` of row `row` of such an array.
template <int NCHR, bool PERM>
__device__ __forceinline__ Mma<__bf16>::F8 lds_piece(const unsigned char* base, int row, int piece) {
  return *reinterpret_cast<const Mma<__bf16>::F8*>(base + row * NCHR * 16 +
                                                   ((piece ^ swz_key<NCHR, PERM>(row)) << 4));
}

template <int DK, int DVS>
struct WyStateLayout {
  static constexpr int C = 64;
  static constexpr int NCQ = DK / 8;  // 16-byte pieces per q / W row
  static constexpr int NCC = C / 8;   // pieces per row of the token-minor arrays
  static constexpr int NCU = DVS / 8;  // pieces per row of the U slice
  static constexpr int NBUF = 2;              // chunk buffers
  static constexpr int oQ = 0;                // q rows [64][dk]
  static constexpr int oW = oQ + C * DK * 2;  // W rows [64][dk]
  static constexpr int oK = oW + C * DK * 2;  // k rows [64][dk]
  static constexpr int oM = oK + C * DK * 2;  // -M rows [64][64]
  static constexpr int oU = oM + C * C * 2;   // U rows of the slice [64][DVS]
  static constexpr int oE = oU + C * DVS * 2; // e^{G_t}, e^{G_n - G_t} (64 each), e^{G_n}: fp32
  static constexpr int BUF = oE + 1024;
  static constexpr int LDO = DVS + 8;         // O rows (16-byte aligned)
  static constexpr int oO = NBUF * BUF;       // two O buffers [64][LDO]
  static constexpr int total = oO + 2 * C * LDO * 2;
  static constexpr bool fits = total <= kLdsLimit;
};

// Workgroup = 2 loader waves and NSW state waves for one state and a slice of DVS = 16 NCT NSW
// value columns; state wave j holds columns 16 NCT j .. 16 NCT (j + 1) - 1 of the slice in its
// accumulators as NCT column tiles.  Chunk c's operands sit in LDS buffer c mod 2, filled by
// direct-to-LDS loads that loader wave c mod 2 issues a whole chunk ahead, so the loads never
// stall the chain and no loader registers hold data.  Two barriers per chunk c:
//   up to A: the state waves read every operand of chunk c into registers;
//   A to B:  the state waves compute
//              V = W S,  R = V - U,  S <- e^{G_n} S - K^T diag(e^{G_n - G_t}) R,
//              O = diag(e^{G_t}) Q S - M R
//            and leave O in an LDS buffer; loader wave c mod 2 refills buffer c mod 2 with
//            chunk c+2, and the other loader wave copies the O rows of chunk c-1 to HBM and
//            waits for its loads of chunk c+1.
//
// Without an erase gate (ERASE false) W = 0: V and W's loads drop out and R = -U.
template <int DK, int NCT, int NSW, bool ERASE>
__global__ __launch_bounds__(64 * (2 + NSW)) void wy_state_kernel(WyArgs a) {
  constexpr int DVS = 16 * NCT * NSW;
  using L = WyStateLayout<DK, DVS>;
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  static_assert(L::fits, "LDS layout exceeds the gfx950 workgroup limit");
  static_assert(DK % 32 == 0, "dk must be a multiple of 32");
  constexpr int C = L::C, NCQ = L::NCQ, NCC = L::NCC;
  constexpr int NTD = DK / 16, NKB = DK / 32;

  __shared__ __attribute__((aligned(1024))) unsigned char smem[L::total];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const bool loader = wave < 2;
  const int cb = loader ? 0 : 16 * NCT * (wave - 2);  // this state wave's first column in the slice

  const int64_t nb = gridDim.x, bid = blockIdx.x;
  const int64_t p = (nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
  const int64_t bh = p / a.nsl;
  const int sl = static_cast<int>(p % a.nsl);
  const int64_t bi = bh / a.H, hi = bh % a.H;
  const int64_t DV = a.DV, H = a.H, T = a.T, nch = a.nch;
  const int64_t col0 = static_cast<int64_t>(sl) * DVS;
  // token stride of q and k (the only [B, T, H?, dk] arrays read here), and of o
  const uint32_t hdk = static_cast<uint32_t>(a.Hk * DK * 2), hdv = static_cast<uint32_t>(H * DV * 2);
  const int64_t hq = hi / (H / a.Hk);  // this state's q / k head

  auto buf = [&](int64_t c) -> unsigned char* { return smem + (c & 1) * L::BUF; };
  auto obuf = [&](int64_t c) -> __bf16* {
    return reinterpret_cast<__bf16*>(smem + L::oO + (c & 1) * C * L::LDO * 2);
  };

  // ---------------- loader waves ----------------
  // per-lane source offsets of the copies, computed once
  constexpr int NQI = C * NCQ / 64, NMI = C * NCC / 64, NUI = C * L::NCU / 64;
  uint32_t offQ[NQI], offW[NQI], offK[NQI], offM[NMI], offU[NUI];
  {
    const int dl = tid & 63;
    dma_offsets<NCQ, false, C * NCQ>(hdk, dl, offQ);
    dma_offsets<NCQ, true, C * NCQ>(DK * 2, dl, offW);
    dma_offsets<NCQ, true, C * NCQ>(hdk, dl, offK);
    dma_offsets<NCC, false, C * NCC>(C * 2, dl, offM);
    dma_offsets<L::NCU, true, C * L::NCU>(static_cast<uint32_t>(DV * 2), dl, offU);
  }
  // chunk c's operands into buffer c mod 2 (q and k rows past the last token arrive as zeros)
  auto dma_chunk = [&](int64_t c) {
    unsigned char* B = buf(c);
    const int64_t t0 = c * C, rr = (bi * T + t0) * a.Hk + hq, cix = bh * nch + c;
    dma_rows<C * NCQ>(make_rsrc(a.q + rr * DK, wy_range(T - t0, a.Hk, DK)), B + L::oQ, offQ);
    if (ERASE) dma_rows<C * NCQ>(make_rsrc(a.W + cix * C * DK, C * DK * 2), B + L::oW, offW);
    dma_rows<C * NCQ>(make_rsrc(a.k + rr * DK, wy_range(T - t0, a.Hk, DK)), B + L::oK, offK);
    dma_rows<C * NCC>(make_rsrc(a.M + cix * C * C, C * C * 2), B + L::oM, offM);
    dma_rows<C * L::NCU>(make_rsrc(a.U + cix * C * DV + col0, static_cast<uint32_t>((C * DV - col0) * 2)),
                         B + L::oU, offU);
    if (lane < kWyE / 4) lds_dma16(make_rsrc(a.E + cix * kWyE, kWyE * 4), B + L::oE, lane * 16);
  };
  // O rows of chunk c from its LDS buffer to HBM, 16 bytes per store; rows past the last token
  // are dropped by the range
  auto store_o = [&](int64_t c) {
    constexpr int NOG = DVS / 8, OPT = C * NOG / 64;
    const __bf16* oO = obuf(c);
    const int64_t t0 = c * C;
    const int64_t rr = (bi * T + t0) * H + hi;
    const int64_t bytes = ((T - t0 - 1) * H + 1) * DV * 2 - col0 * 2;
    const auto ro = make_rsrc(a.o + rr * DV + col0, static_cast<uint32_t>(bytes < 0x7fffffff ? bytes : 0x7fffffff));
#pragma unroll
    for (int j = 0; j < OPT; ++j) {
      const int item = lane + 64 * j, t = item / NOG, part = item % NOG;
      buf_store16(ro, t * hdv + part * 16, *reinterpret_cast<const uint4*>(oO + t * L::LDO + part * 8));
    }
  };

  // ---------------- state waves ----------------
  // S[ct][tl]: column tile ct (slice columns cb + 16 ct + l16); accumulator row 4 g + i holds
  // channel perm_row(tl, 4 g + i), so that the pair fragment of tiles 2 kb, 2 kb + 1 carries
  // channels 32 kb + 8 g .. 32 kb + 8 g + 7 (one 16-byte piece of a q or W row)
  f32x4 S[NCT][NTD];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int tl = 0; tl < NTD; ++tl) {
      S[ct][tl] = zero4();
      if (!loader && a.S0 != nullptr) {
        const int64_t sb = bh * DK * DV + col0 + cb + 16 * ct + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) S[ct][tl][i] = a.S0[sb + (int64_t)perm_row(tl, 4 * g + i) * DV];
      }
    }
  // Complete the initial-state loads here, on every path, so that the chunk loop never waits
  // on vector memory for the accumulators.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // operands, one set for the S chain and one for the read-out:
  //   aw: W rows perm_row(ta, l16) (V tile ta's accumulator row 4 g + i is then token
  //       perm_row(ta, 4 g + i), and R's pair fragments carry tokens 32 kb + 8 g ..), channels
  //       32 kb + 8 g ..;  aq: q rows 16 ta + l16, channels 32 kb + 8 g ..;  mf: -M rows
  //       16 ta + l16, tokens 32 kb + 8 g ..  (one 16-byte read each)
  //   kf: K^T as A fragments, rows = channels perm_row(tl, l16) (S's channel order), tokens
  //       32 kb + 8 g .., by two transposing reads of the k rows: source lane (a, m) = (l16 & 3,
  //       l16 >> 2) of group g points at token 32 kb + 8 g + 4 h + m, channels
  //       perm_row(tl, 4 a) ..;  uv: U at the tokens of V tile ta, this lane's column, the same way
  //   eg: e^{G_t} of this lane's O rows;  dd: e^{G_n - G_t} at V tile ta's tokens;  egn: e^{G_n}
  F8 aw[NKB][4], aq[NKB][4], kf[2][NTD], mf[6];
  bf16x4 uv[NCT][4];
  float eg[4], egn = 0.f;
  float4 dd[4];
  auto read_chain = [&](int64_t c) {
    const unsigned char* B = buf(c);
    const int ta_ = l16 & 3, m_ = l16 >> 2;  // this lane's role as a transposing-read source
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int ta = 0; ta < 4; ++ta)
        if (ERASE) aw[kb][ta] = lds_piece<NCQ, true>(B + L::oW, perm_row(ta, l16), 4 * kb + g);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int col = cb + 16 * ct + 4 * ta_;
#pragma unroll
      for (int ta = 0; ta < 4; ++ta)
        uv[ct][ta] = lds_read_tr4(swz_addr<L::NCU, true>(B + L::oU, perm_row(ta, 4 * g + m_), col >> 3) + 8 * ((col >> 2) & 1));
    }
    const float* E = reinterpret_cast<const float*>(B + L::oE);
#pragma unroll
    for (int ta = 0; ta < 4; ++ta) dd[ta] = *reinterpret_cast<const float4*>(E + C + perm_row(ta, 4 * g));
    egn = E[2 * C];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int tl = 0; tl < NTD; ++tl) {
        const int piece = 4 * (tl >> 1) + ta_;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int row = 32 * kb + 8 * g + 4 * h + m_;
          const bf16x4 v = lds_read_tr4(swz_addr<NCQ, true>(B + L::oK, row, piece) + 8 * (tl & 1));
#pragma unroll
          for (int e = 0; e < 4; ++e) kf[kb][tl][4 * h + e] = v[e];
        }
      }
  };
  auto read_out = [&](int64_t c) {
    const unsigned char* B = buf(c);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) aq[kb][ta] = lds_piece<NCQ, false>(B + L::oQ, 16 * ta + l16, 4 * kb + g);
#pragma unroll
    for (int ta = 0, n = 0; ta < 4; ++ta) {
      mf[n++] = lds_piece<NCC, false>(B + L::oM, 16 * ta + l16, g);
      if (ta >= 2) mf[n++] = lds_piece<NCC, false>(B + L::oM, 16 * ta + l16, 4 + g);
    }
    const float* E = reinterpret_cast<const float*>(B + L::oE);
#pragma unroll
    for (int ta = 0; ta < 4; ++ta) eg[ta] = E[16 * ta + l16];
  };

  // each product runs k-step by k-step across its independent output tiles, so consecutive
  // MFMAs never wait on each other; the chain that carries S (V, R, the update) comes first
  F8 sf[NCT][NKB];  // S of the chunk start as bf16 operand fragments
  F8 rf[NCT][2];    // R (tokens as k)
  auto chain = [&](int64_t c) {
    [[maybe_unused]] const int64_t ch = c;  // for the phase markers
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sf[ct][kb] = acc_pair_frag<__bf16>(S[ct][2 * kb], S[ct][2 * kb + 1]);
    // V = W S
    f32x4 V[NCT][4];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) V[ct][ta] = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int ta = 0; ta < 4; ++ta)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          if (ERASE) V[ct][ta] = MM::mma8(aw[kb][ta], sf[ct][kb], V[ct][ta]);
    GDR_MARK(3);
    // R = V - U (read-out operand) and -R e^{G_n - G_t} (state-update operand), tokens as k
    F8 rs[NCT][2];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 R[4], Rs[4];
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) {
        const float d[4] = {dd[ta].x, dd[ta].y, dd[ta].z, dd[ta].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          R[ta][i] = V[ct][ta][i] - static_cast<float>(uv[ct][ta][i]);
          Rs[ta][i] = -R[ta][i] * d[i];
        }
      }
      rf[ct][0] = acc_pair_frag<__bf16>(R[0], R[1]);
      rf[ct][1] = acc_pair_frag<__bf16>(R[2], R[3]);
      rs[ct][0] = acc_pair_frag<__bf16>(Rs[0], Rs[1]);
      rs[ct][1] = acc_pair_frag<__bf16>(Rs[2], Rs[3]);
    }
    // S <- e^{G_n} S + K^T (-R e^{G_n - G_t})
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int tl = 0; tl < NTD; ++tl)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[ct][tl][i] *= egn;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int tl = 0; tl < NTD; ++tl)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) S[ct][tl] = MM::mma8(kf[kb][tl], rs[ct][kb], S[ct][tl]);
    GDR_MARK(4);
  };
  auto read_out_compute = [&](int64_t c) {
    // O^T tiles: Ot[ct][ta] lane (g, l16) holds O[16 ta + l16][16 ct + 4 g + i];
    // O^T = (Q S)^T diag(e^{G_t}) + R^T (-M)^T
    f32x4 Ot[NCT][4];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) Ot[ct][ta] = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int ta = 0; ta < 4; ++ta)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) Ot[ct][ta] = MM::mma8(sf[ct][kb], aq[kb][ta], Ot[ct][ta]);
#pragma unroll
    for (int ta = 0; ta < 4; ++ta)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) Ot[ct][ta][i] *= eg[ta];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ta = 2 * kb; ta < 4; ++ta) {  // -M is lower triangular: tokens 32.. only reach ta >= 2
        const int m = kb == 0 ? (ta < 2 ? ta : 2 * ta - 2) : 2 * ta - 1;  // (ta, kb) in mf
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) Ot[ct][ta] = MM::mma8(rf[ct][kb], mf[m], Ot[ct][ta]);
      }
    // O rows into the chunk's O buffer, four columns of one token per 8-byte write
    __bf16* oO = obuf(c);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) {
        bf16x4 ob;
#pragma unroll
        for (int i = 0; i < 4; ++i) ob[i] = static_cast<__bf16>(Ot[ct][ta][i]);
        *reinterpret_cast<bf16x4*>(oO + (16 * ta + l16) * L::LDO + cb + 16 * ct + 4 * g) = ob;
      }
  };

  // ---------------- pipeline ----------------
  if (nch > 0) {
    if (wave == 0) {
      dma_chunk(0);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    if (wave == 1 && nch > 1) dma_chunk(1);
  }
  lds_barrier();
  for (int64_t ch = 0; ch < nch; ++ch) {
    // opaque per chunk: keeps lane-dependent LDS addresses from being hoisted out of the loop
    asm volatile("" : "+v"(lane), "+v"(g), "+v"(l16));
    GDR_MARK(0);
    if (!loader) {
      read_chain(ch);
      read_out(ch);
    }
    lds_barrier_keep_vm();  // A: buffer ch mod 2 is free
    GDR_MARK(1);
    if (loader) {
      if (wave == static_cast<int>(ch & 1)) {
        if (ch + 2 < nch) dma_chunk(ch + 2);
      } else {
        if (ch > 0) store_o(ch - 1);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's loads of chunk ch+1
      }
    } else {
      chain(ch);
      read_out_compute(ch);
    }
    GDR_MARK(2);
    lds_barrier_keep_vm();  // B: chunk ch+1 is in buffer (ch+1) mod 2, O of chunk ch in its O buffer
  }
  if (wave == 0 && nch > 0) store_o(nch - 1);

  if (!loader && a.S_T != nullptr) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int64_t sb = bh * DK * DV + col0 + cb + 16 * ct + l16;
#pragma unroll
      for (int tl = 0; tl < NTD; ++tl)
#pragma unroll
        for (int i = 0; i < 4; ++i) a.S_T[sb + (int64_t)perm_row(tl, 4 * g + i) * DV] = S[ct][tl][i];
    }
  }
}

}  // namespace gdr
