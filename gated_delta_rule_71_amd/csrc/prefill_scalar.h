// Chunkwise prefill for a scalar (or no) decay with a scalar (or no) erase gate, software-
// pipelined across chunks on gfx950.
//
// The chunk form is the rank-one one of prefill_kernel.h (MODE 0) with every per-token factor
// kept out of the matrix operands, so the operands are the raw q and k:
//     V = diag(beta_t e^{G_t}) (K S) - X,      (I + A) R = V,
//     O = diag(e^{G_t}) (Q S) - M R,           S' = e^{G_n} S - K^T (diag(e^{G_n - G_t}) R)
// with A[t,i] = beta_t (k_t . k_i) e^{G_t - G_i} (i < t) and M[t,i] = (q_t . k_i) e^{G_t - G_i}
// (i <= t): the exact pairwise decay, safe for any gate values.  ("Recurrent Memory: Write,
// Erase, Decay, Read": section 03 for the linear, reassociable erase and section 04 for the
// decay as prefix sums of log alpha; the scalar gate of section 05's Gated DeltaNet setting.)
//
// Workgroup = 4 key waves + NSW state waves.  Operands live in two LDS buffers (chunk c in one,
// c+1 in the other).  Iteration c of the chunk loop has three barrier-separated intervals:
//     1: key waves 0-1: inverses of the 16x16 diagonal blocks of (I + A) for c;
//        key waves 2-3: M tiles of c                             | state: K S, Q S of c
//     2: key: operands of c+1 from prefetched registers           | state: solve of c
//     3: key: prefetch c+2; waves 0-1: A tiles (and the fp32 diagonal blocks) of c+1
//                                                                 | state: O of c, S update
#pragma once
#include "gdr_common.h"
#include "mfma.h"
#include "prefill_kernel.h"

namespace gdr {

template <int DK, int NSW>
struct ScalarLayout {
  static constexpr int C = 64;
  static constexpr int DVS = 16 * NSW;
  static constexpr int LDT = DK + 8;  // token-major rows (q, k)
  static constexpr int LDD = C + 8;   // channel-major rows (k^T), X^T rows, M rows
  static constexpr int LDA = 48 + 8;  // packed off-diagonal blocks of -A: rows 16..63, cols 0..47
  static constexpr int LDI = 24;
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + C * LDT * 2;
  static constexpr int oKT = oK + C * LDT * 2;
  static constexpr int oX = oKT + DK * LDD * 2;
  static constexpr int oA = oX + DVS * LDD * 2;
  static constexpr int oM = oA + 48 * LDA * 2;
  static constexpr int oI = oM + C * LDD * 2;
  static constexpr int oS = oI + 4 * 16 * LDI * 2;  // fp32: G, e^G, e^{Gn-G}, beta (64 each), e^Gn
  static constexpr int BUF = oS + (4 * C + 4) * 4;   // bytes per buffer
  static constexpr int LDL = 20;                     // column pitch of the fp32 diagonal blocks
  static constexpr int oLD = 2 * BUF;                // fp32 diagonal blocks of A, column-major
  static constexpr int total = oLD + 4 * 16 * LDL * 4;
  static constexpr bool fits = total <= kLdsLimit;
};

typedef int i32x4 __attribute__((ext_vector_type(4)));


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
    // element stores: writing the four values as one 8-byte store gave wrong M rows on the
    // dk <= 64 instantiations (not understood; element stores verified on every shape tested)
    __bf16* dst = prod == 1 ? gM + r * LDD + cc0 : gA + (r - 16) * LDA + cc0;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = o[i];
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

template <int DK, int NSW>
__global__ __launch_bounds__(256 + 64 * NSW) void prefill_scalar_kernel(PrefillArgs<bf16_t> a) {
  using L = ScalarLayout<DK, NSW>;
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  static_assert(L::fits, "LDS layout exceeds the gfx950 workgroup limit");
  static_assert(DK % 32 == 0, "dk must be a multiple of 32");
  constexpr int C = L::C, DVS = L::DVS, LDT = L::LDT, LDD = L::LDD, LDA = L::LDA, LDI = L::LDI;
  constexpr int NTD = DK / 16, NKB = DK / 32;
  constexpr int NCG = DK / 8;              // 8-channel groups of a token row
  constexpr int IPT = C * NCG / 256;       // (token, group) items per key thread for q and k
  constexpr int NXG = DVS / 8;             // 8-column groups of the value slice
  constexpr int XPT = (C * NXG + 255) / 256;

  __shared__ __attribute__((aligned(32))) unsigned char smem[L::total];
  float* Ld = reinterpret_cast<float*>(smem + L::oLD);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches on it
  int lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const bool key = wave < 4;

  const int64_t nb = gridDim.x, bid = blockIdx.x;
  const int64_t p = (nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
  const int64_t bh = p / a.nsl;
  const int sl = static_cast<int>(p % a.nsl);
  const int64_t bi = bh / a.H, hi = bh % a.H;
  const int64_t DV = a.DV, T = a.T, H = a.H;
  const int64_t col0 = static_cast<int64_t>(sl) * DVS;
  const int64_t nch = (T + C - 1) / C;

  auto buf = [&](int64_t c) -> unsigned char* { return smem + (c & 1) * L::BUF; };

  // zero both M buffers: tiles above the diagonal are read as zero and never written
  for (int b2 = 0; b2 < 2; ++b2) {
    uint32_t* z = reinterpret_cast<uint32_t*>(smem + b2 * L::BUF + L::oM);
    for (int i = tid; i < C * LDD / 2; i += blockDim.x) z[i] = 0u;
  }

  // ---------------- key-side prefetch registers ----------------
  // Buffer resources start at token 0 of this (batch, head); a token's row is H rows further.
  const int64_t row0 = bi * T * H + hi;
  const uint32_t tok_rows = static_cast<uint32_t>((T - 1) * H + 1);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + row0 * DK, tok_rows * DK * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + row0 * DK, tok_rows * DK * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + row0 * DV + col0, (tok_rows * DV - col0) * 2);
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(a.wg == nullptr ? a.v : (a.w_kind == kChannel ? a.wg + row0 * DV + col0 : a.wg + row0),
                a.w_kind == kChannel ? (tok_rows * DV - col0) * 2 : tok_rows * 2);
  const __amdgpu_buffer_rsrc_t rla = make_rsrc(a.la == nullptr ? a.q : a.la + row0, tok_rows * 2);
  const __amdgpu_buffer_rsrc_t rbg = make_rsrc(a.bg == nullptr ? a.q : a.bg + row0, tok_rows * 2);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.o + row0 * DV + col0, (tok_rows * DV - col0) * 2);
  const uint32_t hdk2 = static_cast<uint32_t>(H * DK * 2), hdv2 = static_cast<uint32_t>(H * DV * 2);
  const uint32_t h2 = static_cast<uint32_t>(H * 2);

  uint4 pq[IPT], pk[IPT], pv[XPT], pw[XPT];
  uint16_t pws[XPT];
  uint16_t pla = 0, pbeta = 0;

  auto prefetch = [&](int64_t c) {
    const uint32_t t0 = static_cast<uint32_t>(c * C);
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const uint32_t t = (tid / NCG) * IPT + j, cg = tid % NCG;
      pq[j] = buf_load16(rq, (t0 + t) * hdk2 + cg * 16);
      pk[j] = buf_load16(rk, (t0 + t) * hdk2 + cg * 16);
    }
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int item = tid + 256 * j;
      const uint32_t t = item / NXG, xg = item % NXG;
      pv[j] = make_uint4(0, 0, 0, 0);
      pw[j] = make_uint4(0, 0, 0, 0);
      pws[j] = 0x3f80;  // bf16 1.0
      if (item < C * NXG) {
        pv[j] = buf_load16(rv, (t0 + t) * hdv2 + xg * 16);
        if (a.w_kind == kChannel) pw[j] = buf_load16(rw, (t0 + t) * hdv2 + xg * 16);
        if (a.w_kind == kScalar) pws[j] = buf_load_u16(rw, (t0 + t) * h2);
      }
    }
    pla = 0;
    pbeta = 0;
    if (wave == 0) {
      if (a.alpha_kind != kNone) pla = buf_load_u16(rla, (t0 + lane) * h2);
      if (a.b_kind != kNone) pbeta = buf_load_u16(rbg, (t0 + lane) * h2);
    }
  };

  // ---------------- key phase 1: operands of chunk c into its buffer ----------------
  auto key_operands = [&](int64_t c) {
    unsigned char* B = buf(c);
    __bf16* tQ = reinterpret_cast<__bf16*>(B + L::oQ);
    __bf16* tK = reinterpret_cast<__bf16*>(B + L::oK);
    __bf16* kT = reinterpret_cast<__bf16*>(B + L::oKT);
    __bf16* xT = reinterpret_cast<__bf16*>(B + L::oX);
    float* sc = reinterpret_cast<float*>(B + L::oS);
    {
      // this thread holds channels cg*8..cg*8+7 of tokens tb..tb+IPT-1
      const int cg = tid % NCG, tb = (tid / NCG) * IPT;
      uint16_t kh[8][IPT];
#pragma unroll
      for (int j = 0; j < IPT; ++j) {
        *reinterpret_cast<uint4*>(tQ + (tb + j) * LDT + cg * 8) = pq[j];
        *reinterpret_cast<uint4*>(tK + (tb + j) * LDT + cg * 8) = pk[j];
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
        uint16_t* dst = kTu + row * LDD + swz((row >> 3) & 15, tb);
        if constexpr (IPT == 4) {
          *reinterpret_cast<uint2*>(dst) =
              make_uint2(kh[e][0] | (uint32_t(kh[e][1]) << 16), kh[e][2] | (uint32_t(kh[e][3]) << 16));
        } else if constexpr (IPT == 2) {
          *reinterpret_cast<uint32_t*>(dst) = kh[e][0] | (uint32_t(kh[e][1]) << 16);
        } else {
          dst[0] = kh[e][0];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int item = tid + 256 * j;
      if (item < C * NXG) {
        const int t = item / NXG, xg = item % NXG;
        float v8[8], w8[8];
        load8f(reinterpret_cast<const bf16_t*>(&pv[j]), v8);
        if (a.w_kind == kChannel) {
          load8f(reinterpret_cast<const bf16_t*>(&pw[j]), w8);
#pragma unroll
          for (int e = 0; e < 8; ++e) v8[e] *= w8[e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v8[e] *= bf16_to_f32(pws[j]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) xT[(xg * 8 + e) * LDD + swz(2 * xg, t)] = static_cast<__bf16>(v8[e]);
      }
    }
    if (wave == 0) {
      // per-token scalars: G_t (inclusive prefix of log alpha), e^{G_t}, e^{Gn - G_t}, beta_t
      float x = bf16_to_f32(pla);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      const float gn = __shfl(x, 63);
      sc[lane] = x;
      sc[C + lane] = __expf(x);
      sc[2 * C + lane] = __expf(gn - x);
      sc[3 * C + lane] = bf16_to_f32(pbeta);
      if (lane == 0) sc[4 * C] = __expf(gn);
    }
  };

  // ---------------- key phase 2: Gram tiles of chunk c ----------------
  auto key_gram = [&](int64_t c) {
    unsigned char* B = buf(c);
    const __bf16* tQ = reinterpret_cast<const __bf16*>(B + L::oQ);
    const __bf16* tK = reinterpret_cast<const __bf16*>(B + L::oK);
    __bf16* gA = reinterpret_cast<__bf16*>(B + L::oA);
    __bf16* gM = reinterpret_cast<__bf16*>(B + L::oM);
    const float* sc = reinterpret_cast<const float*>(B + L::oS);
    const int prod = wave >> 1;  // 0: A from k k^T, 1: M from q k^T; row blocks {0,3} or {1,2}
    const __bf16* rows = prod == 0 ? tK : tQ;
    if (wave & 1)
      scalar_gram_pair<DK, 1, 2, LDT, LDD, LDA, L::LDL>(rows, tK, prod, g, l16, sc, gA, gM, Ld);
    else
      scalar_gram_pair<DK, 0, 3, LDT, LDD, LDA, L::LDL>(rows, tK, prod, g, l16, sc, gA, gM, Ld);
  };

  // ---------------- key phase 3: inverses of the diagonal blocks of (I + A) ----------------
  // Wave 0 computed the diagonal Gram tiles of row blocks 0 and 3, wave 1 those of 1 and 2;
  // each inverts its own two blocks (lanes 0-15 and 16-31, one column per lane), reading the
  // fp32 tiles it wrote itself, so no barrier separates the two steps.
  auto key_inverse = [&](int64_t c) {
    __bf16* dInv = reinterpret_cast<__bf16*>(buf(c) + L::oI);
    if (wave < 2 && lane < 32) {
      const int blk = (lane < 16) ? (wave == 0 ? 0 : 1) : (wave == 0 ? 3 : 2);
      const int j = l16;
      // column sweep: once x_m is final, every later x_i drops L[i][m] x_m (independent FMAs);
      // column m+1 is read while column m is applied
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
      float4 col[2][4];
      auto load_col = [&](int m, float4* c) {
        const float* p = Ld + (blk * 16 + m) * L::LDL;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          if (4 * q4 + 3 > m) c[q4] = *reinterpret_cast<const float4*>(p + 4 * q4);
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
  };

  // ---------------- state waves ----------------
  const int sw = wave - 4;               // state wave index (valid when !key)
  const int nloc = 16 * sw + l16;        // local value column
  const int64_t sbase = bh * DK * DV + col0 + nloc;
  f32x4 S[NTD];
#pragma unroll
  for (int tl = 0; tl < NTD; ++tl) {
    S[tl] = zero4();
    if (!key && a.S0 != nullptr) {
#pragma unroll
      for (int i = 0; i < 4; ++i) S[tl][i] = a.S0[sbase + (int64_t)(16 * tl + 4 * g + i) * DV];
    }
  }
  F8 rsf[2];  // -R e^{G_n - G_t} as B fragments: from the solve to the state update

  // ---------------- prologue: operands and A tiles of chunk 0 ----------------
  if (key && nch > 0) {
    prefetch(0);
    key_operands(0);
  }
  lds_barrier();
  if (key && nch > 1) prefetch(1);
  if (key && wave < 2 && nch > 0) key_gram(0);
  lds_barrier();

  for (int64_t ch = 0; ch < nch; ++ch) {
    // Lane indices are made opaque once per chunk so that the compiler recomputes the
    // lane-dependent LDS addresses inside the loop instead of holding dozens of them (and the
    // identity used by the inverse) in registers across it, which spilled to scratch; every
    // scratch reload waits for all outstanding global loads and defeated the prefetch.
    asm volatile("" : "+v"(lane), "+v"(g), "+v"(l16));
    const int64_t t0 = ch * C;
    unsigned char* B = buf(ch);
    const float* sc = reinterpret_cast<const float*>(B + L::oS);
    const bool more = ch + 1 < nch;
    f32x4 V[4], O[4], R[4];
    F8 rf0, rf1;

    // ---- interval 1: inverse and M tiles of chunk ch | K S and Q S ----
    GDR_MARK(0);
    if (key) {
      if (wave < 2)
        key_inverse(ch);
      else
        key_gram(ch);
    } else {
      const __bf16* tQ = reinterpret_cast<const __bf16*>(B + L::oQ);
      const __bf16* tK = reinterpret_cast<const __bf16*>(B + L::oK);
      const __bf16* xT = reinterpret_cast<const __bf16*>(B + L::oX);
      F8 sf[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sf[kb] = acc_pair_frag<__bf16>(S[2 * kb], S[2 * kb + 1]);
      // operand fragments of row tile ta+1 are read while the MFMAs of tile ta run
      F8 kf[2][NKB], qf[2][NKB];
      auto load_tile = [&](int ta, F8* kfo, F8* qfo) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          kfo[kb] = lds_pair_frag_k<DK>(tK + (16 * ta + l16) * LDT, 32 * kb, g);
          qfo[kb] = lds_pair_frag_k<DK>(tQ + (16 * ta + l16) * LDT, 32 * kb, g);
        }
      };
      load_tile(0, kf[0], qf[0]);
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) {
        if (ta < 3) load_tile(ta + 1, kf[(ta + 1) & 1], qf[(ta + 1) & 1]);
        const float4 e4 = *reinterpret_cast<const float4*>(sc + C + 16 * ta + 4 * g);
        const float4 b4 = *reinterpret_cast<const float4*>(sc + 3 * C + 16 * ta + 4 * g);
        const bf16x4 x4 =
            *reinterpret_cast<const bf16x4*>(xT + nloc * LDD + swz(2 * (nloc >> 3), 16 * ta + 4 * g));
        V[ta] = zero4();
        O[ta] = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          V[ta] = MM::mma8(kf[ta & 1][kb], sf[kb], V[ta]);
          O[ta] = MM::mma8(qf[ta & 1][kb], sf[kb], O[ta]);
        }
        const float e[4] = {e4.x, e4.y, e4.z, e4.w}, bt[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          V[ta][i] = V[ta][i] * e[i] * bt[i] - static_cast<float>(x4[i]);
          O[ta][i] *= e[i];
        }
      }
    }
    GDR_MARK(1);
    lds_barrier();

    // ---- interval 2: operands of chunk ch+1 | solve ----
    GDR_MARK(2);
    if (key) {
      if (more) key_operands(ch + 1);
    } else {
      const __bf16* gA = reinterpret_cast<const __bf16*>(B + L::oA);
      const __bf16* dInv = reinterpret_cast<const __bf16*>(B + L::oI);
      bf16x4 af[6], tf[4];
#pragma unroll
      for (int i = 0, n = 0; i < 4; ++i) {
        tf[i] = lds_load4(dInv + (16 * i + l16) * LDI + 4 * g);
#pragma unroll
        for (int m = 0; m < i; ++m, ++n) af[n] = lds_load4(gA + (16 * i - 16 + l16) * LDA + 16 * m + 4 * g);
      }
#pragma unroll
      for (int i = 0, n = 0; i < 4; ++i) {
#pragma unroll
        for (int m = 0; m < i; ++m, ++n) V[i] = MM::mma4(af[n], acc_frag4<__bf16>(R[m]), V[i]);
        R[i] = MM::mma4(tf[i], acc_frag4<__bf16>(V[i]), zero4());
      }
      rf0 = acc_pair_frag<__bf16>(R[0], R[1]);
      rf1 = acc_pair_frag<__bf16>(R[2], R[3]);
      f32x4 Rs[4];
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) {
        const float4 r4 = *reinterpret_cast<const float4*>(sc + 2 * C + 16 * ta + 4 * g);
        const float rr[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) Rs[ta][i] = -R[ta][i] * rr[i];
      }
      rsf[0] = acc_pair_frag<__bf16>(Rs[0], Rs[1]);
      rsf[1] = acc_pair_frag<__bf16>(Rs[2], Rs[3]);
    }
    GDR_MARK(3);
    lds_barrier();

    // ---- interval 3: prefetch, A tiles of chunk ch+1 | O and S update ----
    GDR_MARK(4);
    if (key) {
      if (ch + 2 < nch) prefetch(ch + 2);
      if (wave < 2 && more) key_gram(ch + 1);
    } else {
      const __bf16* gM = reinterpret_cast<const __bf16*>(B + L::oM);
      const __bf16* kT = reinterpret_cast<const __bf16*>(B + L::oKT);
      F8 mf[6];
#pragma unroll
      for (int ta = 0, n = 0; ta < 4; ++ta) {
        mf[n++] = lds_pair_frag_k<C>(gM + (16 * ta + l16) * LDD, 0, g);
        if (ta >= 2) mf[n++] = lds_pair_frag_k<C>(gM + (16 * ta + l16) * LDD, 32, g);
      }
      F8 kf[2][2];
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
      load_kt(0, kf[0]);
#pragma unroll
      for (int ta = 0, n = 0; ta < 4; ++ta) {
        O[ta] = MM::mma8(mf[n++], rf0, O[ta]);
        if (ta >= 2) O[ta] = MM::mma8(mf[n++], rf1, O[ta]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t t = static_cast<uint32_t>(t0) + 16 * ta + 4 * g + i;
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(O[ta][i]), ro, t * hdv2 + nloc * 2, 0, 0);
        }
      }
      const F8 sf0 = rsf[0], sf1 = rsf[1];
      const float egn = sc[4 * C];
#pragma unroll
      for (int tl = 0; tl < NTD; ++tl) {
        if (tl + 1 < NTD) load_kt(tl + 1, kf[(tl + 1) & 1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) S[tl][i] *= egn;
        S[tl] = MM::mma8(kf[tl & 1][0], sf0, S[tl]);
        S[tl] = MM::mma8(kf[tl & 1][1], sf1, S[tl]);
      }
    }
    GDR_MARK(5);
    lds_barrier();
  }

  if (!key && a.S_T != nullptr) {
#pragma unroll
    for (int tl = 0; tl < NTD; ++tl)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.S_T[sbase + (int64_t)(16 * tl + 4 * g + i) * DV] = S[tl][i];
  }
}

}  // namespace gdr
