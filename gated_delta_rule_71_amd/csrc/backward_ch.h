// Chunk-local adjoint for a per-channel decay (the Gated DeltaNet-2 and KDA gates), bf16 I/O,
// d_k = 128, d_v = 64 or 128, both orders of erase and decay.
//
// The chunk maps, the chains over the chunks and the checkpoints S_{c-1} and dS_c come from the
// same kernels as for a scalar decay (backward.h); this file replaces only the chunk-local step.
//
// One chunk of n = 64 tokens from the state S_0 that enters it, with c = b . k, X = w . v and the
// per-channel prefix sums G_t of log alpha from the chunk's start (G_{-1} = 0), in the split form
// ("Recurrent Memory: Write, Erase, Decay, Read", sections 03 and 04; the Gated DeltaNet-2
// abstract for the channel-wise decay folded into separate erase factors):
//   erase then decay:  Qh = q e^{G_t}, Kh = k e^{-G_t}, Ch = c e^{G_{t-1}}, Ph = k e^{-G_{t-1}}
//   decay then erase:  Qh = q e^{G_t}, Kh = Ph = k e^{-G_t}, Ch = c e^{G_t}
//   L_P = strict_tril(Ch Ph^T), L_K = strict_tril(Ch Kh^T), M_QK = tril(Qh Kh^T),
//   M_QP = tril(Qh Ph^T), T = (I + L_P)^{-1}
//   R = T (Ch S_0 + L_K X)    (R_t is the erase read of token t)
//   O = Qh S_0 + M_QK X - M_QP R,   S_n = e^{G_n} . Sh,  Sh = S_0 + Kh^T X - Ph^T R
// Its adjoint, given dO and dS_n (dSh = e^{G_n} . dS_n):
//   dR = -M_QP^T dO - Ph dSh,   dV = T^T dR,   dX = M_QK^T dO + Kh dSh + L_K^T dV
//   dM_QK = tril(dO X^T), dM_QP = -tril(dO R^T), dL_K = strict_tril(dV X^T),
//   dL_P = -strict_tril(dV R^T)
//   dQh = dO S_0^T + dM_QK Kh + dM_QP Ph,   dKh = X dSh^T + dM_QK^T Qh + dL_K^T Ch
//   dCh = dV S_0^T + dL_K Kh + dL_P Ph,     dPh = -R dSh^T + dM_QP^T Qh + dL_P^T Ch
// and back through the split factors: dq = dQh e^{G_t}, dk = dKh e^{-G_t} + dPh e^{-G_{t-1}} +
// b . dc, dc = dCh e^{G_{t-1}}, db = k . dc, dv = w . dX, dw = v . dX; the gradient of G_t
// collects dq . q - (dKh e^{-G_t}) . k at t, dc . c - (dPh e^{-G_{t-1}}) . k at t - 1 and
// sum_j dSh . Sh at the last token, and d log alpha_t is its suffix sum over the chunk.  (With the
// decay first every factor sits at G_t and Ph = Kh, so the same code runs with the two key
// families, and the two M and L families, equal.)
//
// The factors stay inside the bf16 and fp32 range while |G_t| <= 76 over the chunk; the products
// only ever pair them as e^{G_t - G_s} with t >= s, or with S_0 and dS_n as e^{G_t} and e^{G_n -
// G_t}.  A chunk past that (or with a non-finite gate) is flagged: bwd_chl_kernel leaves it, and
// bwd_chl_token_kernel differentiates it token by token in fp32 from its checkpoint, exactly for
// any gate values.  bwd_chl_kernel records which chunks it left in a.cflag.
#pragma once

#include "backward.h"

namespace gdr {

constexpr float kChlSpanLimit = 76.f;

// 8 bytes through a buffer resource (reads past its range return zeros)
__device__ __forceinline__ uint2 chl_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ void chl_unpack4(uint2 u, float* f) {
  f[0] = __uint_as_float(u.x << 16);
  f[1] = __uint_as_float(u.x & 0xffff0000u);
  f[2] = __uint_as_float(u.y << 16);
  f[3] = __uint_as_float(u.y & 0xffff0000u);
}
__device__ __forceinline__ uint2 chl_pack4(const float* f) {
  bf16x4 b;
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = static_cast<__bf16>(f[i]);
  return __builtin_bit_cast(uint2, b);
}
// -x for every element of a bf16 fragment (the sign bits)
__device__ __forceinline__ Mma<__bf16>::F8 chl_neg8(const Mma<__bf16>::F8& f) {
  uint4 u = __builtin_bit_cast(uint4, f);
  u.x ^= 0x80008000u;
  u.y ^= 0x80008000u;
  u.z ^= 0x80008000u;
  u.w ^= 0x80008000u;
  return __builtin_bit_cast(Mma<__bf16>::F8, u);
}

// Per-channel prefix sums of log alpha over the chunk by a workgroup of 512 threads (channel
// tid % 128, tokens 16 (tid / 128) .. + 15; the four partial sums are joined through qtot, 4 x 128
// fp32): G[t][ch] into sG (64 x 128 fp32) and, when fGn is given, e^{G_63} into fGn; a chunk with
// any |G_t| > 76 or a non-finite one sets *flag.  Tokens past the state's end read as log alpha =
// 0.  The loads (chl_prefix_load) are issued ahead of the sums, so that their latency overlaps
// other work.  Every thread calls both; the caller zeroes *flag and places a barrier before and
// after chl_prefix.
// x through an empty asm statement: values derived from it are formed where they are used.
__device__ __forceinline__ int chl_opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

struct ChlRaw {
  uint16_t v[16];
};
__device__ __forceinline__ ChlRaw chl_prefix_load(const BwdArgs& a, int64_t rr, int64_t left, int tid) {
  const int ch = tid & 127, q = tid >> 7;
  const auto rla = make_rsrc(a.la + rr * 128, wy_range(left, a.H, 128));
  const uint32_t hdk = static_cast<uint32_t>(a.H * 128 * 2);
  ChlRaw r;
#pragma unroll
  for (int u = 0; u < 16; ++u) r.v[u] = buf_load_u16(rla, (16 * q + u) * hdk + ch * 2);
  return r;
}
__device__ __forceinline__ void chl_prefix(const ChlRaw& raw, float* sG, float* fGn, float* qtot, int* flag,
                                           int tid) {
  const int ch = tid & 127, q = tid >> 7;
  float G[16];
  float run = 0.f;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    run += bf16_to_f32(raw.v[u]);
    G[u] = run;
  }
  qtot[q * 128 + ch] = run;
  lds_barrier();
  float off = 0.f;
  for (int j = 0; j < q; ++j) off += qtot[j * 128 + ch];
  bool ok = true;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const float x = G[u] + off;
    ok = ok && fabsf(x) <= kChlSpanLimit;
    sG[(16 * q + u) * 128 + ch] = x;
  }
  if (fGn != nullptr && q == 3) fGn[ch] = __expf(G[15] + off);
  if (!ok) atomicOr(flag, 1);
}

template <int MODE>
struct ChlLayout {
  static constexpr bool TWO = MODE == 2;
  static constexpr int C = 64, DK = 128, DVH = 64;
  static constexpr int LDT = DK + 8;   // rows of Qh, Kh, Ch, Ph
  static constexpr int LDX = DVH + 8;  // rows of one value half: X, dO, R, and B' / dR / dV
  static constexpr int LDD = C + 8;    // rows of the 64 x 64 Gram matrices
  static constexpr int LDA = 56, LDI = 24, LDL = 20;
  static constexpr int ROWS = C * LDT * 2, HALF = C * LDX * 2, GRAM = C * LDD * 2;
  static constexpr int oQ = 0, oK = ROWS, oC = 2 * ROWS, oP = TWO ? 3 * ROWS : oK;
  static constexpr int OPS = (TWO ? 4 : 3) * ROWS;
  // Gram matrices: L_K (decay first: L), M_QK (decay first: M), M_QP (erase first only), T
  static constexpr int oLK = OPS, oMQK = oLK + GRAM, oMQP = TWO ? oMQK + GRAM : oMQK;
  static constexpr int oT = (TWO ? oMQP : oMQK) + GRAM;
  // one value half: X, dO, R, and W (B' = Ch S_0 + L_K X, then dR, then dV)
  static constexpr int oX = oT + GRAM, oO = oX + HALF, oR = oO + HALF, oW = oR + HALF;
  // fp32: e^{G_n} [128], (unused) [128], scalar db [64], (unused) [64], the flag; the partial
  // sums of the prefix and suffix scans [4][128]
  static constexpr int oF = oW + HALF;
  static constexpr int oQT = oF + (128 + 128 + 64 + 64 + 4) * 4;
  // fixed-order partial sums (no float atomics, so a call's bits do not depend on timing): the
  // per-channel end-of-chunk terms [5][128] and a scalar dw's per-token terms [2][2][2][64]
  static constexpr int oPS = oQT + 4 * 128 * 4;
  static constexpr int total = oPS + (5 * 128 + 8 * 64) * 4;
  // aliases: the prefix sums (fp32 [64][128]) over the half area in the prologue, the pieces of
  // the triangular inverse there too; after the products, G (again) and the per-token gate
  // gradients over the operand area, and (erase first) the gradients of G_{t-1} over the half area
  static constexpr int oG = oX;
  static constexpr int oGA = oX, oLD = oGA + 48 * LDA * 2, oI = oLD + C * LDL * 4;
  static constexpr int oG2 = 0, oDG = TWO ? 32768 : oX, oDGP = oX;
  static_assert(4 * HALF >= 32768 && oI + C * LDI * 2 <= oX + 4 * HALF, "aliases fit the half area");
  static_assert(!TWO || OPS >= 2 * 32768, "G and its gradient fit the operand area");
  static constexpr bool fits = total <= kLdsLimit;
};

// One workgroup of 8 waves per (state, chunk); chunks flagged by chl_prefix are marked in
// a.cflag and left to bwd_chl_token_kernel.  Value columns are taken in halves of 64 (the per-half
// products in LDS); the gradients summed over value columns accumulate in registers across the
// halves.  Global operands (checkpoint fragments, input rows) are loaded ahead of the phase that
// uses them, so that one load latency is paid per phase.
template <int MODE>
__global__ __launch_bounds__(512) void bwd_chl_kernel(BwdArgs a) {
  using L = ChlLayout<MODE>;
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  static_assert(L::fits, "LDS layout exceeds the gfx950 workgroup limit");
  constexpr bool TWO = L::TWO;
  constexpr int C = L::C, DK = L::DK, DVH = L::DVH, LDT = L::LDT, LDX = L::LDX, LDD = L::LDD,
                LDA = L::LDA, LDI = L::LDI, LDL = L::LDL, NT = 512;
  constexpr int NGJ = TWO ? 5 : 3;  // Gram-gradient jobs per wave (40 or 20 over 8 waves)

  __shared__ __attribute__((aligned(32))) unsigned char smem[L::total];
  __bf16* sQ = reinterpret_cast<__bf16*>(smem + L::oQ);
  __bf16* sK = reinterpret_cast<__bf16*>(smem + L::oK);
  __bf16* sC = reinterpret_cast<__bf16*>(smem + L::oC);
  __bf16* sP = reinterpret_cast<__bf16*>(smem + L::oP);
  __bf16* sLK = reinterpret_cast<__bf16*>(smem + L::oLK);
  __bf16* sMQK = reinterpret_cast<__bf16*>(smem + L::oMQK);
  __bf16* sMQP = reinterpret_cast<__bf16*>(smem + L::oMQP);
  __bf16* sT = reinterpret_cast<__bf16*>(smem + L::oT);
  __bf16* sX = reinterpret_cast<__bf16*>(smem + L::oX);
  __bf16* sO = reinterpret_cast<__bf16*>(smem + L::oO);
  __bf16* sR = reinterpret_cast<__bf16*>(smem + L::oR);
  __bf16* sW = reinterpret_cast<__bf16*>(smem + L::oW);
  float* fGn = reinterpret_cast<float*>(smem + L::oF);
  float* fdb = fGn + 256;
  int* sFlag = reinterpret_cast<int*>(fGn + 384);
  float* qtot = reinterpret_cast<float*>(smem + L::oQT);
  float* pGn = reinterpret_cast<float*>(smem + L::oPS);  // [5][128]
  float* pw = pGn + 5 * 128;                             // [half][wave & 1][u][64]
  float* sG = reinterpret_cast<float*>(smem + L::oG);
  __bf16* gA = reinterpret_cast<__bf16*>(smem + L::oGA);
  float* Ld = reinterpret_cast<float*>(smem + L::oLD);
  __bf16* dInv = reinterpret_cast<__bf16*>(smem + L::oI);

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nch = a.nch, DV = a.DV, H = a.H, Hk = a.Hk;
  const int64_t bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int64_t bi = bh / H, hi = bh % H, hk = hi / (H / Hk);
  const int64_t t0 = c * C, left = a.T - t0;
  const int64_t rr = (bi * a.T + t0) * H + hi;   // value-head row of the chunk's first token
  const int64_t rqk = (bi * a.T + t0) * Hk + hk;  // q / k row
  const int64_t cix = bh * nch + c;
  const __bf16* SR = a.SR + cix * DK * DV;
  const __bf16* ST = a.ST + cix * DV * DK;
  const __bf16* GR = a.GR + cix * DK * DV;
  const __bf16* GT = a.GT + cix * DV * DK;
  const uint32_t hdk = static_cast<uint32_t>(H * DK * 2), hqk = static_cast<uint32_t>(Hk * DK * 2);
  const uint32_t hdv = static_cast<uint32_t>(H * DV * 2), h1 = static_cast<uint32_t>(H * 2);
  const uint32_t rng_k = wy_range(left, H, DK), rng_v = wy_range(left, H, DV), rng_1 = wy_range(left, H, 1);
  const auto rq = make_rsrc(a.q + rqk * DK, wy_range(left, Hk, DK));
  const auto rk = make_rsrc(a.k + rqk * DK, wy_range(left, Hk, DK));
  const auto rbc = make_rsrc(a.b_kind == kChannel ? a.bg + rr * DK : a.q, a.b_kind == kChannel ? rng_k : 0u);
  const auto rbs = make_rsrc(a.b_kind == kScalar ? a.bg + rr : a.q, a.b_kind == kScalar ? rng_1 : 0u);
  const auto rv = make_rsrc(a.v + rr * DV, rng_v);
  const auto rwc = make_rsrc(a.w_kind == kChannel ? a.wg + rr * DV : a.v, a.w_kind == kChannel ? rng_v : 0u);
  const auto rws = make_rsrc(a.w_kind == kScalar ? a.wg + rr : a.v, a.w_kind == kScalar ? rng_1 : 0u);
  const auto rdo = make_rsrc(a.dO + rr * DV, rng_v);

  // ---- prologue: zero the Gram matrices (their upper tiles are read as zeros) and the sums;
  // the split's input rows and the rows of S_0 . dS_n are loaded before the prefix sums ----
  for (int i = tid; i < (L::oX - L::oLK) / 16; i += NT)
    reinterpret_cast<uint4*>(smem + L::oLK)[i] = make_uint4(0, 0, 0, 0);
  if (tid < 64) {
    fdb[tid] = 0.f;  // (two terms per token: their sum does not depend on the order)
    if (tid == 0) *sFlag = 0;
  }
  const ChlRaw la_raw = chl_prefix_load(a, rr, left, tid);
  uint2 uq[4], uk[4], ub[4];  // item j: token tid / 32 + 16 j, channels 4 (tid % 32) ..
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int item = tid + NT * j, t = item >> 5, i0 = (item & 31) * 4;
    uq[j] = chl_load8(rq, t * hqk + i0 * 2);
    uk[j] = chl_load8(rk, t * hqk + i0 * 2);
  }
  // (one loop per kind of b: a select between loads into one register would wait for the first)
  if (a.b_kind == kChannel) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int item = tid + NT * j, t = item >> 5, i0 = (item & 31) * 4;
      ub[j] = chl_load8(rbc, t * hdk + i0 * 2);
    }
  } else if (a.b_kind == kScalar) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = (tid + NT * j) >> 5;
      ub[j] = make_uint2(buf_load_u16(rbs, t * h1), 0u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) ub[j] = make_uint2(0u, 0u);
  }
  // sum_j S_0[ch][j] dS_n[ch][j]: channel tid / 4, columns (tid % 4) DV / 4 .. in 8-column pieces
  // (a piece of a tiled16 row is 16 contiguous bytes)
  const int dch = tid >> 2, dq4 = tid & 3, npc = static_cast<int>(DV / 32);
  uint4 us0[4], udn[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (u < npc) {
      const int col = dq4 * (npc * 8) + 8 * u;
      const int64_t o = tiled16(dch, col, DV);
      us0[u] = *reinterpret_cast<const uint4*>(SR + o);
      udn[u] = *reinterpret_cast<const uint4*>(GR + o);
    }
  }
  lds_barrier();
  chl_prefix(la_raw, sG, fGn, qtot, sFlag, tid);
  lds_barrier();
  const bool flagged = *sFlag != 0;
  if (tid == 0) a.cflag[cix] = flagged ? 1 : 0;
  if (flagged) return;  // (uniform) the token kernel takes this chunk
  {
    float dot = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u < npc) {
        float x[8], y[8];
        load8f(reinterpret_cast<const bf16_t*>(&us0[u]), x);
        load8f(reinterpret_cast<const bf16_t*>(&udn[u]), y);
#pragma unroll
        for (int e = 0; e < 8; ++e) dot += x[e] * y[e];
      }
    }
    dot += __shfl_xor(dot, 1);
    dot += __shfl_xor(dot, 2);
    if (dq4 == 0) pGn[dch] = fGn[dch] * dot;  // e^{G_n} <S_0, dS_n> per channel
  }

  // ---- split operands: 4 consecutive channels of one token per item ----
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int item = tid + NT * j, t = item >> 5, i0 = (item & 31) * 4;
    float q4[4], k4[4], c4[4], gt[4], gp[4];
    chl_unpack4(uq[j], q4);
    chl_unpack4(uk[j], k4);
    if (a.b_kind == kChannel) {
      chl_unpack4(ub[j], c4);
    } else {
      const float bs = bf16_to_f32(static_cast<uint16_t>(ub[j].x));
      c4[0] = c4[1] = c4[2] = c4[3] = bs;
    }
    const float4 g4 = *reinterpret_cast<const float4*>(sG + t * 128 + i0);
    const float4 p4 = t > 0 ? *reinterpret_cast<const float4*>(sG + (t - 1) * 128 + i0) : make_float4(0.f, 0.f, 0.f, 0.f);
    gt[0] = g4.x, gt[1] = g4.y, gt[2] = g4.z, gt[3] = g4.w;
    gp[0] = p4.x, gp[1] = p4.y, gp[2] = p4.z, gp[3] = p4.w;
    float oq[4], ok[4], oc[4], op[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c4[e] *= k4[e];
      oq[e] = q4[e] * __expf(gt[e]);
      ok[e] = k4[e] * __expf(-gt[e]);
      oc[e] = c4[e] * __expf(TWO ? gp[e] : gt[e]);
      op[e] = k4[e] * __expf(-gp[e]);
    }
    *reinterpret_cast<uint2*>(sQ + t * LDT + i0) = chl_pack4(oq);
    *reinterpret_cast<uint2*>(sK + t * LDT + i0) = chl_pack4(ok);
    *reinterpret_cast<uint2*>(sC + t * LDT + i0) = chl_pack4(oc);
    if (TWO) *reinterpret_cast<uint2*>(sP + t * LDT + i0) = chl_pack4(op);
  }
  lds_barrier();

  // the first half's v, w and dO rows and its B operands of dS_n and S_0, ahead of their use
  const int pta = wave >> 1, pcv0 = 2 * (wave & 1);
  const int st_t = tid >> 3, st_x0 = (tid & 7) * 8;
  uint4 uv, udo, uw = make_uint4(0, 0, 0, 0);
  uint16_t uws = 0;
  auto load_rows = [&](int c0) {
    const uint32_t off = st_t * hdv + (c0 + st_x0) * 2;
    uv = buf_load16(rv, off);
    udo = buf_load16(rdo, off);
    if (a.w_kind == kChannel)
      uw = buf_load16(rwc, off);
    else if (a.w_kind == kScalar)
      uws = buf_load_u16(rws, st_t * h1);
  };
  F8 dsf[2][4], s0c[2][4];
  auto load_s0c = [&](int c0) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s0c[u][kb] = tiled_row_frag(ST, DK, c0 + 16 * (pcv0 + u) + l16, 32 * kb, g);
  };
  auto load_dsf = [&](int c0) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) dsf[u][kb] = tiled_row_frag(GT, DK, c0 + 16 * (pcv0 + u) + l16, 32 * kb, g);
  };
  load_rows(0);

  // ---- Gram products: family 0 = L_P (to the inverse's pieces; decay first also to sLK as L),
  // 1 = L_K, 2 = M_QK, 3 = M_QP (decay first: families 0 and 2 only) ----
  {
    constexpr int NJ = TWO ? 40 : 20;
    for (int job = wave; job < NJ; job += 8) {
      const int fam = TWO ? job / 10 : (job / 10) * 2, tix = job % 10;
      const int ta = tix >= 6 ? 3 : tix >= 3 ? 2 : tix >= 1 ? 1 : 0, tb = tix - ta * (ta + 1) / 2;
      const __bf16* ar = (fam < 2 ? sC : sQ) + (16 * ta + l16) * LDT;
      const __bf16* br = ((fam == 0 || fam == 3) ? sP : sK) + (16 * tb + l16) * LDT;
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) acc = MM::mma8(lds_load8(ar + 32 * kb + 8 * g), lds_load8(br + 32 * kb + 8 * g), acc);
      const int s = 16 * tb + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * ta + 4 * g + i;
        const bool keep = fam < 2 ? s < t : s <= t;
        const float val = keep ? acc[i] : 0.f;
        if (fam == 0) {
          if (ta > tb)
            gA[(t - 16) * LDA + s] = static_cast<__bf16>(-val);
          else
            Ld[(ta * 16 + (s & 15)) * LDL + (t & 15)] = val;
          if (!TWO) sLK[t * LDD + s] = static_cast<__bf16>(val);
        } else if (fam == 1) {
          sLK[t * LDD + s] = static_cast<__bf16>(val);
        } else if (fam == 2) {
          sMQK[t * LDD + s] = static_cast<__bf16>(val);
        } else {
          sMQP[t * LDD + s] = static_cast<__bf16>(val);
        }
      }
    }
  }
  lds_barrier();
  if (wave < 2 && lane < 32) wy_diag_inverses<LDL, LDI>(Ld, dInv, wave, lane, l16);
  lds_barrier();
  // T = (I + L_P)^{-1}: wave j < 4 forms column block j by blocked forward substitution
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
      for (int e = 0; e < 4; ++e) sT[(16 * i + 4 * g + e) * LDD + 16 * j + l16] = static_cast<__bf16>(R[i][e]);
  }
  lds_barrier();

  // ---- accumulators carried over the value halves ----
  // Gram gradients: job u of this wave = wave + 8 u over (family, lower tile pair); families
  // dM_QK, dM_QP, dL_K, dL_P (decay first: dM, dL), accumulated without the triangular masks
  f32x4 gacc[NGJ];
#pragma unroll
  for (int u = 0; u < NGJ; ++u) gacc[u] = zero4();
  // operand gradients: token tile ta = wave & 3, channel tiles 4 (wave >> 2) + mi
  const int ota = wave & 3, om0 = 4 * (wave >> 2);
  f32x4 aq[4], ak[4], ac[4], ap[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) aq[mi] = ak[mi] = ac[mi] = ap[mi] = zero4();
  // ([token x value] tiles of the per-half products: token tile pta, value tiles pcv0, pcv0 + 1)

  const int nh = static_cast<int>(DV / DVH);
  for (int h = 0; h < nh; ++h) {
    const int c0 = DVH * h;
    // ---- the half's v, w and dO rows (loaded a phase or a half ahead) into X and dO; dS_n (for
    // dSh) and S_0 (for B') as B operands [k = channel][n = value column] of this wave's two value
    // tiles ----
    load_s0c(c0);
    {
      float xf[8], wf[8];
      load8f(reinterpret_cast<const bf16_t*>(&uv), xf);
      if (a.w_kind == kChannel) {
        load8f(reinterpret_cast<const bf16_t*>(&uw), wf);
      } else {
        const float ws = a.w_kind == kScalar ? bf16_to_f32(uws) : 1.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) wf[e] = ws;
      }
      bf16x8 xb;
#pragma unroll
      for (int e = 0; e < 8; ++e) xb[e] = static_cast<__bf16>(xf[e] * wf[e]);
      *reinterpret_cast<bf16x8*>(sX + st_t * LDX + st_x0) = xb;
      *reinterpret_cast<uint4*>(sO + st_t * LDX + st_x0) = udo;
    }
    lds_barrier();
    // ---- B' = Ch S_0 + L_K X, into W ----
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int cv = pcv0 + u;
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        acc = MM::mma8(lds_pair_frag_k<DK>(sC + (16 * pta + l16) * LDT, 32 * kb, g), s0c[u][kb], acc);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        if (ks <= (pta >> 1))
          acc = MM::mma8(lds_pair_frag_k<C>(sLK + (16 * pta + l16) * LDD, 32 * ks, g),
                         lds_col_frag(sX, LDX, 16 * cv + l16, 32 * ks, g, l16), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) sW[(16 * pta + 4 * g + i) * LDX + 16 * cv + l16] = static_cast<__bf16>(acc[i]);
    }
    lds_barrier();
    // ---- R = T B' ----
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int cv = pcv0 + u;
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        if (ks <= (pta >> 1))
          acc = MM::mma8(lds_pair_frag_k<C>(sT + (16 * pta + l16) * LDD, 32 * ks, g),
                         lds_col_frag(sW, LDX, 16 * cv + l16, 32 * ks, g, l16), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) sR[(16 * pta + 4 * g + i) * LDX + 16 * cv + l16] = static_cast<__bf16>(acc[i]);
    }
    lds_barrier();
    load_dsf(c0);
    // dSh = e^{G_n} . dS_n
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const float4 e0 = *reinterpret_cast<const float4*>(fGn + 32 * kb + 4 * g);
      const float4 e1 = *reinterpret_cast<const float4*>(fGn + 32 * kb + 16 + 4 * g);
      const float ee[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) dsf[u][kb][e] = static_cast<__bf16>(static_cast<float>(dsf[u][kb][e]) * ee[e]);
    }
    // ---- dR = -(M_QP^T dO + Ph dSh), into W ----
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int cv = pcv0 + u;
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        acc = MM::mma8(lds_pair_frag_k<DK>(sP + (16 * pta + l16) * LDT, 32 * kb, g), dsf[u][kb], acc);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        if (ks >= (pta >> 1))
          acc = MM::mma8(lds_col_frag(sMQP, LDD, 16 * pta + l16, 32 * ks, g, l16),
                         lds_col_frag(sO, LDX, 16 * cv + l16, 32 * ks, g, l16), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) sW[(16 * pta + 4 * g + i) * LDX + 16 * cv + l16] = static_cast<__bf16>(-acc[i]);
    }
    lds_barrier();
    // ---- dV = T^T dR, into W once every wave has read dR ----
    f32x4 dvt[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int cv = pcv0 + u;
      dvt[u] = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        if (ks >= (pta >> 1))
          dvt[u] = MM::mma8(lds_col_frag(sT, LDD, 16 * pta + l16, 32 * ks, g, l16),
                            lds_col_frag(sW, LDX, 16 * cv + l16, 32 * ks, g, l16), dvt[u]);
    }
    lds_barrier();
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sW[(16 * pta + 4 * g + i) * LDX + 16 * (pcv0 + u) + l16] = static_cast<__bf16>(dvt[u][i]);
    // (v and w at this wave's output positions, for dv and dw below)
    // (one loop per kind of w: a select between loads into one register would wait for the first)
    uint16_t ov[2][4], ow[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ov[u][i] = buf_load_u16(rv, (16 * pta + 4 * g + i) * hdv + (c0 + 16 * (pcv0 + u) + l16) * 2);
    if (a.w_kind == kChannel) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ow[u][i] = buf_load_u16(rwc, (16 * pta + 4 * g + i) * hdv + (c0 + 16 * (pcv0 + u) + l16) * 2);
    } else if (a.w_kind == kScalar) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) ow[u][i] = buf_load_u16(rws, (16 * pta + 4 * g + i) * h1);
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) ow[u][i] = 0;
    }
    lds_barrier();
    // ---- dX = M_QK^T dO + Kh dSh + L_K^T dV: dv = w . dX, dw = v . dX ----
    {
      const auto sv_ = make_rsrc(a.dv + rr * DV, rng_v);
      const auto swc = make_rsrc(a.w_kind == kChannel ? a.dw + rr * DV : a.dv, a.w_kind == kChannel ? rng_v : 0u);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int cv = pcv0 + u;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          acc = MM::mma8(lds_pair_frag_k<DK>(sK + (16 * pta + l16) * LDT, 32 * kb, g), dsf[u][kb], acc);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          if (ks >= (pta >> 1)) {
            acc = MM::mma8(lds_col_frag(sMQK, LDD, 16 * pta + l16, 32 * ks, g, l16),
                           lds_col_frag(sO, LDX, 16 * cv + l16, 32 * ks, g, l16), acc);
            acc = MM::mma8(lds_col_frag(sLK, LDD, 16 * pta + l16, 32 * ks, g, l16),
                           lds_col_frag(sW, LDX, 16 * cv + l16, 32 * ks, g, l16), acc);
          }
        const int col = c0 + 16 * cv + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * pta + 4 * g + i;
          const uint32_t off = t * hdv + col * 2;
          const float vv = bf16_to_f32(ov[u][i]);
          const float ww = a.w_kind == kNone ? 1.f : bf16_to_f32(ow[u][i]);
          buf_store1((bf16_t*)nullptr, sv_, off, acc[i] * ww);
          if (a.w_kind == kChannel) buf_store1((bf16_t*)nullptr, swc, off, acc[i] * vv);
          if (a.w_kind == kScalar) {
            const float x = row_sum16(acc[i] * vv);
            if (l16 == 0) pw[((h * 2 + (wave & 1)) * 2 + u) * 64 + t] = x;
          }
        }
      }
    }
    if (h + 1 < nh) load_rows(c0 + DVH);  // the next half's rows
    // ---- operand gradients: dO S_0^T, X dSh^T, dV S_0^T, -R dSh^T; their B operands
    // [k = value column][n = channel] from the checkpoint rows ----
    F8 s0r[4][2], gnr[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int ch = 16 * (om0 + mi) + l16;
      s0r[mi][0] = tiled_row_frag(SR, static_cast<int>(DV), ch, c0, g);
      gnr[mi][0] = tiled_row_frag(GR, static_cast<int>(DV), ch, c0, g);
    }
    // ---- Gram gradients: dO X^T, -dO R^T, dV X^T, -dV R^T over this half's columns ----
#pragma unroll
    for (int u = 0; u < NGJ; ++u) {
      const int job = wave + 8 * u;
      if (job < (TWO ? 40 : 20)) {
        const int fam = job / 10, tix = job % 10;
        const int ta = tix >= 6 ? 3 : tix >= 3 ? 2 : tix >= 1 ? 1 : 0, tb = tix - ta * (ta + 1) / 2;
        // erase first: fam 0 dM_QK (dO, X), 1 dM_QP (dO, -R), 2 dL_K (dV, X), 3 dL_P (dV, -R);
        // decay first: fam 0 dM (dO; X and -R), 1 dL (dV; X and -R)
        const bool dvrow = TWO ? fam >= 2 : fam == 1;
        const __bf16* ar = (dvrow ? sW : sO) + (16 * ta + l16) * LDX;
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
          const F8 af = lds_pair_frag_k<DVH>(ar, 32 * kv, g);
          const F8 xf = lds_pair_frag_k<DVH>(sX + (16 * tb + l16) * LDX, 32 * kv, g);
          const F8 rf = chl_neg8(lds_pair_frag_k<DVH>(sR + (16 * tb + l16) * LDX, 32 * kv, g));
          if (TWO) {
            gacc[u] = MM::mma8(af, (fam & 1) ? rf : xf, gacc[u]);
          } else {
            gacc[u] = MM::mma8(af, xf, gacc[u]);
            gacc[u] = MM::mma8(af, rf, gacc[u]);
          }
        }
      }
    }
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      if (kv == 1) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const int ch = 16 * (om0 + mi) + l16;
          s0r[mi][1] = tiled_row_frag(SR, static_cast<int>(DV), ch, c0 + 32, g);
          gnr[mi][1] = tiled_row_frag(GR, static_cast<int>(DV), ch, c0 + 32, g);
        }
      }
      const F8 of = lds_pair_frag_k<DVH>(sO + (16 * ota + l16) * LDX, 32 * kv, g);
      const F8 xf = lds_pair_frag_k<DVH>(sX + (16 * ota + l16) * LDX, 32 * kv, g);
      const F8 vf = lds_pair_frag_k<DVH>(sW + (16 * ota + l16) * LDX, 32 * kv, g);
      const F8 rf = chl_neg8(lds_pair_frag_k<DVH>(sR + (16 * ota + l16) * LDX, 32 * kv, g));
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const float en = fGn[16 * (om0 + mi) + l16];
        F8 ds;
#pragma unroll
        for (int e = 0; e < 8; ++e) ds[e] = static_cast<__bf16>(static_cast<float>(gnr[mi][kv][e]) * en);
        aq[mi] = MM::mma8(of, s0r[mi][kv], aq[mi]);
        ak[mi] = MM::mma8(xf, ds, ak[mi]);
        ac[mi] = MM::mma8(vf, s0r[mi][kv], ac[mi]);
        if (TWO)
          ap[mi] = MM::mma8(rf, ds, ap[mi]);
        else
          ak[mi] = MM::mma8(rf, ds, ak[mi]);
      }
    }
    lds_barrier();  // the next half overwrites X, dO, R and W
  }

  // ---- the rest of sum_j dSh . Sh per channel: with Sh = S_0 + Kh^T X - Ph^T R it is
  // sum_t Kh[t] . (X dSh^T)[t] + Ph[t] . (-R dSh^T)[t], the accumulators of dKh and dPh so far ----
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int ch = 16 * (om0 + mi) + l16;
    float x = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * ota + 4 * g + i;
      x += static_cast<float>(sK[t * LDT + ch]) * ak[mi][i];
      if (TWO) x += static_cast<float>(sP[t * LDT + ch]) * ap[mi][i];
    }
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    if (g == 0) pGn[(1 + ota) * 128 + ch] = x;
  }

  // (q, k and b at this wave's accumulator positions, and log alpha again, for the outputs below;
  // the lane's row and column come through an opaque copy of the thread index, so that the
  // offsets are formed here rather than kept in registers, or spilled, from the kernel's start)
  uint16_t eq[4][4], ek[4][4], eb[4][4];
  {
    // (one loop per kind of b: a select between loads into one register would wait for the first)
    const int tl = chl_opaque(tid) & 63, gq = tl >> 4, lq = tl & 15;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * ota + 4 * gq + i, ch = 16 * (om0 + mi) + lq;
        eq[mi][i] = buf_load_u16(rq, t * hqk + ch * 2);
        ek[mi][i] = buf_load_u16(rk, t * hqk + ch * 2);
      }
    if (a.b_kind == kChannel) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          eb[mi][i] = buf_load_u16(rbc, (16 * ota + 4 * gq + i) * hdk + (16 * (om0 + mi) + lq) * 2);
    } else if (a.b_kind == kScalar) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) eb[mi][i] = buf_load_u16(rbs, (16 * ota + 4 * gq + i) * h1);
    } else {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) eb[mi][i] = 0;
    }
  }
  const ChlRaw la_raw2 = chl_prefix_load(a, rr, left, chl_opaque(tid));  // (offsets formed here again)

  // ---- the Gram gradients (masked, bf16) over the half area: dM_QK, dM_QP, dL_K, dL_P (decay
  // first: dM, dL); their upper tiles read as zeros ----
  auto gd = [&](int fam) { return reinterpret_cast<__bf16*>(smem + L::oX + fam * L::HALF); };
  for (int i = tid; i < 4 * L::HALF / 16; i += NT) reinterpret_cast<uint4*>(smem + L::oX)[i] = make_uint4(0, 0, 0, 0);
  lds_barrier();
#pragma unroll
  for (int u = 0; u < NGJ; ++u) {
    const int job = wave + 8 * u;
    if (job < (TWO ? 40 : 20)) {
      const int fam = job / 10, tix = job % 10;
      const int ta = tix >= 6 ? 3 : tix >= 3 ? 2 : tix >= 1 ? 1 : 0, tb = tix - ta * (ta + 1) / 2;
      const bool strict = TWO ? fam >= 2 : fam == 1;
      const int s = 16 * tb + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * ta + 4 * g + i;
        const bool keep = strict ? s < t : s <= t;
        gd(fam)[t * LDD + s] = static_cast<__bf16>(keep ? gacc[u][i] : 0.f);
      }
    }
  }
  lds_barrier();
  // ---- dQh += dM_QK Kh + dM_QP Ph, dKh += dM_QK^T Qh + dL_K^T Ch, dCh += dL_K Kh + dL_P Ph,
  // dPh += dM_QP^T Qh + dL_P^T Ch ----
  {
    const __bf16* dMQK = gd(0);
    const __bf16* dMQP = gd(TWO ? 1 : 0);
    const __bf16* dLK = gd(TWO ? 2 : 1);
    const __bf16* dLP = gd(TWO ? 3 : 1);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int chc = 16 * (om0 + mi) + l16;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const F8 kf = lds_col_frag(sK, LDT, chc, 32 * ks, g, l16);
        const F8 qf = lds_col_frag(sQ, LDT, chc, 32 * ks, g, l16);
        const F8 cf = lds_col_frag(sC, LDT, chc, 32 * ks, g, l16);
        if (ks <= (ota >> 1)) {  // rows of lower-triangular matrices: tokens s <= t
          aq[mi] = MM::mma8(lds_pair_frag_k<C>(dMQK + (16 * ota + l16) * LDD, 32 * ks, g), kf, aq[mi]);
          ac[mi] = MM::mma8(lds_pair_frag_k<C>(dLK + (16 * ota + l16) * LDD, 32 * ks, g), kf, ac[mi]);
          if (TWO) {
            const F8 pf = lds_col_frag(sP, LDT, chc, 32 * ks, g, l16);
            aq[mi] = MM::mma8(lds_pair_frag_k<C>(dMQP + (16 * ota + l16) * LDD, 32 * ks, g), pf, aq[mi]);
            ac[mi] = MM::mma8(lds_pair_frag_k<C>(dLP + (16 * ota + l16) * LDD, 32 * ks, g), pf, ac[mi]);
          }
        }
        if (ks >= (ota >> 1)) {  // columns (transposes): tokens s >= t
          ak[mi] = MM::mma8(lds_col_frag(dMQK, LDD, 16 * ota + l16, 32 * ks, g, l16), qf, ak[mi]);
          ak[mi] = MM::mma8(lds_col_frag(dLK, LDD, 16 * ota + l16, 32 * ks, g, l16), cf, ak[mi]);
          if (TWO) {
            ap[mi] = MM::mma8(lds_col_frag(dMQP, LDD, 16 * ota + l16, 32 * ks, g, l16), qf, ap[mi]);
            ap[mi] = MM::mma8(lds_col_frag(dLP, LDD, 16 * ota + l16, 32 * ks, g, l16), cf, ap[mi]);
          }
        }
      }
    }
  }
  lds_barrier();  // the operand area is reused below

  // ---- back through the split factors; per-token gate gradients ----
  float* sG2 = reinterpret_cast<float*>(smem + L::oG2);
  float* sdG = reinterpret_cast<float*>(smem + L::oDG);
  float* sdGp = reinterpret_cast<float*>(smem + L::oDGP);
  chl_prefix(la_raw2, sG2, nullptr, qtot, sFlag, tid);  // (the same sums as above)
  lds_barrier();
  {
    const auto sq_ = make_rsrc(a.dq + rr * DK, rng_k);
    const auto sk_ = make_rsrc(a.dk + rr * DK, rng_k);
    const auto sb_ = make_rsrc(a.b_kind == kChannel ? a.db + rr * DK : a.dq, a.b_kind == kChannel ? rng_k : 0u);
    float bsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int ch = 16 * (om0 + mi) + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * ota + 4 * g + i;
        const float gt = sG2[t * 128 + ch], gp = t > 0 ? sG2[(t - 1) * 128 + ch] : 0.f;
        const uint32_t offv = t * hdk + ch * 2;
        const float qv = bf16_to_f32(eq[mi][i]), kv = bf16_to_f32(ek[mi][i]);
        const float bv = a.b_kind == kNone ? 0.f : bf16_to_f32(eb[mi][i]);
        const float et = __expf(gt), ept = __expf(-gt);
        const float dq = aq[mi][i] * et;
        const float dkk = ak[mi][i] * ept;
        const float dkp = TWO ? ap[mi][i] * __expf(-gp) : 0.f;
        const float dc = ac[mi][i] * (TWO ? __expf(gp) : et);
        const float cv_ = bv * kv;
        buf_store1((bf16_t*)nullptr, sq_, offv, dq);
        buf_store1((bf16_t*)nullptr, sk_, offv, dkk + dkp + bv * dc);
        if (a.b_kind == kChannel) buf_store1((bf16_t*)nullptr, sb_, offv, kv * dc);
        bsum[i] += kv * dc;
        if (TWO) {
          sdG[t * 128 + ch] = dq * qv - dkk * kv;
          sdGp[t * 128 + ch] = dc * cv_ - dkp * kv;  // (belongs to G_{t-1})
        } else {
          sdG[t * 128 + ch] = dq * qv - dkk * kv + dc * cv_;
        }
      }
    }
    if (a.b_kind == kScalar) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = row_sum16(bsum[i]);
        if (l16 == 0) atomicAdd(&fdb[16 * ota + 4 * g + i], x);
      }
    }
  }
  lds_barrier();
  // ---- d log alpha_t = sum over s >= t of dG_s: channel tid % 128, tokens 16 (tid / 128) ..,
  // the later quarters' totals through qtot; scalar db and dw ----
  {
    const int ch = tid & 127, q = tid >> 7;
    float d[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int t = 16 * q + u;
      d[u] = sdG[t * 128 + ch];
      if (TWO && t + 1 < C) d[u] += sdGp[(t + 1) * 128 + ch];
    }
    if (q == 3)  // the end-of-chunk decay e^{G_n}
      d[15] += (((pGn[ch] + pGn[128 + ch]) + pGn[256 + ch]) + pGn[384 + ch]) + pGn[512 + ch];
#pragma unroll
    for (int u = 14; u >= 0; --u) d[u] += d[u + 1];
    qtot[q * 128 + ch] = d[0];
    lds_barrier();
    float off = 0.f;
    for (int j = q + 1; j < 4; ++j) off += qtot[j * 128 + ch];
    const auto sla = make_rsrc(a.dla + rr * DK, rng_k);
#pragma unroll
    for (int u = 0; u < 16; ++u) buf_store1((bf16_t*)nullptr, sla, (16 * q + u) * hdk + ch * 2, d[u] + off);
    if (tid < 64) {
      if (a.b_kind == kScalar) buf_store1((bf16_t*)nullptr, make_rsrc(a.db + rr, rng_1), tid * h1, fdb[tid]);
      if (a.w_kind == kScalar) {
        float x = 0.f;
        for (int j = 0; j < 4 * nh; ++j) x += pw[j * 64 + tid];
        buf_store1((bf16_t*)nullptr, make_rsrc(a.dw + rr, rng_1), tid * h1, x);
      }
    }
  }
}

// ------------------------------------------------------------------ flagged chunks

// Token-by-token adjoint of a flagged chunk (chl_prefix), exact in fp32 for any gate values.
// One workgroup of DV / 16 waves per (state, chunk): wave w keeps value columns 16 w .. 16 w + 15
// of the state, lane l rows 8 (l / 4) .. 8 (l / 4) + 7 and columns 4 (l % 4) .. + 3 of them.
// The state before each token is recomputed from checkpoints kept at tokens 0, 16, 32 and 48 of
// the chunk (the first from S_{c-1}); the gradient of the state is carried in reverse from dS_c.
// Per token ("Recurrent Memory: Write, Erase, Decay, Read", section 05), with c = b . k, x = w . v:
//   erase then decay:  r = c S,  Z = S - k^T r,  S' = alpha . Z + k^T x
//   decay then erase:  A = alpha . S,  r = c A,  S' = A - k^T r + k^T x
// and o = q S'.  Sums over channels (r, dx, dr) stay inside a wave; sums over value columns
// (dq, dk, dc, d alpha and a scalar dw) are added across waves through LDS, one barrier a token.
template <int MODE>
__global__ __launch_bounds__(512) void bwd_chl_token_kernel(BwdArgs a) {
  constexpr bool TWO = MODE == 2;
  constexpr int C = 64, DK = 128;
  // LDS: the staged q, k, b, log alpha rows (bf16 [64][128]); per-wave partial sums
  // [2][8 waves][5][128] fp32
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * C * DK * 2 + 2 * 8 * 5 * 128 * 4];
  __bf16* tq = reinterpret_cast<__bf16*>(smem);
  __bf16* tk = tq + C * DK;
  __bf16* tb = tk + C * DK;
  __bf16* tl = tb + C * DK;
  float* part = reinterpret_cast<float*>(smem + 4 * C * DK * 2);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int NW = static_cast<int>(a.DV / 16);
  const int64_t nch = a.nch, DV = a.DV, H = a.H, Hk = a.Hk;
  const int64_t bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int64_t bi = bh / H, hi = bh % H, hk = hi / (H / Hk);
  const int64_t t0 = c * C, left = a.T - t0;
  const int64_t rr = (bi * a.T + t0) * H + hi, rqk = (bi * a.T + t0) * Hk + hk;
  const int64_t cix = bh * nch + c;
  const uint32_t hdk = static_cast<uint32_t>(H * DK * 2), hqk = static_cast<uint32_t>(Hk * DK * 2);
  const uint32_t hdv = static_cast<uint32_t>(H * DV * 2), h1 = static_cast<uint32_t>(H * 2);
  const uint32_t rng_k = wy_range(left, H, DK), rng_v = wy_range(left, H, DV), rng_1 = wy_range(left, H, 1);

  if (a.cflag[cix] == 0) return;  // bwd_chl_kernel took this chunk

  // ---- stage q, k, b (per channel, or the scalar in column 0), log alpha ----
  {
    const auto rq = make_rsrc(a.q + rqk * DK, wy_range(left, Hk, DK));
    const auto rk = make_rsrc(a.k + rqk * DK, wy_range(left, Hk, DK));
    const auto rb = make_rsrc(a.b_kind == kChannel ? a.bg + rr * DK : a.bg + rr,
                              a.b_kind == kChannel ? rng_k : a.b_kind == kScalar ? rng_1 : 0u);
    const auto rl = make_rsrc(a.la + rr * DK, rng_k);
    for (int item = tid; item < C * DK / 8; item += 64 * NW) {
      const int t = item / (DK / 8), d0 = (item % (DK / 8)) * 8;
      *reinterpret_cast<uint4*>(tq + t * DK + d0) = buf_load16(rq, t * hqk + d0 * 2);
      *reinterpret_cast<uint4*>(tk + t * DK + d0) = buf_load16(rk, t * hqk + d0 * 2);
      *reinterpret_cast<uint4*>(tl + t * DK + d0) = buf_load16(rl, t * hdk + d0 * 2);
      if (a.b_kind == kChannel) {
        *reinterpret_cast<uint4*>(tb + t * DK + d0) = buf_load16(rb, t * hdk + d0 * 2);
      } else {
        const uint16_t bs = a.b_kind == kScalar ? buf_load_u16(rb, t * h1) : 0;
        uint4 u;
        u.x = u.y = u.z = u.w = static_cast<uint32_t>(bs) * 0x10001u;
        *reinterpret_cast<uint4*>(tb + t * DK + d0) = u;
      }
    }
    if (tid == 0) {  // the scalar-db sums of both partial buffers
      part[4 * 128 + 1] = 0.f;
      part[8 * 5 * 128 + 4 * 128 + 1] = 0.f;
    }
  }
  lds_barrier();

  const int r0 = 8 * (lane >> 2), cl = 4 * (lane & 3), col0 = 16 * w + cl;  // rows r0.., columns col0..
  const __bf16* SR = a.SR + cix * DK * DV;
  const __bf16* GR = a.GR + cix * DK * DV;
  const auto rv = make_rsrc(a.v + rr * DV, rng_v);
  const auto rwc = make_rsrc(a.w_kind == kChannel ? a.wg + rr * DV : a.v, a.w_kind == kChannel ? rng_v : 0u);
  const auto rws = make_rsrc(a.w_kind == kScalar ? a.wg + rr : a.v, a.w_kind == kScalar ? rng_1 : 0u);
  const auto rdo = make_rsrc(a.dO + rr * DV, rng_v);
  auto ld = [&](const __bf16* p, int t, int i) { return static_cast<float>(p[t * DK + i]); };
  // x = w . v of token t at this lane's four columns
  auto xvals = [&](int t, float* x) {
    float vv[4];
    chl_unpack4(chl_load8(rv, t * hdv + col0 * 2), vv);
    if (a.w_kind == kChannel) {
      float ww[4];
      chl_unpack4(chl_load8(rwc, t * hdv + col0 * 2), ww);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = vv[j] * ww[j];
    } else {
      const float ws = a.w_kind == kScalar ? bf16_to_f32(buf_load_u16(rws, t * h1)) : 1.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = vv[j] * ws;
    }
  };
  // sum over the 16 lanes of equal lane % 4 (the channels of a column)
  auto colsum = [&](float v) {
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
  };
  // one forward token on S (rows r0 .. r0 + 7, columns col0 .. col0 + 3)
  auto step = [&](float (&S)[8][4], int t) {
    float x[4];
    xvals(t, x);
    float r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float al = __expf(ld(tl, t, r0 + i)), cc = ld(tb, t, r0 + i) * ld(tk, t, r0 + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!TWO) S[i][j] *= al;
        r[j] += cc * S[i][j];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = colsum(r[j]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float al = __expf(ld(tl, t, r0 + i)), kk = ld(tk, t, r0 + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float z = S[i][j] - kk * r[j];
        S[i][j] = (TWO ? al * z : z) + kk * x[j];
      }
    }
  };

  // the state before token 0 (the checkpoint S_{c-1}), and before tokens 16, 32, 48 (ck)
  auto load_s0 = [&](float (&S)[8][4]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[i][j] = static_cast<float>(SR[tiled16(r0 + i, col0 + j, DV)]);
  };
  float ck[3][8][4];
  {
    float S[8][4];
    load_s0(S);
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      for (int t = 16 * b; t < 16 * b + 16; ++t) step(S, t);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) ck[b][i][j] = S[i][j];
    }
  }
  float Gd[8][4];  // dL/dS_t, from dS_c
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) Gd[i][j] = static_cast<float>(GR[tiled16(r0 + i, col0 + j, DV)]);

  const auto sq_ = make_rsrc(a.dq + rr * DK, rng_k);
  const auto sk_ = make_rsrc(a.dk + rr * DK, rng_k);
  const auto sla = make_rsrc(a.dla + rr * DK, rng_k);
  const auto sbc = make_rsrc(a.b_kind == kChannel ? a.db + rr * DK : a.dq, a.b_kind == kChannel ? rng_k : 0u);
  const auto sv_ = make_rsrc(a.dv + rr * DV, rng_v);
  const auto swc = make_rsrc(a.w_kind == kChannel ? a.dw + rr * DV : a.dv, a.w_kind == kChannel ? rng_v : 0u);
  for (int t = C - 1; t >= 0; --t) {
    // S = the state before token t
    float S[8][4];
    const int b = t >> 4;
    if (b == 0) {
      load_s0(S);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[i][j] = b == 1 ? ck[0][i][j] : b == 2 ? ck[1][i][j] : ck[2][i][j];
    }
    for (int s = 16 * b; s < t; ++s) step(S, s);
    float x[4], dO[4], vv[4];
    xvals(t, x);
    chl_unpack4(chl_load8(rdo, t * hdv + col0 * 2), dO);
    chl_unpack4(chl_load8(rv, t * hdv + col0 * 2), vv);
    // forward of token t, keeping what the adjoint needs
    float al[8], kk[8], cc[8], qq[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      al[i] = __expf(ld(tl, t, r0 + i));
      kk[i] = ld(tk, t, r0 + i);
      cc[i] = ld(tb, t, r0 + i) * kk[i];
      qq[i] = ld(tq, t, r0 + i);
    }
    // A = S (erase first) or alpha . S (decay first), formed where used
    auto Av = [&](int i, int j) { return TWO ? S[i][j] : al[i] * S[i][j]; };
    float r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] += cc[i] * Av(i, j);
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = colsum(r[j]);
    // row partial sums of this lane (4 columns): dq, dk, dc, d alpha
    float pq[8], pk[8], pc[8], pa[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float sq = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float z = Av(i, j) - kk[i] * r[j];
        const float s1 = (TWO ? al[i] * z : z) + kk[i] * x[j];  // S_t
        sq += dO[j] * s1;
        Gd[i][j] += qq[i] * dO[j];  // o_t = q_t S_t
      }
      pq[i] = sq;
    }
    // dx_j = sum_i k_i G_ij
    float dx[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) dx[j] += kk[i] * Gd[i][j];
#pragma unroll
    for (int j = 0; j < 4; ++j) dx[j] = colsum(dx[j]);
    float dr[4];
    if (TWO) {
      // Z = S - k^T r, S' = alpha . Z + k^T x: dZ = alpha . G, dr = -k dZ
      float t4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float sk = 0.f, sa = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float z = S[i][j] - kk[i] * r[j];
          const float dz = al[i] * Gd[i][j];
          sk += Gd[i][j] * x[j] - dz * r[j];
          sa += Gd[i][j] * z;
          t4[j] -= kk[i] * dz;
          Gd[i][j] = dz;
        }
        pk[i] = sk;
        pa[i] = sa * al[i];  // d log alpha = alpha d alpha
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) dr[j] = colsum(t4[j]);
      // r = c S: dc = sum_j S_ij dr_j, dS += c^T dr
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s += S[i][j] * dr[j];
          Gd[i][j] += cc[i] * dr[j];
        }
        pc[i] = s;
      }
    } else {
      // S' = A - k^T r + k^T x, r = c A, A = alpha . S
#pragma unroll
      for (int j = 0; j < 4; ++j) dr[j] = -dx[j];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float sk = 0.f, sc = 0.f, sa = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sk += Gd[i][j] * (x[j] - r[j]);
          sc += Av(i, j) * dr[j];
          const float dA = Gd[i][j] + cc[i] * dr[j];
          sa += dA * S[i][j];
          Gd[i][j] = al[i] * dA;
        }
        pk[i] = sk;
        pc[i] = sc;
        pa[i] = sa * al[i];
      }
    }
    // value-column outputs: dv = w . dx, dw = v . dx
    {
      float ww[4];
      if (a.w_kind == kChannel) {
        chl_unpack4(chl_load8(rwc, t * hdv + col0 * 2), ww);
      } else {
        const float ws = a.w_kind == kScalar ? bf16_to_f32(buf_load_u16(rws, t * h1)) : 1.f;
        ww[0] = ww[1] = ww[2] = ww[3] = ws;
      }
      if ((lane >> 2) == 0) {  // (every lane of a column holds its dx)
        float o4[4], w4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o4[j] = dx[j] * ww[j];
          w4[j] = dx[j] * vv[j];
          buf_store1((bf16_t*)nullptr, sv_, t * hdv + (col0 + j) * 2, o4[j]);
          if (a.w_kind == kChannel) buf_store1((bf16_t*)nullptr, swc, t * hdv + (col0 + j) * 2, w4[j]);
        }
      }
    }
    float wpart = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) wpart += dx[j] * vv[j];
    wpart += __shfl_xor(wpart, 1);
    wpart += __shfl_xor(wpart, 2);
    // row sums over the wave's 16 columns (the 4 lanes of equal lane / 4), then into LDS
    float* pb = part + (t & 1) * 8 * 5 * 128 + w * 5 * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v4[4] = {pq[i], pk[i], pc[i], pa[i]};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v4[u] += __shfl_xor(v4[u], 1);
        v4[u] += __shfl_xor(v4[u], 2);
      }
      if ((lane & 3) == 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) pb[u * 128 + r0 + i] = v4[u];
      }
    }
    if (lane == 0) pb[4 * 128] = wpart;
    lds_barrier();
    if (tid < 128) {
      const float* p0 = part + (t & 1) * 8 * 5 * 128;
      float s[4] = {0.f, 0.f, 0.f, 0.f};
      for (int ww_ = 0; ww_ < NW; ++ww_)
#pragma unroll
        for (int u = 0; u < 4; ++u) s[u] += p0[ww_ * 5 * 128 + u * 128 + tid];
      const float kv = ld(tk, t, tid), bv = ld(tb, t, tid);
      const uint32_t off = t * hdk + tid * 2;
      buf_store1((bf16_t*)nullptr, sq_, off, s[0]);
      buf_store1((bf16_t*)nullptr, sk_, off, s[1] + bv * s[2]);
      buf_store1((bf16_t*)nullptr, sla, off, s[3]);
      if (a.b_kind == kChannel) buf_store1((bf16_t*)nullptr, sbc, off, kv * s[2]);
      if (a.b_kind == kScalar) {
        // db = sum over channels of k . dc: the 128 threads' values through the spare slot
        float x = kv * s[2];
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) x += __shfl_xor(x, d);
        if ((tid & 63) == 0) atomicAdd(&part[(t & 1) * 8 * 5 * 128 + 4 * 128 + 1], x);
      }
    }
    if (tid == 0 && a.w_kind == kScalar) {
      const float* p0 = part + (t & 1) * 8 * 5 * 128;
      float s = 0.f;
      for (int ww_ = 0; ww_ < NW; ++ww_) s += p0[ww_ * 5 * 128 + 4 * 128];
      buf_store1((bf16_t*)nullptr, make_rsrc(a.dw + rr, rng_1), t * h1, s);
    }
    if (a.b_kind == kScalar) {
      lds_barrier();
      if (tid == 0) {
        float* slot = &part[(t & 1) * 8 * 5 * 128 + 4 * 128 + 1];
        buf_store1((bf16_t*)nullptr, make_rsrc(a.db + rr, rng_1), t * h1, *slot);
        *slot = 0.f;
      }
    }
  }
}

}  // namespace gdr
