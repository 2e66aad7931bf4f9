// Backward pass of the chunk form for a scalar decay (or none), bf16 I/O, d_v <= 128.
//
// The recurrence ("Recurrent Memory: Write, Erase, Decay, Read", section 05, with the Gated
// DeltaNet-2 gates) over one chunk of C = 64 tokens, from the state S_0 that enters it, is, with
// g_t the chunk-local prefix sum of log alpha, gamma_t = e^{g_t}, c_t = b_t . k_t, x_t = w_t . v_t:
//
//   (I + L) U = X - Diag(gamma) C S_0,   L[t][s] = e^{g_t - g_s} c_t . k_s   (s < t)
//   O = Diag(gamma) Q S_0 + M U,         M[t][s] = e^{g_t - g_s} q_t . k_s   (s <= t)
//   S_n = gamma_n S_0 + K_n^T U,         K_n[s] = e^{g_n - g_s} k_s
//
// (a scalar decay commutes with the erase, so both orders of the pages are this one map).  Its
// adjoint, given dO and the gradient dS_n of the state that leaves the chunk:
//
//   dU = M^T dO + K_n dS_n,   dV = T^T dU (T = (I + L)^{-1}),   dX = dV
//   dM = tril(dO U^T),        dL = -strict_tril(dV U^T)
//   dq = (dM . Gamma) K + Diag(gamma) dO S_0^T
//   dc = (dL . Gamma) K - Diag(gamma) dV S_0^T
//   dk = (dM . Gamma)^T Q + (dL . Gamma)^T C + Diag(e^{g_n - g_s}) U dS_n^T + b . dc
//   dS_0 = gamma_n dS_n + (Diag(gamma) Q)^T dO - (Diag(gamma) C)^T dV
//
// and the gradient of g_t collects every factor e^{+-g}: the row sums minus the column sums of
// dM . M and dL . L, gamma_t (q_t . dQ_t + c_t . dC_t), -e^{g_n - g_t} k_t . dK_t, and at t = n
// the terms of gamma_n and of every e^{g_n - g_s}; d log alpha_t is its suffix sum in the chunk.
//
// Kernels (one call):
//   1. the per-channel chunk-local kernel (the decay broadcast over channels) forms each chunk's
//      affine map S_n = Ahat S_0 + D, O = Q' S_0 + Z' with Ahat = Diag(e^{G_n}) + A';
//   2. bwd_db_kernel<DK>: Q'^T dO_c for every chunk at once;
//   3. bwd_chain_kernel<DK, false, NS>: S_c = Ahat S_{c-1} + D chunk by chunk, storing S_{c-1};
//   4. bwd_chain_kernel<DK, true, NS>:  dS_{c-1} = Ahat^T dS_c + Q'^T dO_c in reverse, storing dS_c;
//   5. bwd_local_kernel<DK>: every chunk at once, the adjoint above from S_{c-1} and dS_c.
// The checkpoints are bf16, in two tiled layouts each: rows (S[dk][dv]) for products that
// contract over the value columns, and transposed (S^T[dv][dk]) for those over the channels.
#pragma once

#include "prefill_wyc.h"

namespace gdr {

struct BwdArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* la;
  const bf16_t* bg;
  const bf16_t* wg;
  const bf16_t* dO;
  const float* S0;
  const float* dST;
  bf16_t* dq;
  bf16_t* dk;
  bf16_t* dv;
  bf16_t* dla;
  bf16_t* db;
  bf16_t* dw;
  float* dS0;
  // the chunk maps (per-channel chunk-local kernel) and the checkpoints, per chunk index
  // cix = state * nch + chunk, tiled16 as the workspace of the per-channel forward
  const __bf16* Qd;  // [cix][64][dk]   Q'
  const __bf16* Ad;  // [cix][dk][dk]   A'
  const __bf16* Dt;  // [cix][dv][dk]   D^T
  __bf16* Dbt;       // [cix][dv][dk]   (Q'^T dO)^T, for the reverse chain
  const float* Egn;  // [cix][dk + 4]   e^{G_n}
  __bf16* SR;        // [cix][dk][dv]   S_{c-1}
  __bf16* ST;        // [cix][dv][dk]   S_{c-1}^T
  __bf16* GR;        // [cix][dk][dv]   dS_c
  __bf16* GT;        // [cix][dv][dk]   dS_c^T
  int* cflag;        // [cix] per-channel chunk-local adjoint: 1 where the token-by-token kernel runs
  int64_t T, H, DV, nch;
  int alpha_kind, b_kind, w_kind;
  int64_t Hk;  // q / k heads: value head h reads q / k head h / (H / Hk); with Hk < H, dq and dk
               // are written per value head (into the workspace) and summed over each group after
  // chunk-local adjoint: value columns c0 .. c0 + DVh - 1 (DVh <= 128).  Every input gradient is a
  // sum over value columns, so d_v = 256 runs as two launches whose dq, dk, d log alpha, db and
  // (scalar) dw are added afterwards; dv and a per-channel dw are per column.
  int c0, DVh;
};

// Transposing fragment of a tiled16 LDS matrix: lane (g, l16) gets element [k0 + 4 g + e] and
// [k0 + 16 + 4 g + e] (tile-pair order, e < 4) of column `col`, i.e. a row of the transpose.
// ncols: the matrix's column count.
__device__ __forceinline__ Mma<__bf16>::F8 tiled_col_frag(const __bf16* m, int ncols, int col, int k0,
                                                          int g, int l16) {
  Mma<__bf16>::F8 f;
  const int nt = ncols >> 4, ct = col >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = k0 + 16 * h + 4 * g + (l16 >> 2);
    const __bf16* p = m + ((r >> 4) * nt + ct) * 256 + (r & 15) * 16 + 4 * (l16 & 3);
    const bf16x4 v = lds_read_tr4(reinterpret_cast<const unsigned char*>(p));
#pragma unroll
    for (int e = 0; e < 4; ++e) f[4 * h + e] = v[e];
  }
  return f;
}

// Row fragment of a tiled16 matrix (LDS or global): elements [row][k0 + 4 g + e] and
// [row][k0 + 16 + 4 g + e].  `hi` false: the upper four read as zero (past the last column).
__device__ __forceinline__ Mma<__bf16>::F8 tiled_row_frag(const __bf16* m, int ncols, int row, int k0,
                                                          int g, bool hi = true) {
  Mma<__bf16>::F8 f;
  const __bf16* p0 = m + tiled16(row, k0 + 4 * g, ncols);
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 up;
  if (hi) {
    up = *reinterpret_cast<const bf16x4*>(m + tiled16(row, k0 + 16 + 4 * g, ncols));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) up[e] = static_cast<__bf16>(0.f);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = lo[e];
    f[4 + e] = up[e];
  }
  return f;
}

// The same two fragments from a tiled16 matrix staged in LDS with its rows 8 .. 15 of every tile
// holding their two 16-byte pieces swapped: rows r and r + 8 of a tile then fall on different
// banks for these reads (one tile is 512 bytes; unswizzled, rows r and r + 8 share banks).
__device__ __forceinline__ int swz16(int r, int c) {  // element offset of (r, c) inside a tile
  return (r & 15) * 16 + ((((c & 15) >> 3) ^ ((r & 15) >> 3)) << 3) + (c & 7);
}
__device__ __forceinline__ Mma<__bf16>::F8 tiled_row_frag_sw(const __bf16* m, int ncols, int row, int k0, int g) {
  Mma<__bf16>::F8 f;
  const int nt = ncols >> 4;
  const __bf16* t0 = m + ((row >> 4) * nt + (k0 >> 4)) * 256;
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(t0 + swz16(row, 4 * g));
  const bf16x4 up = *reinterpret_cast<const bf16x4*>(t0 + 256 + swz16(row, 4 * g));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = lo[e];
    f[4 + e] = up[e];
  }
  return f;
}
__device__ __forceinline__ Mma<__bf16>::F8 tiled_col_frag_sw(const __bf16* m, int ncols, int col, int k0, int g,
                                                             int l16) {
  Mma<__bf16>::F8 f;
  const int nt = ncols >> 4, ct = col >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = k0 + 16 * h + 4 * g + (l16 >> 2);
    const __bf16* p = m + ((r >> 4) * nt + ct) * 256 + swz16(r, 4 * (l16 & 3));
    const bf16x4 v = lds_read_tr4(reinterpret_cast<const unsigned char*>(p));
#pragma unroll
    for (int e = 0; e < 4; ++e) f[4 * h + e] = v[e];
  }
  return f;
}
// Global offset of the 16-byte piece that lands in LDS slot `lane` of a 1 KB (two-tile) copy in
// the swizzled form above.
__device__ __forceinline__ uint32_t swz16_src(int lane) {
  const int r = (lane & 31) >> 1;
  return static_cast<uint32_t>((lane >> 5) * 512 + r * 32 + (((lane & 1) ^ (r >> 3)) << 4));
}

// Transposing fragment of a row-major LDS array (pitch in elements): column `col`, rows
// k0 + 4 g + e and k0 + 16 + 4 g + e.
__device__ __forceinline__ Mma<__bf16>::F8 lds_col_frag(const __bf16* base, int pitch, int col, int k0,
                                                        int g, int l16) {
  Mma<__bf16>::F8 f;
  const int c0 = col - l16 + 4 * (l16 & 3), m_ = l16 >> 2;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bf16x4 v = lds_read_tr4(reinterpret_cast<const unsigned char*>(base + (k0 + 16 * h + 4 * g + m_) * pitch + c0));
#pragma unroll
    for (int e = 0; e < 4; ++e) f[4 * h + e] = v[e];
  }
  return f;
}

// Sum over the 16 lanes of a row (lanes 16 r .. 16 r + 15), in every lane of the row: four DPP
// row rotations (row_ror 8, 4, 2, 1), no LDS traffic.
__device__ __forceinline__ float row_sum16(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));
  return x;
}

// ------------------------------------------------------------------ chains over the chunks

// Q'^T dO of every chunk, for the reverse chain (chunk-parallel): D_b^T [dv][dk] tiled like D^T.
// One workgroup of four waves per chunk; Q' and the dO rows staged in LDS, lane output
// D_b[16 tl + 4 g + i][16 cv + l16], i.e. four consecutive channels of row 16 cv + l16 of D_b^T.
template <int DK, int DVP>
__global__ __launch_bounds__(256) void bwd_db_kernel(BwdArgs a) {
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  constexpr int C = 64, NTD = DK / 16, LDO = DVP + 8;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C * DK * 2 + C * LDO * 2];
  __bf16* sQ = reinterpret_cast<__bf16*>(smem);
  __bf16* sO = reinterpret_cast<__bf16*>(smem + C * DK * 2);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nch = a.nch, DV = a.DV, H = a.H;
  const int64_t cix = blockIdx.x, bh = cix / nch, c = cix % nch;
  const int64_t bi = bh / H, hi = bh % H, t0 = c * C;
  const int NCV = static_cast<int>(DV / 16);
  const uint4* Q = reinterpret_cast<const uint4*>(a.Qd + cix * C * DK);
  for (int i = tid; i < C * DK / 8; i += 256) reinterpret_cast<uint4*>(sQ)[i] = Q[i];
  const auto rd = make_rsrc(a.dO + ((bi * a.T + t0) * H + hi) * DV, wy_range(a.T - t0, H, DV));
  const uint32_t hdv = static_cast<uint32_t>(H * DV * 2);
  for (int item = tid; item < C * (DV / 8); item += 256) {
    const int t = item / static_cast<int>(DV / 8), x0 = (item % static_cast<int>(DV / 8)) * 8;
    *reinterpret_cast<uint4*>(sO + t * LDO + x0) = buf_load16(rd, t * hdv + x0 * 2);
  }
  lds_barrier();
  __bf16* Db = a.Dbt + cix * DV * DK;
  for (int job = wave; job < NTD * NCV; job += 4) {
    const int tl = job % NTD, cv = job / NTD;
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      acc = MM::mma8(tiled_col_frag(sQ, DK, 16 * tl + l16, 32 * ks, g, l16),
                     lds_col_frag(sO, LDO, 16 * cv + l16, 32 * ks, g, l16), acc);
    bf16x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = static_cast<__bf16>(acc[i]);
    *reinterpret_cast<bf16x4*>(Db + tiled16(16 * cv + l16, 16 * tl + 4 * g, DK)) = o;
  }
}

// The chains: per chunk c, in order (forward) or in reverse,
//   forward: S <- e^{G_n} . S + A' S + D,      storing S_{c-1}
//   reverse: S <- e^{G_n} . S + A'^T S + D_b,  storing dS_c   (D_b = Q'^T dO, above)
// One workgroup per (state, NS x 16 value columns): NS x DK / 32 state waves, state wave sw holding
// channel tiles 2 (sw % NKB) and 2 (sw % NKB) + 1 of slice sw / NKB in its accumulators, plus two
// helper waves:
//   wave 0 copies each chunk's A', the slices' D rows and e^{G_n} into LDS with direct-to-LDS
//     loads, two chunks ahead (three buffers), and before each barrier waits for the next chunk's;
//   wave 1 copies the checkpoints (the bf16 state the state waves leave in an exchange slot each
//     chunk) to HBM, in both tiled layouts.
// The state waves issue no global memory operation inside the loop; one barrier per chunk (the
// exchange has two slots: a slot is rewritten two chunks later, after every wave has passed the
// barrier in between).
template <int DK, int NS>
struct ChainLayout {
  static constexpr int AB = DK * DK * 2;           // A' (tiled, as in HBM)
  static constexpr int DB = NS * 16 * DK * 2;      // D^T rows of the slices (tiled rows, contiguous)
  static constexpr int EB = ((DK + 4) * 4 + 15) / 16 * 16;  // e^{G_n}: (DK + 4) / 4 pieces of 16 bytes
  static constexpr int BUF = (AB + DB + EB + 255) / 256 * 256;
  static constexpr int NSW = NS * DK / 32;         // state waves
  static constexpr int oX = 3 * BUF;               // exchange: [2][NSW][1 KB]
  static constexpr int total = oX + 2 * NSW * 1024;
  static constexpr bool fits = total <= kLdsLimit;
  static constexpr int NDMA = AB / 1024 + DB / 1024 + 1;  // direct-to-LDS loads per chunk
};

// One chain's workgroup bid of nb (the workgroups of that chain); smem: its ChainLayout.
template <int DK, bool REV, int NS>
__device__ __forceinline__ void bwd_chain_body(const BwdArgs& a, int64_t nb, int64_t bid, unsigned char* smem) {
  using L = ChainLayout<DK, NS>;
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  static_assert(L::fits, "LDS layout exceeds the gfx950 workgroup limit");
  static_assert(L::NDMA <= 60, "one chunk's loads must fit the vmcnt range");
  constexpr int NKB = DK / 32, NSW = L::NSW;

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t DV = a.DV, H = a.H, nch = a.nch;
  const int64_t nwg = DV / (16 * NS);  // workgroups per state
  // consecutive workgroup indices go to different XCDs (8, round robin): renumber so that the
  // workgroups of one state share an XCD, and so its L2, for the chunk maps they all read
  const int64_t p = (nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
  const int64_t bh = p / nwg;
  const int sl0 = static_cast<int>(p % nwg) * NS;
  const bool state = wave >= 2;
  const int sw = state ? wave - 2 : 0;
  const int sls = sl0 + sw / NKB, w = sw % NKB;  // this state wave's slice and k-step
  const int col = 16 * sls + l16;
  auto chunk_of = [&](int64_t it) { return REV ? nch - 1 - it : it; };
  auto buf = [&](int64_t it) { return smem + (it % 3) * L::BUF; };
  auto slot = [&](int64_t it) { return smem + L::oX + (it & 1) * NSW * 1024; };

  // ---- wave 0: a chunk's operands into buffer it % 3 ----
  const __bf16* Dsrc = REV ? a.Dbt : a.Dt;
  auto dma = [&](int64_t it) {
    const int64_t cix = bh * nch + chunk_of(it);
    unsigned char* B = buf(it);
    const auto rA = make_rsrc(a.Ad + cix * DK * DK, L::AB);
    const uint32_t src = swz16_src(lane);  // A' in the swizzled tile form
#pragma unroll
    for (int i = 0; i < L::AB / 1024; ++i) lds_dma16(rA, B + 1024 * i, 1024 * i + src);
    const auto rD = make_rsrc(Dsrc + cix * DV * DK + static_cast<int64_t>(sl0) * 16 * DK, L::DB);
#pragma unroll
    for (int i = 0; i < L::DB / 1024; ++i) lds_dma16(rD, B + L::AB + 1024 * i, 1024 * i + lane * 16);
    if (lane < (DK + 4) / 4) lds_dma16(make_rsrc(a.Egn + cix * (DK + 4), (DK + 4) * 4), B + L::AB + L::DB, lane * 16);
  };

  // ---- state waves: S (two channel tiles of one slice) ----
  f32x4 S[2];
  if (state) {
    const float* init = REV ? a.dST : a.S0;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[u][i] = init ? init[(bh * DK + 16 * (2 * w + u) + 4 * g + i) * DV + col] : 0.f;
  }

  if (wave == 0 && nch > 0) {
    dma(0);
    if (nch > 1) dma(1);
  }
  for (int64_t it = 0; it < nch; ++it) {
    if (state) {
      // the state entering this step, bf16, for the other waves and the checkpoint copier
      *reinterpret_cast<F8*>(slot(it) + sw * 1024 + lane * 16) = acc_pair_frag<__bf16>(S[0], S[1]);
    } else if (wave == 0) {
      // this chunk's loads in; the next chunk's (issued after them) may still be in flight
      if (it + 1 < nch)
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(L::NDMA));
      else
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    lds_barrier_keep_vm();
    if (state) {
      const unsigned char* B = buf(it);
      const __bf16* sA = reinterpret_cast<const __bf16*>(B);
      const __bf16* sD = reinterpret_cast<const __bf16*>(B + L::AB);
      const float* sE = reinterpret_cast<const float*>(B + L::AB + L::DB);
      F8 sf[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        sf[kb] = *reinterpret_cast<const F8*>(slot(it) + ((sw / NKB) * NKB + kb) * 1024 + lane * 16);
      f32x4 acc[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tl = 2 * w + u;
        const float4 e4 = *reinterpret_cast<const float4*>(sE + 16 * tl + 4 * g);
        // D^T row col of this slice: tile row (sw / NKB), tile tl
        const bf16x4 d4 = *reinterpret_cast<const bf16x4*>(sD + ((sw / NKB) * (DK / 16) + tl) * 256 + l16 * 16 + 4 * g);
        acc[u][0] = S[u][0] * e4.x + static_cast<float>(d4[0]);
        acc[u][1] = S[u][1] * e4.y + static_cast<float>(d4[1]);
        acc[u][2] = S[u][2] * e4.z + static_cast<float>(d4[2]);
        acc[u][3] = S[u][3] * e4.w + static_cast<float>(d4[3]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tl = 2 * w + u;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const F8 af = REV ? tiled_col_frag_sw(sA, DK, 16 * tl + l16, 32 * kb, g, l16)
                            : tiled_row_frag_sw(sA, DK, 16 * tl + l16, 32 * kb, g);
          acc[u] = MM::mma8(af, sf[kb], acc[u]);
        }
      }
      S[0] = acc[0];
      S[1] = acc[1];
    } else if (wave == 0) {
      // buffer (it + 2) % 3 was last read in step it - 1, before this step's barrier
      if (it + 2 < nch) dma(it + 2);
    } else {
      // checkpoint of this chunk: every state wave's slot entry, both layouts
      const int64_t cix = bh * nch + chunk_of(it);
      __bf16* ckR = (REV ? a.GR : a.SR) + cix * DK * DV;
      __bf16* ckT = (REV ? a.GT : a.ST) + cix * DV * DK;
      // Slot v holds channels 32 (v % NKB) .. + 31 of the 16 columns of slice v / NKB, lane
      // (g, l16) element e carrying channel 4 g + (e & 3) + 16 (e >> 2) of column l16.  Transposed
      // layout: each lane's eight channels as two 8-byte pieces.  Row layout: lane (r, h) gathers
      // channel r's columns 8 h .. 8 h + 7 from eight lanes' slots and writes them as one
      // 16-byte piece (three stores per slot, below the limit of a wave's outstanding stores).
      const int r = lane >> 1, hh = lane & 1;
      const int gr = (r & 15) >> 2, er = (r & 3) + ((r >> 4) << 2);
#pragma unroll 2
      for (int v = 0; v < NSW; ++v) {
        const unsigned char* X = slot(it) + v * 1024;
        const F8 f = *reinterpret_cast<const F8*>(X + lane * 16);
        const int c_ = 16 * (sl0 + v / NKB) + l16, k0 = 32 * (v % NKB) + 4 * g;
        bf16x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = f[e];
          hi[e] = f[4 + e];
        }
        *reinterpret_cast<bf16x4*>(ckT + tiled16(c_, k0, DK)) = lo;
        *reinterpret_cast<bf16x4*>(ckT + tiled16(c_, k0 + 16, DK)) = hi;
        bf16x8 row;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          row[j] = *reinterpret_cast<const __bf16*>(X + (16 * gr + 8 * hh + j) * 16 + 2 * er);
        *reinterpret_cast<bf16x8*>(ckR + tiled16(32 * (v % NKB) + r, 16 * (sl0 + v / NKB) + 8 * hh, DV)) = row;
      }
    }
  }
  if (REV && state && a.dS0 != nullptr) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.dS0[(bh * DK + 16 * (2 * w + u) + 4 * g + i) * DV + col] = S[u][i];
  }
}

template <int DK, bool REV, int NS>
__global__ __launch_bounds__(64 * (2 + NS * DK / 32)) void bwd_chain_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[ChainLayout<DK, NS>::total];
  bwd_chain_body<DK, REV, NS>(a, gridDim.x, blockIdx.x, smem);
}

// Both chains in one launch (they read the same chunk maps but depend on nothing the other
// writes): the first half of the grid runs the forward chain, the second the reverse one.  For
// problems whose chains each fill at most half the chip.  (The second half keeps the XCD
// renumbering when the half is a multiple of 8.)
template <int DK, int NS>
__global__ __launch_bounds__(64 * (2 + NS * DK / 32)) void bwd_chains_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[ChainLayout<DK, NS>::total];
  const int64_t half = gridDim.x / 2;
  if (static_cast<int64_t>(blockIdx.x) < half)
    bwd_chain_body<DK, false, NS>(a, half, blockIdx.x, smem);
  else
    bwd_chain_body<DK, true, NS>(a, half, blockIdx.x - half, smem);
}

// ------------------------------------------------------------------ chunk-local adjoint

template <int DK>
struct BwdLocalLayout {
  static constexpr int C = 64, DVP = 128;
  static constexpr int LDT = DK + 8, LDX = DVP + 8, LDD = C + 8, LDA = 56, LDI = 24, LDL = 20;
  static constexpr int oQ = 0;                      // q rows
  static constexpr int oK = oQ + C * LDT * 2;       // k rows
  static constexpr int oC = oK + C * LDT * 2;       // c = b . k rows
  static constexpr int oX = oC + C * LDT * 2;       // x = w . v, then V, then dV
  static constexpr int oO = oX + C * LDX * 2;       // dO rows
  static constexpr int oU = oO + C * LDX * 2;       // U
  static constexpr int oDU = oU + C * LDX * 2;      // dU
  static constexpr int oM = oDU + C * LDX * 2;      // M, then dM . Gamma
  static constexpr int oT = oM + C * LDD * 2;       // T, then dL . Gamma
  static constexpr int oA = oT + C * LDD * 2;       // -L below the diagonal blocks (rows 16 ..)
  static constexpr int oI = oA + 48 * LDA * 2;      // inverses of the diagonal blocks
  static constexpr int oLD = oI + C * LDI * 2;      // fp32 diagonal blocks of L, column-major
  static constexpr int oF = oLD + C * LDL * 4;      // fp32 g, gamma, dg, b (scalar), dw and db sums
  // per-wave partial sums of d g and of a scalar db [8][C] each, and a scalar dw's per-item terms
  // [C][16], added in a fixed order at the end (no float atomics: a call's bits do not depend on
  // the order in which waves finish)
  static constexpr int oP = oF + 6 * C * 4;
  static constexpr int total = oP + (2 * 8 * C + 16 * C) * 4;
  static constexpr bool fits = total <= kLdsLimit;
};

template <int DK>
__global__ __launch_bounds__(512) void bwd_local_kernel(BwdArgs a) {
  using L = BwdLocalLayout<DK>;
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  static_assert(L::fits, "LDS layout exceeds the gfx950 workgroup limit");
  constexpr int C = L::C, LDT = L::LDT, LDX = L::LDX, LDD = L::LDD, LDA = L::LDA, LDI = L::LDI, LDL = L::LDL;
  constexpr int NKB = DK / 32, NTD = DK / 16, NKVM = L::DVP / 32;
  constexpr int NT = 512, NW = NT / 64;  // threads, waves

  __shared__ __attribute__((aligned(32))) unsigned char smem[L::total];
  __bf16* sQ = reinterpret_cast<__bf16*>(smem + L::oQ);
  __bf16* sK = reinterpret_cast<__bf16*>(smem + L::oK);
  __bf16* sC = reinterpret_cast<__bf16*>(smem + L::oC);
  __bf16* sX = reinterpret_cast<__bf16*>(smem + L::oX);
  __bf16* sO = reinterpret_cast<__bf16*>(smem + L::oO);
  __bf16* sU = reinterpret_cast<__bf16*>(smem + L::oU);
  __bf16* sDU = reinterpret_cast<__bf16*>(smem + L::oDU);
  __bf16* sM = reinterpret_cast<__bf16*>(smem + L::oM);
  __bf16* tT = reinterpret_cast<__bf16*>(smem + L::oT);
  __bf16* gA = reinterpret_cast<__bf16*>(smem + L::oA);
  __bf16* dInv = reinterpret_cast<__bf16*>(smem + L::oI);
  float* Ld = reinterpret_cast<float*>(smem + L::oLD);
  float* fg = reinterpret_cast<float*>(smem + L::oF);  // g_t
  float* fga = fg + C;                                  // gamma_t
  float* fdg = fg + 2 * C;                              // d g_t
  float* fb = fg + 3 * C;                               // scalar b_t
  float* fdw = fg + 4 * C;                              // row sums of dw (scalar w), then of db
  float* pdg = reinterpret_cast<float*>(smem + L::oP);  // [wave][C] partial d g
  float* pdb = pdg + 8 * C;                             // [wave][C] partial scalar db
  float* pdw = pdb + 8 * C;                             // [t][item] partial scalar dw

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nch = a.nch, DV = a.DV, H = a.H;
  const int64_t bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int64_t bi = bh / H, hi = bh % H;
  const int64_t t0 = c * C, left = a.T - t0;
  const int64_t rr = (bi * a.T + t0) * H + hi;
  const int64_t cix = bh * nch + c;
  const int c0 = a.c0, DVh = a.DVh;  // this launch's value columns
  const int NCV = DVh / 16, NKV = (DVh + 31) / 32;
  const __bf16* SR = a.SR + cix * DK * DV;
  const __bf16* ST = a.ST + cix * DV * DK;
  const __bf16* GR = a.GR + cix * DK * DV;
  const __bf16* GT = a.GT + cix * DV * DK;

  // ---- inputs into LDS; the gate prefix sums ----
  const uint32_t oob = 0x80000000u;
  const uint32_t hdk = static_cast<uint32_t>(H * DK * 2), hdv = static_cast<uint32_t>(H * DV * 2), h1 = static_cast<uint32_t>(H * 2);
  const uint32_t rng_k = wy_range(left, H, DK), rng_1 = wy_range(left, H, 1);
  const uint32_t rng_v = wy_range(left, H, DV) - static_cast<uint32_t>(c0 * 2);  // from column c0
  const uint32_t hqk = static_cast<uint32_t>(a.Hk * DK * 2);  // token stride of q and k
  const int64_t rqk = (bi * a.T + t0) * a.Hk + hi / (H / a.Hk);
  const auto rq = make_rsrc(a.q + rqk * DK, wy_range(left, a.Hk, DK));
  const auto rk = make_rsrc(a.k + rqk * DK, wy_range(left, a.Hk, DK));
  const auto rbc = make_rsrc(a.b_kind == kChannel ? a.bg + rr * DK : a.q, a.b_kind == kChannel ? rng_k : 0u);
  const auto rbs = make_rsrc(a.b_kind == kScalar ? a.bg + rr : a.q, a.b_kind == kScalar ? rng_1 : 0u);
  const auto rv = make_rsrc(a.v + rr * DV + c0, rng_v);
  const auto rwc = make_rsrc(a.w_kind == kChannel ? a.wg + rr * DV + c0 : a.v, a.w_kind == kChannel ? rng_v : 0u);
  const auto rws = make_rsrc(a.w_kind == kScalar ? a.wg + rr : a.v, a.w_kind == kScalar ? rng_1 : 0u);
  const auto rdo = make_rsrc(a.dO + rr * DV + c0, rng_v);
  const auto rla = make_rsrc(a.alpha_kind == kScalar ? a.la + rr : a.q, a.alpha_kind == kScalar ? rng_1 : 0u);
  // The checkpoint fragments each wave needs later (one value tile cv = wave and one channel tile
  // tl = wave at most: d_v <= 128 and d_k <= 128 give at most NW of each) are loaded first, with
  // the input rows, so that their latency is paid once.
  static_assert(NTD <= NW && L::DVP / 16 <= NW, "one value tile and one channel tile per wave");
  F8 stf[NKB], gtf[NKB], s0f[NKVM], gnf[NKVM];
  if (wave < NCV) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      stf[kb] = tiled_row_frag(ST, DK, c0 + 16 * wave + l16, 32 * kb, g);  // S_0 column, k = channels
      gtf[kb] = tiled_row_frag(GT, DK, c0 + 16 * wave + l16, 32 * kb, g);  // dS_n column
    }
  }
  if (wave < NTD) {
#pragma unroll
    for (int kv = 0; kv < NKVM; ++kv) {
      if (kv >= NKV) break;
      const bool hiok = 32 * kv + 16 < DVh;
      s0f[kv] = tiled_row_frag(SR, static_cast<int>(DV), 16 * wave + l16, c0 + 32 * kv, g, hiok);  // S_0 row
      gnf[kv] = tiled_row_frag(GR, static_cast<int>(DV), 16 * wave + l16, c0 + 32 * kv, g, hiok);  // dS_n row
    }
  }
  // q, k (and b) rows: every load, then the stores to LDS
  constexpr int NQI = (C * (DK / 8) + NT - 1) / NT, NVI = C * (L::DVP / 8) / NT;
  uint4 uq[NQI], uk[NQI], ub[NQI];
  uint16_t ubs[NQI];
#pragma unroll
  for (int j = 0; j < NQI; ++j) {
    const int item = tid + NT * j;
    const bool in = item < C * (DK / 8);
    const int t = in ? item / (DK / 8) : 0, d0 = in ? (item % (DK / 8)) * 8 : 0;
    const uint32_t off = in ? t * hdk + d0 * 2 : oob, offk = in ? t * hqk + d0 * 2 : oob;
    uq[j] = buf_load16(rq, offk);
    uk[j] = buf_load16(rk, offk);
    ub[j] = buf_load16(rbc, off);
    ubs[j] = buf_load_u16(rbs, in ? t * h1 : oob);
  }
  uint4 uv[NVI], ud[NVI], uw[NVI];
  uint16_t uws[NVI];
#pragma unroll
  for (int j = 0; j < NVI; ++j) {
    const int item = tid + NT * j;
    const int t = item / (L::DVP / 8), x0 = (item % (L::DVP / 8)) * 8;
    const uint32_t off = x0 < DVh ? t * hdv + x0 * 2 : oob;
    uv[j] = buf_load16(rv, off);
    ud[j] = buf_load16(rdo, off);
    uw[j] = buf_load16(rwc, off);
    uws[j] = buf_load_u16(rws, x0 < DVh ? t * h1 : oob);
  }
#pragma unroll
  for (int j = 0; j < NQI; ++j) {
    const int item = tid + NT * j;
    if (item < C * (DK / 8)) {
      const int t = item / (DK / 8), d0 = (item % (DK / 8)) * 8;
      float kf[8], cf[8];
      load8f(reinterpret_cast<const bf16_t*>(&uk[j]), kf);
      if (a.b_kind == kChannel) {
        load8f(reinterpret_cast<const bf16_t*>(&ub[j]), cf);
#pragma unroll
        for (int e = 0; e < 8; ++e) cf[e] *= kf[e];
      } else {
        const float bs = a.b_kind == kScalar ? bf16_to_f32(ubs[j]) : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) cf[e] = bs * kf[e];
      }
      bf16x8 cb;
#pragma unroll
      for (int e = 0; e < 8; ++e) cb[e] = static_cast<__bf16>(cf[e]);
      *reinterpret_cast<uint4*>(sQ + t * LDT + d0) = uq[j];
      *reinterpret_cast<uint4*>(sK + t * LDT + d0) = uk[j];
      *reinterpret_cast<bf16x8*>(sC + t * LDT + d0) = cb;
    }
  }
  // value rows (x = w . v and dO), zero past d_v up to the next multiple of 32 (the contraction
  // step), and the padding of U and dU
#pragma unroll
  for (int j = 0; j < NVI; ++j) {
    const int item = tid + NT * j;
    const int t = item / (L::DVP / 8), x0 = (item % (L::DVP / 8)) * 8;
    float xf[8];
    load8f(reinterpret_cast<const bf16_t*>(&uv[j]), xf);
    if (a.w_kind == kChannel) {
      float wf[8];
      load8f(reinterpret_cast<const bf16_t*>(&uw[j]), wf);
#pragma unroll
      for (int e = 0; e < 8; ++e) xf[e] *= wf[e];
    } else if (a.w_kind == kScalar) {
      const float ws = bf16_to_f32(uws[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) xf[e] *= ws;
    }
    bf16x8 xb;
#pragma unroll
    for (int e = 0; e < 8; ++e) xb[e] = static_cast<__bf16>(xf[e]);
    const bf16x8 zero8 = {};
    *reinterpret_cast<bf16x8*>(sX + t * LDX + x0) = xb;  // (zero past d_v: those loads read zero)
    *reinterpret_cast<uint4*>(sO + t * LDX + x0) = ud[j];
    *reinterpret_cast<bf16x8*>(sU + t * LDX + x0) = zero8;
    *reinterpret_cast<bf16x8*>(sDU + t * LDX + x0) = zero8;
  }
  for (int i = tid; i < C * LDD / 8; i += NT) reinterpret_cast<uint4*>(sM)[i] = make_uint4(0, 0, 0, 0);
  for (int i = tid; i < 2 * 8 * C; i += NT) pdg[i] = 0.f;  // (pdg and pdb)
  if (wave == 0) {
    // inclusive prefix sum of log alpha over the chunk (lane = token)
    float x = a.alpha_kind == kScalar ? bf16_to_f32(buf_load_u16(rla, lane * h1)) : 0.f;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    fg[lane] = x;
    fga[lane] = __expf(x);
    fdg[lane] = 0.f;
    fb[lane] = a.b_kind == kScalar ? bf16_to_f32(buf_load_u16(rbs, lane * h1)) : 0.f;
    fdw[lane] = 0.f;
    fdw[C + lane] = 0.f;
  }
  lds_barrier();
  const float gn = fg[C - 1];

  // ---- Gram tiles: M = Gamma . tril(Q K^T) (bf16), L = Gamma . strict_tril(C K^T) as -L below
  // the diagonal blocks and fp32 diagonal blocks ----
  for (int job = wave; job < 20; job += NW) {
    const int grp = job / 10, tix = job % 10;
    const int ta = tix >= 6 ? 3 : tix >= 3 ? 2 : tix >= 1 ? 1 : 0, tb = tix - ta * (ta + 1) / 2;
    const __bf16* ar = (grp == 0 ? sQ : sC) + (16 * ta + l16) * LDT;
    const __bf16* br = sK + (16 * tb + l16) * LDT;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) acc = MM::mma8(lds_load8(ar + 32 * kb + 8 * g), lds_load8(br + 32 * kb + 8 * g), acc);
    const int s = 16 * tb + l16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * ta + 4 * g + i;
      const bool keep = grp == 0 ? s <= t : s < t;
      const float val = keep ? acc[i] * __expf(fg[t] - fg[s]) : 0.f;
      if (grp == 0)
        sM[t * LDD + s] = static_cast<__bf16>(val);
      else if (ta > tb)
        gA[(t - 16) * LDA + s] = static_cast<__bf16>(-val);
      else
        Ld[(ta * 16 + (s & 15)) * LDL + (t & 15)] = val;
    }
  }
  lds_barrier();
  if (wave < 2 && lane < 32) wy_diag_inverses<LDL, LDI>(Ld, dInv, wave, lane, l16);
  lds_barrier();
  // ---- T = (I + L)^{-1}: wave j < 4 forms column block j by blocked forward substitution ----
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
  // ---- V = X - Diag(gamma) C S_0, in place of X (wave: value tiles cv = wave, wave + NW) ----
  if (wave < NCV) {
    const int cv = wave;
#pragma unroll
    for (int ta = 0; ta < 4; ++ta) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) acc = MM::mma8(lds_pair_frag_k<DK>(sC + (16 * ta + l16) * LDT, 32 * kb, g), stf[kb], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * ta + 4 * g + i;
        __bf16& x = sX[t * LDX + 16 * cv + l16];
        x = static_cast<__bf16>(static_cast<float>(x) - fga[t] * acc[i]);
      }
    }
  }
  lds_barrier();
  // ---- U = T V ----
  for (int cv = wave; cv < NCV; cv += NW) {
    F8 vf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) vf[ks] = lds_col_frag(sX, LDX, 16 * cv + l16, 32 * ks, g, l16);
#pragma unroll
    for (int ta = 0; ta < 4; ++ta) {
      f32x4 acc = MM::mma8(lds_pair_frag_k<C>(tT + (16 * ta + l16) * LDD, 0, g), vf[0], zero4());
      if (ta >= 2) acc = MM::mma8(lds_pair_frag_k<C>(tT + (16 * ta + l16) * LDD, 32, g), vf[1], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) sU[(16 * ta + 4 * g + i) * LDX + 16 * cv + l16] = static_cast<__bf16>(acc[i]);
    }
  }
  // ---- dU = M^T dO + K_n dS_n (M^T row s: tokens t >= s) ----
  if (wave < NCV) {
    const int cv = wave;
    F8 of[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) of[ks] = lds_col_frag(sO, LDX, 16 * cv + l16, 32 * ks, g, l16);
#pragma unroll
    for (int ta = 0; ta < 4; ++ta) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) acc = MM::mma8(lds_pair_frag_k<DK>(sK + (16 * ta + l16) * LDT, 32 * kb, g), gtf[kb], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= __expf(gn - fg[16 * ta + 4 * g + i]);
      if (ta < 2) acc = MM::mma8(lds_col_frag(sM, LDD, 16 * ta + l16, 0, g, l16), of[0], acc);
      acc = MM::mma8(lds_col_frag(sM, LDD, 16 * ta + l16, 32, g, l16), of[1], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) sDU[(16 * ta + 4 * g + i) * LDX + 16 * cv + l16] = static_cast<__bf16>(acc[i]);
    }
  }
  lds_barrier();
  // ---- dV = T^T dU, in place of V (T^T row s: tokens t >= s) ----
  for (int cv = wave; cv < NCV; cv += NW) {
    F8 df[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) df[ks] = lds_col_frag(sDU, LDX, 16 * cv + l16, 32 * ks, g, l16);
#pragma unroll
    for (int ta = 0; ta < 4; ++ta) {
      f32x4 acc = zero4();
      if (ta < 2) acc = MM::mma8(lds_col_frag(tT, LDD, 16 * ta + l16, 0, g, l16), df[0], acc);
      acc = MM::mma8(lds_col_frag(tT, LDD, 16 * ta + l16, 32, g, l16), df[1], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) sX[(16 * ta + 4 * g + i) * LDX + 16 * cv + l16] = static_cast<__bf16>(acc[i]);
    }
  }
  lds_barrier();

  // row sums (over the 16 lanes of a group) and column sums (over the 4 groups and the 4
  // accumulator rows) of a 16 x 16 tile, added to fdg: + rows of tile row ta, - columns of tb
  // (each into this wave's own partial row, in program order)
  auto dg_rows = [&](int ta, f32x4 r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = row_sum16(r[i]);
      if (l16 == 0) pdg[wave * C + 16 * ta + 4 * g + i] += x;
    }
  };
  auto dg_cols = [&](int tb, const f32x4& r) {
    float x = r[0] + r[1] + r[2] + r[3];
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    if (g == 0) pdg[wave * C + 16 * tb + l16] -= x;
  };
  // ---- dM = tril(dO U^T) and dL = -strict_tril(dV U^T); their products with M and L go to dg,
  // dM . Gamma replaces M and dL . Gamma replaces T ----
  for (int job = wave; job < 20; job += NW) {
    const int grp = job / 10, tix = job % 10;
    const int ta = tix >= 6 ? 3 : tix >= 3 ? 2 : tix >= 1 ? 1 : 0, tb = tix - ta * (ta + 1) / 2;
    const __bf16* ar = (grp == 0 ? sO : sX) + (16 * ta + l16) * LDX;
    const __bf16* br = sU + (16 * tb + l16) * LDX;
    f32x4 acc = zero4();
#pragma unroll
    for (int kv = 0; kv < NKVM; ++kv)
      if (kv < NKV) acc = MM::mma8(lds_pair_frag_k<L::DVP>(ar, 32 * kv, g), lds_pair_frag_k<L::DVP>(br, 32 * kv, g), acc);
    const int s = 16 * tb + l16;
    f32x4 e;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * ta + 4 * g + i;
      const bool keep = grp == 0 ? s <= t : s < t;
      const float d = keep ? (grp == 0 ? acc[i] : -acc[i]) : 0.f;
      float m;
      if (grp == 0)
        m = static_cast<float>(sM[t * LDD + s]);
      else
        m = ta > tb ? -static_cast<float>(gA[(t - 16) * LDA + s]) : Ld[(ta * 16 + (s & 15)) * LDL + (t & 15)];
      e[i] = d * m;
      const __bf16 dG = static_cast<__bf16>(keep ? d * __expf(fg[t] - fg[s]) : 0.f);
      if (grp == 0)
        sM[t * LDD + s] = dG;
      else
        tT[t * LDD + s] = dG;
    }
    dg_rows(ta, e);
    dg_cols(tb, e);
  }
  lds_barrier();

  // ---- dq, dc, dk tiles (wave: channel tiles tl = wave, wave + NW; all four token tiles) ----
  const auto sq_ = make_rsrc(a.dq + rr * DK, rng_k);
  const auto sk_ = make_rsrc(a.dk + rr * DK, rng_k);
  const auto sb_ = make_rsrc(a.b_kind == kChannel ? a.db + rr * DK : a.dq, a.b_kind == kChannel ? rng_k : 0u);
  float sdot = 0.f;   // <S_0, dS_n> over this wave's channel tiles
  float ksall = 0.f;  // sum of e^{g_n - g_s} k_s . dK_n[s] over this wave's tiles
  if (wave < NTD) {
    const int tl = wave;
    const int ch = 16 * tl + l16;
    // (s0f, gnf: rows ch of S_0 and dS_n, k = value columns; compile-time indices with a uniform
    // guard, as a register array indexed at run time becomes a chain of selects)
#pragma unroll
    for (int kv = 0; kv < NKVM; ++kv) {
      if (kv >= NKV) break;
#pragma unroll
      for (int e = 0; e < 8; ++e) sdot += static_cast<float>(s0f[kv][e]) * static_cast<float>(gnf[kv][e]);
    }
    F8 kf[2], qf[2], cf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      kf[ks] = lds_col_frag(sK, LDT, ch, 32 * ks, g, l16);
      qf[ks] = lds_col_frag(sQ, LDT, ch, 32 * ks, g, l16);
      cf[ks] = lds_col_frag(sC, LDT, ch, 32 * ks, g, l16);
    }
#pragma unroll
    for (int ta = 0; ta < 4; ++ta) {
      f32x4 aq = zero4(), ac = zero4(), ak = zero4();
#pragma unroll
      for (int kv = 0; kv < NKVM; ++kv) {
        if (kv >= NKV) break;
        aq = MM::mma8(lds_pair_frag_k<L::DVP>(sO + (16 * ta + l16) * LDX, 32 * kv, g), s0f[kv], aq);
        ac = MM::mma8(lds_pair_frag_k<L::DVP>(sX + (16 * ta + l16) * LDX, 32 * kv, g), s0f[kv], ac);
        ak = MM::mma8(lds_pair_frag_k<L::DVP>(sU + (16 * ta + l16) * LDX, 32 * kv, g), gnf[kv], ak);
      }
      f32x4 e;
      float ksum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * ta + 4 * g + i;
        const float ga = fga[t], gk = __expf(gn - fg[t]);
        aq[i] *= ga;    // gamma_t dO S_0^T
        ac[i] *= -ga;   // -gamma_t dV S_0^T
        ak[i] *= gk;    // e^{g_n - g_t} U dS_n^T
        const float kv_ = static_cast<float>(sK[t * LDT + ch]);
        e[i] = static_cast<float>(sQ[t * LDT + ch]) * aq[i] + static_cast<float>(sC[t * LDT + ch]) * ac[i] - kv_ * ak[i];
        ksum += kv_ * ak[i];
      }
      dg_rows(ta, e);
      ksall += ksum;  // the end-of-chunk factor e^{g_n}: every k_s . dK_n[s], summed below
      // intra-chunk terms (dM . Gamma and dL . Gamma are lower triangular)
      const __bf16* dmr = sM + (16 * ta + l16) * LDD;
      const __bf16* dlr = tT + (16 * ta + l16) * LDD;
      aq = MM::mma8(lds_pair_frag_k<C>(dmr, 0, g), kf[0], aq);
      ac = MM::mma8(lds_pair_frag_k<C>(dlr, 0, g), kf[0], ac);
      if (ta >= 2) {
        aq = MM::mma8(lds_pair_frag_k<C>(dmr, 32, g), kf[1], aq);
        ac = MM::mma8(lds_pair_frag_k<C>(dlr, 32, g), kf[1], ac);
      }
      if (ta < 2) {
        ak = MM::mma8(lds_col_frag(sM, LDD, 16 * ta + l16, 0, g, l16), qf[0], ak);
        ak = MM::mma8(lds_col_frag(tT, LDD, 16 * ta + l16, 0, g, l16), cf[0], ak);
      }
      ak = MM::mma8(lds_col_frag(sM, LDD, 16 * ta + l16, 32, g, l16), qf[1], ak);
      ak = MM::mma8(lds_col_frag(tT, LDD, 16 * ta + l16, 32, g, l16), cf[1], ak);
      // c = b . k: dk += b . dc, db = k . dc
      float bsum[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * ta + 4 * g + i;
        const uint32_t off = t * hdk + ch * 2;
        const float kv_ = static_cast<float>(sK[t * LDT + ch]);
        float bv = 0.f;
        if (a.b_kind == kChannel)
          bv = bf16_to_f32(buf_load_u16(rbc, off));
        else if (a.b_kind == kScalar)
          bv = fb[t];
        ak[i] += bv * ac[i];
        bsum[i] = kv_ * ac[i];
        buf_store1((bf16_t*)nullptr, sq_, off, aq[i]);
        buf_store1((bf16_t*)nullptr, sk_, off, ak[i]);
        if (a.b_kind == kChannel) buf_store1((bf16_t*)nullptr, sb_, off, bsum[i]);
      }
      if (a.b_kind == kScalar) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = bsum[i];
          x += __shfl_xor(x, 1);
          x += __shfl_xor(x, 2);
          x += __shfl_xor(x, 4);
          x += __shfl_xor(x, 8);
          if (l16 == 0) pdb[wave * C + 16 * ta + 4 * g + i] += x;
        }
      }
    }
  }
  // gamma_n <S_0, dS_n> and the k . dK_n terms, both at the last token
  sdot = __expf(gn) * sdot + ksall;
  sdot += __shfl_xor(sdot, 1);
  sdot += __shfl_xor(sdot, 2);
  sdot += __shfl_xor(sdot, 4);
  sdot += __shfl_xor(sdot, 8);
  sdot += __shfl_xor(sdot, 16);
  sdot += __shfl_xor(sdot, 32);
  if (lane == 0) pdg[wave * C + C - 1] += sdot;
  // ---- dv = w . dV and dw = v . dV ----
  const auto sv_ = make_rsrc(a.dv + rr * DV + c0, rng_v);
  const auto swc = make_rsrc(a.w_kind == kChannel ? a.dw + rr * DV + c0 : a.dv, a.w_kind == kChannel ? rng_v : 0u);
  for (int item = tid; item < C * (DVh / 8); item += NT) {
    const int t = item / (DVh / 8), x0 = (item % (DVh / 8)) * 8;
    const uint32_t off = t * hdv + x0 * 2;
    float dx[8], vv[8], ww[8];
    load8f(reinterpret_cast<const bf16_t*>(sX + t * LDX + x0), dx);
    const uint4 uv = buf_load16(rv, off);
    load8f(reinterpret_cast<const bf16_t*>(&uv), vv);
    if (a.w_kind == kChannel) {
      const uint4 uw = buf_load16(rwc, off);
      load8f(reinterpret_cast<const bf16_t*>(&uw), ww);
    } else {
      const float ws = a.w_kind == kScalar ? bf16_to_f32(buf_load_u16(rws, t * h1)) : 1.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ww[j] = ws;
    }
    bf16x8 ov, ow;
    float wsum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ov[j] = static_cast<__bf16>(dx[j] * ww[j]);
      ow[j] = static_cast<__bf16>(dx[j] * vv[j]);
      wsum += dx[j] * vv[j];
    }
    buf_store16(sv_, off, __builtin_bit_cast(uint4, ov));
    if (a.w_kind == kChannel) buf_store16(swc, off, __builtin_bit_cast(uint4, ow));
    if (a.w_kind == kScalar) pdw[t * 16 + item % (DVh / 8)] = wsum;
  }
  lds_barrier();
  // ---- per-token outputs: d log alpha (suffix sums of dg in the chunk), scalar db and dw ----
  if (wave == 0) {
    const uint32_t off = lane * h1;
    float dgs = 0.f, dbs = 0.f, dws = 0.f;  // the partial sums in a fixed order
    for (int w = 0; w < NW; ++w) {
      dgs += pdg[w * C + lane];
      dbs += pdb[w * C + lane];
    }
    for (int j = 0; j < DVh / 8; ++j) dws += pdw[lane * 16 + j];
    fdw[lane] = dws;
    fdw[C + lane] = dbs;
    if (a.alpha_kind == kScalar) {
      float x = dgs;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_down(x, d);
        if (lane + d < 64) x += y;
      }
      buf_store1((bf16_t*)nullptr, make_rsrc(a.dla + rr, rng_1), off, x);
    }
    if (a.b_kind == kScalar) buf_store1((bf16_t*)nullptr, make_rsrc(a.db + rr, rng_1), off, fdw[C + lane]);
    if (a.w_kind == kScalar) buf_store1((bf16_t*)nullptr, make_rsrc(a.dw + rr, rng_1), off, fdw[lane]);
  }
}

// dS0 of an empty sequence: the state passes through unchanged, so dS0 = dS_T (zeros when absent).
__global__ __launch_bounds__(256) void bwd_pass_state_kernel(const float* dST, float* dS0, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) dS0[i] = dST != nullptr ? dST[i] : 0.f;
}

// Partial gradients added up: dst[r][d] = sum over j < G of src0[r G + j][d] (+ src1[r G + j][d]).
// Grouped heads: the per-value-head dq and dk summed over the H / Hk value heads that share each
// q / k head; d_v = 256: the two column halves' partial sums.  One thread per element.
__global__ __launch_bounds__(256) void bwd_sum_kernel(const bf16_t* src0, const bf16_t* src1, bf16_t* dst,
                                                      int64_t rows, int64_t G, int64_t width) {
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (item >= rows * width) return;
  const int64_t r = item / width, d = item % width;
  float acc = 0.f;
  for (int64_t j = 0; j < G; ++j) {
    const int64_t i = (r * G + j) * width + d;
    acc += bf16_to_f32(src0[i].x);
    if (src1 != nullptr) acc += bf16_to_f32(src1[i].x);
  }
  dst[item].x = f32_to_bf16(acc);
}

}  // namespace gdr
