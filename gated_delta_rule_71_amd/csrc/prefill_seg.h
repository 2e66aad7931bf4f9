// Chunkwise prefill as one fused kernel per (state, segment of chunks), for d_k = d_v = 128.
//
// Each workgroup walks the chunks of one segment of one state.  Per 32-token chunk it forms the
// chunk's operands in LDS (prefix sums of log alpha, split factors, Gram products, the triangular
// inverse, W and Y) and then advances the state, whose 128 value columns live in the MFMA
// accumulators of its eight waves (wave w holds columns 16 w .. 16 w + 15, all 128 rows).  No
// chunk data goes through HBM: the next chunk's inputs arrive in LDS by direct-to-LDS loads while
// the current chunk is computed.
//
// Chunk form ("Recurrent Memory: Write, Erase, Decay, Read": section 03, the erase is linear and
// reassociates over a chunk; section 04, the decay enters through prefix sums G_t of log alpha;
// the Gated DeltaNet-2 abstract, a channel-wise decay absorbed into separate erase factors).  With
// c = b . k, X = w . v and per-channel prefix sums G_t of log alpha from the chunk's start
// (G_{-1} = 0, G_n = G_31):
//   decay after the erase (MODE 2):
//     Qs = q e^{G_t},  Ks = k e^{-G_t},  Cs = c e^{G_{t-1}},  Ps = k e^{-G_{t-1}},
//     L_P = strict_tril(Cs Ps^T),  L_K = strict_tril(Cs Ks^T),  M_QK = tril(Qs Ks^T),
//     M_QP = tril(Qs Ps^T),  T = (I + L_P)^{-1},  W = T Cs,  Y = T L_K X,
//     R = W S + Y  (R_t = c_t S_{t-1}: the erase reads)
//     O = Qs S - M_QP R + M_QK X,       S' = e^{G_n} . (S + Ks^T X - Ps^T R)
//   decay before the erase (MODE 1; also a scalar decay, where both orders agree):
//     Cs = c e^{G_t},  L = strict_tril(Cs Ks^T),  M = tril(Qs Ks^T),  T = (I + L)^{-1},
//     W = T Cs,  Y = -T X,  R = W S + Y,  O = Qs S - M R,  S' = e^{G_n} . (S - Ks^T R)
// Every factor lies in the fp32 and bf16 range while |G_t| <= 76 for all t of the chunk; the
// Gram products only ever combine them as e^{G_t - G_s} with t >= s.  A chunk past that is run
// token by token in fp32 on the register-resident state instead: exact for any gate values.
//
// Segments.  A state's chunks are split into segments so that enough workgroups run at once.  The
// state entering segment s > 0 is not known when it starts, so its workgroup carries, next to the
// state N from zero, the segment's transition Phi (dk x dk, from the identity: the same products
// with X = 0), and writes for every chunk Q~ = (the chunk's read-out of Phi), a 32 x dk matrix:
//   S_exit(s) = Phi_s S_enter(s) + N_s,   o_c = O_c(N) + Q~_c S_enter(s)
// (the recurrence is affine in the state: "How Linear Attention Remembers", Analytical Framework).
// A second kernel chains S_enter over the segments; a third adds Q~_c S_enter(s) to o.
#pragma once
#include "gdr_common.h"
#include "mfma.h"
#include "prefill_kernel.h"
#include "prefill_wy.h"

namespace gdr {

struct SegArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* la;
  const bf16_t* bg;
  const bf16_t* wg;
  const float* S0;
  bf16_t* o;
  float* S_T;
  __bf16* Qt;     // [state][nch] blocks of 32 x dk: Q~ of every chunk of segments > 0 (seg_qt_pos)
  __bf16* On;     // [state][nch] blocks of 32 x dv: the read-out of N, same chunks (seg_on_pos)
  float* Nseg;    // [state][nseg] blocks of dk x dv: state from zero over segment s > 0 (seg_acc_pos)
  float* Pseg;    // [state][nseg][dk][dk] transition of segment s (s > 0)
  float* Eseg;    // [state][nseg] blocks of dk x dv, slot 1: the state leaving segment 0 (seg_acc_pos)
  __bf16* Ebf;    // [state][nseg][dv][dk] the state entering segment s, bf16, transposed, pair order
  int64_t T, H, Hk, nch;
  int64_t nseg, L;  // segments per state, chunks per segment (the last may be shorter)
  int alpha_kind, b_kind, w_kind;
};

constexpr float kSegSpanLimit = 76.f;
constexpr int kSegC = 32;  // tokens per chunk
constexpr int kSegThreads = 512;  // threads of a segment workgroup

__device__ __forceinline__ void unpack4(uint2 u, float* f) {
  f[0] = __uint_as_float(u.x << 16);
  f[1] = __uint_as_float(u.x & 0xffff0000u);
  f[2] = __uint_as_float(u.y << 16);
  f[3] = __uint_as_float(u.y & 0xffff0000u);
}
__device__ __forceinline__ uint2 pack4(const float* f) {
  bf16x4 b;
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = static_cast<__bf16>(f[i]);
  return __builtin_bit_cast(uint2, b);
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 v) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
}
// x through an empty asm statement: the compiler can neither see its value nor move it out of a
// loop, so what is derived from it is recomputed where it is used
__device__ __forceinline__ int opaque_v(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// One 16-byte direct-to-LDS load per lane from `bytes` bytes at `base` (pieces past them arrive as
// zeros): lane L's piece lands at lds + 16 L.  Issued from an asm statement, so the compiler does
// not count it as a write to LDS and inserts no wait for it before later LDS reads, which it would
// otherwise do before every transposing read; the kernel waits for these loads itself
// (s_waitcnt vmcnt(0), then a barrier) before anything reads the staging.
__device__ __forceinline__ void seg_dma16(const void* base, uint32_t bytes, unsigned char* lds, uint32_t off) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = static_cast<int>(static_cast<uint32_t>(p));
  r.y = static_cast<int>(static_cast<uint32_t>(p >> 32) & 0xffffu);  // stride 0, no swizzle
  r.z = static_cast<int>(bytes);
  r.w = 0x00020000;
  const uint32_t m0 = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(off), "s"(r)
               : "memory", "m0");
}

// Positions inside one chunk's block of the segment read-outs, in the order the correction kernel
// takes them as MFMA operands, so that each of its loads is contiguous across the wave.  On holds
// O[t][col] (the read-out of N) as the accumulators of the chunk kernel: [t / 16][col / 16][lane]
// [4], lane = 16 ((col % 16) / 4) + t % 16.  Qt holds Q~[t][ch] as B operands over the channels:
// [t / 16][ch / 32][lane][8], the 8 being channels 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3 of
// the 32-channel block, g = (ch % 16) / 4.
// N and the state leaving segment 0 keep the chunk kernel's accumulator order:
// [col / 16][row / 16][lane][4], lane = 16 ((row % 16) / 4) + col % 16, the 4 being row % 4.
__device__ __forceinline__ int seg_acc_pos(int row, int col) {
  return (((col >> 4) * 8 + (row >> 4)) * 64 + ((row & 15) >> 2) * 16 + (col & 15)) * 4 + (row & 3);
}
__device__ __forceinline__ int seg_on_pos(int t, int col) {
  return (((t >> 4) * 8 + (col >> 4)) * 64 + ((col & 15) >> 2) * 16 + (t & 15)) * 4 + (col & 3);
}
__device__ __forceinline__ int seg_qt_pos(int t, int ch) {
  return (((t >> 4) * 4 + (ch >> 5)) * 64 + ((ch & 15) >> 2) * 16 + (t & 15)) * 8 + ((ch >> 4) & 1) * 4 + (ch & 3);
}

// Sums over the 16 lanes of a row (lanes 16 r .. 16 r + 15): the inclusive prefix up to this lane,
// by DPP row shifts (lanes past the row's start add zero), and the value of the row's lane 15.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float row_prefix16(float x) {
  x += dpp_row<0x111>(x);  // row_shr:1
  x += dpp_row<0x112>(x);  // row_shr:2
  x += dpp_row<0x114>(x);  // row_shr:4
  x += dpp_row<0x118>(x);  // row_shr:8
  return x;
}
__device__ __forceinline__ float row_lane15(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x15f, 0xf, 0xf, false));
}

// Fragment of column `col` (this lane's, col = tile + l16) of a token-major LDS array over the 32
// tokens of a chunk, in tile-pair order: lane holds tokens 4 g + (e & 3) + 16 (e >> 2).
__device__ __forceinline__ bf16x8 seg_col_frag(const __bf16* base, int pitch, int col, int g, int l16) {
  const int c0 = col - l16 + 4 * (l16 & 3), m_ = l16 >> 2;
  bf16x8 f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bf16x4 v = lds_read_tr4(reinterpret_cast<const unsigned char*>(base + (16 * h + 4 * g + m_) * pitch + c0));
#pragma unroll
    for (int e = 0; e < 4; ++e) f[4 * h + e] = v[e];
  }
  return f;
}

// Staging of one chunk's inputs in LDS: [32 tokens][128] bf16 per per-channel input, rows of 256
// bytes without padding, the 16 pieces of 16 bytes of row t permuted by XOR with t & 15 (so that
// the 16 rows one read touches fall on distinct banks); 32 bf16 per scalar gate.
__device__ __forceinline__ int stage_off(int t, int c) {  // byte offset of element (t, c), c % 4 == 0
  return t * 256 + ((((c >> 3) ^ t) & 15) << 4) + ((c & 4) << 1);
}

template <int MODE, int AK, int BK, int WK>
struct SegLayout {
  static constexpr int DK = 128, DV = 128, C = kSegC;
  static constexpr bool TWO = MODE == 2;
  static constexpr int LDT = DK + 8;  // token-major rows of dk (or dv) bf16
  static constexpr int LDD = C + 8;   // rows of 32 x 32 matrices
  static constexpr int LDA = 16 + 8;  // the off-diagonal block of -L_P (rows 16..31, cols 0..15), transposed
  static constexpr int LDL = 20;      // fp32 rows of the diagonal blocks of L_P / L
  static constexpr int LDI = 24;      // bf16 rows of their inverses (over the same area)
  static constexpr int ROWS = C * LDT * 2;
  static constexpr int MAT = C * LDD * 2;
  // operand buffer of one chunk: Qs, Cs, Ks (MODE 1: -Ks), -Ps (MODE 2), X, each [32][LDT]
  static constexpr int pQ = 0, pC = ROWS, pK = 2 * ROWS, pP = 3 * ROWS, pX = (TWO ? 4 : 3) * ROWS;
  static constexpr int PB = pX + ROWS;
  // Gram buffer of one chunk: (-L_10)^T [16][LDA], -M_QP / -M, L_K, M_QK [32][LDD] (the last two
  // MODE 2 only), per diagonal block of L_P / L a [16][LDL] fp32 area: the block's rows, then its
  // inverse D = (I + L_bb)^{-1} in bf16 [16][LDI]
  static constexpr int gA = 0, gM = 16 * LDA * 2, gLK = gM + MAT, gMQK = gLK + (TWO ? MAT : 0);
  static constexpr int gLD = gMQK + (TWO ? MAT : 0);
  static constexpr int GB = gLD + 2 * 16 * LDL * 4;
  // two of each (the chunk being advanced and the next one), then e^{G_n} [2][DK] fp32, the
  // per-wave flags [8], and the staging of the inputs of the chunk after
  static constexpr int oP0 = 0, oG0 = 2 * PB, oF = oG0 + 2 * GB, oFL = oF + 2 * DK * 4;
  static constexpr int oS = (oFL + 8 * 4 + 1023) / 1024 * 1024;
  static constexpr int CH = C * DK * 2;                 // one per-channel input: 8 KB
  static constexpr int SC = 256;                        // one scalar gate (32 bf16, padded)
  static constexpr int sQ = oS, sK = sQ + CH, sV = sK + CH;
  static constexpr int sLA = sV + CH;
  static constexpr int sB = sLA + (AK == kChannel ? CH : SC);
  static constexpr int sW = sB + (BK == kChannel ? CH : SC);
  static constexpr int total = sW + (WK == kChannel ? CH : SC);
  static constexpr bool fits = total <= kLdsLimit;
  static_assert(PB % 16 == 0 && GB % 16 == 0 && gM % 16 == 0 && gLD % 16 == 0 && oF % 16 == 0 &&
                    oFL % 16 == 0 && oS % 1024 == 0 && CH % 1024 == 0,
                "aligned arrays (each 1 KB direct-to-LDS load of the staging fills 1 KB of LDS)");
};

// Forward substitution for D = (I + L)^{-1}, L strictly lower 16 x 16 (seg_inv_sweep2: two blocks
// at once): lane (row i = l16, quarter g) holds row i of -L (all 16 entries) and
// D[i][4 g .. 4 g + 3].  At step
// M, row M of D is final; a DPP row broadcast (row_newbcast:M) hands D[M][4 g + c] to every lane
// of the 16-lane group, which adds -L[i][M] times it (a no-op for rows i <= M, where L[i][M] = 0).
template <int M>
__device__ __forceinline__ void seg_inv_sweep(float (&d)[4], const float (&nl)[16]) {
  if constexpr (M < 15) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float dm =
          __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, d[c]), 0x150 + M, 0xf, 0xf, true));
      d[c] = fmaf(dm, nl[M], d[c]);
    }
    seg_inv_sweep<M + 1>(d, nl);
  }
}
template <int M>
__device__ __forceinline__ void seg_inv_sweep2(float (&d)[2][4], const float (&nl)[2][16]) {
  if constexpr (M < 15) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float dm =
            __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, d[b][c]), 0x150 + M, 0xf, 0xf, true));
        d[b][c] = fmaf(dm, nl[b][M], d[b][c]);
      }
    seg_inv_sweep2<M + 1>(d, nl);
  }
}

// Gate values at one token for four channels: a channel gate's four channels, a scalar gate's
// value four times, or `none` (the absent gate's value) four times.
template <int KIND>
__device__ __forceinline__ void stage_gate4(const unsigned char* st, int t, int c, float none, float* f) {
  if constexpr (KIND == kChannel) {
    unpack4(*reinterpret_cast<const uint2*>(st + stage_off(t, c)), f);
  } else if constexpr (KIND == kScalar) {
    const float v = static_cast<float>(reinterpret_cast<const __bf16*>(st)[t]);
    f[0] = f[1] = f[2] = f[3] = v;
  } else {
    f[0] = f[1] = f[2] = f[3] = none;
  }
}
// One element (t, c) of a staged per-channel input.
__device__ __forceinline__ float stage_elem(const unsigned char* st, int t, int c) {
  return static_cast<float>(*reinterpret_cast<const __bf16*>(st + stage_off(t, c & ~3) + 2 * (c & 3)));
}

// The work of one (state, segment) workgroup of 8 waves.  PHI: the segment starts from an unknown
// state, so the workgroup also carries the segment's transition and writes the read-outs of N and
// of Phi (On, Qt) for the correction (every segment but the first).  AK, BK, WK: the kinds of
// log alpha (scalar or channel), b (scalar or channel) and w (none, scalar or channel).
//
// Two chunks are in flight: while the state advances through chunk c (its operands in buffer
// c & 1), the scan, split and Gram products of chunk c + 1 fill the other buffer, and the inputs of
// chunk c + 2 arrive in the staging.  One chunk takes three barriers:
//   A0  the inputs of chunk c + 1 are in the staging
//       split of c + 1 (all waves); then, for chunk c: U, T and R
//   A1  the operands of c + 1 are in their buffer; its flags are known
//       loads of chunk c + 2 (waves 2 and 3); Gram products of c + 1; for chunk c: the read-outs
//       and the state update
//   A2
// (The read-outs wait until after A1 so that the two windows carry about equal work: the split
// is vector-ALU work that the first window cannot hide.)
// A chunk whose gates leave the range of the chunk form ("flagged") runs token by token from its
// staged inputs; the loads of the chunk after it wait for that, and the pipeline refills.
// The barriers wait for LDS operations only, so loads and stores stay in flight across them.
template <int MODE, int AK, int BK, int WK, bool PHI>
__device__ __forceinline__ void seg_body(const SegArgs& a, unsigned char* smem, int64_t bh, int64_t seg) {
  using L = SegLayout<MODE, AK, BK, WK>;
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  constexpr bool TWO = L::TWO;
  constexpr int C = kSegC, DK = 128, DV = 128, LDT = L::LDT, LDD = L::LDD, LDA = L::LDA,
                LDL = L::LDL, NT = 512;

  int* sFlag = reinterpret_cast<int*>(smem + L::oFL);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t H = a.H, Hk = a.Hk, T = a.T, nch = a.nch;
  const int64_t bi = bh / H, hi = bh % H, hk = hi / (H / Hk);
  const int64_t c_begin = seg * a.L;
  const int64_t c_end = c_begin + a.L < nch ? c_begin + a.L : nch;
  const uint32_t hqk = static_cast<uint32_t>(Hk * DK * 2), hdk = static_cast<uint32_t>(H * DK * 2);
  const uint32_t hdv = static_cast<uint32_t>(H * DV * 2), h1 = static_cast<uint32_t>(H * 2);
  auto pbuf = [&](int par) { return smem + L::oP0 + par * L::PB; };
  auto gbuf = [&](int par) { return smem + L::oG0 + par * L::GB; };

  // tiles of -M_QP / -M, L_K and M_QK above the diagonal are never written but are read as zero
#pragma unroll
  for (int b = 0; b < 2; ++b)
    for (int i = tid; i < (L::gLD - L::gM) / 16; i += NT)
      reinterpret_cast<uint4*>(gbuf(b) + L::gM)[i] = make_uint4(0, 0, 0, 0);

  // ---- state tiles: N (value column col) and Phi (channel column col), rows 16 m + 4 g + i ----
  f32x4 SN[8], SP[8];
  {
    const int lane = tid & 63, g = lane >> 4, col = 16 * wave + (lane & 15);
    const float* S0 = (!PHI && a.S0 != nullptr) ? a.S0 + bh * DK * DV : nullptr;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * m + 4 * g + i;
        SN[m][i] = S0 ? S0[row * DV + col] : 0.f;
        if constexpr (PHI) SP[m][i] = (row == col) ? 1.f : 0.f;
      }
  }

  // ---- direct-to-LDS loads of chunk c's inputs (every wave: one 1 KB load of each per-channel
  // input; wave 0 also the scalar gates) ----
  uint16_t scA = 0, scB = 0, scW = 0;  // wave 0, lane t: token t's scalar gates in flight
  // per input: this state's first row, its row stride, and the bytes from the first row to the end
  // of the last (reads past that return zeros: the ragged last chunk)
  struct In {
    const unsigned char* p;
    uint32_t stride;
    int64_t end;
  };
  auto in_of = [&](const bf16_t* x, int64_t heads, int64_t head, int64_t width) {
    const int64_t stride = heads * width * 2;
    return In{reinterpret_cast<const unsigned char*>(x + (bi * T * heads + head) * width),
              static_cast<uint32_t>(stride), (T - 1) * stride + width * 2};
  };
  const In inQ = in_of(a.q, Hk, hk, DK), inK = in_of(a.k, Hk, hk, DK), inV = in_of(a.v, H, hi, DV);
  const In inA = in_of(a.la, H, hi, AK == kChannel ? DK : 1), inB = in_of(a.bg, H, hi, BK == kChannel ? DK : 1);
  const In inW = in_of(a.wg, H, hi, WK == kChannel ? DV : 1);
  // two: waves 2 and 3 issue every per-channel load (four row groups each) and wave 0 the scalar
  // gates, else each wave its own row group
  auto stage = [&](int64_t c, int lane, bool two) {
    const int64_t t0 = c * C;
    // a per-channel array is 8 loads of 1 KB (row group j: rows 4 j .. 4 j + 3)
    auto rows = [&](const In& in, int dst) {
      const int64_t off = t0 * in.stride, left = in.end - off;
      const uint32_t bytes = static_cast<uint32_t>(left < 0x7fffffff ? left : 0x7fffffff);
      const int slot = lane & 15;
      if (two && wave < 2) return;  // (wave 0: the scalar gates only)
      for (int u = 0; u < (two ? 4 : 1); ++u) {
        const int j = two ? 4 * (wave - 2) + u : wave;
        const int t = 4 * j + (lane >> 4);
        const int piece = (slot ^ t) & 15;
        seg_dma16(in.p + off, bytes, smem + dst + 1024 * j, static_cast<uint32_t>(t) * in.stride + piece * 16);
      }
    };
    // a scalar gate: one bf16 per token into a register of wave 0's lane t (written to LDS once
    // the wave has waited for its loads)
    auto scalar = [&](const In& in, uint16_t& dst) {
      if (wave == 0 && lane < C) {
        const int64_t off = t0 * in.stride, left = in.end - off;
        const auto r = make_rsrc(in.p + off, static_cast<uint32_t>(left < 0x7fffffff ? left : 0x7fffffff));
        dst = buf_load_u16(r, static_cast<uint32_t>(lane) * in.stride);
      }
    };
    rows(inQ, L::sQ);
    rows(inK, L::sK);
    rows(inV, L::sV);
    if constexpr (AK == kChannel) rows(inA, L::sLA);
    if constexpr (AK == kScalar) scalar(inA, scA);
    if constexpr (BK == kChannel) rows(inB, L::sB);
    if constexpr (BK == kScalar) scalar(inB, scB);
    if constexpr (WK == kChannel) rows(inW, L::sW);
    if constexpr (WK == kScalar) scalar(inW, scW);
  };
  // every wave waits for its staging loads; wave 0 then writes the scalar gates it holds
  auto arrive = [&](int lane) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (wave == 0 && lane < C) {
      if constexpr (AK == kScalar) reinterpret_cast<uint16_t*>(smem + L::sLA)[lane] = scA;
      if constexpr (BK == kScalar) reinterpret_cast<uint16_t*>(smem + L::sB)[lane] = scB;
      if constexpr (WK == kScalar) reinterpret_cast<uint16_t*>(smem + L::sW)[lane] = scW;
    }
  };
  auto flagged_now = [&]() {
    const int4 f0 = reinterpret_cast<const int4*>(sFlag)[0], f1 = reinterpret_cast<const int4*>(sFlag)[1];
    return (f0.x | f0.y | f0.z | f0.w | f1.x | f1.y | f1.z | f1.w) != 0;
  };

  // ---- scan and split of the staged chunk into operand buffer par: prefix sums of log alpha over
  // the chunk, per channel (this lane's tokens l16 + 16 j of channels ch0 .. ch0 + 3), e^{G_n},
  // the wave's range flag, then the split operands and X ----
  auto split = [&](int par, int lane) {
    const int g = lane >> 4, l16 = lane & 15, ch0 = 16 * wave + 4 * g;
    const unsigned char* st = smem;
    __bf16* tQ = reinterpret_cast<__bf16*>(pbuf(par) + L::pQ);
    __bf16* tC = reinterpret_cast<__bf16*>(pbuf(par) + L::pC);
    __bf16* tK = reinterpret_cast<__bf16*>(pbuf(par) + L::pK);
    __bf16* tP = reinterpret_cast<__bf16*>(pbuf(par) + L::pP);
    __bf16* tX = reinterpret_cast<__bf16*>(pbuf(par) + L::pX);
    float* fG = reinterpret_cast<float*>(smem + L::oF) + par * DK;
    float G[2][4], la[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      stage_gate4<AK>(st + L::sLA, l16 + 16 * j, ch0, 0.f, la[j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) G[j][i] = row_prefix16(la[j][i]);
    }
    bool ok = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      G[1][i] += row_lane15(G[0][i]);  // + G_15
      ok = ok && fabsf(G[0][i]) <= kSegSpanLimit && fabsf(G[1][i]) <= kSegSpanLimit;  // (NaN fails too)
      if (l16 == 15) fG[ch0 + i] = __expf(G[1][i]);  // G_n = G_31
    }
    const bool wave_ok = __all(ok);
    if (lane == 0) sFlag[wave] = wave_ok ? 0 : 1;

    // (all reads of both tokens first, so that their latencies overlap)
    float q4[2][4], k4[2][4], c4[2][4], x4[2][4], w4[2][4];
    {
      uint2 rq[2], rk[2], rv[2], rb[2], rw[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = l16 + 16 * j;
        rq[j] = *reinterpret_cast<const uint2*>(st + L::sQ + stage_off(t, ch0));
        rk[j] = *reinterpret_cast<const uint2*>(st + L::sK + stage_off(t, ch0));
        rv[j] = *reinterpret_cast<const uint2*>(st + L::sV + stage_off(t, ch0));
        if constexpr (BK == kChannel) rb[j] = *reinterpret_cast<const uint2*>(st + L::sB + stage_off(t, ch0));
        if constexpr (WK == kChannel) rw[j] = *reinterpret_cast<const uint2*>(st + L::sW + stage_off(t, ch0));
        if constexpr (BK != kChannel) stage_gate4<BK>(st + L::sB, t, ch0, 0.f, c4[j]);
        if constexpr (WK != kChannel) stage_gate4<WK>(st + L::sW, t, ch0, 1.f, w4[j]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        unpack4(rq[j], q4[j]);
        unpack4(rk[j], k4[j]);
        unpack4(rv[j], x4[j]);
        if constexpr (BK == kChannel) unpack4(rb[j], c4[j]);
        if constexpr (WK == kChannel) unpack4(rw[j], w4[j]);
      }
    }
    // e^{G_t} and e^{-G_t}; e^{G_{t-1}} and e^{-G_{t-1}} (decay after the erase) are the previous
    // token's: the row's lane l16 - 1 (DPP row_shr:1), row lane 15 of the first 16 tokens for
    // token 16, and 1 for token 0
    float eq[2][4], er[2][4], ep[2][4], epr[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        eq[j][i] = __expf(G[j][i]);
        er[j][i] = __builtin_amdgcn_rcpf(eq[j][i]);
      }
      if (TWO) {
        const float e0 = dpp_row<0x111>(eq[0][i]), r0 = dpp_row<0x111>(er[0][i]);
        const float e1 = dpp_row<0x111>(eq[1][i]), r1 = dpp_row<0x111>(er[1][i]);
        const float e15 = row_lane15(eq[0][i]), r15 = row_lane15(er[0][i]);
        ep[0][i] = l16 == 0 ? 1.f : e0;
        epr[0][i] = l16 == 0 ? 1.f : r0;
        ep[1][i] = l16 == 0 ? e15 : e1;
        epr[1][i] = l16 == 0 ? r15 : r1;
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = l16 + 16 * j;
      float oq[4], ok_[4], oc[4], op[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c4[j][i] *= k4[j][i];
        x4[j][i] *= w4[j][i];
        oq[i] = q4[j][i] * eq[j][i];
        ok_[i] = k4[j][i] * er[j][i];
        if (TWO) {
          oc[i] = c4[j][i] * ep[j][i];
          op[i] = -k4[j][i] * epr[j][i];  // stored negated
        } else {
          oc[i] = c4[j][i] * eq[j][i];
          ok_[i] = -ok_[i];  // stored negated
        }
      }
      *reinterpret_cast<uint2*>(tQ + t * LDT + ch0) = pack4(oq);
      *reinterpret_cast<uint2*>(tK + t * LDT + ch0) = pack4(ok_);
      *reinterpret_cast<uint2*>(tC + t * LDT + ch0) = pack4(oc);
      if (TWO) *reinterpret_cast<uint2*>(tP + t * LDT + ch0) = pack4(op);
      *reinterpret_cast<uint2*>(tX + t * LDT + ch0) = pack4(x4[j]);
    }
  };

  // ---- Gram tiles of operand buffer par into Gram buffer par: 6 jobs = 2 row operands x 3 lower
  // tile pairs (waves 2-7) ----
  // Waves 2-7 take one tile pair each (job = wave - 2: row operand Cs or Qs, lower tile pair
  // (ta, tb)); waves 0 and 1 form the diagonal tiles of L_P / L again and invert them, which the
  // jobs with ta = tb then leave out.
  auto gram = [&](int par, int lane) {
    const int g = lane >> 4, l16 = lane & 15;
    const __bf16* tQ = reinterpret_cast<const __bf16*>(pbuf(par) + L::pQ);
    const __bf16* tC = reinterpret_cast<const __bf16*>(pbuf(par) + L::pC);
    const __bf16* tK = reinterpret_cast<const __bf16*>(pbuf(par) + L::pK);
    const __bf16* tP = reinterpret_cast<const __bf16*>(pbuf(par) + L::pP);
    __bf16* gA = reinterpret_cast<__bf16*>(gbuf(par) + L::gA);
    __bf16* gM = reinterpret_cast<__bf16*>(gbuf(par) + L::gM);
    __bf16* gLK = reinterpret_cast<__bf16*>(gbuf(par) + L::gLK);
    __bf16* gMQK = reinterpret_cast<__bf16*>(gbuf(par) + L::gMQK);
    float* Ld = reinterpret_cast<float*>(gbuf(par) + L::gLD);
    const bool diag = wave < 2;
    const int job = diag ? 0 : wave - 2, grp = diag ? 0 : job / 3, tix = job % 3;
    const int ta = diag ? wave : tix >= 1 ? 1 : 0, tb = diag ? wave : tix == 2 ? 1 : 0;
    const bool need2 = TWO && !diag;
    if (!diag && grp == 0 && ta == tb && !TWO) return;  // (decay first: only L_P, formed by wave ta)
    const __bf16* ar = (grp == 0 ? tC : tQ) + (16 * ta + l16) * LDT;
    const __bf16* br = ((TWO && grp == 0) ? tP : tK) + (16 * tb + l16) * LDT;
    const __bf16* cr = (grp == 0 ? tK : tP) + (16 * tb + l16) * LDT;
    F8 fa[4], fb[4], fc[4];
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
      fa[kb] = lds_load8(ar + 32 * kb + 8 * g);
      fb[kb] = lds_load8(br + 32 * kb + 8 * g);
      if (need2) fc[kb] = lds_load8(cr + 32 * kb + 8 * g);
    }
    f32x4 acc1 = zero4(), acc2 = zero4();
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
      acc1 = MM::mma8(fa[kb], fb[kb], acc1);
      if (need2) acc2 = MM::mma8(fa[kb], fc[kb], acc2);
    }
    // which: 0 = -L_P / -L (strict; the off-diagonal block transposed -> gA, the diagonal
    // blocks -> Ld negated back), 1 = -M_QP / -M, 2 = L_K (strict), 3 = M_QK (inclusive).  The
    // products against the negated key family (which 0 and 1) arrive negated.
    auto store_tile = [&](int which, const f32x4& acc) {
      const int r0 = 16 * ta + 4 * g, cc = 16 * tb + l16;
      if (ta > tb) {
        if (which == 0) {  // (-L_10)^T: row l16, columns 4 g .. 4 g + 3
          float a4[4] = {acc[0], acc[1], acc[2], acc[3]};
          *reinterpret_cast<uint2*>(gA + l16 * LDA + 4 * g) = pack4(a4);
          return;
        }
        __bf16* dst = (which == 1 ? gM : which == 2 ? gLK : gMQK) + r0 * LDD + cc;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i * LDD] = static_cast<__bf16>(acc[i]);
        return;
      }
      const int lim = (which == 0 || which == 2) ? cc + 1 : cc;  // keep rows r >= lim
      if (which == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = r0 + i;
          Ld[(ta * 16 + (r & 15)) * LDL + (cc & 15)] = r >= lim ? -acc[i] : 0.f;
        }
        return;
      }
      __bf16* dst = (which == 1 ? gM : which == 2 ? gLK : gMQK) + r0 * LDD + cc;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i * LDD] = static_cast<__bf16>(r0 + i >= lim ? acc[i] : 0.f);
    };
    if (diag) {
      store_tile(0, acc1);
    } else if (TWO) {
      if (grp != 0 || ta != tb) store_tile(grp == 0 ? 0 : 3, acc1);
      store_tile(grp == 0 ? 2 : 1, acc2);
    } else {
      store_tile(grp == 0 ? 0 : 1, acc1);
    }
    // a diagonal block of L_P / L: its inverse D by seg_inv_sweep, from the rows this wave just
    // wrote (the wave's own LDS writes precede its reads), over the same area
    if (diag) {
      float* Lb = Ld + ta * 16 * LDL;
      float nl[16], d[4];
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const float4 v = *reinterpret_cast<const float4*>(Lb + l16 * LDL + 4 * c4);
        nl[4 * c4] = -v.x;
        nl[4 * c4 + 1] = -v.y;
        nl[4 * c4 + 2] = -v.z;
        nl[4 * c4 + 3] = -v.w;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) d[e] = (4 * g + e == l16) ? 1.f : 0.f;
      seg_inv_sweep<0>(d, nl);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): every lane's reads of the rows are done
      *reinterpret_cast<uint2*>(reinterpret_cast<__bf16*>(Lb) + l16 * L::LDI + 4 * g) = pack4(d);
    }
  };

  // ---- the state through chunk c, part 1: U = Cs S (channel contraction, N and Phi), Z = L_K X
  // (MODE 2) or -X; T = (I + L)^{-1} (the diagonal blocks' inverses from the Gram waves, the
  // off-diagonal block by three small MFMAs in every wave); R = T U + T Z.  Leaves R (over the
  // tokens), X's column and S's bf16 fragments (sfN, sfP) for the read-outs and part 2. ----
  auto chain1 = [&](int par, int lane, F8& rfN, F8& rfP, F8& xf, F8 (&sfN)[4], F8 (&sfP)[4]) {
    const int g = lane >> 4, l16 = lane & 15, col = 16 * wave + l16;
    const __bf16* tC = reinterpret_cast<const __bf16*>(pbuf(par) + L::pC);
    const __bf16* tX = reinterpret_cast<const __bf16*>(pbuf(par) + L::pX);
    const __bf16* gA = reinterpret_cast<const __bf16*>(gbuf(par) + L::gA);
    const __bf16* gLK = reinterpret_cast<const __bf16*>(gbuf(par) + L::gLK);
    const float* Ld = reinterpret_cast<const float*>(gbuf(par) + L::gLD);
    // operand loads first: their latencies overlap the conversions and the sweep
    F8 cfr[2][4];  // rows 16 ta + l16 of Cs, channels 32 kb + pair(g)
#pragma unroll
    for (int ta = 0; ta < 2; ++ta)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) cfr[ta][kb] = lds_pair_frag_k<DK>(tC + (16 * ta + l16) * LDT, 32 * kb, g);
    // D_b[l16][4 g .. 4 g + 3] (the Gram waves' inverses of the diagonal blocks)
    const bf16x4 d0 = lds_load4(reinterpret_cast<const __bf16*>(Ld) + l16 * L::LDI + 4 * g);
    const bf16x4 d1 = lds_load4(reinterpret_cast<const __bf16*>(Ld + 16 * LDL) + l16 * L::LDI + 4 * g);
    const bf16x4 nl10t = lds_load4(gA + l16 * LDA + 4 * g);  // (-L_10)^T [l16][4 g ..]
    xf = seg_col_frag(tX, LDT, col, g, l16);                 // X column col over the tokens
    F8 lkf[2];
    if (TWO) {
#pragma unroll
      for (int ta = 0; ta < 2; ++ta) lkf[ta] = lds_pair_frag_k<C>(gLK + (16 * ta + l16) * LDD, 0, g);
    }
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sfN[kb] = acc_pair_frag<__bf16>(SN[2 * kb], SN[2 * kb + 1]);
      if constexpr (PHI) sfP[kb] = acc_pair_frag<__bf16>(SP[2 * kb], SP[2 * kb + 1]);
    }
    // U (the N and Phi tiles share each Cs fragment)
    f32x4 UN[2], UP[2];
#pragma unroll
    for (int ta = 0; ta < 2; ++ta) {
      UN[ta] = zero4();
      UP[ta] = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        UN[ta] = MM::mma8(cfr[ta][kb], sfN[kb], UN[ta]);
        if constexpr (PHI) UP[ta] = MM::mma8(cfr[ta][kb], sfP[kb], UP[ta]);
      }
    }
    F8 zf;  // Z over the tokens (k) for column col
    if (TWO) {
      const f32x4 z0 = MM::mma8(lkf[0], xf, zero4()), z1 = MM::mma8(lkf[1], xf, zero4());
      zf = acc_pair_frag<__bf16>(z0, z1);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) zf[e] = -xf[e];
    }
    // T as A operands: rows 16 ta + l16, tokens in pair order.  D_b[l16][4 g .. 4 g + 3] is that
    // layout already; T_10 arrives in it as the accumulator of T_10^T = D_0^T ((-L_10)^T D_1^T).
    f32x4 id;
#pragma unroll
    for (int e = 0; e < 4; ++e) id[e] = (4 * g + e == l16) ? 1.f : 0.f;
    const f32x4 D0 = MM::mma4(d0, acc_frag4<__bf16>(id), zero4());                      // D_0[4 g + i][l16]
    const f32x4 Qm = MM::mma4(nl10t, d1, zero4());                                       // (-L_10)^T D_1^T
    const f32x4 T10t = MM::mma4(acc_frag4<__bf16>(D0), acc_frag4<__bf16>(Qm), zero4());  // T_10[l16][4 g + i]
    F8 tf0, tf1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tf0[e] = d0[e];
      tf0[4 + e] = static_cast<__bf16>(0.f);
      tf1[e] = static_cast<__bf16>(T10t[e]);
      tf1[4 + e] = d1[e];
    }
    // R = T (U + Z), tokens 16 ta + 4 g + i, column col
    const F8 ufN = acc_pair_frag<__bf16>(UN[0], UN[1]);
    F8 ufP;
    if constexpr (PHI) ufP = acc_pair_frag<__bf16>(UP[0], UP[1]);
    f32x4 RN[2], RP[2];
    RN[0] = MM::mma8(tf0, ufN, MM::mma8(tf0, zf, zero4()));
    RN[1] = MM::mma8(tf1, ufN, MM::mma8(tf1, zf, zero4()));
    if constexpr (PHI) {
      RP[0] = MM::mma8(tf0, ufP, zero4());
      RP[1] = MM::mma8(tf1, ufP, zero4());
    }
    rfN = acc_pair_frag<__bf16>(RN[0], RN[1]);
    if constexpr (PHI) rfP = acc_pair_frag<__bf16>(RP[0], RP[1]);
  };
  // ---- the read-outs of chunk c: O^T = S^T Qs^T - R^T M^T (+ X^T M_QK^T) from S's fragments as
  // they entered the chunk; to o, or (a segment from an unknown state) O(N) and Q~ to On and Qt ----
  auto readout = [&](int64_t c, int par, int lane, const F8& rfN, const F8& rfP, const F8& xf, const F8 (&sfN)[4],
                     const F8 (&sfP)[4]) {
    const int g = lane >> 4, l16 = lane & 15, ch0 = 16 * wave + 4 * g;
    const __bf16* tQ = reinterpret_cast<const __bf16*>(pbuf(par) + L::pQ);
    const __bf16* gM = reinterpret_cast<const __bf16*>(gbuf(par) + L::gM);
    const __bf16* gMQK = reinterpret_cast<const __bf16*>(gbuf(par) + L::gMQK);
    // O^T: lane holds O[token 16 ta + l16][column 16 w + 4 g + i]
    const int64_t t0 = c * C;
    const auto ro = make_rsrc(a.o + ((bi * T + t0) * H + hi) * DV, wy_range(T - t0, H, DV));
#pragma unroll
    for (int ta = 0; ta < 2; ++ta) {
      F8 qf[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) qf[kb] = lds_pair_frag_k<DK>(tQ + (16 * ta + l16) * LDT, 32 * kb, g);
      const F8 mf = lds_pair_frag_k<C>(gM + (16 * ta + l16) * LDD, 0, g);
      F8 mqf;
      if (TWO) mqf = lds_pair_frag_k<C>(gMQK + (16 * ta + l16) * LDD, 0, g);
      f32x4 oN = zero4(), oP = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        oN = MM::mma8(sfN[kb], qf[kb], oN);
        if constexpr (PHI) oP = MM::mma8(sfP[kb], qf[kb], oP);
      }
      oN = MM::mma8(rfN, mf, oN);
      if constexpr (PHI) oP = MM::mma8(rfP, mf, oP);
      if (TWO) oN = MM::mma8(xf, mqf, oN);
      float o4[4] = {oN[0], oN[1], oN[2], oN[3]};
      if constexpr (PHI) {
        // straight from the accumulators: seg_on_pos / seg_qt_pos of (16 ta + l16, 16 w + 4 g)
        float p4[4] = {oP[0], oP[1], oP[2], oP[3]};
        __bf16* on = a.On + (bh * nch + c) * C * DV;
        __bf16* qt = a.Qt + (bh * nch + c) * C * DK;
        *reinterpret_cast<uint2*>(on + ((ta * 8 + wave) * 64 + lane) * 4) = pack4(o4);
        *reinterpret_cast<uint2*>(qt + ((ta * 4 + (wave >> 1)) * 64 + lane) * 8 + (wave & 1) * 4) = pack4(p4);
      } else {
        buf_store8(ro, static_cast<uint32_t>(16 * ta + l16) * hdv + ch0 * 2, pack4(o4));
      }
    }
  };

  // ---- part 2: S += Ks^T X + (-Ps)^T R (MODE 2) or S += (-Ks)^T R (MODE 1), then
  // S = e^{G_n} . S ----
  auto chain2 = [&](int par, int lane, const F8& rfN, const F8& rfP, const F8& xf) {
    const int g = lane >> 4, l16 = lane & 15;
    const __bf16* tK = reinterpret_cast<const __bf16*>(pbuf(par) + L::pK);
    const __bf16* tP = reinterpret_cast<const __bf16*>(pbuf(par) + L::pP);
    const float* fG = reinterpret_cast<const float*>(smem + L::oF) + par * DK;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const F8 kf = seg_col_frag(tK, LDT, 16 * m + l16, g, l16);
      if (TWO) {
        const F8 pf = seg_col_frag(tP, LDT, 16 * m + l16, g, l16);
        SN[m] = MM::mma8(kf, xf, SN[m]);
        SN[m] = MM::mma8(pf, rfN, SN[m]);
        if constexpr (PHI) SP[m] = MM::mma8(pf, rfP, SP[m]);
      } else {
        SN[m] = MM::mma8(kf, rfN, SN[m]);
        if constexpr (PHI) SP[m] = MM::mma8(kf, rfP, SP[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float4 f = *reinterpret_cast<const float4*>(fG + 16 * m + 4 * g);
      SN[m][0] *= f.x;
      SN[m][1] *= f.y;
      SN[m][2] *= f.z;
      SN[m][3] *= f.w;
      if constexpr (PHI) {
        SP[m][0] *= f.x;
        SP[m][1] *= f.y;
        SP[m][2] *= f.z;
        SP[m][3] *= f.w;
      }
    }
  };

  // ---- a flagged chunk c, token by token in fp32 from its staged inputs, on the
  // register-resident tiles: one tile per loop (keeps the values the loop carries to 32); is_n: an
  // N tile (takes X, read-outs to o or On), else Phi (read-outs to Qt) ----
  auto token = [&](int64_t c, int lane) {
    const int g = lane >> 4, l16 = lane & 15, col = 16 * wave + l16;
    const unsigned char* st = smem;
    const int64_t t0 = c * C;
    const auto ro = make_rsrc(a.o + ((bi * T + t0) * H + hi) * DV, wy_range(T - t0, H, DV));
    __bf16* qt = PHI ? a.Qt + (bh * nch + c) * C * DK : nullptr;
    __bf16* on = PHI ? a.On + (bh * nch + c) * C * DV : nullptr;
    auto run_tile = [&](f32x4 (&S)[8], bool is_n) {
#pragma unroll 1
      for (int t = 0; t < C; ++t) {
        auto decay = [&](int m, float* f) {
          float l4[4];
          stage_gate4<AK>(st + L::sLA, t, 16 * m + 4 * g, 0.f, l4);
#pragma unroll
          for (int i = 0; i < 4; ++i) f[i] = __expf(l4[i]);
        };
        float r = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          float k4[4], c4[4], a4[4];
          unpack4(*reinterpret_cast<const uint2*>(st + L::sK + stage_off(t, 16 * m + 4 * g)), k4);
          stage_gate4<BK>(st + L::sB, t, 16 * m + 4 * g, 0.f, c4);
          if (!TWO) decay(m, a4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (!TWO) S[m][i] *= a4[i];  // decay first
            r += c4[i] * k4[i] * S[m][i];
          }
        }
        r += __shfl_xor(r, 16);
        r += __shfl_xor(r, 32);
        float x = 0.f;
        if (is_n) {
          float wv;
          if constexpr (WK == kChannel) wv = stage_elem(st + L::sW, t, col);
          else if constexpr (WK == kScalar) wv = static_cast<float>(reinterpret_cast<const __bf16*>(st + L::sW)[t]);
          else wv = 1.f;
          x = stage_elem(st + L::sV, t, col) * wv;
        }
        float y = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          float q4[4], k4[4], a4[4];
          unpack4(*reinterpret_cast<const uint2*>(st + L::sQ + stage_off(t, 16 * m + 4 * g)), q4);
          unpack4(*reinterpret_cast<const uint2*>(st + L::sK + stage_off(t, 16 * m + 4 * g)), k4);
          if (TWO) decay(m, a4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float sv = S[m][i] - k4[i] * r;
            if (TWO) sv *= a4[i];
            sv += k4[i] * x;
            S[m][i] = sv;
            y += q4[i] * sv;
          }
        }
        y += __shfl_xor(y, 16);
        y += __shfl_xor(y, 32);
        if (g == 0) {
          if (!is_n)
            qt[seg_qt_pos(t, col)] = static_cast<__bf16>(y);
          else if (PHI)
            on[seg_on_pos(t, col)] = static_cast<__bf16>(y);
          else
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, static_cast<__bf16>(y)),
                                                  ro, static_cast<uint32_t>(t) * hdv + col * 2, 0, 0);
        }
      }
    };
    run_tile(SN, true);
    if constexpr (PHI) run_tile(SP, false);
  };

  // ---- prologue: the first chunk's operands (and the loads of the second) ----
  bool flag_cur = false;  // (uniform) chunk c is flagged
  if (c_begin < c_end) {
    const int lane = opaque_v(tid) & 63;
    stage(c_begin, lane, false);
    arrive(lane);
    lds_barrier_keep_vm();
    split(0, lane);
    lds_barrier_keep_vm();
    flag_cur = flagged_now();
    if (!flag_cur) {
      if (c_begin + 1 < c_end) stage(c_begin + 1, lane, false);
      gram(0, lane);
    }
    lds_barrier_keep_vm();
  }

  int par = 0;  // operand buffer of chunk c
  for (int64_t c = c_begin; c < c_end; ++c, par ^= 1) {
    // the lane from an opaque copy of the thread index: values derived from it are recomputed
    // where used instead of being kept across the loop in registers the chunk needs
    const int lane = opaque_v(tid) & 63;
    const bool has_next = c + 1 < c_end;
    bool flag_next = false;
    if (flag_cur) {
      // the staging still holds chunk c: nothing was loaded after it
      token(c, lane);
      lds_barrier_keep_vm();
      if (has_next) {  // refill: chunk c + 1 from its loads to its Gram products
        stage(c + 1, lane, false);
        arrive(lane);
        lds_barrier_keep_vm();
        split(par ^ 1, lane);
        lds_barrier_keep_vm();
        flag_next = flagged_now();
        if (!flag_next) {
          if (c + 2 < c_end) stage(c + 2, lane, false);
          gram(par ^ 1, lane);
        }
        lds_barrier_keep_vm();
      }
      flag_cur = flag_next;
      continue;
    }
    arrive(lane);
    lds_barrier_keep_vm();  // A0: chunk c + 1's inputs are in the staging
    split(par ^ 1, lane);  // (past the segment's end: stale staging into an unused buffer)
    __builtin_amdgcn_sched_barrier(0);
    F8 rfN, rfP, xf, sfN[4], sfP[4];
    chain1(par, lane, rfN, rfP, xf, sfN, sfP);
    lds_barrier_keep_vm();  // A1: chunk c + 1's operands are in their buffer, its flags known
    if (has_next) flag_next = flagged_now();
    if (has_next && !flag_next) {
      // waves 2 and 3 issue the loads of chunk c + 2 (wave 0 its scalar gates); then the Gram
      // products (waves 0 and 1 the diagonal blocks and their inverses)
      if ((wave == 0 || wave == 2 || wave == 3) && c + 2 < c_end) stage(c + 2, lane, true);
      gram(par ^ 1, lane);
    }
    readout(c, par, lane, rfN, rfP, xf, sfN, sfP);
    chain2(par, lane, rfN, rfP, xf);
    lds_barrier_keep_vm();  // A2
    flag_cur = flag_next;
  }

  // ---- end of the segment: the final state (one segment), or N, Phi and E_1 (from segment 0) ----
  const int lane = tid & 63, g = lane >> 4, col = 16 * wave + (lane & 15);
  if (a.nseg == 1) {
    if (a.S_T != nullptr) {
      float* St = a.S_T + bh * DK * DV;
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) St[(16 * m + 4 * g + i) * DV + col] = SN[m][i];
    }
  } else {
    const int64_t sb = bh * a.nseg + seg;
    float* No = PHI ? a.Nseg + sb * DK * DV : a.Eseg + (sb + 1) * DK * DV;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      *reinterpret_cast<f32x4*>(No + ((wave * 8 + m) * 64 + lane) * 4) = SN[m];  // seg_acc_pos
      if constexpr (PHI) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a.Pseg[sb * DK * DK + (16 * m + 4 * g + i) * DK + col] = SP[m][i];
      }
    }
  }
}

template <int MODE, int AK, int BK, int WK>
__global__ __launch_bounds__(kSegThreads) void seg_kernel(SegArgs a) {
  using L = SegLayout<MODE, AK, BK, WK>;
  static_assert(L::fits, "LDS layout exceeds the gfx950 workgroup limit");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[L::total];
  const int64_t bh = blockIdx.x / a.nseg, seg = blockIdx.x % a.nseg;
  if (seg == 0)
    seg_body<MODE, AK, BK, WK, false>(a, smem, bh, seg);
  else
    seg_body<MODE, AK, BK, WK, true>(a, smem, bh, seg);
}

// x = hi + lo in bf16 (hi the rounding of x, lo that of the remainder): products of such pairs
// taken as hi hi + hi lo + lo hi carry about 16 significant bits, where one bf16 product keeps 8.
__device__ __forceinline__ void seg_split8(const float* x, Mma<__bf16>::F8& hi, Mma<__bf16>::F8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi[e] = static_cast<__bf16>(x[e]);
    lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(hi[e]));
  }
}


// ---- segment chain: E_{s+1} = Phi_s E_s + N_s ----
// E_1 is segment 0's exit state (seg_kernel writes it to Eseg slot 1).  Writes every E_s
// (1 <= s < nseg) as bf16, transposed and in pair order, into Ebf for the correction, and E_nseg
// into S_T.  One workgroup of 4 waves per (state, 16 NT value columns); wave w computes rows
// 32 w .. 32 w + 31 of E (two 16-row tiles by NT 16-column tiles) on MFMA, in the three-term
// bf16 form of seg_split8 with fp32 accumulation (two partial sums over the k blocks, so that the
// dependent MFMA chains are half as long).  The two row tiles of wave w are, as accumulators,
// exactly the B operands of k block w for every wave: each step passes them through LDS.  Phi and
// N are loaded two segments ahead of their use.
template <int NT>
__global__ __launch_bounds__(256) void seg_chain_kernel(SegArgs a) {
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  constexpr int DK = 128, DV = 128, kChainNT = NT, kChainCols = 16 * NT, NB = DV / kChainCols;
  __shared__ __attribute__((aligned(16))) uint4 sB[2][4][kChainNT][2][64];  // [buffer][kb][n][hi, lo][lane]
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  // (the workgroups of one state on one XCD, so that its L2 serves them each segment's Phi)
  const int64_t nb = gridDim.x, bid = blockIdx.x;
  const int64_t p = (nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
  const int64_t bh = p / NB, c0 = (p % NB) * kChainCols;
  const int64_t nseg = a.nseg;

  f32x4 acc[2][kChainNT];  // [row tile 2 w + mt][column tile n]: rows 32 w + 16 mt + 4 g + i, column c0 + 16 n + l16
  {
    // (seg_acc_pos: column tile c0 / 16 + n, row tile 2 w + mt, this lane)
    const float* E1 = a.Eseg + (bh * nseg + 1) * DK * DV;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int n = 0; n < kChainNT; ++n)
        acc[mt][n] = *reinterpret_cast<const f32x4*>(E1 + (((c0 / 16 + n) * 8 + 2 * w + mt) * 64 + lane) * 4);
  }
  // Phi rows 32 w + 16 mt + l16, channels 32 kb + 16 h + 4 g .. + 3, and N at the accumulator
  // positions, of one segment
  using PhiRegs = float4[2][4][2];
  using NRegs = f32x4[2][kChainNT];
  auto load = [&](int64_t s, PhiRegs& ph, NRegs& nx) {
    const float* P = a.Pseg + (bh * nseg + s) * DK * DK;
    const float* Nn = a.Nseg + (bh * nseg + s) * DK * DV;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          ph[mt][kb][h] = *reinterpret_cast<const float4*>(P + (32 * w + 16 * mt + l16) * DK + 32 * kb + 16 * h + 4 * g);
#pragma unroll
      for (int n = 0; n < kChainNT; ++n)
        nx[mt][n] = *reinterpret_cast<const f32x4*>(Nn + (((c0 / 16 + n) * 8 + 2 * w + mt) * 64 + lane) * 4);
    }
  };
  // E_{s+1} = Phi_s E_s + N_s with E_s in acc
  auto step = [&](int64_t s, const PhiRegs& ph, const NRegs& nx) {
    const int buf = static_cast<int>(s & 1);
    // E_s: its bf16 transposed copy and its B operands
    __bf16* eb = a.Ebf + (bh * nseg + s) * DV * DK;
#pragma unroll
    for (int n = 0; n < kChainNT; ++n) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        float e4[4] = {acc[mt][n][0], acc[mt][n][1], acc[mt][n][2], acc[mt][n][3]};
        *reinterpret_cast<uint2*>(eb + (c0 + 16 * n + l16) * DK + 32 * w + 8 * g + 4 * mt) = pack4(e4);
      }
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = acc[0][n][i];
        x[4 + i] = acc[1][n][i];
      }
      F8 hi, lo;
      seg_split8(x, hi, lo);
      sB[buf][w][n][0][lane] = __builtin_bit_cast(uint4, hi);
      sB[buf][w][n][1][lane] = __builtin_bit_cast(uint4, lo);
    }
    lds_barrier();
    F8 ah[2][4], al[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float x[8] = {ph[mt][kb][0].x, ph[mt][kb][0].y, ph[mt][kb][0].z, ph[mt][kb][0].w,
                            ph[mt][kb][1].x, ph[mt][kb][1].y, ph[mt][kb][1].z, ph[mt][kb][1].w};
        seg_split8(x, ah[mt][kb], al[mt][kb]);
      }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int n = 0; n < kChainNT; ++n) acc[mt][n] = nx[mt][n];
    F8 bfr[4][kChainNT][2];  // all B operands first, so that their LDS latencies overlap
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int n = 0; n < kChainNT; ++n)
#pragma unroll
        for (int hl = 0; hl < 2; ++hl) bfr[kb][n][hl] = __builtin_bit_cast(F8, sB[buf][kb][n][hl][lane]);
    f32x4 acc2[2][kChainNT];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int n = 0; n < kChainNT; ++n) acc2[mt][n] = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int n = 0; n < kChainNT; ++n) {
        const F8 bh_ = bfr[kb][n][0], bl_ = bfr[kb][n][1];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          f32x4& t = kb < 2 ? acc[mt][n] : acc2[mt][n];
          t = MM::mma8(ah[mt][kb], bh_, t);
          t = MM::mma8(ah[mt][kb], bl_, t);
          t = MM::mma8(al[mt][kb], bh_, t);
        }
      }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int n = 0; n < kChainNT; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][n][i] += acc2[mt][n][i];
  };
  // two register sets, each loaded two segments ahead of its use; loads are unconditional (past
  // the end they repeat the last segment, unused), so the compiler's wait before one set's use
  // leaves the other set's loads in flight
  if (nseg > 1) {
    const int64_t last = nseg - 1;
    PhiRegs pA, pB;
    NRegs nA, nB;
    load(1, pA, nA);
    load(2 < last ? 2 : last, pB, nB);
    __builtin_amdgcn_sched_barrier(0);
    for (int64_t s = 1; s < nseg; s += 2) {
      step(s, pA, nA);
      load(s + 2 < last ? s + 2 : last, pA, nA);
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < nseg) step(s + 1, pB, nB);
      load(s + 3 < last ? s + 3 : last, pB, nB);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (a.S_T != nullptr) {
    float* St = a.S_T + bh * DK * DV;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int n = 0; n < kChainNT; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) St[(32 * w + 16 * mt + 4 * g + i) * DV + c0 + 16 * n + l16] = acc[mt][n][i];
  }
}

constexpr int kFixGroup = 8;  // chunks per correction workgroup
constexpr int kFixRing = 4;   // chunk slots of the correction's LDS ring (inputs two chunks ahead)

// ---- correction: o_c = O_c(N) + Q~_c E_s for every chunk c of segments s > 0 ----
// One workgroup of 4 waves per (state, segment s > 0, group of up to 8 of its chunks); wave w takes
// value column tiles 2 w, 2 w + 1 and keeps their rows of E_s^T (Ebf: transposed, each 32-channel
// block in the pair order of seg_qt_pos) as A operands for the whole group.  O^T tile (columns
// 16 n + 4 g + i, tokens 16 ta + l16) = O(N)^T + E^T Q~^T: On supplies the accumulators and Qt the
// B operands; o is only written.  Each chunk's Qt and On blocks (8 KB each, contiguous) arrive in
// a ring of four LDS slots by direct-to-LDS loads, every wave issuing a quarter of them, two chunks
// ahead of their use: the slot refilled in iteration i held chunk i - 2, whose reads all waves
// finished before the barrier of iteration i - 1.  So a chunk's 16 KB is read from HBM once per
// workgroup (not once per wave) and no registers hold loads in flight; one barrier per chunk.
__global__ __launch_bounds__(256) void seg_fix_kernel(SegArgs a) {
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  constexpr int DK = 128, DV = 128, C = kSegC;
  constexpr int SLOT = 2 * C * DK * 2;  // Qt block, then On block
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kFixRing * SLOT];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  // (32-bit index arithmetic: the grid is far below 2^31 workgroups)
  const uint32_t ngrp = static_cast<uint32_t>((a.L + kFixGroup - 1) / kFixGroup);
  const uint32_t nsm1 = static_cast<uint32_t>(a.nseg - 1);
  // consecutive workgroup indices go to different XCDs (8, round robin): renumber so that the
  // groups of one (state, segment) share an XCD, and so its L2, for the entering state they all read
  const uint32_t nb = gridDim.x, bid = blockIdx.x;
  uint32_t blk = (nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
  const uint32_t grp = blk % ngrp;
  blk /= ngrp;
  const int64_t s = 1 + blk % nsm1, bh = blk / nsm1;
  const int64_t seg_end = (s + 1) * a.L < a.nch ? (s + 1) * a.L : a.nch;
  const int64_t c0 = s * a.L + static_cast<int64_t>(grp) * kFixGroup;
  const int64_t c1 = c0 + kFixGroup < seg_end ? c0 + kFixGroup : seg_end;
  if (c0 >= c1) return;  // past the end of a shorter last segment (uniform: before any load)
  const int n = static_cast<int>(c1 - c0);
  const int64_t bi = bh / a.H, hi = bh % a.H;
  const uint32_t hdv = static_cast<uint32_t>(a.H * DV * 2);
  const __bf16* eb = a.Ebf + (bh * a.nseg + s) * DV * DK;
  F8 ef[2][4];
#pragma unroll
  for (int nn = 0; nn < 2; ++nn)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      ef[nn][kb] = *reinterpret_cast<const F8*>(eb + (16 * (2 * wave + nn) + l16) * DK + 32 * kb + 8 * g);

  // chunk c0 + i (clamped to the group's last chunk, so that every iteration issues the same
  // number of loads) into slot `slot`: this wave's 1 KB pieces 2 wave, 2 wave + 1 of each block
  auto issue = [&](int i, int slot) {
    const int64_t c = c0 + (i < n ? i : n - 1);
    const unsigned char* qt = reinterpret_cast<const unsigned char*>(a.Qt + (bh * a.nch + c) * C * DK);
    const unsigned char* on = reinterpret_cast<const unsigned char*>(a.On + (bh * a.nch + c) * C * DV);
    unsigned char* dst = ring + slot * SLOT;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int piece = 2 * wave + p;
      seg_dma16(qt + piece * 1024, 1024, dst + piece * 1024, 16 * lane);
      seg_dma16(on + piece * 1024, 1024, dst + C * DK * 2 + piece * 1024, 16 * lane);
    }
  };
  constexpr int kLoadsPerChunk = 4;  // direct-to-LDS loads one wave issues per chunk
  // s_waitcnt immediate: at most 2 chunks' loads outstanding (gfx9 encoding: vmcnt bits 3:0 and
  // 15:14, expcnt and lgkmcnt at their maxima); loads complete in order, so chunk i's are done
  constexpr int kWaitRing = 0x0F70 | (2 * kLoadsPerChunk & 0xF) | (((2 * kLoadsPerChunk >> 4) & 3) << 14);

  issue(0, 0);
  issue(1, 1);
  for (int i = 0; i < n; ++i) {
    issue(i + 2, (i + 2) & (kFixRing - 1));
    __builtin_amdgcn_s_waitcnt(kWaitRing);
    lds_barrier_keep_vm();  // every wave's pieces of chunk i are in
    const unsigned char* slot = ring + (i & (kFixRing - 1)) * SLOT;
    const int64_t t0 = (c0 + i) * C;
    const auto ro = make_rsrc(a.o + ((bi * a.T + t0) * a.H + hi) * DV, wy_range(a.T - t0, a.H, DV));
#pragma unroll
    for (int ta = 0; ta < 2; ++ta) {
      F8 q[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) q[kb] = *reinterpret_cast<const F8*>(slot + ((ta * 4 + kb) * 64 + lane) * 16);
      const uint32_t t = static_cast<uint32_t>(16 * ta + l16);
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) {
        float o4[4];
        unpack4(*reinterpret_cast<const uint2*>(slot + C * DK * 2 + ((ta * 8 + 2 * wave + nn) * 64 + lane) * 8), o4);
        f32x4 acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = o4[e];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc = MM::mma8(ef[nn][kb], q[kb], acc);
        float r4[4] = {acc[0], acc[1], acc[2], acc[3]};
        buf_store8(ro, t * hdv + (16 * (2 * wave + nn) + 4 * g) * 2, pack4(r4));
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // the clamped loads past the group land before exit
}

}  // namespace gdr
