// Chunkwise prefill of the gated delta rule on gfx950: one fused kernel.
//
// One workgroup (4 waves) owns one (batch, head) state and a slice of DVS = 16*NSW value
// columns; it walks the chunks of 64 tokens in order and keeps its slice of S in the
// accumulator registers of NSW "state waves" (16 columns each) for the whole sequence.
// Columns of S evolve independently (the transition multiplies S from the left:
// "Recurrent Memory: Write, Erase, Decay, Read", section 05), which is what makes the
// column slicing exact.
//
// Chunk form (derived by unrolling the recurrence over a chunk; section 03 of the same
// page notes that the linear erase reassociates into a chunkwise-parallel form, section
// 04 that the decay enters as prefix sums of log alpha, and the Gated DeltaNet-2 abstract
// that a channel-wise decay is absorbed into separate erase factors).  With entering
// state S, local prefix sums G_t of log alpha (G_0 = 0), c = b . k and x = w . v:
//
// MODE 0 (scalar decay, either order) and MODE 1 (per-channel decay applied before the
// erase) are rank one per token: u_t = x_t - c_t Diag(alpha_t) S_{t-1}, S_t = Diag(alpha_t)
// S_{t-1} + k_t^T u_t.  With Chat_t = c_t e^{G_t}, Khat_i = k_i e^{-G_i}, Qhat_t = q_t e^{G_t},
// Kbar_i = k_i e^{G_n - G_i} and A = strict_tril(Chat Khat^T), M = tril(Qhat Khat^T):
//     (I + A) R = Chat S - X                 (R = -U)
//     O = Qhat S - M R,     S' = e^{G_n} . S - Kbar^T R
// MODE 2 (per-channel decay after the erase, the unified equation's order): the erase
// of token i uses the decay-absorbed key alpha_i . k_i while the write uses k_i, so two
// key families appear.  With Chat_t = c_t e^{G_{t-1}}, Phat_i = k_i e^{-G_{i-1}},
// Pbar_i = k_i e^{G_n - G_{i-1}}, L_P = strict_tril(Chat Phat^T), L_K = strict_tril(Chat
// Khat^T), M_QK = tril(Qhat Khat^T), M_QP = tril(Qhat Phat^T):
//     (I + L_P) R = Chat S + L_K X           (R_t = c_t S_{t-1}, the erase reads)
//     O  = Qhat S + M_QK X - M_QP R,   S' = e^{G_n} . S + Kbar^T X - Pbar^T R
//
// Per-channel exponentials are split around a reference G_ref = G_31 (mid-chunk) in the
// products that do not involve S (e^{G_t - G_ref} on row operands, e^{G_ref - G_i} on
// column operands, each factor clamped at e^80), and the S-side products use the same row
// operands against e^{G_ref} . S.  Scalar decay uses the exact pairwise mask
// e^{G_t - G_i} instead.
//
// The unit-lower-triangular solve runs as blocked forward substitution over 16-row
// blocks on the state waves (R_i = T_ii (V_i - sum_{m<i} L_im R_m)), with the four
// 16x16 diagonal inverses T_ii computed once per chunk in fp32 by substitution.
//
// Phases per chunk (barriers between): A gate prefix sums and scaled operands into LDS;
// B Gram tiles on MFMA; C diagonal inverses; D state waves: S-side products, solve,
// read-out, state update.
#pragma once
#include "gdr_common.h"
#include "mfma.h"

// Phase markers: no-ops unless a profiling build defines GDR_MARK before including this file.
#ifndef GDR_MARK
#define GDR_MARK(id) ((void)0)
#endif

namespace gdr {

constexpr int kLdsLimit = 163840;  // bytes of LDS one gfx950 workgroup may use
// s_waitcnt immediate that waits for vmcnt = 0 only (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt in bits 6:4, lgkmcnt in bits 11:8; the last two left at their maxima)
constexpr int kWaitVmcnt0 = 0x0F70;

template <typename OT, int DK, int NSW, int MODE>
struct PrefillLayout {
  static constexpr int C = 64;
  static constexpr int DVS = 16 * NSW;
  // row pitches (elements) of token-major operands and of channel-major / 64-wide arrays: padded
  // by 8 against bank conflicts, except at dk = 256, whose unpadded layout is what fits in LDS
  static constexpr int PAD = DK >= 256 ? 0 : 8;
  static constexpr int LDT = DK + PAD;
  static constexpr int LDD = C + PAD;
  static constexpr int LDI = 24;      // row pitch of the diagonal inverses
  static constexpr int ES = sizeof(OT);
  static constexpr bool TWO = MODE == 2;
  static constexpr int NCG = DK / 8;  // 8-channel groups in the gate preparation
  static constexpr int NSEG = (256 / NCG) < C ? (256 / NCG) : C;
  static constexpr int TPS = C / NSEG;  // tokens per thread in the gate preparation
  static constexpr int SEG_BYTES = NSEG * DK * 4;
  static constexpr int GRAM_BYTES = C * LDD * ES;
  static constexpr int oQ = 0;                                   // Qhat   [C][LDT]
  static constexpr int oC = oQ + C * LDT * ES;                   // Chat   [C][LDT]
  static constexpr int oK = oC + C * LDT * ES;                   // Khat   [C][LDT]
  static constexpr int oP = oK + C * LDT * ES;                   // Phat   [C][LDT] (MODE 2)
  static constexpr int oDP = oP + (TWO ? C * LDT * ES : 0);      // -Pbar^T / -Kbar^T [DK][LDD]
  static constexpr int oDK = oDP + DK * LDD * ES;                // Kbar^T [DK][LDD] (MODE 2)
  static constexpr int oX = oDK + (TWO ? DK * LDD * ES : 0);     // X^T    [DVS][LDD]
  static constexpr int oGA = oX + DVS * LDD * ES;                // -L (solve) / segment sums
  static constexpr int oGM = oGA + (GRAM_BYTES > SEG_BYTES ? GRAM_BYTES : SEG_BYTES);  // -M
  static constexpr int oGLK = oGM + GRAM_BYTES;                  // L_K (MODE 2)
  static constexpr int oGMQK = oGLK + (TWO ? GRAM_BYTES : 0);    // M_QK (MODE 2)
  static constexpr int oINV = oGMQK + (TWO ? GRAM_BYTES : 0);    // T_ii [4][16][LDI]
  static constexpr int LDL = 20;                                 // column pitch of L_ii
  static constexpr int oLD = oINV + 4 * 16 * LDI * ES;           // fp32 L_ii, column-major [4][16][LDL]
  static constexpr int oF = oLD + 4 * 16 * LDL * 4;              // fp32 per-channel / per-token
  static constexpr int NF = MODE == 0 ? 2 * C + 8 : 4 * DK + 4;  // + robust-chunk flag
  static constexpr int total = oF + NF * 4;
  static constexpr bool fits = total <= kLdsLimit;
};

template <typename IO>
struct PrefillArgs {
  const IO* q;
  const IO* k;
  const IO* v;
  const IO* la;
  const IO* bg;
  const IO* wg;
  const float* S0;
  IO* o;
  float* S_T;
  int64_t T, H, DV;
  int alpha_kind, b_kind, w_kind;
  int nsl;     // value slices per state
  int64_t Hk;  // q / k heads (H is a multiple): value head h reads q / k head h / (H / Hk)
};

// 8 consecutive I/O elements starting at p (16-byte aligned for bf16) as fp32.
__device__ __forceinline__ void load8f(const bf16_t* p, float* out) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = __uint_as_float(w[j] << 16);
    out[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8f(const float* p, float* out) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// Raw buffer resource over `bytes` bytes from `base` (gfx9 descriptor word 3).  Loads past the
// range return zero and stores past it are dropped, which pads the ragged last chunk.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}
// Raw 16-bit load; converted to fp32 only where the value is used, so that issuing the load
// does not wait for it.
__device__ __forceinline__ uint16_t buf_load_u16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// Eight consecutive I/O elements held in registers in their I/O encoding: a prefetch issues the
// load and nothing waits for it until the values are converted.
template <typename IO>
struct Raw8;
template <>
struct Raw8<bf16_t> {
  uint4 u;
};
template <>
struct Raw8<float> {
  float4 a, b;
};
__device__ __forceinline__ Raw8<bf16_t> raw8_load(const bf16_t* p) {
  return {*reinterpret_cast<const uint4*>(p)};
}
__device__ __forceinline__ Raw8<float> raw8_load(const float* p) {
  const float4* q = reinterpret_cast<const float4*>(p);
  return {q[0], q[1]};
}
__device__ __forceinline__ void raw8_zero(Raw8<bf16_t>& r) { r.u = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void raw8_zero(Raw8<float>& r) {
  r.a = make_float4(0.f, 0.f, 0.f, 0.f);
  r.b = r.a;
}
__device__ __forceinline__ void raw8_cvt(const Raw8<bf16_t>& r, float* out) {
  load8f(reinterpret_cast<const bf16_t*>(&r.u), out);
}
__device__ __forceinline__ void raw8_cvt(const Raw8<float>& r, float* out) {
  out[0] = r.a.x; out[1] = r.a.y; out[2] = r.a.z; out[3] = r.a.w;
  out[4] = r.b.x; out[5] = r.b.y; out[6] = r.b.z; out[7] = r.b.w;
}
__device__ __forceinline__ void raw8_buf(Raw8<bf16_t>& r, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
  r.u = buf_load16(rs, off);
}
__device__ __forceinline__ void raw8_buf(Raw8<float>& r, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
  r.a = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  r.b = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0));
}
__device__ __forceinline__ void raw1_buf(bf16_t& x, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
  x.x = buf_load_u16(rs, off);
}
__device__ __forceinline__ void raw1_buf(float& x, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
  x = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
}
__device__ __forceinline__ void buf_store1(bf16_t*, __amdgpu_buffer_rsrc_t rs, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), rs, off, 0, 0);
}
__device__ __forceinline__ void buf_store1(float*, __amdgpu_buffer_rsrc_t rs, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, off, 0, 0);
}
__device__ __forceinline__ float raw1_cvt(bf16_t x) { return bf16_to_f32(x.x); }
__device__ __forceinline__ float raw1_cvt(float x) { return x; }
__device__ __forceinline__ void raw1_zero(bf16_t& x) { x.x = 0; }
__device__ __forceinline__ void raw1_zero(float& x) { x = 0.f; }

template <typename OT>
__device__ __forceinline__ void lds_store8(OT* p, const float* v) {
  typename Mma<OT>::F8 f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = to_ot<OT>(v[j]);
  *reinterpret_cast<typename Mma<OT>::F8*>(p) = f;
}

__device__ __forceinline__ float exp_clamped(float x) { return __expf(fminf(x, 80.f)); }

// Channel-major rows (k^T, X^T) hold 64 tokens; quads of 4 tokens are stored at quad ^ key(row)
// so that transposed writes from lanes with different rows hit different banks.  Reads of 4
// consecutive tokens from a quad boundary stay contiguous.
__device__ __forceinline__ int swz(int row_key, int t) { return (((t >> 2) ^ row_key) << 2) | (t & 3); }

// N (1, 2 or 4) consecutive elements as one LDS store.
template <int N>
__device__ __forceinline__ void lds_store_run(__bf16* p, const __bf16* v) {
  static_assert(N == 1 || N == 2 || N == 4, "runs of 1, 2 or 4 elements");
  uint32_t h[N];
#pragma unroll
  for (int j = 0; j < N; ++j) h[j] = __builtin_bit_cast(uint16_t, v[j]);
  if constexpr (N == 4) {
    *reinterpret_cast<uint2*>(p) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  } else if constexpr (N == 2) {
    *reinterpret_cast<uint32_t*>(p) = h[0] | (h[1] << 16);
  } else {
    p[0] = v[0];
  }
}
template <int N>
__device__ __forceinline__ void lds_store_run(float* p, const float* v) {
  static_assert(N == 1 || N == 2 || N == 4, "runs of 1, 2 or 4 elements");
  if constexpr (N == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  } else if constexpr (N == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  } else {
    p[0] = v[0];
  }
}

// Fragment from two 4-element runs of an LDS row (k = 4 consecutive values each).
template <typename OT>
__device__ __forceinline__ typename Mma<OT>::F8 lds_two_quads(const OT* row, int pa, int pb) {
  const typename Mma<OT>::F4 lo = lds_load4(row + pa), hi = lds_load4(row + pb);
  typename Mma<OT>::F8 f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = lo[j];
    f[4 + j] = hi[j];
  }
  return f;
}

template <typename IO, typename OT, int DK, int NSW, int MODE>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs<IO> a) {
  using L = PrefillLayout<OT, DK, NSW, MODE>;
  using MM = Mma<OT>;
  using F8 = typename MM::F8;
  static_assert(L::fits, "LDS layout exceeds the gfx950 workgroup limit");
  constexpr int C = L::C, DVS = L::DVS, LDT = L::LDT, LDD = L::LDD, LDI = L::LDI;
  constexpr int NTD = DK / 16;         // 16-row tiles of the state slice
  constexpr int NKB = (DK + 31) / 32;  // 32-wide k blocks over dk
  constexpr bool TWO = MODE == 2;

  __shared__ __attribute__((aligned(32))) unsigned char smem[L::total];
  OT* tQ = reinterpret_cast<OT*>(smem + L::oQ);
  OT* tC = reinterpret_cast<OT*>(smem + L::oC);
  OT* tK = reinterpret_cast<OT*>(smem + L::oK);
  OT* tP = reinterpret_cast<OT*>(smem + L::oP);
  OT* dP = reinterpret_cast<OT*>(smem + L::oDP);
  OT* dK = reinterpret_cast<OT*>(smem + L::oDK);
  OT* xT = reinterpret_cast<OT*>(smem + L::oX);
  OT* gA = reinterpret_cast<OT*>(smem + L::oGA);
  float* segtot = reinterpret_cast<float*>(smem + L::oGA);  // aliases gA (phase A only)
  OT* gM = reinterpret_cast<OT*>(smem + L::oGM);
  OT* gLK = reinterpret_cast<OT*>(smem + L::oGLK);
  OT* gMQK = reinterpret_cast<OT*>(smem + L::oGMQK);
  OT* dInv = reinterpret_cast<OT*>(smem + L::oINV);
  float* Ld = reinterpret_cast<float*>(smem + L::oLD);
  float* fF = reinterpret_cast<float*>(smem + L::oF);
  // MODE 0: fF = [G_t (64) | e^{G_t} (64) | e^{G_n}];  MODE 1/2: [G_ref | G_n | e^{G_ref} | e^{G_n}]
  float* sG = fF;
  float* sEG = fF + C;
  float* sEGn = fF + 2 * C;
  float* fRef = fF;
  float* fGn = fF + DK;
  float* fEref = fF + 2 * DK;
  float* fEGn = fF + 3 * DK;
  int* sRobust = reinterpret_cast<int*>(fF + 4 * DK);  // MODE 1/2: this chunk takes the exact path
  // Largest |G_t - G_ref| (per channel, within a chunk) for which the split exponentials stay
  // below the e^80 clamp; chunks beyond it run token by token (robust path, exact).
  constexpr float kSpanLimit = 76.f;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches on it
  int lane = tid & 63, g = lane >> 4, l16 = lane & 15;

  // Block -> (state, slice).  Blocks are dealt round-robin to the 8 XCDs; consecutive
  // pairs p land on one XCD, so the slices of one head share that XCD's L2.
  const int64_t nb = gridDim.x, bid = blockIdx.x;
  const int64_t p = (nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
  const int64_t bh = p / a.nsl;
  const int sl = static_cast<int>(p % a.nsl);
  const int64_t bi = bh / a.H, hi = bh % a.H;
  const int64_t DV = a.DV;
  const int64_t col0 = static_cast<int64_t>(sl) * DVS;

  // Gram outputs: tiles above the diagonal are never written and must read as zero.
  {
    float* z = reinterpret_cast<float*>(smem + L::oGM);
    const int nz = (L::oINV - L::oGM) / 4;
    for (int i = tid; i < nz; i += 256) z[i] = 0.f;
  }

  const bool sside = wave < NSW;
  const int nloc = 16 * wave + l16;  // state wave: local value column
  const int64_t sbase = bh * DK * DV + col0 + nloc;
  f32x4 S[NTD];
#pragma unroll
  for (int tl = 0; tl < NTD; ++tl) {
    S[tl] = zero4();
    if (sside && a.S0 != nullptr) {
#pragma unroll
      for (int i = 0; i < 4; ++i) S[tl][i] = a.S0[sbase + (int64_t)(16 * tl + 4 * g + i) * DV];
    }
  }

  const int64_t nch = (a.T + C - 1) / C;

  // ---------------- prefetch registers ----------------
  // Each thread holds, for the next chunk: channels d0..d0+7 of tokens ts*TPS.. (q, k, b, log
  // alpha) and one 8-column group of one token of v and w.  Loaded while the current chunk
  // computes; tokens past the end read as zero (identity padding).
  constexpr int NCG = L::NCG, NSEG = L::NSEG, TPS = L::TPS;
  constexpr int NXG = DVS / 8;
  constexpr int XPT = (NXG * C + 255) / 256;
  int ts = tid / NCG, d0 = (tid % NCG) * 8;
  const bool act = ts < NSEG;
  Raw8<IO> pq[TPS], pk[TPS], pb[TPS], pla[TPS], pv[XPT], pw[XPT];
  IO pbs[TPS], pws[XPT], pla0;
  // Buffer resources are rebased at each chunk's first token, so offsets stay below 64 token
  // rows whatever T is; rows past the last token fall outside the range and load as zero.
  constexpr uint32_t ES = sizeof(IO);
  const uint32_t hdk = static_cast<uint32_t>(a.H * DK) * ES, hdv = static_cast<uint32_t>(a.H * DV) * ES;
  const uint32_t hqk = static_cast<uint32_t>(a.Hk * DK) * ES;  // token stride of q and k
  const uint32_t h1 = static_cast<uint32_t>(a.H) * ES;
  const int64_t hq = hi / (a.H / a.Hk);                         // this state's q / k head
  auto prefetch = [&](int64_t c) {
    const int64_t t0 = c * C;
    const int64_t rr = (bi * a.T + t0) * a.H + hi;  // row of the chunk's first token
    const int64_t left = a.T - t0;                  // tokens from t0 to the end, >= 1
    auto range = [&](int64_t width) -> uint32_t {
      const int64_t bytes = ((left - 1) * a.H + 1) * width * ES;
      return static_cast<uint32_t>(bytes < 0x7fffffff ? bytes : 0x7fffffff);
    };
    // Every load is issued unconditionally (no branch, so no wait at a join): a gate kind that
    // is absent gets an empty range and inactive lanes an out-of-range offset; both read zero.
    const uint32_t oob = 0x80000000u;
    const uint32_t vb = range(DV) - static_cast<uint32_t>(col0) * ES;
    const auto rv = make_rsrc(a.v + rr * DV + col0, vb);
    const auto rwc = make_rsrc(a.w_kind == kChannel ? a.wg + rr * DV + col0 : a.v, a.w_kind == kChannel ? vb : 0u);
    const auto rws = make_rsrc(a.w_kind == kScalar ? a.wg + rr : a.v, a.w_kind == kScalar ? range(1) : 0u);
    const int64_t rqk = (bi * a.T + t0) * a.Hk + hq;  // q / k row of the chunk's first token
    const int64_t qkb = ((left - 1) * a.Hk + 1) * DK * ES;
    const uint32_t qkr = static_cast<uint32_t>(qkb < 0x7fffffff ? qkb : 0x7fffffff);
    const auto rq = make_rsrc(a.q + rqk * DK, qkr);
    const auto rk = make_rsrc(a.k + rqk * DK, qkr);
    const auto rbc = make_rsrc(a.b_kind == kChannel ? a.bg + rr * DK : a.q, a.b_kind == kChannel ? range(DK) : 0u);
    const auto rbs = make_rsrc(a.b_kind == kScalar ? a.bg + rr : a.q, a.b_kind == kScalar ? range(1) : 0u);
    const auto rla = make_rsrc(a.alpha_kind == kChannel ? a.la + rr * DK : (a.alpha_kind == kScalar ? a.la + rr : a.q),
                               a.alpha_kind == kChannel ? range(DK) : (a.alpha_kind == kScalar ? range(1) : 0u));
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int item = tid + 256 * j;
      const uint32_t t = item / NXG, xg = item % NXG;
      const bool in = item < NXG * C;
      const uint32_t xo = in ? t * hdv + xg * 8 * ES : oob;
      raw8_buf(pv[j], rv, xo);
      raw8_buf(pw[j], rwc, xo);
      raw1_buf(pws[j], rws, in ? t * h1 : oob);
    }
    if (MODE == 0) raw1_buf(pla0, rla, wave == 0 ? static_cast<uint32_t>(lane) * h1 : oob);
#pragma unroll
    for (int u = 0; u < TPS; ++u) {
      const uint32_t t = ts * TPS + u;
      const uint32_t ko = act ? t * hdk + d0 * ES : oob;
      const uint32_t qo = act ? t * hqk + d0 * ES : oob;
      raw8_buf(pq[u], rq, qo);
      raw8_buf(pk[u], rk, qo);
      raw8_buf(pb[u], rbc, ko);
      raw1_buf(pbs[u], rbs, act ? t * h1 : oob);
      if (MODE != 0) raw8_buf(pla[u], rla, ko);
    }
  };
  if (nch > 0) prefetch(0);

  for (int64_t ch = 0; ch < nch; ++ch) {
    // Opaque per chunk: keeps the compiler from hoisting every per-lane LDS address out of the
    // chunk loop, which would hold them in registers for the whole kernel.
    asm volatile("" : "+v"(lane), "+v"(g), "+v"(l16), "+v"(ts), "+v"(d0));
    const int64_t t0 = ch * C;
    const int nval = static_cast<int>(a.T - t0 < C ? a.T - t0 : C);
    auto row_of = [&](int t) -> int64_t { return (bi * a.T + t0 + t) * a.H + hi; };
    if (MODE != 0 && tid == 0) sRobust[0] = 0;
    lds_barrier();  // the previous chunk's readers of every LDS array are done
    GDR_MARK(0);

    // ---------------- phase A: X^T, gate prefix sums, scaled operands ----------------
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int item = tid + 256 * j;
      if (item < NXG * C) {
        const int xg = item % NXG, t = item / NXG;
        float x[8];
        raw8_cvt(pv[j], x);
        if (a.w_kind == kChannel) {
          float w[8];
          raw8_cvt(pw[j], w);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= w[e];
        } else if (a.w_kind == kScalar) {
          const float w = raw1_cvt(pws[j]);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) xT[(xg * 8 + e) * LDD + t] = to_ot<OT>(x[e]);
      }
    }

    float la8[TPS][8], G8[TPS][8];
    if (MODE == 0) {
      if (wave == 0) {
        float x = raw1_cvt(pla0);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(x, off);
          if (lane >= off) x += y;
        }
        sG[lane] = x;
        sEG[lane] = __expf(x);
        if (lane == 63) sEGn[0] = __expf(x);
      }
    } else {
      if (act) {
        float run[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < TPS; ++u) {
          raw8_cvt(pla[u], la8[u]);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            run[j] += la8[u][j];
            G8[u][j] = run[j];
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) segtot[ts * DK + d0 + j] = run[j];
      }
      lds_barrier();
      if (tid < DK) {
        float run = 0.f;
        for (int s = 0; s < NSEG; ++s) {
          const float tv = segtot[s * DK + tid];
          segtot[s * DK + tid] = run;
          run += tv;
        }
        const float ref = segtot[(NSEG / 2) * DK + tid];
        fRef[tid] = ref;
        fGn[tid] = run;
        fEref[tid] = __expf(ref);
        fEGn[tid] = __expf(run);
        if (fmaxf(fabsf(ref), fabsf(run - ref)) > kSpanLimit || !(run == run)) sRobust[0] = 1;
      }
    }
    lds_barrier();
    const bool robust = MODE != 0 && sRobust[0] != 0;

    GDR_MARK(1);
    if (act) {
      float off[8], ref[8], egr[8];
      if (MODE != 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          off[j] = segtot[ts * DK + d0 + j];
          ref[j] = fRef[d0 + j];
          egr[j] = __expf(fGn[d0 + j] - ref[j]);  // e^{G_n - G_ref}
        }
      }
      OT pdp[8][TPS], pdk[8][TPS];
#pragma unroll
      for (int u = 0; u < TPS; ++u) {
        const int t = ts * TPS + u;
        float q[8], k[8], c[8];
        raw8_cvt(pq[u], q);
        raw8_cvt(pk[u], k);
        if (a.b_kind == kChannel) {
          raw8_cvt(pb[u], c);
#pragma unroll
          for (int j = 0; j < 8; ++j) c[j] *= k[j];
        } else {
          const float bs = a.b_kind == kScalar ? raw1_cvt(pbs[u]) : 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) c[j] = bs * k[j];
        }
        float oq[8], oc[8], ok[8], op[8], odp[8], odk[8];
        if (MODE != 0 && robust) {
          // exact path: raw q, c = b . k, k and log alpha, token-major
          OT* laArr = TWO ? tP : dP;
          const int lpitch = TWO ? LDT : ((C * LDT <= DK * LDD) ? LDT : DK);
          lds_store8(tQ + t * LDT + d0, q);
          lds_store8(tC + t * LDT + d0, c);
          lds_store8(tK + t * LDT + d0, k);
          lds_store8(laArr + t * lpitch + d0, la8[u]);
          continue;
        }
        if (MODE == 0) {
          const float fk = __expf(sG[C - 1] - sG[t]);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            oq[j] = q[j];
            oc[j] = c[j];
            ok[j] = k[j];
            odp[j] = -k[j] * fk;
          }
        } else {
          // A chunk on this path has every |G_t - G_ref| and |G_n - G_ref| within the span
          // limit, so each factor below stays inside the fp32 range; reciprocals replace the
          // exponentials of negated arguments.
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float G = G8[u][j] + off[j];
            const float eq = __expf(G - ref[j]);          // e^{G_t - G_ref}
            const float er = __builtin_amdgcn_rcpf(eq);   // e^{G_ref - G_t}
            oq[j] = q[j] * eq;
            ok[j] = k[j] * er;
            if (MODE == 1) {
              oc[j] = c[j] * eq;
              odp[j] = -(ok[j] * egr[j]);                 // -k e^{G_n - G_t}
            } else {
              const float ep = __expf(G - la8[u][j] - ref[j]);  // e^{G_{t-1} - G_ref}
              const float epr = __builtin_amdgcn_rcpf(ep);
              oc[j] = c[j] * ep;
              op[j] = k[j] * epr;
              odp[j] = -(op[j] * egr[j]);                 // -k e^{G_n - G_{t-1}}
              odk[j] = ok[j] * egr[j];                    // k e^{G_n - G_t}
            }
          }
        }
        lds_store8(tQ + t * LDT + d0, oq);
        lds_store8(tC + t * LDT + d0, oc);
        lds_store8(tK + t * LDT + d0, ok);
        if (TWO) lds_store8(tP + t * LDT + d0, op);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pdp[j][u] = to_ot<OT>(odp[j]);
          if (TWO) pdk[j][u] = to_ot<OT>(odk[j]);
        }
      }
      if (!(MODE != 0 && robust)) {
        // channel-major rows d0..d0+7: this thread's TPS tokens as one store per row and quad of
        // 4 tokens (quads are swizzled apart, so a run of 8 at dk = 256 is two stores)
        constexpr int RUN = TPS < 4 ? TPS : 4;
#pragma unroll
        for (int r0 = 0; r0 < TPS; r0 += RUN) {
          const int pos = swz((d0 >> 3) & 15, ts * TPS + r0);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            lds_store_run<RUN>(dP + (d0 + j) * LDD + pos, pdp[j] + r0);
            if (TWO) lds_store_run<RUN>(dK + (d0 + j) * LDD + pos, pdk[j] + r0);
          }
        }
      }
    }
    lds_barrier();
    GDR_MARK(2);

    // ---------------- phase B: Gram tiles of the lower triangle ----------------
    // 20 jobs = 2 row operands x 10 tile pairs (ta >= tb), 5 per wave.  Row operand 0 is Chat
    // (the solve products), 1 is Qhat (the read-out products).  MODE 0/1: one product per job
    // against Khat.  MODE 2: two products sharing the row fragment, against Phat and Khat
    // (job 0: L_P, L_K; job 1: M_QK, M_QP).  The next job's fragments are loaded before the
    // current job's MFMAs.
    if (!robust) {
      constexpr int JPW = 5;
      F8 fa[2][NKB], fb[2][NKB], fc[2][NKB];
      auto job_of = [&](int jj, int& grp, int& ta, int& tb) {
        const int job = wave + 4 * jj;
        grp = job / 10;
        const int tix = job % 10;
        ta = tix >= 6 ? 3 : tix >= 3 ? 2 : tix >= 1 ? 1 : 0;
        tb = tix - ta * (ta + 1) / 2;
      };
      auto load_job = [&](int jj, int bsel) {
        int grp, ta, tb;
        job_of(jj, grp, ta, tb);
        const OT* ar = (grp == 0 ? tC : tQ) + (16 * ta + l16) * LDT;
        const OT* br = ((TWO && grp == 0) ? tP : tK) + (16 * tb + l16) * LDT;
        const OT* cr = (grp == 0 ? tK : tP) + (16 * tb + l16) * LDT;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          fa[bsel][kb] = lds_std_frag_k<DK>(ar, 32 * kb, g);
          fb[bsel][kb] = lds_std_frag_k<DK>(br, 32 * kb, g);
          if (TWO) fc[bsel][kb] = lds_std_frag_k<DK>(cr, 32 * kb, g);
        }
      };
      // which: 0 = solve matrix (strict; off-diagonal -> gA as -L, diagonal -> Ld in fp32),
      // 1 = M used with R (inclusive, stored as -M), 2 = L_K (strict), 3 = M_QK (inclusive)
      auto store_tile = [&](int which, int ta, int tb, const f32x4& acc) {
        if (ta > tb) {  // below the diagonal block: every entry is kept (uniform branch)
          const int r0 = 16 * ta + 4 * g, cc = 16 * tb + l16;
          OT* dst = (which == 0 ? gA : which == 1 ? gM : which == 2 ? gLK : gMQK) + r0 * LDD + cc;
          const float sgn = which <= 1 ? -1.f : 1.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float val = acc[i] * sgn;
            if (MODE == 0) val *= __expf(sG[r0 + i] - sG[cc]);
            dst[i * LDD] = to_ot<OT>(val);
          }
          return;
        }
        const bool strict = which == 0 || which == 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * ta + 4 * g + i, cc = 16 * tb + l16;
          const bool keep = strict ? (cc < r) : (cc <= r);
          float val = 0.f;
          if (keep) {
            val = acc[i];
            if (MODE == 0) val *= __expf(sG[r] - sG[cc]);
          }
          if (which == 0) {
            if (ta > tb)
              gA[r * LDD + cc] = to_ot<OT>(-val);
            else
              Ld[(ta * 16 + (cc & 15)) * L::LDL + (r & 15)] = val;
          } else if (which == 1) {
            gM[r * LDD + cc] = to_ot<OT>(-val);
          } else if (which == 2) {
            gLK[r * LDD + cc] = to_ot<OT>(val);
          } else {
            gMQK[r * LDD + cc] = to_ot<OT>(val);
          }
        }
      };
      load_job(0, 0);
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj) {
        const int cur = jj & 1;
        if (jj + 1 < JPW) load_job(jj + 1, cur ^ 1);
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
    lds_barrier();
    GDR_MARK(3);

    // ---------------- phase C: inverses of the four 16x16 diagonal blocks ----------------
    // The next chunk's loads are issued where each wave would otherwise wait: waves 0-2 while
    // wave 3 inverts, wave 3 at the start of phase D.
    if (wave != 3 && ch + 1 < nch) prefetch(ch + 1);
    // Lane (blk, j) solves column j of block blk by a column sweep: once x_m is final, every
    // later x_i drops L[i][m] x_m (independent FMAs); column m+1 is read while m is applied.
    if (wave == 3 && !robust) {
      const int blk = g, j = l16;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
      float4 col[2][4];
      auto load_col = [&](int m, float4* cv) {
        const float* p = Ld + (blk * 16 + m) * L::LDL;
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
      for (int i = 0; i < 16; ++i) dInv[(blk * 16 + i) * LDI + j] = to_ot<OT>(x[i]);
    }
    lds_barrier();
    GDR_MARK(4);
    if (wave == 3 && ch + 1 < nch) prefetch(ch + 1);

    // ---------------- phase D (exact path): token by token, fp32 ----------------
    // The recurrence itself on this wave's 16 columns: each lane holds rows 16*tl + 4g + i of
    // column nloc, so the two dk-reductions are a partial sum plus two cross-lane-group adds.
    if (MODE != 0 && robust && sside) {
      const OT* laArr = TWO ? tP : dP;
      const int lpitch = TWO ? LDT : ((C * LDT <= DK * LDD) ? LDT : DK);
      for (int t = 0; t < nval; ++t) {
        float qd[NTD][4], kd[NTD][4], cd[NTD][4], al[NTD][4];
#pragma unroll
        for (int tl = 0; tl < NTD; ++tl) {
          const int d = 16 * tl + 4 * g;
          const auto q4 = lds_load4(tQ + t * LDT + d);
          const auto k4 = lds_load4(tK + t * LDT + d);
          const auto c4 = lds_load4(tC + t * LDT + d);
          const auto l4 = lds_load4(laArr + t * lpitch + d);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            qd[tl][i] = static_cast<float>(q4[i]);
            kd[tl][i] = static_cast<float>(k4[i]);
            cd[tl][i] = static_cast<float>(c4[i]);
            al[tl][i] = __expf(static_cast<float>(l4[i]));
          }
        }
        const float x = static_cast<float>(xT[nloc * LDD + t]);
        if (!TWO) {  // decay first
#pragma unroll
          for (int tl = 0; tl < NTD; ++tl)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[tl][i] *= al[tl][i];
        }
        float r = 0.f;
#pragma unroll
        for (int tl = 0; tl < NTD; ++tl)
#pragma unroll
          for (int i = 0; i < 4; ++i) r += cd[tl][i] * S[tl][i];
        r += __shfl_xor(r, 16);
        r += __shfl_xor(r, 32);
        float y = 0.f;
#pragma unroll
        for (int tl = 0; tl < NTD; ++tl)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float sv = S[tl][i] - kd[tl][i] * r;
            if (TWO) sv *= al[tl][i];
            sv += kd[tl][i] * x;
            S[tl][i] = sv;
            y += qd[tl][i] * sv;
          }
        y += __shfl_xor(y, 16);
        y += __shfl_xor(y, 32);
        if (g == 0) st(a.o, row_of(t) * DV + col0 + nloc, y);
      }
    }

    // ---------------- phase D: state waves ----------------
    if (sside && !robust) {
      // (1) S (scaled by e^{G_ref} for a per-channel decay) as B fragments, tile-pair order
      F8 sf[NKB];
      float4 er4[NTD];
      if (MODE != 0) {
#pragma unroll
        for (int tl = 0; tl < NTD; ++tl) er4[tl] = *reinterpret_cast<const float4*>(fEref + 16 * tl + 4 * g);
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int tl = 2 * kb + (j >> 2), i = j & 3;
          float val = 0.f;
          if (tl < NTD) {
            val = S[tl][i];
            if (MODE != 0) val *= reinterpret_cast<const float*>(&er4[tl])[i];
          }
          sf[kb][j] = to_ot<OT>(val);
        }
      }
      // (2) V = Chat S, O = Qhat S
      f32x4 V[4], O[4];
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) {
        V[ta] = zero4();
        O[ta] = zero4();
        const OT* cr = tC + (16 * ta + l16) * LDT;
        const OT* qr = tQ + (16 * ta + l16) * LDT;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          V[ta] = MM::mma8(lds_pair_frag_k<DK>(cr, 32 * kb, g), sf[kb], V[ta]);
          O[ta] = MM::mma8(lds_pair_frag_k<DK>(qr, 32 * kb, g), sf[kb], O[ta]);
        }
        if (MODE == 0) {
          const float4 e4 = *reinterpret_cast<const float4*>(sEG + 16 * ta + 4 * g);
          const float e[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            V[ta][i] *= e[i];
            O[ta][i] *= e[i];
          }
        }
      }
      // (3) value side: MODE 0/1 subtract X; MODE 2 add L_K X and M_QK X
      const OT* xr = xT + nloc * LDD;
      F8 xf[2];
      xf[0] = lds_load8(xr + 8 * g);
      xf[1] = lds_load8(xr + 32 + 8 * g);
      if (!TWO) {
#pragma unroll
        for (int ta = 0; ta < 4; ++ta) {
          const auto x4 = lds_load4(xr + 16 * ta + 4 * g);
#pragma unroll
          for (int i = 0; i < 4; ++i) V[ta][i] -= static_cast<float>(x4[i]);
        }
      } else {
#pragma unroll
        for (int ta = 0; ta < 4; ++ta) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            if (kb == 1 && ta < 2) continue;
            V[ta] = MM::mma8(lds_load8(gLK + (16 * ta + l16) * LDD + 32 * kb + 8 * g), xf[kb], V[ta]);
            O[ta] = MM::mma8(lds_load8(gMQK + (16 * ta + l16) * LDD + 32 * kb + 8 * g), xf[kb], O[ta]);
          }
        }
      }
      // (4) blocked forward substitution: R_i = T_ii (V_i - sum_{m<i} L_im R_m)
      f32x4 R[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int m = 0; m < i; ++m)
          V[i] = MM::mma4(lds_load4(gA + (16 * i + l16) * LDD + 16 * m + 4 * g),
                          acc_frag4<OT>(R[m]), V[i]);
        R[i] = MM::mma4(lds_load4(dInv + (16 * i + l16) * LDI + 4 * g), acc_frag4<OT>(V[i]),
                        zero4());
      }
      F8 rf[2];
      rf[0] = acc_pair_frag<OT>(R[0], R[1]);
      rf[1] = acc_pair_frag<OT>(R[2], R[3]);
      // (5) O -= M R   (gM holds -M)
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (kb == 1 && ta < 2) continue;
          O[ta] = MM::mma8(lds_pair_frag_k<C>(gM + (16 * ta + l16) * LDD, 32 * kb, g), rf[kb], O[ta]);
        }
      }
      // (6) read-out
      // rows past the last token fall outside the buffer range and are dropped
      {
        const int64_t rr = (bi * a.T + t0) * a.H + hi;
        const int64_t bytes = (((a.T - t0) - 1) * a.H + 1) * DV * static_cast<int64_t>(sizeof(IO)) -
                              col0 * static_cast<int64_t>(sizeof(IO));
        const auto ro = make_rsrc(a.o + rr * DV + col0, static_cast<uint32_t>(bytes < 0x7fffffff ? bytes : 0x7fffffff));
        const uint32_t hdvo = static_cast<uint32_t>(a.H * DV) * sizeof(IO);
#pragma unroll
        for (int ta = 0; ta < 4; ++ta)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            buf_store1(a.o, ro, (16 * ta + 4 * g + i) * hdvo + nloc * sizeof(IO), O[ta][i]);
      }
      // (7) S <- e^{G_n} . S (+ Kbar^T X) - P^T R   (dP holds -P^T)
#pragma unroll
      for (int tl = 0; tl < NTD; ++tl) {
        if (MODE == 0) {
          const float e = sEGn[0];
#pragma unroll
          for (int i = 0; i < 4; ++i) S[tl][i] *= e;
        } else {
          const float4 e4 = *reinterpret_cast<const float4*>(fEGn + 16 * tl + 4 * g);
          S[tl][0] *= e4.x;
          S[tl][1] *= e4.y;
          S[tl][2] *= e4.z;
          S[tl][3] *= e4.w;
        }
        const int key = (2 * tl + (l16 >> 3)) & 15;  // swizzle key of row 16 tl + l16
        const OT* pr = dP + (16 * tl + l16) * LDD;
        if (TWO) {
          const OT* kr = dK + (16 * tl + l16) * LDD;
          S[tl] = MM::mma8(lds_two_quads(kr, swz(key, 8 * g), swz(key, 8 * g + 4)), xf[0], S[tl]);
          S[tl] = MM::mma8(lds_two_quads(kr, swz(key, 32 + 8 * g), swz(key, 36 + 8 * g)), xf[1], S[tl]);
        }
        S[tl] = MM::mma8(lds_two_quads(pr, swz(key, 4 * g), swz(key, 16 + 4 * g)), rf[0], S[tl]);
        S[tl] = MM::mma8(lds_two_quads(pr, swz(key, 32 + 4 * g), swz(key, 48 + 4 * g)), rf[1], S[tl]);
      }
    }
    GDR_MARK(5);
  }

  if (sside && a.S_T != nullptr) {
#pragma unroll
    for (int tl = 0; tl < NTD; ++tl)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.S_T[sbase + (int64_t)(16 * tl + 4 * g + i) * DV] = S[tl][i];
  }
}

}  // namespace gdr
