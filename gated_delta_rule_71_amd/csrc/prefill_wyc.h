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
// range; W, Qhat, Pbar and Kbar themselves only carry e^{non-positive} factors.  A chunk whose
// prefix sums span more than kSpanLimit nats (or are not finite) is flagged, and the state kernel
// runs it token by token from the raw inputs instead (exact for any gate values).
#pragma once
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
  // workspace, per chunk index cix = state * nch + chunk
  __bf16* W;   // [cix][64][dk]  W
  __bf16* Qp;  // [cix][64][dk]  Qhat (unsplit)
  __bf16* Pn;  // [cix][dk][64]  -Pbar^T (MODE 1: -Kbar^T)
  __bf16* Kb;  // [cix][dk][64]  Kbar^T (MODE 2)
  __bf16* Mn;  // [cix][64][64]  -M_QP (MODE 1: -M), zero above the diagonal
  __bf16* Y;   // [cix][dv][64]  Y^T
  __bf16* Z;   // [cix][64][dv]  Z (MODE 2)
  __bf16* Xt;  // [cix][dv][64]  X^T (MODE 2)
  float* Egn;  // [cix][dk]      e^{G_n}
  int* flag;   // [cix]          1: exact token path
  int64_t T, H, DV, nch;
  int b_kind, w_kind;
  int nsl;     // value slices per state (state kernel)
  int64_t Hk;  // q / k heads (H is a multiple): value head h reads q / k head h / (H / Hk)
};

constexpr float kWycSpanLimit = 76.f;

// ------------------------------------------------------------------ chunk-local kernel

template <int DK, int DVP, int MODE>
struct WycPrepLayout {
  static constexpr bool TWO = MODE == 2;
  static constexpr int C = 64;
  static constexpr int LDT = DK + 8;
  static constexpr int LDX = DVP + 8;
  static constexpr int LDD = C + 8;
  static constexpr int LDA = 48 + 8;
  static constexpr int LDI = 24;
  static constexpr int LDL = 20;
  static constexpr int NCG = DK / 8;
  static constexpr int NSEG = (256 / NCG) < C ? (256 / NCG) : C;
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
};

template <int DK, int DVP, int MODE>
__global__ __launch_bounds__(256) void wyc_prep_kernel(WycArgs a) {
  using L = WycPrepLayout<DK, DVP, MODE>;
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  static_assert(L::fits, "LDS layout exceeds the gfx950 workgroup limit");
  static_assert(DK % 32 == 0, "dk must be a multiple of 32");
  constexpr bool TWO = L::TWO;
  constexpr int C = L::C, LDT = L::LDT, LDX = L::LDX, LDD = L::LDD, LDA = L::LDA, LDI = L::LDI,
                LDL = L::LDL;
  constexpr int NCG = L::NCG, NSEG = L::NSEG, TPS = L::TPS, NKB = DK / 32;

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
  const auto rla = make_rsrc(a.la + rr * DK, wy_range(left, H, DK));
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
    a.Egn[cix * DK + tid] = __expf(run);
    if (fmaxf(fabsf(ref), fabsf(run - ref)) > kWycSpanLimit || !(run == run)) sFlag[0] = 1;
  }
  GDR_PMARK(0);
  lds_barrier();
  const bool robust = sFlag[0] != 0;
  if (tid == 0) a.flag[cix] = robust ? 1 : 0;
  if (robust) return;  // the state kernel runs this chunk token by token from the raw inputs

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
      bf16x8 oq, oc, ok, op, oqp;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float G = G8[u][j] + off[j];
        const float eq = __expf(G - ref[j]);          // e^{G_t - G_ref}
        const float er = __builtin_amdgcn_rcpf(eq);   // e^{G_ref - G_t}
        oq[j] = static_cast<__bf16>(q[j] * eq);
        ok[j] = static_cast<__bf16>(k[j] * er);
        oqp[j] = static_cast<__bf16>(q[j] * eq * eref[j]);  // q e^{G_t}
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
      *reinterpret_cast<bf16x8*>(a.Qp + (cix * C + t) * DK + d0) = oqp;
    }
  }
  // tiles above the diagonal of -M, L_K and M_QK are never written by the Gram phase but are
  // read as zero by the products below (the three arrays are contiguous)
  for (int i = tid; i < (L::oT - L::oM) / 4; i += 256) reinterpret_cast<uint32_t*>(gM)[i] = 0u;
  GDR_PMARK(1);
  lds_barrier();

  // ---- Gram tiles: 20 jobs = 2 row operands x 10 tile pairs, 5 per wave ----
  {
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
  GDR_PMARK(2);
  lds_barrier();

  // ---- diagonal inverses (waves 0-1) | -M_QP out (waves 2-3) ----
  if (wave < 2) {
    if (lane < 32) wy_diag_inverses<LDL, LDI>(Ld, dInv, wave, lane, l16);
  } else {
    __bf16* Mo = a.Mn + cix * C * C;
    for (int item = tid - 128; item < C * 8; item += 128) {
      const int r = item >> 3, part = item & 7;
      *reinterpret_cast<uint4*>(Mo + r * C + part * 8) = *reinterpret_cast<const uint4*>(gM + r * LDD + part * 8);
    }
    if (TWO) {  // X^T out: item = column * 8 + part holds tokens 8 part .. 8 part + 7
      __bf16* Xo = a.Xt + cix * DV * C;
      for (int item = tid - 128; item < DV * 8; item += 128) {
        const int col = item >> 3, part = item & 7;
        bf16x8 xv;
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[e] = tX[(8 * part + e) * LDX + col];
        *reinterpret_cast<bf16x8*>(Xo + col * C + 8 * part) = xv;
      }
    }
  }
  GDR_PMARK(3);
  lds_barrier();

  // ---- -Pbar^T (and Kbar^T) out: the split Phat (Khat) columns times e^{G_n - G_ref}; 16-byte
  // pieces of channel rows, so every store instruction writes whole row segments ----
  {
    __bf16* Po = a.Pn + cix * DK * C;
    __bf16* Ko = a.Kb + cix * DK * C;
    const __bf16* src = TWO ? tP : tK;
    for (int item = tid; item < DK * 8; item += 256) {
      const int d = item >> 3, part = item & 7;
      const float f = fEgr[d];
      bf16x8 pv, kv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = static_cast<__bf16>(-static_cast<float>(src[(8 * part + e) * LDT + d]) * f);
        if (TWO) kv[e] = static_cast<__bf16>(static_cast<float>(tK[(8 * part + e) * LDT + d]) * f);
      }
      *reinterpret_cast<bf16x8*>(Po + d * C + 8 * part) = pv;
      if (TWO) *reinterpret_cast<bf16x8*>(Ko + d * C + 8 * part) = kv;
    }
  }
  // ---- T = (I + L_P)^{-1}: wave j solves column block j on the identity ----
  {
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

  // ---- products, as transposed tiles so that each lane stores four consecutive columns ----
  // B fragments of T^T (and of L_K^T, M_QK^T) are pair fragments of the rows of T (L_K, M_QK).
  auto row_frags = [&](const __bf16* m, F8* f) {  // 6 fragments: lower-triangular 64 x 64
#pragma unroll
    for (int ta = 0, n = 0; ta < 4; ++ta) {
      f[n++] = lds_pair_frag_k<C>(m + (16 * ta + l16) * LDD, 0, g);
      if (ta >= 2) f[n++] = lds_pair_frag_k<C>(m + (16 * ta + l16) * LDD, 32, g);
    }
  };
  // column tile of a token-major LDS array as A fragments: 8 tokens (tile-pair order) of column
  // col per lane, times `scale`
  auto col_frags = [&](const __bf16* base, int pitch, int col, float scale, F8* f) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = 32 * ks + 4 * g + (e & 3) + (e >> 2) * 16;
        f[ks][e] = static_cast<__bf16>(static_cast<float>(base[t * pitch + col]) * scale);
      }
  };
  // D^T tiles of (lower-triangular 64 x 64 B-side matrix) x (A-side 64 x 16 tile): out[ta] lane
  // holds D[token 16 ta + l16][column 4 g + i]
  auto tr_product = [&](const F8* af, const F8* bf, bool strict, f32x4* out) {
#pragma unroll
    for (int ta = 0, n = 0; ta < 4; ++ta) {
      out[ta] = MM::mma8(af[0], bf[n++], zero4());
      if (ta >= 2) out[ta] = MM::mma8(af[1], bf[n++], out[ta]);
    }
    (void)strict;
  };
  // upright tiles of (lower-triangular 64 x 64 A-side matrix) x (64 x 16 B-side tile): out[ta] lane
  // holds D[token 16 ta + 4 g + i][column l16]
  auto up_product = [&](const F8* af, const F8* bf, f32x4* out) {
#pragma unroll
    for (int ta = 0, n = 0; ta < 4; ++ta) {
      out[ta] = MM::mma8(af[n++], bf[0], zero4());
      if (ta >= 2) out[ta] = MM::mma8(af[n++], bf[1], out[ta]);
    }
  };
  // upright tiles out as a [column][64] array: four consecutive tokens per 8-byte store
  auto store_up_t = [&](__bf16* dst, int col0c, const f32x4* t4, float sgn) {
#pragma unroll
    for (int ta = 0; ta < 4; ++ta) {
      bf16x4 ob;
#pragma unroll
      for (int i = 0; i < 4; ++i) ob[i] = static_cast<__bf16>(t4[ta][i] * sgn);
      *reinterpret_cast<bf16x4*>(dst + (col0c + l16) * C + 16 * ta + 4 * g) = ob;
    }
  };
  auto store_tr = [&](__bf16* dst, int64_t pitch, int col0c, const f32x4* t4, float sgn) {
#pragma unroll
    for (int ta = 0; ta < 4; ++ta) {
      bf16x4 ob;
#pragma unroll
      for (int i = 0; i < 4; ++i) ob[i] = static_cast<__bf16>(t4[ta][i] * sgn);
      *reinterpret_cast<bf16x4*>(dst + (16 * ta + l16) * pitch + col0c + 4 * g) = ob;
    }
  };
  {
    F8 tfr[6];
    row_frags(tT, tfr);
    // W = T Chat (unsplit: the split Chat times e^{G_ref} per channel)
    __bf16* Wo = a.W + cix * C * DK;
    for (int ct = wave; ct < DK / 16; ct += 4) {
      const int col = 16 * ct + l16;
      F8 cf[2];
      col_frags(tC, LDT, col, fEref[col], cf);
      f32x4 D[4];
      tr_product(cf, tfr, false, D);
      store_tr(Wo, DK, 16 * ct, D, 1.f);
    }
    const int nct_u = static_cast<int>(DV / 16);
    __bf16* Yo = a.Y + cix * C * DV;
    if (TWO) {
      F8 lkf[6], mqf[6];
      row_frags(gLK, lkf);
      row_frags(gMQK, mqf);
      __bf16* Zo = a.Z + cix * C * DV;
      for (int ct = wave; ct < nct_u; ct += 4) {
        const int col = 16 * ct + l16;
        F8 xf[2];
        col_frags(tX, LDX, col, 1.f, xf);
        // L_K X as upright tiles (lane: rows 16 ta + 4 g + i, column col), whose tile pairs are
        // the A fragments of (T L_K X)^T
        f32x4 LKX[4];
#pragma unroll
        for (int ta = 0, n = 0; ta < 4; ++ta) {
          LKX[ta] = MM::mma8(lkf[n++], xf[0], zero4());
          if (ta >= 2) LKX[ta] = MM::mma8(lkf[n++], xf[1], LKX[ta]);
        }
        F8 lf[2];
        lf[0] = acc_pair_frag<__bf16>(LKX[0], LKX[1]);
        lf[1] = acc_pair_frag<__bf16>(LKX[2], LKX[3]);
        f32x4 D[4];
        up_product(tfr, lf, D);
        store_up_t(Yo, 16 * ct, D, 1.f);
        tr_product(xf, mqf, false, D);
        store_tr(Zo, DV, 16 * ct, D, 1.f);
      }
    } else {
      for (int ct = wave; ct < nct_u; ct += 4) {
        const int col = 16 * ct + l16;
        F8 xf[2];
        col_frags(tX, LDX, col, 1.f, xf);
        f32x4 D[4];
        up_product(tfr, xf, D);
        store_up_t(Yo, 16 * ct, D, -1.f);
      }
    }
  }
  GDR_PMARK(5);
}

// ------------------------------------------------------------------ state kernel

template <int DK, int NCT, int MODE>
struct WycStateLayout {
  static constexpr bool TWO = MODE == 2;
  static constexpr int C = 64;
  static constexpr int DVS = 16 * NCT;
  static constexpr int LDT = DK + 8;
  static constexpr int LDD = C + 8;
  static constexpr int LDZ = DVS + 8;
  static constexpr int CHT = (DK * LDD > C * LDT ? DK * LDD : C * LDT) * 2;  // channel-major or token-major
  // set 1 (single buffer): Qhat rows and W rows (raw q and k rows on the exact path)
  static constexpr int oQ = 0;
  static constexpr int oW = oQ + C * LDT * 2;
  static constexpr int SET1 = oW + C * LDT * 2;
  // set 2 (two buffers), offsets within a buffer
  static constexpr int oP = 0;              // -Pbar^T [dk][LDD] (exact path: c rows [64][LDT])
  static constexpr int oKb = oP + CHT;      // Kbar^T (exact path: log alpha rows)
  static constexpr int oM = oKb + CHT;      // -M [64][LDD]
  static constexpr int oY = oM + C * LDD * 2;     // Y^T [DVS][LDD]
  static constexpr int oZ = oY + DVS * LDD * 2;   // Z rows [64][LDZ] (MODE 2)
  static constexpr int oX = oZ + (TWO ? C * LDZ * 2 : 0);  // X^T [DVS][LDD]
  static constexpr int oS = oX + DVS * LDD * 2;   // fp32 e^{G_n} [dk], flag
  static constexpr int BUF = oS + (DK + 4) * 4;
  static constexpr int total = SET1 + 2 * BUF;
  static constexpr bool fits = total <= kLdsLimit;
};

// Workgroup = 2 loader waves and one state wave for one state and DVS = 16 NCT value columns.
// Per chunk c, two barrier-separated intervals:
//   1: loaders write set 2 of chunk c+1 (its own buffer); state: Qhat S and W S of chunk c (or
//      the whole chunk token by token when it is flagged)
//   2: loaders write set 1 of chunk c+1 (Qhat, W: the state wave is done with them);
//      state: R = W S + Y, O = Qhat S + Z - M R out, S <- e^{G_n} . S (+ Kbar^T X) - Pbar^T R
template <int DK, int NCT, int MODE>
__global__ __launch_bounds__(192) void wyc_state_kernel(WycArgs a) {
  using L = WycStateLayout<DK, NCT, MODE>;
  using MM = Mma<__bf16>;
  using F8 = MM::F8;
  static_assert(L::fits, "LDS layout exceeds the gfx950 workgroup limit");
  static_assert(DK % 32 == 0, "dk must be a multiple of 32");
  constexpr bool TWO = L::TWO;
  constexpr int C = L::C, DVS = L::DVS, LDT = L::LDT, LDD = L::LDD, LDZ = L::LDZ;
  constexpr int NTD = DK / 16, NKB = DK / 32;
  constexpr int NLT = 128;
  constexpr int NCG = DK / 8, IPT = C * NCG / NLT;   // 16-byte row items per loader thread
  constexpr int CPT = DK * (C / 8) / NLT;            // 16-byte items of a [dk][64] array
  constexpr int MPT = C * C / 8 / NLT;
  constexpr int NXG = DVS / 8, XPT = (C * NXG + NLT - 1) / NLT;

  __shared__ __attribute__((aligned(32))) unsigned char smem[L::total];
  __bf16* tQ = reinterpret_cast<__bf16*>(smem + L::oQ);
  __bf16* tW = reinterpret_cast<__bf16*>(smem + L::oW);
  auto buf = [&](int64_t c) -> unsigned char* { return smem + L::SET1 + (c & 1) * L::BUF; };

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
  const uint32_t hqk = static_cast<uint32_t>(a.Hk * DK * 2);  // token stride of q and k
  const int64_t hq = hi / (H / a.Hk);                        // this state's q / k head
  const uint32_t h1 = static_cast<uint32_t>(H * 2);
  const uint32_t oob = 0x80000000u;

  // ---------------- loaders ----------------
  auto read_flag = [&](int64_t c) -> int {
    const auto rf = make_rsrc(a.flag + bh * nch + c, 4);
    return __builtin_amdgcn_readfirstlane(__builtin_amdgcn_raw_buffer_load_b32(rf, 0, 0, 0));
  };
  // x = w . v for this slice, transposed into X^T (value column major, swizzled token quads)
  auto store_x = [&](int64_t c, __bf16* xT) {
    const int64_t t0 = c * C, rr = (bi * T + t0) * H + hi;
    const uint32_t vb = wy_range(T - t0, H, DV) - static_cast<uint32_t>(col0) * 2;
    const auto rv = make_rsrc(a.v + rr * DV + col0, vb);
    const auto rwc = make_rsrc(a.w_kind == kChannel ? a.wg + rr * DV + col0 : a.v, a.w_kind == kChannel ? vb : 0u);
    const auto rws = make_rsrc(a.w_kind == kScalar ? a.wg + rr : a.v, a.w_kind == kScalar ? wy_range(T - t0, H, 1) : 0u);
    uint4 vv[XPT], ww[XPT];
    uint16_t wsv[XPT];
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int item = tid + NLT * j;
      const bool in = item < C * NXG;
      const uint32_t t = item / NXG, xg = item % NXG;
      vv[j] = buf_load16(rv, in ? t * hdv + xg * 16 : oob);
      ww[j] = buf_load16(rwc, in ? t * hdv + xg * 16 : oob);
      wsv[j] = buf_load_u16(rws, in ? t * h1 : oob);
    }
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int item = tid + NLT * j;
      if (item < C * NXG) {
        const int t = item / NXG, xg = item % NXG;
        float x[8];
        load8f(reinterpret_cast<const bf16_t*>(&vv[j]), x);
        if (a.w_kind == kChannel) {
          float w8[8];
          load8f(reinterpret_cast<const bf16_t*>(&ww[j]), w8);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= w8[e];
        } else if (a.w_kind == kScalar) {
          const float ws = bf16_to_f32(wsv[j]);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= ws;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) xT[(xg * 8 + e) * LDD + swz(2 * xg, t)] = static_cast<__bf16>(x[e]);
      }
    }
  };
  // set 2 of chunk c: -Pbar^T, Kbar^T, -M, Y^T, Z, X^T, e^{G_n}, flag (exact path: c, log alpha, X^T)
  auto store_set2 = [&](int64_t c, int robust) {
    unsigned char* B = buf(c);
    __bf16* tP = reinterpret_cast<__bf16*>(B + L::oP);
    __bf16* tKb = reinterpret_cast<__bf16*>(B + L::oKb);
    __bf16* gM = reinterpret_cast<__bf16*>(B + L::oM);
    __bf16* yT = reinterpret_cast<__bf16*>(B + L::oY);
    __bf16* zs = reinterpret_cast<__bf16*>(B + L::oZ);
    __bf16* xT = reinterpret_cast<__bf16*>(B + L::oX);
    float* sc = reinterpret_cast<float*>(B + L::oS);
    const int64_t cix = bh * nch + c;
    if (tid < DK) {
      const auto re = make_rsrc(a.Egn + cix * DK, DK * 4);
      sc[tid] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(re, tid * 4, 0, 0));
    }
    if (tid == 0) reinterpret_cast<int*>(sc + DK)[0] = robust;
    if (robust) store_x(c, xT);
    if (robust) {
      // raw c = b . k and log alpha rows, token-major
      const int64_t t0 = c * C, rr = (bi * T + t0) * H + hi, rqk = (bi * T + t0) * a.Hk + hq;
      const auto rk = make_rsrc(a.k + rqk * DK, wy_range(T - t0, a.Hk, DK));
      const auto rla = make_rsrc(a.la + rr * DK, wy_range(T - t0, H, DK));
      const auto rbc = make_rsrc(a.b_kind == kChannel ? a.bg + rr * DK : a.q, a.b_kind == kChannel ? wy_range(T - t0, H, DK) : 0u);
      const auto rbs = make_rsrc(a.b_kind == kScalar ? a.bg + rr : a.q, a.b_kind == kScalar ? wy_range(T - t0, H, 1) : 0u);
#pragma unroll
      for (int j = 0; j < IPT; ++j) {
        const uint32_t t = (tid / NCG) * IPT + j, cg = tid % NCG;
        const uint4 kk = buf_load16(rk, t * hqk + cg * 16);
        const uint4 bb = buf_load16(rbc, t * hdk + cg * 16);
        const uint16_t bs = buf_load_u16(rbs, t * h1);
        float k8[8], c8[8];
        load8f(reinterpret_cast<const bf16_t*>(&kk), k8);
        if (a.b_kind == kChannel) {
          load8f(reinterpret_cast<const bf16_t*>(&bb), c8);
#pragma unroll
          for (int e = 0; e < 8; ++e) c8[e] *= k8[e];
        } else {
          const float b1 = a.b_kind == kScalar ? bf16_to_f32(bs) : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) c8[e] = b1 * k8[e];
        }
        bf16x8 cb;
#pragma unroll
        for (int e = 0; e < 8; ++e) cb[e] = static_cast<__bf16>(c8[e]);
        *reinterpret_cast<bf16x8*>(tP + t * LDT + cg * 8) = cb;
        *reinterpret_cast<uint4*>(tKb + t * LDT + cg * 8) = buf_load16(rla, t * hdk + cg * 16);
      }
      return;
    }
    const auto rp = make_rsrc(a.Pn + cix * DK * C, DK * C * 2);
    const auto rm = make_rsrc(a.Mn + cix * C * C, C * C * 2);
    const auto ry = make_rsrc(a.Y + (cix * DV + col0) * C, DVS * C * 2);
    const auto rx = make_rsrc(TWO ? a.Xt + (cix * DV + col0) * C : a.Y, DVS * C * 2);
    const auto rz = make_rsrc(TWO ? a.Z + cix * C * DV + col0 : a.Y, static_cast<uint32_t>((C * DV - col0) * 2));
    const auto rkb = make_rsrc(TWO ? a.Kb + cix * DK * C : a.Pn, DK * C * 2);
    uint4 pp[CPT], pkb[CPT], pm[MPT], py[XPT], px[XPT], pz[XPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      pp[j] = buf_load16(rp, (tid + NLT * j) * 16);
      if (TWO) pkb[j] = buf_load16(rkb, (tid + NLT * j) * 16);
    }
#pragma unroll
    for (int j = 0; j < MPT; ++j) pm[j] = buf_load16(rm, (tid + NLT * j) * 16);
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int item = tid + NLT * j;
      const uint32_t t = item / NXG, xg = item % NXG;
      const bool in = item < C * NXG;
      py[j] = buf_load16(ry, in ? item * 16 : oob);  // [DVS][64]: item = column * 8 + part
      if (TWO) {
        px[j] = buf_load16(rx, in ? item * 16 : oob);
        pz[j] = buf_load16(rz, in ? (t * DV + xg * 8) * 2 : oob);
      }
    }
    // [dk][64] arrays: item = row * 8 + part holds tokens 8 part .. 8 part + 7 of row `row`
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int item = tid + NLT * j, row = item >> 3, part = item & 7, key = (row >> 3) & 15;
      __bf16* dp = tP + row * LDD;
      *reinterpret_cast<uint2*>(dp + swz(key, 8 * part)) = make_uint2(pp[j].x, pp[j].y);
      *reinterpret_cast<uint2*>(dp + swz(key, 8 * part + 4)) = make_uint2(pp[j].z, pp[j].w);
      if (TWO) {
        __bf16* dk = tKb + row * LDD;
        *reinterpret_cast<uint2*>(dk + swz(key, 8 * part)) = make_uint2(pkb[j].x, pkb[j].y);
        *reinterpret_cast<uint2*>(dk + swz(key, 8 * part + 4)) = make_uint2(pkb[j].z, pkb[j].w);
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
        // [column][64] slices: tokens 8 part .. 8 part + 7 of one column as two swizzled quads
        const int col = item >> 3, part = item & 7, key = 2 * (col >> 3);
        __bf16* yr = yT + col * LDD;
        *reinterpret_cast<uint2*>(yr + swz(key, 8 * part)) = make_uint2(py[j].x, py[j].y);
        *reinterpret_cast<uint2*>(yr + swz(key, 8 * part + 4)) = make_uint2(py[j].z, py[j].w);
        if (TWO) {
          __bf16* xr = xT + col * LDD;
          *reinterpret_cast<uint2*>(xr + swz(key, 8 * part)) = make_uint2(px[j].x, px[j].y);
          *reinterpret_cast<uint2*>(xr + swz(key, 8 * part + 4)) = make_uint2(px[j].z, px[j].w);
          const int t = item / NXG, xg = item % NXG;
          *reinterpret_cast<uint4*>(zs + t * LDZ + xg * 8) = pz[j];
        }
      }
    }
  };
  // set 1 of chunk c: Qhat and W rows (exact path: raw q and k rows)
  auto store_set1 = [&](int64_t c, int robust) {
    const int64_t cix = bh * nch + c;
    const int64_t t0 = c * C, rqk = (bi * T + t0) * a.Hk + hq;
    const auto ra = robust ? make_rsrc(a.q + rqk * DK, wy_range(T - t0, a.Hk, DK)) : make_rsrc(a.Qp + cix * C * DK, C * DK * 2);
    const auto rb = robust ? make_rsrc(a.k + rqk * DK, wy_range(T - t0, a.Hk, DK)) : make_rsrc(a.W + cix * C * DK, C * DK * 2);
    const uint32_t pitch = robust ? hqk : DK * 2;
    uint4 pa[IPT], pb[IPT];
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const uint32_t t = (tid / NCG) * IPT + j, cg = tid % NCG;
      pa[j] = buf_load16(ra, t * pitch + cg * 16);
      pb[j] = buf_load16(rb, t * pitch + cg * 16);
    }
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const uint32_t t = (tid / NCG) * IPT + j, cg = tid % NCG;
      *reinterpret_cast<uint4*>(tQ + t * LDT + cg * 8) = pa[j];
      *reinterpret_cast<uint4*>(tW + t * LDT + cg * 8) = pb[j];
    }
  };

  // ---------------- state wave ----------------
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
  f32x4 Ot[NCT][4], V[NCT][4];  // across the two intervals of a chunk

  // Ot = (Qhat S)^T tiles and V = W S tiles: one stream of eight 16-row tiles (Qhat then W)
  auto qs_ws = [&]() {
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

  // A operand tiles of a channel-major [dk][64] array (swizzled token quads), tile-pair order
  auto load_ct = [&](const __bf16* arr, int tl, F8* o) {
    const int row = 16 * tl + l16, key = (row >> 3) & 15;
    const __bf16* kr = arr + row * LDD;
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

  auto second = [&](int64_t c) {
    const unsigned char* B = buf(c);
    const __bf16* tP = reinterpret_cast<const __bf16*>(B + L::oP);
    const __bf16* tKb = reinterpret_cast<const __bf16*>(B + L::oKb);
    const __bf16* gM = reinterpret_cast<const __bf16*>(B + L::oM);
    const __bf16* yT = reinterpret_cast<const __bf16*>(B + L::oY);
    const __bf16* zs = reinterpret_cast<const __bf16*>(B + L::oZ);
    const __bf16* xT = reinterpret_cast<const __bf16*>(B + L::oX);
    const float* sc = reinterpret_cast<const float*>(B + L::oS);
    F8 mf[6];
#pragma unroll
    for (int ta = 0, n = 0; ta < 4; ++ta) {
      mf[n++] = lds_pair_frag_k<C>(gM + (16 * ta + l16) * LDD, 0, g);
      if (ta >= 2) mf[n++] = lds_pair_frag_k<C>(gM + (16 * ta + l16) * LDD, 32, g);
    }
    // R = V + Y as tile-pair fragments; X fragments for Kbar^T X
    F8 rf[NCT][2], xf[NCT][2];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int n = 16 * ct + l16;
      f32x4 R[4];
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) {
        const bf16x4 y4 = *reinterpret_cast<const bf16x4*>(yT + n * LDD + swz(2 * (n >> 3), 16 * ta + 4 * g));
#pragma unroll
        for (int i = 0; i < 4; ++i) R[ta][i] = V[ct][ta][i] + static_cast<float>(y4[i]);
      }
      rf[ct][0] = acc_pair_frag<__bf16>(R[0], R[1]);
      rf[ct][1] = acc_pair_frag<__bf16>(R[2], R[3]);
      if (TWO) {
        const int key = 2 * (n >> 3);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x4 lo = lds_load4(xT + n * LDD + swz(key, 32 * kb + 4 * g));
          const bf16x4 hi = lds_load4(xT + n * LDD + swz(key, 32 * kb + 16 + 4 * g));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xf[ct][kb][e] = lo[e];
            xf[ct][kb][4 + e] = hi[e];
          }
        }
      }
    }
    // O^T += Z^T + R^T (-M)^T, then O out (four columns of one token per 8-byte store)
    const int64_t t0 = c * C;
    const int64_t rr = (bi * T + t0) * H + hi;
    const int64_t bytes = ((T - t0 - 1) * H + 1) * DV * 2 - col0 * 2;
    const auto ro = make_rsrc(a.o + rr * DV + col0, static_cast<uint32_t>(bytes < 0x7fffffff ? bytes : 0x7fffffff));
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int ta = 0, n = 0; ta < 4; ++ta) {
        Ot[ct][ta] = MM::mma8(rf[ct][0], mf[n++], Ot[ct][ta]);
        if (ta >= 2) Ot[ct][ta] = MM::mma8(rf[ct][1], mf[n++], Ot[ct][ta]);
        if (TWO) {
          const bf16x4 z4 = *reinterpret_cast<const bf16x4*>(zs + (16 * ta + l16) * LDZ + 16 * ct + 4 * g);
#pragma unroll
          for (int i = 0; i < 4; ++i) Ot[ct][ta][i] += static_cast<float>(z4[i]);
        }
        bf16x4 ob;
#pragma unroll
        for (int i = 0; i < 4; ++i) ob[i] = static_cast<__bf16>(Ot[ct][ta][i]);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ob), ro,
                                              (16 * ta + l16) * hdv + (16 * ct + 4 * g) * 2, 0, 0);
      }
    // S <- e^{G_n} . S (+ Kbar^T X) + (-Pbar^T) R
    F8 pf[4][2], kf[4][2];
#pragma unroll
    for (int tl = 0; tl < 3; ++tl) {
      load_ct(tP, tl, pf[tl]);
      if (TWO) load_ct(tKb, tl, kf[tl]);
    }
#pragma unroll
    for (int tl = 0; tl < NTD; ++tl) {
      if (tl + 3 < NTD) {
        load_ct(tP, tl + 3, pf[(tl + 3) & 3]);
        if (TWO) load_ct(tKb, tl + 3, kf[(tl + 3) & 3]);
      }
      const float4 e4 = *reinterpret_cast<const float4*>(sc + 16 * tl + 4 * g);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        S[ct][tl][0] *= e4.x;
        S[ct][tl][1] *= e4.y;
        S[ct][tl][2] *= e4.z;
        S[ct][tl][3] *= e4.w;
        if (TWO) {
          S[ct][tl] = MM::mma8(kf[tl & 3][0], xf[ct][0], S[ct][tl]);
          S[ct][tl] = MM::mma8(kf[tl & 3][1], xf[ct][1], S[ct][tl]);
        }
        S[ct][tl] = MM::mma8(pf[tl & 3][0], rf[ct][0], S[ct][tl]);
        S[ct][tl] = MM::mma8(pf[tl & 3][1], rf[ct][1], S[ct][tl]);
      }
    }
  };

  // the recurrence itself, token by token in fp32, for a flagged chunk: each lane holds rows
  // 16 tl + 4 g + i of its columns, so both dk-reductions are a partial sum plus two
  // cross-lane-group adds
  auto exact = [&](int64_t c) {
    const unsigned char* B = buf(c);
    const __bf16* tC = reinterpret_cast<const __bf16*>(B + L::oP);
    const __bf16* tLa = reinterpret_cast<const __bf16*>(B + L::oKb);
    const __bf16* xT = reinterpret_cast<const __bf16*>(B + L::oX);
    const int64_t t0 = c * C;
    const int nval = static_cast<int>(T - t0 < C ? T - t0 : C);
    const int64_t rr = (bi * T + t0) * H + hi;
    for (int t = 0; t < nval; ++t) {
      float qd[NTD][4], kd[NTD][4], cd[NTD][4], al[NTD][4];
#pragma unroll
      for (int tl = 0; tl < NTD; ++tl) {
        const int d = 16 * tl + 4 * g;
        const bf16x4 q4 = lds_load4(tQ + t * LDT + d);
        const bf16x4 k4 = lds_load4(tW + t * LDT + d);
        const bf16x4 c4 = lds_load4(tC + t * LDT + d);
        const bf16x4 l4 = lds_load4(tLa + t * LDT + d);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qd[tl][i] = static_cast<float>(q4[i]);
          kd[tl][i] = static_cast<float>(k4[i]);
          cd[tl][i] = static_cast<float>(c4[i]);
          al[tl][i] = __expf(static_cast<float>(l4[i]));
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int n = 16 * ct + l16;
        const float x = static_cast<float>(xT[n * LDD + swz(2 * (n >> 3), t)]);
        if (!TWO) {  // decay first
#pragma unroll
          for (int tl = 0; tl < NTD; ++tl)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[ct][tl][i] *= al[tl][i];
        }
        float r = 0.f;
#pragma unroll
        for (int tl = 0; tl < NTD; ++tl)
#pragma unroll
          for (int i = 0; i < 4; ++i) r += cd[tl][i] * S[ct][tl][i];
        r += __shfl_xor(r, 16);
        r += __shfl_xor(r, 32);
        float y = 0.f;
#pragma unroll
        for (int tl = 0; tl < NTD; ++tl)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float sv = S[ct][tl][i] - kd[tl][i] * r;
            if (TWO) sv *= al[tl][i];
            sv += kd[tl][i] * x;
            S[ct][tl][i] = sv;
            y += qd[tl][i] * sv;
          }
        y += __shfl_xor(y, 16);
        y += __shfl_xor(y, 32);
        if (g == 0) a.o[(rr + static_cast<int64_t>(t) * H) * DV + col0 + n].x = f32_to_bf16(y);
      }
    }
  };

  // ---------------- pipeline ----------------
  int nflag = 0;  // loaders: flag of the chunk whose set 1 comes next
  if (loader && nch > 0) {
    nflag = read_flag(0);
    store_set2(0, nflag);
    store_set1(0, nflag);
  }
  lds_barrier();
  for (int64_t ch = 0; ch < nch; ++ch) {
    asm volatile("" : "+v"(lane), "+v"(g), "+v"(l16));
    const bool more = ch + 1 < nch;
    int robust = 0;
    GDR_MARK(0);
    if (loader) {
      if (more) {
        nflag = read_flag(ch + 1);
        store_set2(ch + 1, nflag);
      }
    } else {
      robust = reinterpret_cast<const int*>(reinterpret_cast<const float*>(buf(ch) + L::oS) + DK)[0];
      if (robust)
        exact(ch);
      else
        qs_ws();
    }
    GDR_MARK(1);
    lds_barrier();
    GDR_MARK(2);
    if (loader) {
      if (more) store_set1(ch + 1, nflag);
    } else if (!robust) {
      second(ch);
    }
    GDR_MARK(3);
    lds_barrier();
    GDR_MARK(4);
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
