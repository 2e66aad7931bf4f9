/*
 * Plain CPU oracle for the generalized gated delta-rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file or the library built from it; only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark use it.
 *
 * What it computes (fp64 throughout, one token at a time, no blocking):
 *
 *   S_t = Diag(alpha_t) (I - k_t^T (b_t . k_t)) S_{t-1} + k_t^T (w_t . v_t)
 *   o_t = q_t S_t
 *
 * with row vectors q_t, k_t in R^dk, v_t in R^dv and a dk x dv state S per
 * (batch, head). Sources, on the pages:
 *   - "Recurrent Memory: Write, Erase, Decay, Read", section 01 (write
 *     S <- S + k^T v and read o = qS, row-vector convention), section 03 (the
 *     delta rule: read, delta, write back; the Householder erase form),
 *     section 04 (decay; survival as exp of a sum of log alpha) and section 05
 *     (the unified equation Diag(alpha)(I - beta k^T k) S + beta k^T v).
 *   - "How Linear Attention Remembers" summary, Analytical Framework
 *     (S_t = T_t(S_{t-1}) + W_t and o_t = q_t^T S_t: the read sees this
 *     token's write).
 *   - Gated DeltaNet-2 abstract (channel-wise erase gate b_t on the key side,
 *     channel-wise write gate w_t on the value side; reduces to KDA when both
 *     collapse to one scalar and to Gated DeltaNet when the decay does too).
 *
 * Readings taken where the pages leave a step open:
 *   - Gated DeltaNet-2's equation is not printed. b_t weights the read used for
 *     erasure (key side), w_t scales the written value (value side); with
 *     b = w = beta the unified equation of section 05 comes back exactly.
 *   - Order: section 05 applies the erase first and the decay after it
 *     (ORDER_ERASE_THEN_DECAY, the default). ORDER_DECAY_THEN_ERASE applies the
 *     decay to S_{t-1} first, then reads, erases and writes. The two agree when
 *     alpha is a scalar.
 *   - Gates arrive as log alpha (section 04 works in logs), b and w as values.
 *     A gate "kind" of NONE means alpha = 1, b = 0, w = 1.
 *   - No scale on q, no normalisation of q or k inside the recurrence.
 *
 * Inputs are float32 arrays (bf16 and fp32 inputs are exact in fp32); every
 * operation is done in double. Columns of S evolve independently (the
 * transition multiplies S from the left), so independent (batch, head,
 * column block) chains run on separate OpenMP threads; each column's
 * arithmetic is the same sequence of operations whatever the split.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { KIND_NONE = 0, KIND_SCALAR = 1, KIND_CHANNEL = 2 };
enum { ORDER_ERASE_THEN_DECAY = 0, ORDER_DECAY_THEN_ERASE = 1 };

int gdr_oracle_version(void) { return 1; }

/* Gate value for (token row `row`, channel j): NONE -> dflt, SCALAR -> one per
 * (b, t, h), CHANNEL -> one per channel. */
static double gate_at(const float* g, int kind, int64_t row, int64_t width,
                      int64_t j, double dflt) {
  if (kind == KIND_NONE || g == NULL) return dflt;
  if (kind == KIND_SCALAR) return (double)g[row];
  return (double)g[row * width + j];
}

/* One (batch, head) chain restricted to state columns [n0, n1). */
static void run_chain(int64_t B, int64_t H, int64_t T, int64_t DK, int64_t DV,
                      int64_t bi, int64_t hi, int64_t n0, int64_t n1,
                      const float* q, const float* k, const float* v,
                      const float* log_alpha, int alpha_kind,
                      const float* bg, int b_kind, const float* wg, int w_kind,
                      int order, const double* S0, double* o, double* S_T) {
  (void)B;
  const int64_t nc = n1 - n0;
  double* S = (double*)calloc((size_t)(DK * nc), sizeof(double));
  double* alpha = (double*)malloc((size_t)DK * sizeof(double));
  double* c = (double*)malloc((size_t)DK * sizeof(double));
  double* x = (double*)malloc((size_t)nc * sizeof(double));
  double* r = (double*)malloc((size_t)nc * sizeof(double));
  const int64_t sbase = (bi * H + hi) * DK * DV;

  if (S0 != NULL)
    for (int64_t d = 0; d < DK; ++d)
      for (int64_t n = 0; n < nc; ++n) S[d * nc + n] = S0[sbase + d * DV + n0 + n];

  for (int64_t t = 0; t < T; ++t) {
    const int64_t row = (bi * T + t) * H + hi; /* token row in [B, T, H] */
    const float* qt = q + row * DK;
    const float* kt = k + row * DK;
    const float* vt = v + row * DV;

    for (int64_t d = 0; d < DK; ++d) {
      alpha[d] = exp(gate_at(log_alpha, alpha_kind, row, DK, d, 0.0));
      c[d] = gate_at(bg, b_kind, row, DK, d, 0.0) * (double)kt[d];
    }
    for (int64_t n = 0; n < nc; ++n)
      x[n] = gate_at(wg, w_kind, row, DV, n0 + n, 1.0) * (double)vt[n0 + n];

    if (order == ORDER_DECAY_THEN_ERASE) /* decay: S <- Diag(alpha) S */
      for (int64_t d = 0; d < DK; ++d)
        for (int64_t n = 0; n < nc; ++n) S[d * nc + n] *= alpha[d];

    /* read for the erase: r = (b . k) S */
    for (int64_t n = 0; n < nc; ++n) r[n] = 0.0;
    for (int64_t d = 0; d < DK; ++d)
      for (int64_t n = 0; n < nc; ++n) r[n] += c[d] * S[d * nc + n];

    /* erase: S <- S - k^T r */
    for (int64_t d = 0; d < DK; ++d)
      for (int64_t n = 0; n < nc; ++n) S[d * nc + n] -= (double)kt[d] * r[n];

    if (order == ORDER_ERASE_THEN_DECAY) /* decay: S <- Diag(alpha) S */
      for (int64_t d = 0; d < DK; ++d)
        for (int64_t n = 0; n < nc; ++n) S[d * nc + n] *= alpha[d];

    /* write: S <- S + k^T (w . v) */
    for (int64_t d = 0; d < DK; ++d)
      for (int64_t n = 0; n < nc; ++n) S[d * nc + n] += (double)kt[d] * x[n];

    /* read out: o_t = q_t S_t */
    for (int64_t n = 0; n < nc; ++n) {
      double acc = 0.0;
      for (int64_t d = 0; d < DK; ++d) acc += (double)qt[d] * S[d * nc + n];
      o[row * DV + n0 + n] = acc;
    }
  }

  if (S_T != NULL)
    for (int64_t d = 0; d < DK; ++d)
      for (int64_t n = 0; n < nc; ++n) S_T[sbase + d * DV + n0 + n] = S[d * nc + n];

  free(S);
  free(alpha);
  free(c);
  free(x);
  free(r);
}

/*
 * Layouts (row-major, contiguous):
 *   q, k       [B, T, H, DK]      v, o        [B, T, H, DV]
 *   log_alpha  [B, T, H] (SCALAR) or [B, T, H, DK] (CHANNEL) or NULL (NONE)
 *   b          [B, T, H] (SCALAR) or [B, T, H, DK] (CHANNEL) or NULL (NONE)
 *   w          [B, T, H] (SCALAR) or [B, T, H, DV] (CHANNEL) or NULL (NONE)
 *   S0, S_T    [B, H, DK, DV]; S0 may be NULL (zero state), S_T may be NULL.
 * n_threads <= 0 uses the OpenMP default. Returns 0, or -1 on bad arguments.
 */
int gdr_oracle_forward(int64_t B, int64_t H, int64_t T, int64_t DK, int64_t DV,
                       const float* q, const float* k, const float* v,
                       const float* log_alpha, int alpha_kind,
                       const float* b, int b_kind, const float* w, int w_kind,
                       int order, const double* S0, double* o, double* S_T,
                       int n_threads) {
  if (B < 0 || H < 0 || T < 0 || DK <= 0 || DV <= 0) return -1;
  if (q == NULL || k == NULL || v == NULL || o == NULL) return -1;
  if (alpha_kind < 0 || alpha_kind > 2 || b_kind < 0 || b_kind > 2 || w_kind < 0 || w_kind > 2)
    return -1;
  if (order != ORDER_ERASE_THEN_DECAY && order != ORDER_DECAY_THEN_ERASE) return -1;

  /* Split columns so that there are at least ~4 chains per thread. */
  int nt = 1;
#ifdef _OPENMP
  nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#endif
  int64_t nblk = 1;
  while (B * H * nblk < 4 * (int64_t)nt && DV % (2 * nblk) == 0 && DV / (2 * nblk) >= 8) nblk *= 2;
  const int64_t width = DV / nblk;
  const int64_t jobs = B * H * nblk;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
  for (int64_t j = 0; j < jobs; ++j) {
    const int64_t blk = j % nblk;
    const int64_t bh = j / nblk;
    run_chain(B, H, T, DK, DV, bh / H, bh % H, blk * width, (blk + 1) * width, q, k, v,
              log_alpha, alpha_kind, b, b_kind, w, w_kind, order, S0, o, S_T);
  }
  return 0;
}
