/* Host checks of the CPU oracle (oracle/gdr_oracle.c), built with AddressSanitizer and
 * UndefinedBehaviorSanitizer: every gate kind, both orders, ragged shapes and several thread
 * counts run over exactly sized heap buffers (so any read or write past a tensor is caught), the
 * argument checks return -1, and two closed forms of the recurrence hold ("Recurrent Memory:
 * Write, Erase, Decay, Read", section 01: one write read back gives (q . k) v; section 04: with
 * no erase and no write the state decays by exp of the summed log alpha).  Exits with the number
 * of failures. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int gdr_oracle_forward(int64_t B, int64_t H, int64_t T, int64_t DK, int64_t DV, const float* q, const float* k,
                       const float* v, const float* log_alpha, int alpha_kind, const float* b, int b_kind,
                       const float* w, int w_kind, int order, const double* S0, double* o, double* S_T,
                       int n_threads);

static int fails = 0;
#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);         \
      ++fails;                                                    \
    }                                                             \
  } while (0)

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static float urand(void) { /* xorshift64*, uniform in [-1, 1) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (float)((double)((rng * 0x2545f4914f6cdd1dull) >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}
static float* fill(int64_t n, float lo, float hi) {
  float* p = malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
  for (int64_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5f * (urand() + 1.f);
  return p;
}

static void run_shapes(void) {
  const int64_t shapes[][5] = {{1, 1, 1, 4, 4}, {2, 3, 7, 8, 12}, {1, 2, 65, 16, 16}, {3, 1, 0, 4, 8}, {0, 2, 5, 4, 4}};
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
    const int64_t B = shapes[s][0], H = shapes[s][1], T = shapes[s][2], DK = shapes[s][3], DV = shapes[s][4];
    const int64_t rows = B * T * H;
    for (int ak = 0; ak <= 2; ++ak)
      for (int bk = 0; bk <= 2; ++bk)
        for (int wk = 0; wk <= 2; ++wk)
          for (int order = 0; order <= 1; ++order) {
            float* q = fill(rows * DK, -1.f, 1.f);
            float* k = fill(rows * DK, -0.3f, 0.3f);
            float* v = fill(rows * DV, -1.f, 1.f);
            float* la = ak ? fill(rows * (ak == 2 ? DK : 1), -1.f, 0.f) : NULL;
            float* b = bk ? fill(rows * (bk == 2 ? DK : 1), 0.f, 1.f) : NULL;
            float* w = wk ? fill(rows * (wk == 2 ? DV : 1), 0.f, 1.f) : NULL;
            double* S0 = malloc((size_t)(B * H * DK * DV + 1) * sizeof(double));
            for (int64_t i = 0; i < B * H * DK * DV; ++i) S0[i] = 0.02 * urand();
            double* o = malloc((size_t)(rows * DV + 1) * sizeof(double));
            double* ST = malloc((size_t)(B * H * DK * DV + 1) * sizeof(double));
            for (int threads = 1; threads <= 3; threads += 2) {
              const int rc = gdr_oracle_forward(B, H, T, DK, DV, q, k, v, la, ak, b, bk, w, wk, order,
                                                (s & 1) ? S0 : NULL, o, ST, threads);
              CHECK(rc == 0);
              for (int64_t i = 0; i < rows * DV; ++i) CHECK(isfinite(o[i]));
            }
            free(q), free(k), free(v), free(la), free(b), free(w), free(S0), free(o), free(ST);
          }
  }
}

static void closed_forms(void) {
  enum { DK = 8, DV = 8 };
  float q[DK], k[DK], v[DV];
  for (int i = 0; i < DK; ++i) q[i] = urand(), k[i] = urand();
  for (int j = 0; j < DV; ++j) v[j] = urand();
  double o[DV], S[DK * DV];
  /* one write from zero, read by q: o = (q . k) v */
  CHECK(gdr_oracle_forward(1, 1, 1, DK, DV, q, k, v, NULL, 0, NULL, 0, NULL, 0, 0, NULL, o, S, 1) == 0);
  double qk = 0;
  for (int i = 0; i < DK; ++i) qk += (double)q[i] * k[i];
  for (int j = 0; j < DV; ++j) CHECK(fabs(o[j] - qk * v[j]) <= 1e-12 * (1 + fabs(qk * v[j])));
  /* three tokens with w = 0 and no erase: S_3 = exp(sum log alpha) S0 per channel */
  float q3[3 * DK], k3[3 * DK], v3[3 * DV], la3[3 * DK], w3[3] = {0.f, 0.f, 0.f};
  for (int i = 0; i < 3 * DK; ++i) q3[i] = urand(), k3[i] = urand(), la3[i] = -0.5f * (urand() + 1.f);
  for (int j = 0; j < 3 * DV; ++j) v3[j] = urand();
  double S0[DK * DV], o3[3 * DV];
  for (int i = 0; i < DK * DV; ++i) S0[i] = urand();
  CHECK(gdr_oracle_forward(1, 1, 3, DK, DV, q3, k3, v3, la3, 2, NULL, 0, w3, 1, 0, S0, o3, S, 1) == 0);
  for (int i = 0; i < DK; ++i) {
    const double f = exp((double)la3[i] + la3[DK + i] + la3[2 * DK + i]);
    for (int j = 0; j < DV; ++j) CHECK(fabs(S[i * DV + j] - f * S0[i * DV + j]) <= 1e-12);
  }
}

static void bad_arguments(void) {
  float x[16] = {0};
  double o[16], S[16];
  CHECK(gdr_oracle_forward(-1, 1, 1, 2, 2, x, x, x, NULL, 0, NULL, 0, NULL, 0, 0, NULL, o, S, 1) == -1);
  CHECK(gdr_oracle_forward(1, 1, 1, 0, 2, x, x, x, NULL, 0, NULL, 0, NULL, 0, 0, NULL, o, S, 1) == -1);
  CHECK(gdr_oracle_forward(1, 1, 1, 2, 2, NULL, x, x, NULL, 0, NULL, 0, NULL, 0, 0, NULL, o, S, 1) == -1);
  CHECK(gdr_oracle_forward(1, 1, 1, 2, 2, x, x, x, x, 3, NULL, 0, NULL, 0, 0, NULL, o, S, 1) == -1);
  CHECK(gdr_oracle_forward(1, 1, 1, 2, 2, x, x, x, NULL, 0, NULL, 0, NULL, 0, 2, NULL, o, S, 1) == -1);
}

int main(void) {
  run_shapes();
  closed_forms();
  bad_arguments();
  printf("oracle checks: %d failure(s)\n", fails);
  return fails;
}
