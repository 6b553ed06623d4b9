/* The fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitizers.py): every entry point on small problems that cover
 * each flag, both io dtypes, shared and per-head angles, one-token and ragged
 * lengths, the forget gates and the per-head query multipliers.  Checks only
 * that the calls succeed and give finite results; the values are pinned by
 * the oracle's own tests. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/arp_oracle.h"

static int failures = 0;
#define EXPECT(cond)                                                               \
  do {                                                                             \
    if (!(cond)) {                                                                 \
      fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);            \
      ++failures;                                                                  \
    }                                                                              \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* splitmix64, uniform in [-1, 1) */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) / 4503599627370496.0 - 1.0;
}

static uint16_t to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static int all_finite(const double* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) return 0;
  return 1;
}

static void run_case(int64_t B, int64_t H, int64_t L, int64_t d, int64_t G, int dtype, uint32_t flags,
                     int head_scale) {
  const int64_t n = B * H * L * d, P = d / 2;
  void *q, *k, *v, *dout;
  const size_t es = dtype == ORACLE_DTYPE_F32 ? 4 : 2;
  q = malloc(n * es); k = malloc(n * es); v = malloc(n * es); dout = malloc(n * es);
  float* phi = malloc(sizeof(float) * B * G * L * P);
  float* alibi = malloc(sizeof(float) * H);
  float* logf = malloc(sizeof(float) * B * H * L);
  float* lam = malloc(sizeof(float) * H);
  void* bufs[4] = {q, k, v, dout};
  for (int j = 0; j < 4; ++j)
    for (int64_t i = 0; i < n; ++i) {
      const float x = (float)(urand() * 0.5);
      if (dtype == ORACLE_DTYPE_F32) ((float*)bufs[j])[i] = x;
      else ((uint16_t*)bufs[j])[i] = to_bf16(x);
    }
  for (int64_t i = 0; i < B * G * L * P; ++i) phi[i] = (float)(urand() * 0.8);
  for (int64_t h = 0; h < H; ++h) { alibi[h] = (float)(0.05 * (h + 1)); lam[h] = (float)(1.0 + 0.25 * h); }
  for (int64_t i = 0; i < B * H * L; ++i) logf[i] = (float)(-0.1 - 0.4 * (urand() + 1.0));

  oracle_problem p;
  memset(&p, 0, sizeof p);
  p.batch = B; p.heads = H; p.seqlen = L; p.head_dim = d; p.phi_heads = G;
  p.io_dtype = dtype; p.flags = flags; p.scale = 1.0 / sqrt((double)d);
  p.q = q; p.k = k; p.v = v; p.phi = phi; p.alibi_slopes = alibi; p.logf = logf;
  p.head_scale = head_scale ? lam : NULL;

  double* theta = malloc(sizeof(double) * B * G * L * P);
  EXPECT(oracle_theta(&p, theta) == ORACLE_OK);
  EXPECT(all_finite(theta, B * G * L * P));
  double* srow = malloc(sizeof(double) * L);
  EXPECT(oracle_scores_row(&p, B - 1, H - 1, L - 1, srow) == ORACLE_OK);
  EXPECT(all_finite(srow, L));
  const int64_t nrows = B * H * L;
  int64_t* rows = malloc(sizeof(int64_t) * nrows);
  for (int64_t r = 0; r < nrows; ++r) rows[r] = r;
  double* out = malloc(sizeof(double) * nrows * d);
  EXPECT(oracle_attention_rows(&p, rows, nrows, 2, out) == ORACLE_OK);
  EXPECT(all_finite(out, nrows * d));
  double *dq = malloc(sizeof(double) * n), *dk = malloc(sizeof(double) * n), *dv = malloc(sizeof(double) * n);
  double* dth = malloc(sizeof(double) * B * H * L * P);
  double* dphi = malloc(sizeof(double) * B * G * L * P);
  double* dlogf = malloc(sizeof(double) * B * H * L);
  EXPECT(oracle_backward(&p, dout, 2, dq, dk, dv, dth, dphi, dlogf) == ORACLE_OK);
  EXPECT(all_finite(dq, n) && all_finite(dk, n) && all_finite(dv, n));
  EXPECT(all_finite(dth, B * H * L * P) && all_finite(dphi, B * G * L * P));
  if (flags & ORACLE_FORGET) EXPECT(all_finite(dlogf, B * H * L));
  /* out-of-range rows and a bad problem are rejected, not read */
  int64_t badrow = nrows;
  EXPECT(oracle_attention_rows(&p, &badrow, 1, 1, out) != ORACLE_OK);
  oracle_problem bad = p;
  bad.phi_heads = 2 * H + 1;
  EXPECT(oracle_theta(&bad, theta) != ORACLE_OK);
  free(q); free(k); free(v); free(dout); free(phi); free(alibi); free(logf); free(lam);
  free(theta); free(srow); free(rows); free(out); free(dq); free(dk); free(dv); free(dth);
  free(dphi); free(dlogf);
}

int main(void) {
  const uint32_t R = ORACLE_ROTATE_QK, V = ORACLE_ROTATE_V, A = ORACLE_ALIBI,
                 X = ORACLE_SCAN_EXCLUSIVE, F = ORACLE_FORGET;
  const uint32_t flag_sets[] = {0, R, R | V, R | V | A, R | X, R | V | A | F, V | F};
  const int64_t lens[] = {1, 2, 17};
  for (size_t f = 0; f < sizeof flag_sets / sizeof flag_sets[0]; ++f)
    for (size_t l = 0; l < 3; ++l)
      for (int dt = 0; dt < 2; ++dt) {
        run_case(2, 3, lens[l], 8, 3, dt, flag_sets[f], (int)(f & 1));
        run_case(1, 2, lens[l], 4, 1, dt, flag_sets[f], (int)((f + 1) & 1));
      }
  /* generators and small helpers */
  {
    uint64_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, o[4];
    oracle_philox4x64_10(ctr, key, o);
    float bound[2 * 8], phi[2 * 2 * 5 * 8];
    for (int i = 0; i < 16; ++i) bound[i] = 0.1f * (float)(i + 1);
    oracle_random_phi(2, 2, 5, 8, 42, 7, bound, phi);
    for (int i = 0; i < 2 * 2 * 5 * 8; ++i) EXPECT(fabsf(phi[i]) <= bound[(i / (5 * 8)) % 2 * 8 + i % 8]);
    double tau[3] = {1, 2, 0.5}, gam[3] = {0, 1, -1}, lam[3];
    oracle_adascale_lambda(tau, gam, 3, 5000, 1000, lam);
    EXPECT(lam[0] == 1.0);
    double th[6];
    float steps[6] = {3.0f, 3.0f, -7.0f, 1e30f, -1e30f, 0.f};
    oracle_angle_scan(steps, 2, 3, 1, 0, th);
    double w[6];
    oracle_wrap_array(th, 6, w);
    for (int i = 0; i < 6; ++i) EXPECT(!isfinite(th[i]) || (w[i] >= -M_PI && w[i] < M_PI));
    float x[4] = {1, 2, 3, 4};
    double ang[2] = {0.5, -2.0}, r[4];
    oracle_rotate_rows(x, ORACLE_DTYPE_F32, ang, 1, 4, 1, r);
    EXPECT(all_finite(r, 4));
  }
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle checks passed\n");
  return 0;
}
