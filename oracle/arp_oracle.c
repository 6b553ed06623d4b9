/*
 * arp_oracle.c -- plain fp64 CPU oracle for causal attention with accumulated
 * SO(2) rotations.
 *
 * TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
 * benchmark's CPU-baseline leg call it; the GPU library never does, and the
 * two share no source.  It is written to be read against the pages, not to be
 * fast: every step is the plain definition, computed in double precision from
 * the exact bits the GPU reads (fp32, or bf16 widened by a 16-bit shift).
 *
 * Sources (page title, then the place on it):
 *  [ACC]  "Why Do Accumulated Transformations Extrapolate?" (arXiv 2606.24975)
 *  [ADA]  "AdaRoPE: Not All Attention Heads Should Rotate and Scale Equally"
 *         (arXiv 2607.19363)
 *  [POST] "The RoPE decay curve everyone plots is noise ..." (dev.to)
 *
 * What is computed, step by step:
 *  1. Accumulated angles.  Each position t carries a block-diagonal step
 *     rotation with one angle phi_t[p] per two-dimensional block p; the
 *     blocks commute, so the product of steps is a rotation by the summed
 *     angle ([ACC] Sec. 5, "SO(2) notation").  The route from source j to
 *     query i holds the steps j+1 .. i ([ACC] Sec. 2.2, eq. (6)), so the
 *     angle attached to position t is the inclusive sum
 *         Theta_t[p] = sum_{s <= t} phi_s[p],
 *     and the route rotation is the difference Theta_i - Theta_j.
 *     (ORACLE_SCAN_EXCLUSIVE gives the exclusive sum over s < t.)
 *  2. Rotation.  Block p acts on the adjacent pair (x[2p], x[2p+1]) as
 *         R(a) = [[cos a, -sin a], [sin a, cos a]]
 *     ([ADA] Sec. 2.1 eq. (1) and the preliminaries' eq. (7)-(8); [POST] rope()).
 *     q~_t = R(Theta_t) q_t, k~_t = R(Theta_t) k_t, and v~_t = R(Theta_t) v_t
 *     when values are transported.  Then
 *         <q~_i, k~_j> = q_i^T R(Theta_j - Theta_i) k_j = q_i^T P_{j->i} k_j,
 *     the routed score of [ACC] eq. (7)-(8), with P_{j->i} a rotation by
 *     minus the summed angles of steps j+1..i ([ACC] App. B.8, position-only
 *     case; App. B.2 writes the step as e^{-i psi_t}).
 *  2b. Per-head query scale (AdaScale, [ADA] Sec. 3.3): each head's query is
 *     multiplied by its inverse temperature lambda_h before anything else,
 *     q_i <- lambda_h q_i, so the logit becomes lambda_h scale <q~_i, k~_j>;
 *     keys and values are untouched (the page applies it to the query only).
 *     Without a head scale lambda_h = 1.
 *  3. Scores s_ij = scale * <q~_i, k~_j> - m_h (i - j) [distance bias on]
 *     + sum_{s=j+1}^{i} log f_s [forget gate on], for the causal set j <= i
 *     ([ACC] eq. (2), (11); [ADA] eq. (5); the forget gate is the logit term of
 *     the PaTH reading notes' Sec. 2.5, one gate f_s per token and head, which
 *     [ACC] Sec. 4 names beside the distance bias as far-mass control).  The
 *     gate sum is accumulated here over s = j+1..i directly, not as a
 *     difference of prefix sums.
 *  4. Softmax over j <= i, computed in two passes: the row maximum M, then
 *     w_ij = exp(s_ij - M) and l_i = sum_j w_ij ([ACC] eq. (2)).
 *  5. Aggregation c_i = sum_j (w_ij / l_i) P_{j->i} v_j ([ACC] eq. (4)); with
 *     value transport this is R(Theta_i)^T sum_j alpha_ij v~_j, without it the
 *     plain sum of eq. (3).
 *
 * Gradients (oracle_backward): the chain rule through steps 1-5 as written,
 * for an upstream gradient g_i = dL/dc_i.  The pages train these models with
 * learned angles ([ACC] "Model variants"), which needs dL/dphi; nothing about
 * the gradient is stated on the pages beyond the forward definition, so this
 * is that definition differentiated by hand:
 *  - value transport: c_i = R(Theta_i)^T o~_i, so dL/do~_i = R(Theta_i) g_i;
 *  - softmax: with alpha_ij = w_ij / l_i and D_i = <dL/do~_i, o~_i>,
 *    dL/ds_ij = alpha_ij (<dL/do~_i, v~_j> - D_i);
 *  - head scale: q_i = lambda_h q_raw_i, so dL/dq_raw_i = lambda_h dL/dq_i;
 *  - scores: dL/dq~_i = scale sum_j dL/ds_ij k~_j, dL/dk~_j = scale
 *    sum_i dL/ds_ij q~_i, dL/dv~_j = sum_i alpha_ij dL/do~_i;
 *  - rotation: x~ = R(a) x gives dL/dx = R(a)^T dL/dx~ and, per pair,
 *    dL/da = <dL/dx~, J x~> with J = [[0, -1], [1, 0]] (dR/da = R J = J R);
 *    the transport step contributes -<dL/do~_i, J o~_i> at position i;
 *  - scan: Theta_t sums phi_s over s <= t, so dL/dphi_s sums dL/dTheta_t over
 *    t >= s (t > s for the exclusive scan), and over the heads that share one
 *    angle stream.  The wrap into [-pi, pi) has derivative 1.
 */
#include "arp_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_PI 3.14159265358979323846

/* Widen one stored element to double.  bf16 is the top half of an fp32. */
static double load_elem(const void* base, int32_t dtype, int64_t idx) {
  if (dtype == ORACLE_DTYPE_F32) {
    return (double)((const float*)base)[idx];
  }
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Step 1: prefix sum along the sequence, one running total per (segment, pair). */
void oracle_angle_scan(const float* phi, int64_t nseg, int64_t seqlen, int64_t npairs,
                       int exclusive, double* theta) {
  for (int64_t s = 0; s < nseg; ++s) {
    for (int64_t p = 0; p < npairs; ++p) {
      double run = 0.0;
      for (int64_t t = 0; t < seqlen; ++t) {
        int64_t idx = (s * seqlen + t) * npairs + p;
        if (exclusive) {
          theta[idx] = run;
          run += (double)phi[idx];
        } else {
          run += (double)phi[idx];
          theta[idx] = run;
        }
      }
    }
  }
}

/* ---- Step angles drawn on the fly ----------------------------------------
 * Philox4x64-10, the counter-based generator of Salmon, Moraes, Dror and Shaw
 * ("Parallel random numbers: as easy as 1, 2, 3", SC 2011).  A block of four
 * 64-bit words is a pure function of a 256-bit counter and a 128-bit key: ten
 * rounds, each multiplying words 0 and 2 by two fixed odd constants; the low
 * halves of the products become words 3 and 1, the high halves xor'd with
 * the other two words and the key become words 2 and 0; between rounds the
 * key grows by two Weyl increments (the golden ratio and sqrt(3) - 1 in
 * 64-bit fixed point). */
__extension__ typedef unsigned __int128 oracle_u128;

void oracle_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
  const uint64_t m0 = 0xD2E7470EE14C6C93ull, m1 = 0xCA5A826395121157ull;
  const uint64_t w0 = 0x9E3779B97F4A7C15ull, w1 = 0xBB67AE8584CAA73Bull;
  uint64_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint64_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += w0;
      k1 += w1;
    }
    const oracle_u128 p0 = (oracle_u128)m0 * c[0];
    const oracle_u128 p1 = (oracle_u128)m1 * c[2];
    const uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
    const uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
  for (int i = 0; i < 4; ++i) out[i] = c[i];
}

/* The random variant's step angles ("Why Do Accumulated Transformations
 * Extrapolate?", App. D "Model variants": independent per position and pair,
 * uniform on (-f_b, f_b), redrawn every forward pass).  One Philox block
 * serves two consecutive positions (t even and odd) of four consecutive pairs:
 * the block for (b, g, t, p) sits at counter (c, step, 0, 0), key (seed, 0),
 * with c = ((b * phi_heads + g) * ceil(seqlen / 2) + t / 2) * (npairs / 4) +
 * p / 4; word p mod 4 holds the pair, its low 32 bits for even t and high 32
 * bits for odd t.  Those 32 bits w give u = w * 2^-32 in [0, 1), and
 * phi = bound[g][p] * (2u - 1), formed in fp64 (exactly, but for the final
 * product) and rounded once to fp32.  step numbers the draws (one per
 * forward pass).  npairs must be a multiple of 4. */
void oracle_random_phi(int64_t batch, int64_t phi_heads, int64_t seqlen, int64_t npairs,
                       uint64_t seed, uint64_t step, const float* bound, float* phi) {
  const uint64_t key[2] = {seed, 0};
  const int64_t half_len = (seqlen + 1) / 2, groups = npairs / 4;
  for (int64_t s = 0; s < batch * phi_heads; ++s) {
    const int64_t g = s % phi_heads;
    for (int64_t t = 0; t < seqlen; ++t) {
      for (int64_t p = 0; p < npairs; ++p) {
        const uint64_t c = (uint64_t)((s * half_len + t / 2) * groups + p / 4);
        const uint64_t ctr[4] = {c, step, 0, 0};
        uint64_t words[4];
        oracle_philox4x64_10(ctr, key, words);
        const uint64_t w = words[p % 4];
        const uint32_t bits = (t % 2 == 0) ? (uint32_t)w : (uint32_t)(w >> 32);
        const double u = (double)bits * (1.0 / 4294967296.0); /* 2^-32 */
        phi[(s * seqlen + t) * npairs + p] = (float)((double)bound[g * npairs + p] * (2.0 * u - 1.0));
      }
    }
  }
}

/* x - 2 pi k with k chosen so the result lies in [-pi, pi). */
double oracle_wrap(double x) {
  /* fmod's remainder is exact, and the one correction step is exact too (a
   * difference of two doubles within a factor of two of each other), so the
   * result is x - k 2pi with no rounding at all, in [-pi, pi) for every
   * finite x.  (A quotient-and-multiply reduction rounds twice and leaves the
   * range once |x| passes ~2^53.) */
  const double two_pi = 2.0 * ORACLE_PI;
  double r = fmod(x, two_pi);
  if (r >= ORACLE_PI) r -= two_pi;
  else if (r < -ORACLE_PI) r += two_pi;
  return r;
}

void oracle_wrap_array(const double* x, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_wrap(x[i]);
}

/* Step 2 for one vector: y = R(a) x per pair, or R(a)^T x when inverse. */
static void rotate_vec(const double* x, const double* angle, int64_t npairs, int inverse,
                       double* y) {
  for (int64_t p = 0; p < npairs; ++p) {
    double c = cos(angle[p]);
    double s = sin(angle[p]);
    if (inverse) s = -s;
    double a = x[2 * p];
    double b = x[2 * p + 1];
    y[2 * p] = a * c - b * s;
    y[2 * p + 1] = a * s + b * c;
  }
}

void oracle_rotate_rows(const void* x, int32_t io_dtype, const double* angle, int64_t nrows,
                        int64_t dim, int inverse, double* out) {
  int64_t npairs = dim / 2;
  double* row = (double*)malloc(sizeof(double) * (size_t)dim);
  if (!row) return;
  for (int64_t r = 0; r < nrows; ++r) {
    for (int64_t c = 0; c < dim; ++c) row[c] = load_elem(x, io_dtype, r * dim + c);
    rotate_vec(row, angle + r * npairs, npairs, inverse, out + r * dim);
  }
  free(row);
}

static int check_problem(const oracle_problem* p) {
  if (!p || p->batch <= 0 || p->heads <= 0 || p->seqlen <= 0 || p->head_dim <= 0) return ORACLE_ERR_ARG;
  if (p->head_dim % 2 != 0) return ORACLE_ERR_ARG;
  if (p->phi_heads != 1 && p->phi_heads != p->heads) return ORACLE_ERR_ARG;
  if (p->io_dtype != ORACLE_DTYPE_F32 && p->io_dtype != ORACLE_DTYPE_BF16) return ORACLE_ERR_ARG;
  if (!p->q || !p->k || !p->v || !p->phi) return ORACLE_ERR_ARG;
  if ((p->flags & ORACLE_ALIBI) && !p->alibi_slopes) return ORACLE_ERR_ARG;
  if ((p->flags & ORACLE_FORGET) && !p->logf) return ORACLE_ERR_ARG;
  return ORACLE_OK;
}

int oracle_theta(const oracle_problem* p, double* theta) {
  int rc = check_problem(p);
  if (rc) return rc;
  oracle_angle_scan(p->phi, p->batch * p->phi_heads, p->seqlen, p->head_dim / 2,
                    (p->flags & ORACLE_SCAN_EXCLUSIVE) != 0, theta);
  return ORACLE_OK;
}

/* Everything one (b, h) needs for rows i <= imax: unwrapped angles, and the
 * rotated keys and values of positions 0..imax. */
typedef struct head_state {
  int64_t n;        /* positions held: imax + 1 */
  double* theta;    /* [n, P] */
  double* krot;     /* [n, d] */
  double* vrot;     /* [n, d] */
} head_state;

static void head_free(head_state* hs) {
  free(hs->theta);
  free(hs->krot);
  free(hs->vrot);
  memset(hs, 0, sizeof *hs);
}

static int head_build(const oracle_problem* p, int64_t b, int64_t h, int64_t imax, head_state* hs) {
  const int64_t d = p->head_dim, P = d / 2, L = p->seqlen;
  const int64_t hphi = (p->phi_heads == 1) ? 0 : h;
  const int64_t n = imax + 1;
  memset(hs, 0, sizeof *hs);
  hs->n = n;
  hs->theta = (double*)malloc(sizeof(double) * (size_t)(n * P));
  hs->krot = (double*)malloc(sizeof(double) * (size_t)(n * d));
  hs->vrot = (double*)malloc(sizeof(double) * (size_t)(n * d));
  if (!hs->theta || !hs->krot || !hs->vrot) {
    head_free(hs);
    return ORACLE_ERR_NOMEM;
  }
  /* Step 1 on this head's angle stream (only the first n positions are needed). */
  const float* phi = p->phi + (b * p->phi_heads + hphi) * L * P;
  oracle_angle_scan(phi, 1, n, P, (p->flags & ORACLE_SCAN_EXCLUSIVE) != 0, hs->theta);
  /* Step 2 on keys and values. */
  const int64_t base = ((b * p->heads + h) * L) * d;
  double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
  if (!tmp) {
    head_free(hs);
    return ORACLE_ERR_NOMEM;
  }
  for (int64_t j = 0; j < n; ++j) {
    for (int64_t c = 0; c < d; ++c) tmp[c] = load_elem(p->k, p->io_dtype, base + j * d + c);
    if (p->flags & ORACLE_ROTATE_QK) {
      rotate_vec(tmp, hs->theta + j * P, P, 0, hs->krot + j * d);
    } else {
      memcpy(hs->krot + j * d, tmp, sizeof(double) * (size_t)d);
    }
    for (int64_t c = 0; c < d; ++c) tmp[c] = load_elem(p->v, p->io_dtype, base + j * d + c);
    if (p->flags & ORACLE_ROTATE_V) {
      rotate_vec(tmp, hs->theta + j * P, P, 0, hs->vrot + j * d);
    } else {
      memcpy(hs->vrot + j * d, tmp, sizeof(double) * (size_t)d);
    }
  }
  free(tmp);
  return ORACLE_OK;
}

/* Step 2b: the query multiplier of head h (1 without a head scale). */
static double head_lambda(const oracle_problem* p, int64_t h) {
  return p->head_scale ? (double)p->head_scale[h] : 1.0;
}

void oracle_adascale_lambda(const double* tau, const double* gamma, int64_t heads, double L,
                            double L_ref, double* lambda) {
  const double len = L > L_ref ? L : L_ref;
  for (int64_t h = 0; h < heads; ++h) lambda[h] = pow(log(1.0 + len / L_ref), gamma[h]) / tau[h];
}

/* Step 3 for row i: scores[j] for j = 0..i.  qrot is scratch of length d. */
static void row_scores(const oracle_problem* p, const head_state* hs, int64_t b, int64_t h,
                       int64_t i, double* qrot, double* scores) {
  const int64_t d = p->head_dim, P = d / 2, L = p->seqlen;
  const int64_t base = ((b * p->heads + h) * L) * d;
  double* qraw = qrot + d; /* caller gives 2*d doubles */
  const double lam = head_lambda(p, h);
  for (int64_t c = 0; c < d; ++c) qraw[c] = lam * load_elem(p->q, p->io_dtype, base + i * d + c);
  if (p->flags & ORACLE_ROTATE_QK) {
    rotate_vec(qraw, hs->theta + i * P, P, 0, qrot);
  } else {
    memcpy(qrot, qraw, sizeof(double) * (size_t)d);
  }
  const double slope = (p->flags & ORACLE_ALIBI) ? (double)p->alibi_slopes[h] : 0.0;
  for (int64_t j = 0; j <= i; ++j) {
    const double* kj = hs->krot + j * d;
    double dot = 0.0;
    for (int64_t c = 0; c < d; ++c) dot += qrot[c] * kj[c];
    scores[j] = p->scale * dot - slope * (double)(i - j);
  }
  if (p->flags & ORACLE_FORGET) {
    /* sum_{s=j+1}^{i} log f_s, from j = i (empty) down to 0 */
    const float* lf = p->logf + (b * p->heads + h) * L;
    double gate = 0.0;
    for (int64_t j = i; j >= 0; --j) {
      scores[j] += gate;
      gate += (double)lf[j];
    }
  }
}

int oracle_scores_row(const oracle_problem* p, int64_t b, int64_t h, int64_t i, double* out) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (b < 0 || b >= p->batch || h < 0 || h >= p->heads || i < 0 || i >= p->seqlen) return ORACLE_ERR_ARG;
  head_state hs;
  rc = head_build(p, b, h, i, &hs);
  if (rc) return rc;
  double* q2 = (double*)malloc(sizeof(double) * (size_t)(2 * p->head_dim));
  if (!q2) {
    head_free(&hs);
    return ORACLE_ERR_NOMEM;
  }
  row_scores(p, &hs, b, h, i, q2, out);
  free(q2);
  head_free(&hs);
  return ORACLE_OK;
}

/* Steps 3-5 for one row. */
static int attention_row(const oracle_problem* p, const head_state* hs, int64_t b, int64_t h,
                         int64_t i, double* out) {
  const int64_t d = p->head_dim, P = d / 2;
  double* scores = (double*)malloc(sizeof(double) * (size_t)(i + 1));
  double* work = (double*)malloc(sizeof(double) * (size_t)(3 * d));
  if (!scores || !work) {
    free(scores);
    free(work);
    return ORACLE_ERR_NOMEM;
  }
  double* qrot = work;      /* 2*d: rotated query + raw query */
  double* acc = work + 2 * d;
  row_scores(p, hs, b, h, i, qrot, scores);

  /* Step 4, pass 1: the row maximum over the causal set. */
  double m = scores[0];
  for (int64_t j = 1; j <= i; ++j)
    if (scores[j] > m) m = scores[j];
  /* Step 4, pass 2, and step 5: weights, their sum, and the weighted values. */
  double l = 0.0;
  for (int64_t c = 0; c < d; ++c) acc[c] = 0.0;
  for (int64_t j = 0; j <= i; ++j) {
    double w = exp(scores[j] - m);
    l += w;
    const double* vj = hs->vrot + j * d;
    for (int64_t c = 0; c < d; ++c) acc[c] += w * vj[c];
  }
  for (int64_t c = 0; c < d; ++c) acc[c] /= l;
  if (p->flags & ORACLE_ROTATE_V) {
    /* Bring the sum of R(Theta_j) v_j back to the query's frame: R(Theta_i)^T. */
    rotate_vec(acc, hs->theta + i * P, P, 1, out);
  } else {
    memcpy(out, acc, sizeof(double) * (size_t)d);
  }
  free(scores);
  free(work);
  return ORACLE_OK;
}

int oracle_attention_rows(const oracle_problem* p, const int64_t* rows, int64_t nrows,
                          int nthreads, double* out) {
  int rc = check_problem(p);
  if (rc) return rc;
  const int64_t L = p->seqlen, BH = p->batch * p->heads;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= BH * L) return ORACLE_ERR_ARG;

  /* Highest query position requested per (b, h). */
  int64_t* imax = (int64_t*)malloc(sizeof(int64_t) * (size_t)BH);
  if (!imax) return ORACLE_ERR_NOMEM;
  for (int64_t bh = 0; bh < BH; ++bh) imax[bh] = -1;
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t bh = rows[r] / L, i = rows[r] % L;
    if (i > imax[bh]) imax[bh] = i;
  }
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  for (int64_t bh = 0; bh < BH && rc == ORACLE_OK; ++bh) {
    if (imax[bh] < 0) continue;
    const int64_t b = bh / p->heads, h = bh % p->heads;
    head_state hs;
    rc = head_build(p, b, h, imax[bh], &hs);
    if (rc) break;
    int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t r = 0; r < nrows; ++r) {
      if (rows[r] / L != bh) continue;
      err |= attention_row(p, &hs, b, h, rows[r] % L, out + r * p->head_dim);
    }
    head_free(&hs);
    rc = err;
  }
  free(imax);
  return rc;
}

/* ---------------------------------------------------------------------------
 * Gradients.
 * ------------------------------------------------------------------------- */

/* <x, J a> for one pair: J a = (-a1, a0). */
static double pair_cross(const double* x, const double* a) { return -x[0] * a[1] + x[1] * a[0]; }

/* One (b, h): all gradients of the head, O(L^2 d). dtheta_h is [L, P]. */
static int backward_head(const oracle_problem* p, const void* dout, int64_t b, int64_t h,
                         double* dq, double* dk, double* dv, double* dtheta_h, double* dlogf_h) {
  const int64_t d = p->head_dim, P = d / 2, L = p->seqlen;
  const int64_t base = ((b * p->heads + h) * L) * d;
  const int qk = (p->flags & ORACLE_ROTATE_QK) != 0, tv = (p->flags & ORACLE_ROTATE_V) != 0;
  const double slope = (p->flags & ORACLE_ALIBI) ? (double)p->alibi_slopes[h] : 0.0;
  head_state hs;
  int rc = head_build(p, b, h, L - 1, &hs);
  if (rc) return rc;
  double* qrot = (double*)calloc((size_t)(L * d), sizeof(double));
  double* dorot = (double*)calloc((size_t)(L * d), sizeof(double));  /* dL/do~ */
  double* otil = (double*)calloc((size_t)(L * d), sizeof(double));   /* o~ */
  double* dqt = (double*)calloc((size_t)(L * d), sizeof(double));
  double* dkt = (double*)calloc((size_t)(L * d), sizeof(double));
  double* dvt = (double*)calloc((size_t)(L * d), sizeof(double));
  double* alpha = (double*)malloc(sizeof(double) * (size_t)L);
  double* raw = (double*)malloc(sizeof(double) * (size_t)d);
  if (!qrot || !dorot || !otil || !dqt || !dkt || !dvt || !alpha || !raw) {
    rc = ORACLE_ERR_NOMEM;
    goto done;
  }
  const double lam = head_lambda(p, h);
  for (int64_t t = 0; t < L; ++t) {
    for (int64_t c = 0; c < d; ++c) raw[c] = lam * load_elem(p->q, p->io_dtype, base + t * d + c);
    if (qk) rotate_vec(raw, hs.theta + t * P, P, 0, qrot + t * d);
    else memcpy(qrot + t * d, raw, sizeof(double) * (size_t)d);
    for (int64_t c = 0; c < d; ++c) raw[c] = load_elem(dout, p->io_dtype, base + t * d + c);
    if (tv) rotate_vec(raw, hs.theta + t * P, P, 0, dorot + t * d);
    else memcpy(dorot + t * d, raw, sizeof(double) * (size_t)d);
  }
  for (int64_t i = 0; i < L; ++i) {
    /* forward row: scores, normalised weights alpha_ij, o~_i */
    const double* qi = qrot + i * d;
    double m = -INFINITY;
    for (int64_t j = 0; j <= i; ++j) {
      const double* kj = hs.krot + j * d;
      double dot = 0.0;
      for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];
      alpha[j] = p->scale * dot - slope * (double)(i - j);
    }
    if (p->flags & ORACLE_FORGET) {
      /* sum_{s=j+1}^{i} log f_s, from j = i (empty) down to 0 */
      const float* lf = p->logf + (b * p->heads + h) * L;
      double gate = 0.0;
      for (int64_t j = i; j >= 0; --j) {
        alpha[j] += gate;
        gate += (double)lf[j];
      }
    }
    for (int64_t j = 0; j <= i; ++j)
      if (alpha[j] > m) m = alpha[j];
    double l = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
      alpha[j] = exp(alpha[j] - m);
      l += alpha[j];
    }
    double* oi = otil + i * d;
    for (int64_t j = 0; j <= i; ++j) {
      alpha[j] /= l;
      const double* vj = hs.vrot + j * d;
      for (int64_t c = 0; c < d; ++c) oi[c] += alpha[j] * vj[c];
    }
    /* backward row */
    const double* gi = dorot + i * d;
    double Di = 0.0;
    for (int64_t c = 0; c < d; ++c) Di += gi[c] * oi[c];
    /* gate gradient: the logit s_ij holds log f_s for j < s <= i, so
       dlogf_s collects sum_{j < s} dS_ij from every row i >= s */
    double pre = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
      const double* vj = hs.vrot + j * d;
      const double* kj = hs.krot + j * d;
      double dp = 0.0;
      for (int64_t c = 0; c < d; ++c) dp += gi[c] * vj[c];
      const double ds = alpha[j] * (dp - Di);
      if (dlogf_h && j + 1 <= i) {
        pre += ds;                 /* sum_{j' <= j} dS_ij' = sum_{j' < s} for s = j + 1 */
        dlogf_h[j + 1] += pre;
      }
      for (int64_t c = 0; c < d; ++c) {
        dqt[i * d + c] += p->scale * ds * kj[c];
        dkt[j * d + c] += p->scale * ds * qi[c];
        dvt[j * d + c] += alpha[j] * gi[c];
      }
    }
  }
  for (int64_t t = 0; t < L; ++t) {
    const double* th = hs.theta + t * P;
    for (int64_t pp = 0; pp < P; ++pp) {
      double g = 0.0;
      if (qk) {
        g += pair_cross(dqt + t * d + 2 * pp, qrot + t * d + 2 * pp);
        g += pair_cross(dkt + t * d + 2 * pp, hs.krot + t * d + 2 * pp);
      }
      if (tv) {
        g += pair_cross(dvt + t * d + 2 * pp, hs.vrot + t * d + 2 * pp);
        g -= pair_cross(dorot + t * d + 2 * pp, otil + t * d + 2 * pp);
      }
      dtheta_h[t * P + pp] = g;
    }
    double* oq = dq + base + t * d;
    double* ok = dk + base + t * d;
    double* ov = dv + base + t * d;
    if (qk) {
      rotate_vec(dqt + t * d, th, P, 1, oq);
      rotate_vec(dkt + t * d, th, P, 1, ok);
    } else {
      memcpy(oq, dqt + t * d, sizeof(double) * (size_t)d);
      memcpy(ok, dkt + t * d, sizeof(double) * (size_t)d);
    }
    if (tv) rotate_vec(dvt + t * d, th, P, 1, ov);
    else memcpy(ov, dvt + t * d, sizeof(double) * (size_t)d);
    for (int64_t c = 0; c < d; ++c) oq[c] *= lam;  /* through q = lambda_h q_raw */
  }
done:
  free(qrot);
  free(dorot);
  free(otil);
  free(dqt);
  free(dkt);
  free(dvt);
  free(alpha);
  free(raw);
  head_free(&hs);
  return rc;
}

int oracle_backward(const oracle_problem* p, const void* dout, int nthreads, double* dq,
                    double* dk, double* dv, double* dtheta, double* dphi, double* dlogf) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!dout || !dq || !dk || !dv || !dtheta || !dphi) return ORACLE_ERR_ARG;
  if ((p->flags & ORACLE_FORGET) && !dlogf) return ORACLE_ERR_ARG;
  const int64_t B = p->batch, H = p->heads, L = p->seqlen, P = p->head_dim / 2;
  const int gated = (p->flags & ORACLE_FORGET) != 0;
  if (gated) memset(dlogf, 0, sizeof(double) * (size_t)(B * H * L));
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int64_t bh = 0; bh < B * H; ++bh)
    err |= backward_head(p, dout, bh / H, bh % H, dq, dk, dv, dtheta + bh * L * P,
                         gated ? dlogf + bh * L : NULL);
  if (err) return err;
  /* dphi_s = sum over heads sharing the stream, and over t >= s (t > s exclusive). */
  const int excl = (p->flags & ORACLE_SCAN_EXCLUSIVE) != 0;
  memset(dphi, 0, sizeof(double) * (size_t)(B * p->phi_heads * L * P));
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h) {
      const int64_t g = (p->phi_heads == 1) ? 0 : h;
      const double* dth = dtheta + (b * H + h) * L * P;
      double* out = dphi + (b * p->phi_heads + g) * L * P;
      for (int64_t pp = 0; pp < P; ++pp) {
        double run = 0.0;
        for (int64_t s = L - 1; s >= 0; --s) {
          if (excl) {
            out[s * P + pp] += run;
            run += dth[s * P + pp];
          } else {
            run += dth[s * P + pp];
            out[s * P + pp] += run;
          }
        }
      }
    }
  return ORACLE_OK;
}
