/*
 * arp_oracle.h -- plain fp64 CPU oracle for causal attention with accumulated
 * SO(2) rotations.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only callers.  The GPU library neither
 * links nor calls this code, and this file shares no source with it.
 *
 * Every pointer here is a host pointer.  Every output is fp64.
 *
 * Layouts (row-major, last index fastest):
 *   q, k, v       [batch, heads, seqlen, head_dim]        fp32 or bf16 bit patterns
 *   phi           [batch, phi_heads, seqlen, head_dim/2]  fp32
 *   alibi_slopes  [heads]                                 fp32
 *   theta         [batch, phi_heads, seqlen, head_dim/2]  fp64
 * phi_heads is 1 (one angle stream shared by every head) or equal to heads.
 */
#ifndef ARP_ORACLE_H
#define ARP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Flags.  Same meaning as the GPU library's, defined here on their own. */
#define ORACLE_ROTATE_QK 1u      /* rotate q and k by their accumulated angles    */
#define ORACLE_ROTATE_V 2u       /* transport values along the route (eq. (4))    */
#define ORACLE_ALIBI 4u          /* add the distance bias -m_h (i - j)            */
#define ORACLE_SCAN_EXCLUSIVE 16u /* Theta_t sums steps s < t instead of s <= t   */
#define ORACLE_FORGET 64u        /* add the forget-gate bias sum_{s=j+1}^{i} log f_s */

#define ORACLE_DTYPE_F32 0
#define ORACLE_DTYPE_BF16 1

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

typedef struct oracle_problem {
  int64_t batch, heads, seqlen, head_dim;
  int64_t phi_heads;  /* 1 or heads */
  int32_t io_dtype;   /* ORACLE_DTYPE_F32 or ORACLE_DTYPE_BF16 (uint16 bit patterns) */
  uint32_t flags;     /* ORACLE_* flags above */
  double scale;       /* logit scale applied to <q~, k~> (e.g. 1/sqrt(head_dim)) */
  const void* q;
  const void* k;
  const void* v;
  const float* phi;
  const float* alibi_slopes; /* read only when ORACLE_ALIBI is set */
  const float* logf;         /* [batch, heads, seqlen] log forget gates; read only with ORACLE_FORGET */
  const float* head_scale;   /* NULL, or [heads]: per-head query multipliers lambda_h (AdaScale) */
} oracle_problem;

/* Prefix sum of step angles along the sequence, one segment per (outer, pair).
 * phi and theta are [nseg, seqlen, npairs].  Unwrapped fp64. */
void oracle_angle_scan(const float* phi, int64_t nseg, int64_t seqlen, int64_t npairs,
                       int exclusive, double* theta);

/* Philox4x64-10 block for counter ctr and key (Salmon et al., SC 2011). */
void oracle_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]);

/* Random step angles phi [batch, phi_heads, seqlen, npairs] (fp32), uniform
 * on (-bound[g][p], bound[g][p]); bound is [phi_heads, npairs] fp32 and npairs
 * a multiple of 4.  One Philox block (key (seed, 0), counter (c, step, 0, 0))
 * covers positions 2m, 2m+1 of pairs 4j..4j+3 of one (b, g); the arp_oracle.c
 * definition gives c and which 32 bits each element takes. */
void oracle_random_phi(int64_t batch, int64_t phi_heads, int64_t seqlen, int64_t npairs,
                       uint64_t seed, uint64_t step, const float* bound, float* phi);

/* AdaScale's per-head, length-aware inverse temperature ("AdaRoPE: Not All
 * Attention Heads Should Rotate and Scale Equally", Sec. 3.3, AdaScale):
 *   lambda_h(L) = (1 / tau_h) * [ln(1 + max(L, L_ref) / L_ref)]^gamma_h
 * for heads h = 0..heads-1, in fp64. */
void oracle_adascale_lambda(const double* tau, const double* gamma, int64_t heads, double L,
                            double L_ref, double* lambda);

/* Reduce an angle into [-pi, pi). */
double oracle_wrap(double x);
void oracle_wrap_array(const double* x, int64_t n, double* out);

/* Rotate rows of x ([nrows, dim], fp32 or bf16 bits) pair by pair by the angles
 * in angle ([nrows, dim/2], fp64).  inverse != 0 applies R(a)^T. */
void oracle_rotate_rows(const void* x, int32_t io_dtype, const double* angle, int64_t nrows,
                        int64_t dim, int inverse, double* out);

/* Accumulated angles of the whole problem: [batch, phi_heads, seqlen, head_dim/2]. */
int oracle_theta(const oracle_problem* p, double* theta);

/* Scores s_{i,j} for j = 0..i of row (b, h, i): out has i+1 entries. */
int oracle_scores_row(const oracle_problem* p, int64_t b, int64_t h, int64_t i, double* out);

/* Attention output rows.  rows[r] = (b * heads + h) * seqlen + i.
 * out is [nrows, head_dim].  nthreads <= 0 lets OpenMP choose. */
int oracle_attention_rows(const oracle_problem* p, const int64_t* rows, int64_t nrows,
                          int nthreads, double* out);

/* Gradients of the attention output (oracle_attention_rows over every row)
 * for an upstream gradient dout ([batch, heads, seqlen, head_dim], same io
 * dtype as q).  Outputs, all fp64:
 *   dq, dk, dv  [batch, heads, seqlen, head_dim]
 *   dtheta      [batch, heads, seqlen, head_dim/2]   dL/dTheta per head
 *   dphi        [batch, phi_heads, seqlen, head_dim/2]
 *   dlogf       [batch, heads, seqlen]  dL/d(log f_s), required with
 *               ORACLE_FORGET (else may be NULL): the logit s_ij holds
 *               log f_s for j < s <= i, so dlogf_s = sum_{i >= s} sum_{j < s} dS_ij
 * O(seqlen^2 head_dim) per head; OpenMP over heads. */
int oracle_backward(const oracle_problem* p, const void* dout, int nthreads, double* dq,
                    double* dk, double* dv, double* dtheta, double* dphi, double* dlogf);

#ifdef __cplusplus
}
#endif

#endif /* ARP_ORACLE_H */
