/*
 * arp.h -- C ABI of libarp.so: causal softmax attention with accumulated,
 * token-dependent SO(2) rotations, for AMD MI355X (gfx950).
 *
 * The method ("Why Do Accumulated Transformations Extrapolate?", arXiv
 * 2606.24975):
 *  - each position t carries one step angle phi_t[p] per two-dimensional
 *    rotary block p; blocks commute, so a route of steps is a rotation by
 *    the summed angle (Sec. 5, "SO(2) notation");
 *  - the route from source j to query i holds the steps j+1..i (Sec. 2.2,
 *    eq. (6)), so position t gets the inclusive prefix sum
 *    Theta_t = sum_{s<=t} phi_s and the route is a rotation by
 *    Theta_j - Theta_i (App. B.8 fixes the sign: a position-only route by
 *    k steps of angle w is R(-w k));
 *  - q, k (and v, with value transport) are rotated by R(Theta_t), the pair
 *    map [[cos, -sin], [sin, cos]] on elements (2p, 2p+1) (AdaRoPE, "AdaRoPE:
 *    Not All Attention Heads Should Rotate and Scale Equally", Sec. 2.1
 *    eq. (1));
 *  - scores s_ij = scale <q~_i, k~_j> - m_h (i - j) [distance bias] over the
 *    causal set j <= i, softmax, and the transported sum
 *    c_i = sum_j alpha_ij P_{j->i} v_j (eq. (2), (4), (8), (11)); with value
 *    transport the library returns R(Theta_i)^T sum_j alpha_ij R(Theta_j) v_j,
 *    which is exactly eq. (4).
 * RoPE is the special case of a constant phi_t[p] = theta_p (AdaRoPE
 * Sec. 2.1), NoPE the case without ARP_ROTATE_QK.
 *
 * Conventions for every entry point:
 *  - Tensors are caller-owned DEVICE memory, C-contiguous:
 *      q, k, v, o : [batch, heads, seqlen, head_dim]     (dtype of the desc)
 *      phi, theta : [batch, phi_heads, seqlen, head_dim/2] float32,
 *                   phi_heads = 1 with ARP_PHI_SHARED_HEADS, else heads
 *      alibi      : [heads] float32 slopes m_h (ARP_ALIBI only)
 *    Rotary pair p is elements (2p, 2p+1) of the last axis.
 *  - Every tensor pointer must be 16-byte aligned (token ids: 4 bytes); the
 *    scan state and every workspace must be 256-byte aligned.  A misaligned
 *    pointer returns ARP_ERR_ALIGNMENT with nothing launched.
 *  - stream is a hipStream_t (NULL: the default stream).  Work is enqueued
 *    asynchronously; nothing is synchronised; no host memory is touched.
 *  - The library allocates nothing.  It uses two caller-provided buffers:
 *      scan_state (arp_scan_state_bytes): the look-back status words of the
 *        angle scan.  Zero-fill it once before its first use and never write
 *        to it afterwards: each scan leaves it ready for the next one (it
 *        keeps two halves and alternates between them), so one buffer serves
 *        any number of calls and problem sizes, as long as each call's
 *        arp_scan_state_bytes fits in it.
 *      workspace (arp_workspace_bytes): the rotated bf16 keys (and values)
 *        of the pre-rotation path; no initialisation needed.
 *    Calls that share a buffer must be ordered (same stream).
 *  - Arguments are validated on the host before anything is enqueued; an
 *    error code means nothing was launched.  ARP_ERR_HIP reports a failed
 *    launch; faults inside kernels surface at the caller's next sync.
 */
#ifndef ARP_H
#define ARP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ARP_ABI_VERSION 2

typedef enum arp_status {
  ARP_OK = 0,
  ARP_ERR_INVALID_ARG = 1, /* null desc/pointer, bad size, odd head_dim, unknown flag or dtype */
  ARP_ERR_UNSUPPORTED = 2, /* well-formed but not built: head_dim other than 64 or 128 */
  ARP_ERR_ALIGNMENT = 3,   /* a tensor pointer is not 16-byte aligned, or a scan
                              state or workspace not 256-byte aligned */
  ARP_ERR_WORKSPACE = 4,   /* scan state or workspace null or smaller than required */
  ARP_ERR_HIP = 5,         /* a kernel launch failed */
  ARP_ERR_SCRATCH = 6      /* arp_forward_noalloc: the problem exceeds its scratch */
} arp_status;

typedef enum arp_dtype {
  ARP_DTYPE_F32 = 0,  /* fp32 I/O, fp32 arithmetic throughout */
  ARP_DTYPE_BF16 = 1  /* bf16 I/O, bf16 matrix-core products, fp32 accumulation */
} arp_dtype;

/* Flags (arp_desc.flags). */
#define ARP_ROTATE_QK 0x1u        /* rotate q and k by R(Theta_t) */
#define ARP_ROTATE_V 0x2u         /* value transport (eq. (4)): rotate v, un-rotate o */
#define ARP_ALIBI 0x4u            /* add the distance bias -m_h (i - j) to every score */
#define ARP_PHI_SHARED_HEADS 0x8u /* phi/theta have one head shared by all heads */
#define ARP_SCAN_EXCLUSIVE 0x10u  /* Theta_t = sum_{s<t} phi_s (route steps j..i-1) */
#define ARP_FUSED_ROTATION 0x20u  /* bf16: rotate k/v while staging tiles in LDS
                                     instead of a separate pre-rotation pass */
#define ARP_FORGET_GATE 0x40u     /* add the forget-gate bias sum_{s=j+1}^{i} log f_s (bf16,
                                     pre-rotation path; arp_forward_ex,
                                     arp_backward_ex and the _ex decode calls) */
#define ARP_HEAD_SCALE 0x80u      /* multiply head h's queries by head_scale[h] (AdaScale) */
#define ARP_ALL_FLAGS 0xFFu

typedef struct arp_desc {
  int32_t batch;
  int32_t heads;
  int32_t seqlen;
  int32_t head_dim;  /* even; 64 or 128 are built */
  int32_t dtype;     /* arp_dtype of q, k, v, o */
  uint32_t flags;    /* ARP_* flags above */
  float scale;       /* logit scale; <= 0 selects 1/sqrt(head_dim) */
  int32_t reserved;  /* must be 0 */
  /* With ARP_HEAD_SCALE: device float32 [heads], 16-byte aligned, each head's
   * query multiplier lambda_h -- AdaScale's per-head, length-aware inverse
   * temperature ("AdaRoPE: Not All Attention Heads Should Rotate and Scale
   * Equally", Sec. 3.3; arp_adascale_lambda computes it), applied to the
   * query only (q_i <- lambda_h q_i, same section and Sec. 3.4), so the logit
   * is lambda_h * scale * <q~_i, k~_j>; keys, values and caches are
   * unchanged.  Every attention entry point honours it (forward, training,
   * backward, decode; arp_rotate and the angle scans do not read it).
   * Without the flag it must be NULL (ARP_ERR_INVALID_ARG otherwise). */
  const float* head_scale;
} arp_desc;

/* ARP_ABI_VERSION of the loaded library. */
int arp_abi_version(void);

/* Static, never-NULL description of a status code. */
const char* arp_status_string(int status);

/* Host-only validation of a descriptor (no launch; head_scale is checked for
 * presence and alignment only, never dereferenced). */
arp_status arp_check(const arp_desc* desc);

/* Host-only: AdaScale's inverse temperatures ("AdaRoPE", Sec. 3.3)
 *   lambda[h] = (1 / tau[h]) * [ln(1 + max(L, L_ref) / L_ref)]^gamma[h]
 * for h < heads, evaluated in fp64 and rounded once to fp32; L is the context
 * length the queries attend over (seqlen for a whole-sequence pass), L_ref the
 * reference length.  tau, gamma, lambda are HOST arrays of heads floats.
 * ARP_ERR_INVALID_ARG for heads < 1, L < 1, L_ref < 1, a NULL array, or a
 * tau that is not finite and positive.  Copy the result to the device and
 * pass it as arp_desc.head_scale.  The scale is a constant of the library's
 * calls: a caller training tau and gamma gets dL/dlambda_h =
 * (1 / lambda_h) sum_{b,i} <dL/dq_{b,h,i}, q_{b,h,i}> from arp_backward's dq. */
arp_status arp_adascale_lambda(int32_t heads, const float* tau, const float* gamma, int64_t L,
                               int64_t L_ref, float* lambda);

/* Bytes of the angle scan's look-back state for desc (0 when desc is invalid).
 * The state must be zero before first use; every call leaves it ready for the next. */
size_t arp_scan_state_bytes(const arp_desc* desc);

/* Bytes of the operand workspace for desc: the rotated bf16 k~ (and v~ with
 * ARP_ROTATE_V) of the pre-rotation path, per-tile key-norm maxima, and with
 * ARP_FORGET_GATE the gate prefix and its tile bases and chunk totals; 0 for
 * fp32 I/O or ARP_FUSED_ROTATION (and when desc is invalid). */
size_t arp_workspace_bytes(const arp_desc* desc);

/* a1. Accumulated angles: theta[b,g,t,p] = wrap(sum_{s<=t} phi[b,g,s,p]) in
 * [-pi, pi) (exclusive sum with ARP_SCAN_EXCLUSIVE).  Each fp32 step is
 * converted to 48-bit fixed-point turns and summed exactly as integers (the
 * wrap is the integer overflow), single pass with chained look-back across
 * chunks of the sequence; each output is the correctly rounded fp32 of a sum
 * within 2^-48 turn of the exact one.  Method: Sec. 5 "SO(2) notation" and
 * eq. (6). */
arp_status arp_angle_scan(const arp_desc* desc, const float* phi, float* theta, void* scan_state,
                          size_t scan_state_bytes, void* stream);

/* a1 with the step angles generated inside the kernel instead of read from a
 * phi tensor (the theta written is bit-identical to arp_angle_scan's on the
 * phi the generator defines; same flags and errors as arp_angle_scan, and the
 * same scan state where one is taken).  Angle heads: 1 with
 * ARP_PHI_SHARED_HEADS, else heads.
 *
 * arp_angle_scan_random: the method paper's random variant (App. D "Model
 *   variants": steps independent per position and pair, uniform on
 *   (-f_b, f_b), redrawn every forward pass, shared by the heads of a layer).
 *   bound: float32 [angle heads, head_dim/2] device, the f_b (RoPE's
 *   10000^(-2b/d) in the paper).  seed keys the draws, step numbers them (pass
 *   a new step per forward pass).  Definition: one Philox4x64-10 block
 *   (Salmon et al., SC 2011; key (seed, 0), counter (c, step, 0, 0)) per two
 *   positions 2m, 2m+1 and four pairs 4j..4j+3 of one (b, g), with
 *   c = ((b * angle_heads + g) * ceil(seqlen / 2) + m) * (head_dim / 8) + j;
 *   word p % 4 serves pair p, its low 32 bits position 2m and its high 32 bits
 *   position 2m+1; bits w give phi = bound[g][p] * (2 w 2^-32 - 1), in fp64,
 *   rounded once to fp32.
 * arp_angle_scan_tokens: the learned token-rotation variant (same section: an
 *   angle vector per token identity), phi[b, g, t, p] = table[tokens[b, t], g, p].
 *   tokens: int32 [batch, seqlen] device (4-byte aligned), ids outside
 *   [0, vocab) are clamped into it; table: float32 [vocab, angle heads,
 *   head_dim/2] device.
 * arp_angle_scan_const: position-independent steps, phi[b, g, t, p] =
 *   freq[g, p] (RoPE: 10000^(-2p/d); AdaRoPE's per-head learned frequencies,
 *   AdaRoPE Sec. 3.3, AdaFreq): theta_t = (t + 1) freq, wrapped (t freq with
 *   ARP_SCAN_EXCLUSIVE), formed directly as an integer multiple of the
 *   fixed-point step, without a scan or its state.  freq: float32
 *   [angle heads, head_dim/2] device. */
arp_status arp_angle_scan_random(const arp_desc* desc, uint64_t seed, uint64_t step,
                                 const float* bound, float* theta, void* scan_state,
                                 size_t scan_state_bytes, void* stream);
arp_status arp_angle_scan_tokens(const arp_desc* desc, const int32_t* tokens, const float* table,
                                 int64_t vocab, float* theta, void* scan_state,
                                 size_t scan_state_bytes, void* stream);
arp_status arp_angle_scan_const(const arp_desc* desc, const float* freq, float* theta,
                                void* stream);

/* The random variant's steps written out: phi float32 [batch, angle heads,
 * seqlen, head_dim/2] device, exactly the phi arp_angle_scan_random scans
 * (same seed, step, bound).  For callers that need the draws themselves. */
arp_status arp_random_phi(const arp_desc* desc, uint64_t seed, uint64_t step, const float* bound,
                          float* phi, void* stream);

/* a2 for keys and values (bf16 pre-rotation pass): writes R(Theta_t) k_t (or
 * k_t without ARP_ROTATE_QK) and, with ARP_ROTATE_V, R(Theta_t) v_t as bf16
 * into the workspace, with each 64-key tile's largest |k~|, in the layout
 * arp_attn_rotated reads.  v is read (and required) only with ARP_ROTATE_V.
 * The queries are rotated by arp_attn_rotated itself.
 * Method: AdaRoPE Sec. 2.1 eq. (1); RoPE post, rope(). */
arp_status arp_rotate_kv(const arp_desc* desc, const void* k, const void* v, const float* theta,
                         void* workspace, size_t workspace_bytes, void* stream);

/* a1 and a2 for keys in one launch: the angle scan (as arp_angle_scan) with
 * the pre-rotation pass of arp_rotate_kv in its epilogue -- the threads that
 * produce a token's angles rotate that token's k (and v) rows for every head
 * of the angle stream, so the angles are not read back.  theta and the
 * workspace receive exactly what arp_angle_scan then arp_rotate_kv write (bit
 * for bit).  bf16 pre-rotation path only (ARP_ERR_UNSUPPORTED for fp32 I/O or
 * ARP_FUSED_ROTATION); v is read (and required) only with ARP_ROTATE_V.
 * Method: AdaRoPE Sec. 2.1 eq. (1) applied to the accumulated angles of
 * "Why Do Accumulated Transformations Extrapolate?" eq. (7). */
arp_status arp_angle_scan_rotate_kv(const arp_desc* desc, const float* phi, const void* k,
                                    const void* v, float* theta, void* scan_state,
                                    size_t scan_state_bytes, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* a2 for the queries, then a3-a6, over the keys (and transported values) that
 * arp_rotate_kv left in the workspace (bf16): q (the caller's, [batch, heads,
 * seqlen, head_dim]) rotated by R(Theta_i) and multiplied by the logit scale
 * in the kernel's prologue; scores, causal mask, distance bias, online
 * softmax, P V, and the value-transport epilogue o_i = R(Theta_i)^T o~_i.
 * Without ARP_ROTATE_V the values are the caller's v, read here (and
 * required); with it, v~ from the workspace (v may be NULL).  Method: eq.
 * (2)-(4), (8), (11).  theta is read with ARP_ROTATE_QK or ARP_ROTATE_V,
 * alibi with ARP_ALIBI.  The bf16 kernels take sin/cos from the hardware's
 * sine and cosine of turns: angles are expected as the scan writes them, in
 * [-pi, pi) (absolute error below 3e-7 there; it grows with |theta|). */
arp_status arp_attn_rotated(const arp_desc* desc, const void* q, const void* v, const float* theta,
                            const float* alibi, void* o, void* workspace, size_t workspace_bytes,
                            void* stream);

/* a2-a6: attention given accumulated angles.  bf16: arp_rotate_kv then
 * arp_attn_rotated, or one kernel that rotates while staging with
 * ARP_FUSED_ROTATION.  fp32: one kernel, rotation fused into staging. */
arp_status arp_attn_fwd(const arp_desc* desc, const void* q, const void* k, const void* v,
                        const float* theta, const float* alibi, void* o, void* workspace,
                        size_t workspace_bytes, void* stream);

/* a1-a6: the whole forward pass, (q, k, v, phi, flags) -> o.  theta receives
 * the accumulated angles (caller-owned, same layout as phi). */
arp_status arp_forward(const arp_desc* desc, const void* q, const void* k, const void* v,
                       const float* phi, const float* alibi, float* theta, void* o,
                       void* scan_state, size_t scan_state_bytes, void* workspace,
                       size_t workspace_bytes, void* stream);

/* For callers that cannot allocate or pass buffers -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: arp_forward
 * with the scan state and the operand workspace in a device array the library
 * owns (one per GPU, 64 MiB, held until the process ends), so the call needs
 * nothing but the inputs and outputs and allocates nothing.  Same arguments,
 * flags, kernels and results as arp_forward (ARP_FUSED_ROTATION included).
 * Limits: arp_scan_state_bytes(desc) <= 24 MiB and arp_workspace_bytes(desc)
 * <= 40 MiB, else ARP_ERR_SCRATCH with nothing launched (the pre-rotation
 * path's operands take 2 head_dim bytes per token and head, 4 with
 * ARP_ROTATE_V: ~327 (164) thousand tokens x heads at head_dim 64, half that
 * at 128; ARP_FUSED_ROTATION and fp32 I/O need no operand workspace).  The first call on a device clears the scan-state region with a
 * kernel on its stream; every call on that GPU shares the array, so calls that
 * overlap on one GPU (different streams or threads without ordering) race. */
arp_status arp_forward_noalloc(const arp_desc* desc, const void* q, const void* k, const void* v,
                               const float* phi, const float* alibi, float* theta, void* o,
                               void* stream);

/* Training forward (bf16 pre-rotation path, or fp32 I/O): arp_forward that
 * also writes lse[b,h,i] (float32 [batch, heads, seqlen]), the base-2
 * log-sum-exp of row i's scaled logits: log2 sum_{j<=i} 2^(log2(e) s_ij).
 * The backward pass recomputes the softmax from it.  ARP_ERR_UNSUPPORTED
 * for bf16 with ARP_FUSED_ROTATION. */
arp_status arp_forward_train(const arp_desc* desc, const void* q, const void* k, const void* v,
                             const float* phi, const float* alibi, float* theta, void* o,
                             float* lse, void* scan_state, size_t scan_state_bytes,
                             void* workspace, size_t workspace_bytes, void* stream);

/* The whole forward with every option: arp_forward plus
 *  - lse (NULL, or float32 [batch, heads, seqlen]: as in arp_forward_train),
 *  - logf (required with ARP_FORGET_GATE, else ignored): float32
 *    [batch, heads, seqlen] log forget gates log f_t; score (i, j) gets
 *    sum_{s=j+1}^{i} log f_s, the route's product of gates outside the
 *    exponential (the PaTH reading notes' Sec. 2.5; named as far-mass control
 *    beside the distance bias in Sec. 4 of the method paper).  Gates are at
 *    most 1: values log f_t > 0 are taken as 0.
 * bf16 with the pre-rotation path only (ARP_ERR_UNSUPPORTED otherwise); every
 * other entry point but arp_backward_ex, arp_decode_prefill_ex and
 * arp_decode_step_ex returns ARP_ERR_INVALID_ARG when ARP_FORGET_GATE is set. */
arp_status arp_forward_ex(const arp_desc* desc, const void* q, const void* k, const void* v,
                          const float* phi, const float* alibi, const float* logf, float* theta,
                          void* o, float* lse, void* scan_state, size_t scan_state_bytes,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the backward workspace for desc (0 for an invalid desc or fp32
 * with forget gates): the operands of the gradient kernels (rotated q scaled
 * by scale*log2(e), k, v and the rotated upstream gradient; bf16 row-major
 * and transposed, or fp32 row-major for fp32 I/O), per-row statistics, the
 * reverse scan's chunk totals and, with forget gates, the gate prefix and
 * the dS sums.  No initialisation needed. */
size_t arp_backward_workspace_bytes(const arp_desc* desc);

/* Gradients: given the forward's inputs, theta, o and lse (from
 * arp_forward_train, same desc) and the upstream gradient dout = dL/do
 * ([batch, heads, seqlen, head_dim], the dtype of q), writes
 *   dq, dk, dv  [batch, heads, seqlen, head_dim], the dtype of q
 *   dtheta      float32 [batch, heads, seqlen, head_dim/2]: dL/dTheta per head
 *   dphi        float32, phi's layout: dL/dphi_s = sum over t >= s (t > s with
 *               ARP_SCAN_EXCLUSIVE) of dL/dTheta_t, summed over the heads that
 *               share an angle stream.
 * The chain rule through eq. (2)-(4), (6)-(8) and the rotation AdaRoPE
 * Sec. 2.1 eq. (1) defines (dR/da = R J, J = [[0,-1],[1,0]]); the wrap into
 * [-pi, pi) has derivative 1.  The ALiBi slopes and the scale are constants.
 * bf16: matrix-core kernels; fp32 I/O: fp32 FMAs throughout (the workspace
 * then holds fp32 operands).  ARP_FUSED_ROTATION is ignored. */
arp_status arp_backward(const arp_desc* desc, const void* q, const void* k, const void* v,
                        const float* theta, const float* alibi, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, float* dtheta,
                        float* dphi, void* workspace, size_t workspace_bytes, void* stream);

/* arp_backward with the forget gates (ARP_FORGET_GATE; logf and dlogf are
 * then required, else ignored): o and lse from arp_forward_ex with the same
 * desc and logf (float32 [batch, heads, seqlen]); additionally writes
 *   dlogf       float32 [batch, heads, seqlen]: dL/d(log f_s).
 * Score (i, j) holds log f_s for j < s <= i (the PaTH reading notes' Sec. 2.5),
 * so dlogf_s = sum_{i >= s} sum_{j < s} dS_ij with dS_ij = dL/ds_ij.  It is
 * formed as sum_{t < s} (c_t - r_t) from the column sums c_t = sum_i dS_it and
 * the row sums r_t = sum_j dS_tj of the computed dS, an identity for any
 * lower-triangular matrix (the rows of the exact dS also sum to zero).  Gates
 * above 1 are taken as 1 by the forward, so dlogf_s = 0 where log f_s > 0.
 * The workspace (arp_backward_workspace_bytes with the flag set) also holds
 * the gate prefix and the dS sums.  Gates are bf16 only (ARP_ERR_UNSUPPORTED
 * for fp32 I/O).  Without the flag this is arp_backward. */
arp_status arp_backward_ex(const arp_desc* desc, const void* q, const void* k, const void* v,
                           const float* theta, const float* alibi, const float* logf, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* dtheta, float* dphi, float* dlogf, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ---- decode: one new token per sequence against a key/value cache ----
 * desc.seqlen is the cache capacity Lmax; bf16 only.  Caches hold the keys and
 * values already rotated by their own accumulated angles, bf16
 * [batch, heads, Lmax, head_dim]: a token's rotation never changes once it is
 * written, since the route from j to i is R(Theta_j - Theta_i) (eq. (6)-(8),
 * Sec. 5), applied through the query's rotation.  The angle state is
 * uint64 [batch, phi_heads, head_dim/2]: the running sum of the steps in
 * 48-bit fixed-point turns (plus half a turn), the arithmetic of
 * arp_angle_scan, so decoded angles are bit-identical to a full scan's. */

/* Bytes of the decode step's workspace (partial results of the split-key
 * attention) for a cache of desc.seqlen tokens; 0 unless bf16. */
size_t arp_decode_workspace_bytes(const arp_desc* desc);

/* Fill cache rows [0, len) from a prompt and set the state after len tokens.
 * k, v: [batch, heads, len, head_dim] (raw); phi, theta: [batch, phi_heads,
 * len, head_dim/2], theta from arp_angle_scan (or arp_forward) over the same
 * len tokens.  len = 0 only resets the state (k, v, phi, theta may be NULL). */
arp_status arp_decode_prefill(const arp_desc* desc, int32_t len, const void* k, const void* v,
                              const float* phi, const float* theta, void* kcache, void* vcache,
                              uint64_t* state, void* stream);

/* One decode step at position pos (0 <= pos < Lmax, the same for every
 * sequence; rows 0..pos-1 of the caches filled): q, k, v [batch, heads,
 * head_dim] and phi [batch, phi_heads, head_dim/2] are the new token's.
 * Advances the state, writes the token's wrapped angles to theta
 * [batch, phi_heads, head_dim/2], appends its rotated k, v at row pos, and
 * writes o [batch, heads, head_dim]: causal attention of the token over rows
 * 0..pos, with the flags' rotation, distance bias and value transport --
 * the row pos of arp_forward over the whole sequence. */
arp_status arp_decode_step(const arp_desc* desc, int32_t pos, const void* q, const void* k,
                           const void* v, const float* phi, const float* alibi, uint64_t* state,
                           float* theta, void* kcache, void* vcache, void* o, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Decode with forget gates (ARP_FORGET_GATE; without it these are
 * arp_decode_prefill and arp_decode_step).  Two more caller-owned buffers:
 *   gcache  double [batch, heads, Lmax]: G_j = log2(e) * sum_{s<=j} min(log f_s, 0)
 *           of each cached key (the gate prefix, in fp64 so that G_t - G_j stays
 *           exact to fp32 rounding however long the context),
 *   gstate  double [batch, heads]: sum_{s<t} min(log f_s, 0) of the tokens so
 *           far, in fp64.
 * prefill_ex takes the prompt's gates logf float32 [batch, heads, len] (NULL
 * when len = 0) and sets gcache rows [0, len) and gstate; step_ex takes the
 * new token's logf float32 [batch, heads], adds G_t - G_j to the score of
 * every cached key j (the route's product of gates outside the exponential,
 * the PaTH reading notes' Sec. 2.5), appends G_t and advances gstate: the
 * row pos of arp_forward_ex over the whole sequence with the same gates.
 * Gates above 1 are taken as 1.  With the flag, logf, gcache and gstate are
 * required (ARP_ERR_INVALID_ARG) and 16-byte aligned (ARP_ERR_ALIGNMENT). */
arp_status arp_decode_prefill_ex(const arp_desc* desc, int32_t len, const void* k, const void* v,
                                 const float* phi, const float* theta, const float* logf,
                                 void* kcache, void* vcache, uint64_t* state, double* gcache,
                                 double* gstate, void* stream);
arp_status arp_decode_step_ex(const arp_desc* desc, int32_t pos, const void* q, const void* k,
                              const void* v, const float* phi, const float* alibi,
                              const float* logf, uint64_t* state, float* theta, void* kcache,
                              void* vcache, double* gcache, double* gstate, void* o,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Diagnostic: out = R(theta) x (or R(theta)^T x when inverse != 0) in fp32.
 * x has the desc's dtype and q's layout; out is float32 of the same shape. */
arp_status arp_rotate(const arp_desc* desc, const void* x, const float* theta, float* out,
                      int inverse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ARP_H */
