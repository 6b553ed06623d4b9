// arp_internal.hpp -- host-side interface between the C ABI layer (api.hip)
// and the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/arp.h"

namespace arp {

// Problem geometry derived once from a validated descriptor.
struct Geometry {
  int B, H, L, D, P;   // batch, heads, seqlen, head_dim, pairs (D/2)
  int Hphi;            // angle heads: 1 (shared) or H
  int dtype;           // arp_dtype
  uint32_t flags;
  float scale;         // resolved logit scale
  int Lp;              // seqlen padded for the pre-rotated operands (multiple of 256)
  const float* hscale; // device [H] per-head query multipliers (ARP_HEAD_SCALE), else null
};

// ---- buffers ----------------------------------------------------------------
// scan state: a 256-byte header and two interleaved halves of 64-bit
//   look-back status words, [B*Hphi][nchunks][P] per half (angle_scan.hip).
// workspace:  [ k~ (bf16, [B*H, Lp, D]) | v~ (bf16, [B*H, Lp, D], with ARP_ROTATE_V only)
//               | kmax (fp32, [B*H, Lp/64]) | gate prefix (ARP_FORGET_GATE) ]
//   for bf16 without ARP_FUSED_ROTATION; empty otherwise.
struct ScanPlan {
  int rows_per_thread;  // tokens each thread scans serially (T)
  int min_blocks;       // workgroups per CU the kernel is built for (launch bounds)
  int chunk;            // tokens per workgroup
  int nchunks;          // chunks per (batch, angle head) segment
};
// rotating: the plan of the scan with the key rotation in its epilogue
// (chunks that hold whole 64-key tiles)
ScanPlan scan_plan(const Geometry& g, bool rotating = false);
size_t scan_state_bytes(const Geometry& g);  // upper bound over every plan
struct WorkspaceLayout {
  size_t k_off, v_off, operand_bytes;          // each operand block (v~ only with ARP_ROTATE_V)
  size_t kmax_off;                             // float [B*H][Lp/64]: max |k~| per key tile
  size_t gate_off;                             // float [B*H][Lp]: gate prefix within its
                                               //   64-token tile (ARP_FORGET_GATE)
  size_t gate_base_off;                        // double [B*H][Lp/64]: the prefix before each tile
  size_t gate_tot_off;                         // double [B*H][gate_chunks]: chunk totals
  size_t total;
};
constexpr int KEY_TILE = 64;  // keys per tile of the attention kernel (and per kmax entry)
WorkspaceLayout workspace_layout(const Geometry& g);

// ---- launchers (enqueue only; return hipSuccess or the launch error) -------
hipError_t launch_angle_scan(const Geometry& g, const float* phi, float* theta, void* scan_state,
                             hipStream_t stream);
// The scan with its step angles generated in the kernel: the random
// variant's uniform draws (Philox4x64-10 keyed by seed, draw number step;
// bound [Hphi, P]) or a learned per-token table (tokens [B, L], table
// [vocab, Hphi, P]); constant per-pair frequencies (freq [Hphi, P]) in
// closed form, without a scan.
hipError_t launch_angle_scan_random(const Geometry& g, uint64_t seed, uint64_t step,
                                    const float* bound, float* theta, void* scan_state,
                                    hipStream_t stream);
hipError_t launch_angle_scan_tokens(const Geometry& g, const int32_t* tokens, const float* table,
                                    int vocab, float* theta, void* scan_state, hipStream_t stream);
hipError_t launch_angle_scan_const(const Geometry& g, const float* freq, float* theta,
                                   hipStream_t stream);
// The random draws written out as phi [B, Hphi, L, P].
hipError_t launch_random_phi(const Geometry& g, uint64_t seed, uint64_t step, const float* bound,
                             float* phi, hipStream_t stream);
// The angle scan with the pre-rotation pass in its epilogue: each scan
// thread rotates the k (and v) rows of the angles it has just produced, so
// the angles are not read back and one launch is saved.  Same outputs, bit
// for bit, as launch_angle_scan then launch_rotate_kv (which it falls back to
// when the scan's chunks do not cover whole 64-key tiles).
struct KeyRotation {
  const void* k;
  const void* v;   // read with ARP_ROTATE_V only
  uint16_t* kr;    // k~ [B*H, Lp, D] (rows past L written as zeros)
  uint16_t* vr;    // v~ [B*H, Lp, D] with ARP_ROTATE_V, else NULL
  float* kmax;     // [B*H, Lp/64]: the largest |k~| of each 64-key tile
};
hipError_t launch_angle_scan_rotate(const Geometry& g, const float* phi, float* theta,
                                    void* scan_state, const KeyRotation& rot, hipStream_t stream);
// k~ (and v~ with ARP_ROTATE_V) into the workspace, with the key-norm maxima
hipError_t launch_rotate_kv(const Geometry& g, const void* k, const void* v, const float* theta,
                            uint16_t* kr, uint16_t* vr, float* kmax, hipStream_t stream);
// q: the caller's raw q (rotated in the kernel's prologue); v: V rows, vrows
// per head (the workspace's v~ with vrows = Lp, or the caller's v with L)
hipError_t launch_attn_bf16_rotated(const Geometry& g, const uint16_t* q, const uint16_t* kr,
                                    const uint16_t* v, int vrows, const float* kmax,
                                    const float* theta, const float* alibi, const float* gate2,
                                    const double* gbase, uint16_t* o, float* lse,
                                    hipStream_t stream);
// Forget gates: with G_t = log2 e * sum_{s <= t} min(logf[b, h, s], 0) (fp64
// accumulation; padded to Lp with the last value), the prefix is kept relative
// to 64-token tiles so that it stays exact however long the sequence:
//   gbase[b*H + h][c] = G_{64c - 1} (0 for c = 0), double
//   gate2[b*H + h][t] = fp32(G_t - gbase[t / 64])   (|.| <= 64 max|log f| log2 e)
// and a logit's bias G_i - G_j = fp32(gbase[i/64] - gbase[j/64]) + gate2[i] -
// gate2[j], the tile difference rounded once.  totals holds one double per
// (b*H + h, chunk of GATE_CHUNK tokens).
constexpr int GATE_CHUNK = 1024;
constexpr int GATE_TILE = 64;
inline int gate_chunks(const Geometry& g) { return (g.Lp + GATE_CHUNK - 1) / GATE_CHUNK; }
hipError_t launch_gate_scan(const Geometry& g, const float* logf, float* gate2, double* gbase,
                            double* totals, hipStream_t stream);
hipError_t launch_attn_bf16_fused(const Geometry& g, const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, const float* theta, const float* alibi,
                                  uint16_t* o, hipStream_t stream);
// lse (nullable): [B, H, L] base-2 log-sum-exp of each row's scaled logits
// Compute units of the current device (queried on every call: launches size
// their grids by it; 256 if the query fails).
inline int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

hipError_t launch_attn_f32(const Geometry& g, const float* q, const float* k, const float* v,
                           const float* theta, const float* alibi, float* o, float* lse,
                           hipStream_t stream);
hipError_t launch_rotate_diag(const Geometry& g, const void* x, const float* theta, float* out,
                              int inverse, hipStream_t stream);

// ---- backward (bf16) --------------------------------------------------------
// Operands the gradient kernels read, in the backward workspace (per head):
//   qs, k, v, dout   bf16 [B*H, Lp, D]: q~ * scale * log2 e, k~, v~, do~
//   qsT, kT, doutT   bf16 [B*H, D, Lp]: transposes of qs, k, dout
//   stats            fp32 [B*H, Lp/64, 128]: per 64-row tile, -lse (-inf past L)
//                    then -D = -<do~, o~> (0 past L), negated for the MFMA
//                    accumulator input
struct BwdOperands {
  uint16_t* qs;
  uint16_t* qsT;
  uint16_t* k;
  uint16_t* kT;
  uint16_t* v;
  uint16_t* dout;
  uint16_t* doutT;
  float* stats;
  float* tstat;  // per 64-token tile: max |q~ scale log2 e|, max |k~|, max_i (-lse_i - slope2 i), 0
  // forget gates only (else null): the gate prefix in the forward's tiled
  // form (gate2 fp32 [B*H, Lp] within each 64-token tile, gbase double
  // [B*H, Lp/64] the prefix before each tile), and fp32 [B*H, Lp] the sums of
  // dS over each key's column and over each query's row
  const float* gate2;
  float* colsum;
  float* rowsum;
  const double* gbase;
};
struct BwdArgs {
  const uint16_t *q, *k, *v, *o, *dout;  // caller tensors [B, H, L, D]
  const float *theta, *lse, *alibi;
  uint16_t *dq, *dk, *dv;                // caller gradients [B, H, L, D]
  float* dtheta;                         // caller [B, H, L, P]
  float* dphi;                           // caller [B, Hphi, L, P]
  float* totals;                         // workspace [B*Hphi, ceil(L/256), P]
  const float* logf;                     // caller [B, H, L] log forget gates (gated only)
  float* dlogf;                          // caller [B, H, L] out: dL/d(log f) (gated only)
  double* gate_tot;                      // workspace [B*H, gate_chunks] (gated only)
  BwdOperands ops;
};
struct BwdWorkspaceLayout {
  size_t operand_bytes;  // one bf16 [B*H, Lp, D] block
  size_t stats_off, tstat_off, totals_off;
  size_t gate_off, gate_base_off, gate_tot_off, colsum_off, rowsum_off;  // gated only
  size_t total;
};
BwdWorkspaceLayout bwd_workspace_layout(const Geometry& g);
hipError_t launch_backward_bf16(const Geometry& g, const BwdArgs& a, hipStream_t stream);

// fp32 I/O backward (plain FMAs; no forget gates)
struct BwdF32Args {
  const float *q, *k, *v, *o, *dout;  // caller tensors [B, H, L, D]
  const float *theta, *lse, *alibi;
  float *dq, *dk, *dv;                 // caller gradients [B, H, L, D]
  float* dtheta;                       // caller [B, H, L, P]
  float* dphi;                         // caller [B, Hphi, L, P]
  float* totals;                       // workspace [B*Hphi, ceil(L/256), P]
  float *qs, *kr, *vr, *dor;           // workspace [B*H, L, D]: q~ scale log2 e, k~, v~, do~
  float *nl, *nd;                      // workspace [B*H, L]: -lse, -D
};
hipError_t launch_backward_f32(const Geometry& g, const BwdF32Args& a, hipStream_t stream);

// ---- decode (bf16; Geometry.L is the cache capacity) ------------------------
struct DecodeArgs {
  int pos;                      // position of the new token (cache rows 0..pos attended)
  const uint16_t *q, *k, *v;    // [B, H, D] the new token
  const float *phi, *alibi;     // phi [B, Hphi, P] the new token's steps
  uint64_t* state;              // [B, Hphi, P] angle sums, 48-bit turns + 2^47
  float* theta;                 // [B, Hphi, P] out: the new token's angles
  uint16_t *kcache, *vcache;    // [B, H, L, D] pre-rotated k~, v~
  uint16_t* o;                  // [B, H, D]
  float* part;                  // workspace: [B*H, ceil(L/256), D + 2] partial results
  const float* logf;            // [B, H] the new token's log forget gate (gated only)
  double* gcache;               // [B, H, L] gate prefixes G_j of the cached keys (gated only)
  double* gstate;               // [B, H] running sum of min(log f, 0) (gated only)
};
size_t decode_workspace_bytes(const Geometry& g);
hipError_t launch_decode_prefill(const Geometry& g, int len, const uint16_t* k, const uint16_t* v,
                                 const float* phi, const float* theta, uint16_t* kcache,
                                 uint16_t* vcache, uint64_t* state, const float* logf,
                                 double* gcache, double* gstate, hipStream_t stream);
hipError_t launch_decode_step(const Geometry& g, const DecodeArgs& a, hipStream_t stream);

}  // namespace arp
