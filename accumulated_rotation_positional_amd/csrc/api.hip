// api.hip -- the C ABI of libarp.so (declared in include/arp.h).
//
// Host side only: validate the descriptor and pointers, derive the problem
// geometry, carve the caller's workspace, and enqueue kernels on the caller's
// stream.  Nothing here allocates, synchronises, or touches device memory
// from the host.
#include <math.h>
#include <string.h>

#include <mutex>

#include "arp_internal.hpp"

namespace arp {

namespace {

constexpr size_t ALIGN = 256;
size_t align_up(size_t x) { return (x + ALIGN - 1) & ~(ALIGN - 1); }

bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

arp_status make_geometry(const arp_desc* d, Geometry* g) {
  if (d == nullptr) return ARP_ERR_INVALID_ARG;
  if (d->batch <= 0 || d->heads <= 0 || d->seqlen <= 0 || d->head_dim <= 0) return ARP_ERR_INVALID_ARG;
  if (d->head_dim % 2 != 0) return ARP_ERR_INVALID_ARG;
  if (d->dtype != ARP_DTYPE_F32 && d->dtype != ARP_DTYPE_BF16) return ARP_ERR_INVALID_ARG;
  if ((d->flags & ~ARP_ALL_FLAGS) != 0u) return ARP_ERR_INVALID_ARG;
  if (d->reserved != 0) return ARP_ERR_INVALID_ARG;
  if (!(d->scale == d->scale) || isinf(d->scale)) return ARP_ERR_INVALID_ARG;
  // Sizes: every tensor index must fit comfortably in 64 bits and the grids in
  // their limits; the sequence is capped at 2^24 tokens.
  if (d->seqlen > (1 << 24) || (long long)d->batch * d->heads > 65535) return ARP_ERR_INVALID_ARG;
  if (((d->flags & ARP_HEAD_SCALE) != 0) != (d->head_scale != nullptr)) return ARP_ERR_INVALID_ARG;
  if (d->head_scale != nullptr && ((uintptr_t)d->head_scale & 15u) != 0) return ARP_ERR_ALIGNMENT;
  if (d->head_dim != 64 && d->head_dim != 128) return ARP_ERR_UNSUPPORTED;
  g->B = d->batch;
  g->H = d->heads;
  g->L = d->seqlen;
  g->D = d->head_dim;
  g->P = d->head_dim / 2;
  g->Hphi = (d->flags & ARP_PHI_SHARED_HEADS) ? 1 : d->heads;
  g->dtype = d->dtype;
  g->flags = d->flags;
  g->scale = d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)d->head_dim);
  g->Lp = (int)(((long long)d->seqlen + 255) / 256 * 256);
  g->hscale = d->head_scale;
  return ARP_OK;
}

bool needs_operands(const Geometry& g) {
  return g.dtype == ARP_DTYPE_BF16 && !(g.flags & ARP_FUSED_ROTATION);
}

arp_status check_buffer(const void* p, size_t have, size_t need) {
  if (need == 0) return ARP_OK;
  if (p == nullptr || have < need) return ARP_ERR_WORKSPACE;
  if (((uintptr_t)p & (ALIGN - 1)) != 0) return ARP_ERR_ALIGNMENT;
  return ARP_OK;
}
arp_status check_ws(const Geometry& g, const void* ws, size_t bytes) {
  return check_buffer(ws, bytes, workspace_layout(g).total);
}
arp_status check_scan_state(const Geometry& g, const void* st, size_t bytes) {
  return check_buffer(st, bytes, align_up(scan_state_bytes(g)));
}

arp_status hip_status(hipError_t e) { return e == hipSuccess ? ARP_OK : ARP_ERR_HIP; }
arp_status fused_status(hipError_t e) {
  return e == hipErrorNotSupported ? ARP_ERR_UNSUPPORTED : hip_status(e);
}

bool rotates(const Geometry& g) { return (g.flags & (ARP_ROTATE_QK | ARP_ROTATE_V)) != 0; }
bool gated(const Geometry& g) { return (g.flags & ARP_FORGET_GATE) != 0; }

}  // namespace

namespace {

// The pre-rotation path's two launches over a carved workspace: k~ (and v~
// with value transport), then the attention kernel, which rotates q itself
// and reads V rows from v~ or, without value transport, the caller's v.
hipError_t launch_rotation_pass(const Geometry& g, const void* k, const void* v,
                                const float* theta, char* ws, hipStream_t s) {
  const WorkspaceLayout lay = workspace_layout(g);
  return launch_rotate_kv(g, k, v, theta, reinterpret_cast<uint16_t*>(ws + lay.k_off),
                          (g.flags & ARP_ROTATE_V) ? reinterpret_cast<uint16_t*>(ws + lay.v_off)
                                                   : nullptr,
                          reinterpret_cast<float*>(ws + lay.kmax_off), s);
}

// a1 and the pre-rotation pass in one launch (the bf16 pre-rotation path)
hipError_t launch_scan_and_rotation(const Geometry& g, const float* phi, float* theta,
                                    void* scan_state, const void* k, const void* v, char* ws,
                                    hipStream_t s) {
  const WorkspaceLayout lay = workspace_layout(g);
  const KeyRotation kr{k, v, reinterpret_cast<uint16_t*>(ws + lay.k_off),
                       (g.flags & ARP_ROTATE_V) ? reinterpret_cast<uint16_t*>(ws + lay.v_off)
                                                : nullptr,
                       reinterpret_cast<float*>(ws + lay.kmax_off)};
  return launch_angle_scan_rotate(g, phi, theta, scan_state, kr, s);
}

hipError_t launch_attention(const Geometry& g, const void* q, const void* v, const float* theta,
                            const float* alibi, const float* gate2, const double* gbase, void* o,
                            float* lse, const char* ws, hipStream_t s) {
  const WorkspaceLayout lay = workspace_layout(g);
  const bool rv = (g.flags & ARP_ROTATE_V) != 0;
  const uint16_t* vrows = rv ? reinterpret_cast<const uint16_t*>(ws + lay.v_off)
                             : static_cast<const uint16_t*>(v);
  return launch_attn_bf16_rotated(g, static_cast<const uint16_t*>(q),
                                  reinterpret_cast<const uint16_t*>(ws + lay.k_off), vrows,
                                  rv ? g.Lp : g.L, reinterpret_cast<const float*>(ws + lay.kmax_off),
                                  theta, alibi, gate2, gbase, static_cast<uint16_t*>(o), lse, s);
}

}  // namespace

WorkspaceLayout workspace_layout(const Geometry& g) {
  WorkspaceLayout lay{};
  size_t off = 0;
  if (needs_operands(g)) {
    lay.operand_bytes = align_up((size_t)g.B * g.H * g.Lp * g.D * sizeof(uint16_t));
    lay.k_off = off;
    off += lay.operand_bytes;
    if (g.flags & ARP_ROTATE_V) {  // v~; without value transport the caller's v is read
      lay.v_off = off;
      off += lay.operand_bytes;
    }
    lay.kmax_off = off;
    off += align_up((size_t)g.B * g.H * (g.Lp / KEY_TILE) * sizeof(float));
    if (g.flags & ARP_FORGET_GATE) {
      lay.gate_off = off;
      off += align_up((size_t)g.B * g.H * g.Lp * sizeof(float));
      lay.gate_base_off = off;
      off += align_up((size_t)g.B * g.H * (g.Lp / GATE_TILE) * sizeof(double));
      lay.gate_tot_off = off;
      off += align_up((size_t)g.B * g.H * gate_chunks(g) * sizeof(double));
    }
  }
  lay.total = off;
  return lay;
}

BwdWorkspaceLayout bwd_workspace_layout(const Geometry& g) {
  BwdWorkspaceLayout lay{};
  if (g.dtype == ARP_DTYPE_F32) {
    // four fp32 operand blocks [B*H, L, D], then -lse and -D, then the reverse scan's totals
    lay.operand_bytes = align_up((size_t)g.B * g.H * g.L * g.D * sizeof(float));
    lay.stats_off = 4 * lay.operand_bytes;
    lay.tstat_off = lay.stats_off + align_up((size_t)g.B * g.H * g.L * 2 * sizeof(float));
    lay.totals_off = lay.tstat_off;
    const size_t nch = ((size_t)g.L + 255) / 256;
    lay.total = lay.totals_off + align_up((size_t)g.B * g.Hphi * nch * g.P * sizeof(float));
    return lay;
  }
  lay.operand_bytes = align_up((size_t)g.B * g.H * g.Lp * g.D * sizeof(uint16_t));
  lay.stats_off = 7 * lay.operand_bytes;
  lay.tstat_off = lay.stats_off + align_up((size_t)g.B * g.H * g.Lp * 2 * sizeof(float));
  lay.totals_off = lay.tstat_off + align_up((size_t)g.B * g.H * (g.Lp / KEY_TILE) * 4 * sizeof(float));
  const size_t nch = ((size_t)g.L + 255) / 256;
  size_t off = lay.totals_off + align_up((size_t)g.B * g.Hphi * nch * g.P * sizeof(float));
  if (g.flags & ARP_FORGET_GATE) {
    const size_t per_token = align_up((size_t)g.B * g.H * g.Lp * sizeof(float));
    lay.gate_off = off;
    lay.gate_base_off = off + per_token;
    lay.gate_tot_off =
        lay.gate_base_off + align_up((size_t)g.B * g.H * (g.Lp / GATE_TILE) * sizeof(double));
    off = lay.gate_tot_off + align_up((size_t)g.B * g.H * gate_chunks(g) * sizeof(double));
    lay.colsum_off = off;
    lay.rowsum_off = off + per_token;
    off += 2 * per_token;
  }
  lay.total = off;
  return lay;
}

}  // namespace arp

using namespace arp;

extern "C" {

int arp_abi_version(void) { return ARP_ABI_VERSION; }

const char* arp_status_string(int status) {
  switch (status) {
    case ARP_OK: return "ok";
    case ARP_ERR_INVALID_ARG: return "invalid argument";
    case ARP_ERR_UNSUPPORTED: return "unsupported configuration";
    case ARP_ERR_ALIGNMENT:
      return "pointer misaligned (tensors: 16 bytes; scan state and workspaces: 256 bytes)";
    case ARP_ERR_WORKSPACE: return "workspace missing or too small";
    case ARP_ERR_HIP: return "HIP launch failed";
    case ARP_ERR_SCRATCH:
      return "problem exceeds the no-alloc scratch (24 MiB scan state, 40 MiB operands)";
    default: return "unknown status";
  }
}

arp_status arp_check(const arp_desc* desc) {
  Geometry g;
  return make_geometry(desc, &g);
}

arp_status arp_adascale_lambda(int32_t heads, const float* tau, const float* gamma, int64_t L,
                               int64_t L_ref, float* lambda) {
  if (heads < 1 || L < 1 || L_ref < 1 || tau == nullptr || gamma == nullptr || lambda == nullptr)
    return ARP_ERR_INVALID_ARG;
  for (int32_t h = 0; h < heads; ++h)
    if (!(tau[h] > 0.f) || isinf(tau[h]) || !(gamma[h] == gamma[h]) || isinf(gamma[h]))
      return ARP_ERR_INVALID_ARG;
  const double len = (double)(L > L_ref ? L : L_ref);
  const double growth = log(1.0 + len / (double)L_ref);
  for (int32_t h = 0; h < heads; ++h)
    lambda[h] = (float)(pow(growth, (double)gamma[h]) / (double)tau[h]);
  return ARP_OK;
}

size_t arp_scan_state_bytes(const arp_desc* desc) {
  Geometry g;
  if (make_geometry(desc, &g) != ARP_OK) return 0;
  return align_up(scan_state_bytes(g));
}

size_t arp_workspace_bytes(const arp_desc* desc) {
  Geometry g;
  if (make_geometry(desc, &g) != ARP_OK) return 0;
  return workspace_layout(g).total;
}

arp_status arp_angle_scan(const arp_desc* desc, const float* phi, float* theta, void* scan_state,
                          size_t scan_state_bytes, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (phi == nullptr || theta == nullptr) return ARP_ERR_INVALID_ARG;
  if (!aligned16(phi) || !aligned16(theta)) return ARP_ERR_ALIGNMENT;
  if ((st = check_scan_state(g, scan_state, scan_state_bytes)) != ARP_OK) return st;
  return hip_status(launch_angle_scan(g, phi, theta, scan_state, (hipStream_t)stream));
}

arp_status arp_angle_scan_random(const arp_desc* desc, uint64_t seed, uint64_t step,
                                 const float* bound, float* theta, void* scan_state,
                                 size_t scan_state_bytes, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (bound == nullptr || theta == nullptr) return ARP_ERR_INVALID_ARG;
  if (!aligned16(bound) || !aligned16(theta)) return ARP_ERR_ALIGNMENT;
  if ((st = check_scan_state(g, scan_state, scan_state_bytes)) != ARP_OK) return st;
  return hip_status(
      launch_angle_scan_random(g, seed, step, bound, theta, scan_state, (hipStream_t)stream));
}

arp_status arp_angle_scan_tokens(const arp_desc* desc, const int32_t* tokens, const float* table,
                                 int64_t vocab, float* theta, void* scan_state,
                                 size_t scan_state_bytes, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (tokens == nullptr || table == nullptr || theta == nullptr || vocab < 1 || vocab > INT32_MAX)
    return ARP_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(tokens) & 3) != 0 || !aligned16(table) || !aligned16(theta))
    return ARP_ERR_ALIGNMENT;
  if ((st = check_scan_state(g, scan_state, scan_state_bytes)) != ARP_OK) return st;
  return hip_status(launch_angle_scan_tokens(g, tokens, table, (int)vocab, theta, scan_state,
                                             (hipStream_t)stream));
}

arp_status arp_angle_scan_const(const arp_desc* desc, const float* freq, float* theta,
                                void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (freq == nullptr || theta == nullptr) return ARP_ERR_INVALID_ARG;
  if (!aligned16(freq) || !aligned16(theta)) return ARP_ERR_ALIGNMENT;
  return hip_status(launch_angle_scan_const(g, freq, theta, (hipStream_t)stream));
}

arp_status arp_random_phi(const arp_desc* desc, uint64_t seed, uint64_t step, const float* bound,
                          float* phi, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (bound == nullptr || phi == nullptr) return ARP_ERR_INVALID_ARG;
  if (!aligned16(bound) || !aligned16(phi)) return ARP_ERR_ALIGNMENT;
  return hip_status(launch_random_phi(g, seed, step, bound, phi, (hipStream_t)stream));
}

arp_status arp_rotate_kv(const arp_desc* desc, const void* k, const void* v, const float* theta,
                         void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (gated(g)) return ARP_ERR_INVALID_ARG;  // the gate input: arp_forward_ex
  if (!needs_operands(g)) return ARP_ERR_UNSUPPORTED;
  const bool rv = (g.flags & ARP_ROTATE_V) != 0;
  if (k == nullptr || (rv && v == nullptr) || (rotates(g) && theta == nullptr))
    return ARP_ERR_INVALID_ARG;
  if (!aligned16(k) || (v && !aligned16(v)) || (theta && !aligned16(theta))) return ARP_ERR_ALIGNMENT;
  if ((st = check_ws(g, workspace, workspace_bytes)) != ARP_OK) return st;
  return hip_status(launch_rotation_pass(g, k, v, theta, static_cast<char*>(workspace),
                                         (hipStream_t)stream));
}

arp_status arp_angle_scan_rotate_kv(const arp_desc* desc, const float* phi, const void* k,
                                    const void* v, float* theta, void* scan_state,
                                    size_t scan_state_bytes, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (gated(g)) return ARP_ERR_INVALID_ARG;  // the gate input: arp_forward_ex
  if (!needs_operands(g)) return ARP_ERR_UNSUPPORTED;
  const bool rv = (g.flags & ARP_ROTATE_V) != 0;
  if (phi == nullptr || theta == nullptr || k == nullptr || (rv && v == nullptr))
    return ARP_ERR_INVALID_ARG;
  if (!aligned16(phi) || !aligned16(theta) || !aligned16(k) || (v && !aligned16(v)))
    return ARP_ERR_ALIGNMENT;
  if ((st = check_scan_state(g, scan_state, scan_state_bytes)) != ARP_OK) return st;
  if ((st = check_ws(g, workspace, workspace_bytes)) != ARP_OK) return st;
  return hip_status(launch_scan_and_rotation(g, phi, theta, scan_state, k, v,
                                             static_cast<char*>(workspace), (hipStream_t)stream));
}

arp_status arp_attn_rotated(const arp_desc* desc, const void* q, const void* v, const float* theta,
                            const float* alibi, void* o, void* workspace, size_t workspace_bytes,
                            void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (gated(g)) return ARP_ERR_INVALID_ARG;  // the gate input: arp_forward_ex
  if (!needs_operands(g)) return ARP_ERR_UNSUPPORTED;
  const bool rv = (g.flags & ARP_ROTATE_V) != 0;
  if (q == nullptr || o == nullptr || (!rv && v == nullptr) || (rotates(g) && theta == nullptr) ||
      ((g.flags & ARP_ALIBI) && alibi == nullptr))
    return ARP_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(o) || (v && !aligned16(v)) || (theta && !aligned16(theta)) ||
      (alibi && !aligned16(alibi)))
    return ARP_ERR_ALIGNMENT;
  if ((st = check_ws(g, workspace, workspace_bytes)) != ARP_OK) return st;
  return hip_status(launch_attention(g, q, v, theta, alibi, nullptr, nullptr, o, nullptr,
                                     static_cast<const char*>(workspace), (hipStream_t)stream));
}

arp_status arp_attn_fwd(const arp_desc* desc, const void* q, const void* k, const void* v,
                        const float* theta, const float* alibi, void* o, void* workspace,
                        size_t workspace_bytes, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (gated(g)) return ARP_ERR_INVALID_ARG;  // the gate input: arp_forward_ex
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr ||
      (rotates(g) && theta == nullptr) || ((g.flags & ARP_ALIBI) && alibi == nullptr))
    return ARP_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (theta && !aligned16(theta)) || (alibi && !aligned16(alibi)))
    return ARP_ERR_ALIGNMENT;
  if ((st = check_ws(g, workspace, workspace_bytes)) != ARP_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (g.dtype == ARP_DTYPE_F32)
    return hip_status(launch_attn_f32(g, static_cast<const float*>(q), static_cast<const float*>(k),
                                      static_cast<const float*>(v), theta, alibi,
                                      static_cast<float*>(o), nullptr, s));
  if (g.flags & ARP_FUSED_ROTATION)
    return fused_status(launch_attn_bf16_fused(
        g, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
        static_cast<const uint16_t*>(v), theta, alibi, static_cast<uint16_t*>(o), s));
  st = arp_rotate_kv(desc, k, v, theta, workspace, workspace_bytes, stream);
  if (st != ARP_OK) return st;
  return arp_attn_rotated(desc, q, v, theta, alibi, o, workspace, workspace_bytes, stream);
}

arp_status arp_forward(const arp_desc* desc, const void* q, const void* k, const void* v,
                       const float* phi, const float* alibi, float* theta, void* o,
                       void* scan_state, size_t scan_state_bytes, void* workspace,
                       size_t workspace_bytes, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (gated(g)) return ARP_ERR_INVALID_ARG;  // the gate input: arp_forward_ex
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || phi == nullptr ||
      theta == nullptr || ((g.flags & ARP_ALIBI) && alibi == nullptr))
    return ARP_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(phi) ||
      !aligned16(theta) || (alibi && !aligned16(alibi)))
    return ARP_ERR_ALIGNMENT;
  if ((st = check_scan_state(g, scan_state, scan_state_bytes)) != ARP_OK) return st;
  if ((st = check_ws(g, workspace, workspace_bytes)) != ARP_OK) return st;
  if (needs_operands(g)) {  // bf16 pre-rotation path: the scan rotates the keys too
    hipStream_t s = (hipStream_t)stream;
    char* ws = static_cast<char*>(workspace);
    if (launch_scan_and_rotation(g, phi, theta, scan_state, k, v, ws, s) != hipSuccess)
      return ARP_ERR_HIP;
    return hip_status(launch_attention(g, q, v, theta, alibi, nullptr, nullptr, o, nullptr, ws, s));
  }
  st = arp_angle_scan(desc, phi, theta, scan_state, scan_state_bytes, stream);
  if (st != ARP_OK) return st;
  return arp_attn_fwd(desc, q, k, v, theta, alibi, o, workspace, workspace_bytes, stream);
}

arp_status arp_forward_train(const arp_desc* desc, const void* q, const void* k, const void* v,
                             const float* phi, const float* alibi, float* theta, void* o,
                             float* lse, void* scan_state, size_t scan_state_bytes,
                             void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (gated(g)) return ARP_ERR_INVALID_ARG;  // the gate input: arp_forward_ex
  const bool f32 = g.dtype == ARP_DTYPE_F32;
  if (!needs_operands(g) && !f32) return ARP_ERR_UNSUPPORTED;  // the fused rotation
  if (lse == nullptr) return ARP_ERR_INVALID_ARG;
  if (!aligned16(lse)) return ARP_ERR_ALIGNMENT;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || phi == nullptr ||
      theta == nullptr || ((g.flags & ARP_ALIBI) && alibi == nullptr))
    return ARP_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(phi) ||
      !aligned16(theta) || (alibi && !aligned16(alibi)))
    return ARP_ERR_ALIGNMENT;
  if ((st = check_scan_state(g, scan_state, scan_state_bytes)) != ARP_OK) return st;
  if ((st = check_ws(g, workspace, workspace_bytes)) != ARP_OK) return st;
  if (f32) {
    st = arp_angle_scan(desc, phi, theta, scan_state, scan_state_bytes, stream);
    if (st != ARP_OK) return st;
    return hip_status(launch_attn_f32(g, static_cast<const float*>(q), static_cast<const float*>(k),
                                      static_cast<const float*>(v), theta, alibi,
                                      static_cast<float*>(o), lse, (hipStream_t)stream));
  }
  hipStream_t s = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  if (launch_scan_and_rotation(g, phi, theta, scan_state, k, v, ws, s) != hipSuccess)
    return ARP_ERR_HIP;
  return hip_status(launch_attention(g, q, v, theta, alibi, nullptr, nullptr, o, lse, ws, s));
}

arp_status arp_forward_ex(const arp_desc* desc, const void* q, const void* k, const void* v,
                          const float* phi, const float* alibi, const float* logf, float* theta,
                          void* o, float* lse, void* scan_state, size_t scan_state_bytes,
                          void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (!needs_operands(g)) {
    // fp32 I/O or the fused rotation: no gate there; lse from the fp32 kernel only
    if (gated(g)) return ARP_ERR_UNSUPPORTED;
    if (lse != nullptr)
      return g.dtype == ARP_DTYPE_F32
                 ? arp_forward_train(desc, q, k, v, phi, alibi, theta, o, lse, scan_state,
                                     scan_state_bytes, workspace, workspace_bytes, stream)
                 : ARP_ERR_UNSUPPORTED;
    return arp_forward(desc, q, k, v, phi, alibi, theta, o, scan_state, scan_state_bytes,
                       workspace, workspace_bytes, stream);
  }
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || phi == nullptr ||
      theta == nullptr || ((g.flags & ARP_ALIBI) && alibi == nullptr) || (gated(g) && logf == nullptr))
    return ARP_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(phi) ||
      !aligned16(theta) || (alibi && !aligned16(alibi)) || (lse && !aligned16(lse)) ||
      (gated(g) && !aligned16(logf)))
    return ARP_ERR_ALIGNMENT;
  if ((st = check_scan_state(g, scan_state, scan_state_bytes)) != ARP_OK) return st;
  if ((st = check_ws(g, workspace, workspace_bytes)) != ARP_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const WorkspaceLayout lay = workspace_layout(g);
  char* ws = static_cast<char*>(workspace);
  if (launch_scan_and_rotation(g, phi, theta, scan_state, k, v, ws, s) != hipSuccess)
    return ARP_ERR_HIP;
  float* gate2 = gated(g) ? reinterpret_cast<float*>(ws + lay.gate_off) : nullptr;
  double* gbase = gated(g) ? reinterpret_cast<double*>(ws + lay.gate_base_off) : nullptr;
  if (gated(g) && launch_gate_scan(g, logf, gate2, gbase,
                                   reinterpret_cast<double*>(ws + lay.gate_tot_off), s) != hipSuccess)
    return ARP_ERR_HIP;
  return hip_status(launch_attention(g, q, v, theta, alibi, gate2, gbase, o, lse, ws, s));
}

size_t arp_backward_workspace_bytes(const arp_desc* desc) {
  Geometry g;
  if (make_geometry(desc, &g) != ARP_OK) return 0;
  if (g.dtype == ARP_DTYPE_F32 && gated(g)) return 0;
  return bwd_workspace_layout(g).total;
}

arp_status arp_backward_ex(const arp_desc* desc, const void* q, const void* k, const void* v,
                           const float* theta, const float* alibi, const float* logf, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* dtheta, float* dphi, float* dlogf, void* workspace,
                           size_t workspace_bytes, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  const bool f32 = g.dtype == ARP_DTYPE_F32;
  if (f32 && gated(g)) return ARP_ERR_UNSUPPORTED;  // gates: bf16 only
  const void* in[] = {q, k, v, o, lse, dout, dq, dk, dv, dtheta, dphi};
  for (const void* p : in)
    if (p == nullptr) return ARP_ERR_INVALID_ARG;
  if ((rotates(g) && theta == nullptr) || ((g.flags & ARP_ALIBI) && alibi == nullptr) ||
      (gated(g) && (logf == nullptr || dlogf == nullptr)))
    return ARP_ERR_INVALID_ARG;
  for (const void* p : in)
    if (!aligned16(p)) return ARP_ERR_ALIGNMENT;
  if ((theta && !aligned16(theta)) || (alibi && !aligned16(alibi))) return ARP_ERR_ALIGNMENT;
  if (gated(g) && (!aligned16(logf) || !aligned16(dlogf))) return ARP_ERR_ALIGNMENT;
  const BwdWorkspaceLayout lay = bwd_workspace_layout(g);
  if ((st = check_buffer(workspace, workspace_bytes, lay.total)) != ARP_OK) return st;
  char* ws = static_cast<char*>(workspace);
  if (f32) {
    auto fblk = [&](int i) { return reinterpret_cast<float*>(ws + i * lay.operand_bytes); };
    BwdF32Args f{};
    f.q = static_cast<const float*>(q);
    f.k = static_cast<const float*>(k);
    f.v = static_cast<const float*>(v);
    f.o = static_cast<const float*>(o);
    f.dout = static_cast<const float*>(dout);
    f.theta = theta;
    f.lse = lse;
    f.alibi = alibi;
    f.dq = static_cast<float*>(dq);
    f.dk = static_cast<float*>(dk);
    f.dv = static_cast<float*>(dv);
    f.dtheta = dtheta;
    f.dphi = dphi;
    f.totals = reinterpret_cast<float*>(ws + lay.totals_off);
    f.qs = fblk(0);
    f.kr = fblk(1);
    f.vr = fblk(2);
    f.dor = fblk(3);
    f.nl = reinterpret_cast<float*>(ws + lay.stats_off);
    f.nd = f.nl + (size_t)g.B * g.H * g.L;
    return hip_status(launch_backward_f32(g, f, (hipStream_t)stream));
  }
  auto blk = [&](int i) { return reinterpret_cast<uint16_t*>(ws + i * lay.operand_bytes); };
  BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(dout);
  a.theta = theta;
  a.lse = lse;
  a.alibi = alibi;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.dtheta = dtheta;
  a.dphi = dphi;
  a.totals = reinterpret_cast<float*>(ws + lay.totals_off);
  a.ops = BwdOperands{blk(0), blk(1), blk(2), blk(3), blk(4), blk(5), blk(6),
                      reinterpret_cast<float*>(ws + lay.stats_off),
                      reinterpret_cast<float*>(ws + lay.tstat_off), nullptr, nullptr, nullptr,
                      nullptr};
  hipStream_t s = (hipStream_t)stream;
  if (gated(g)) {
    float* gate2 = reinterpret_cast<float*>(ws + lay.gate_off);
    a.logf = logf;
    a.dlogf = dlogf;
    a.gate_tot = reinterpret_cast<double*>(ws + lay.gate_tot_off);
    double* gbase = reinterpret_cast<double*>(ws + lay.gate_base_off);
    a.ops.gate2 = gate2;
    a.ops.gbase = gbase;
    a.ops.colsum = reinterpret_cast<float*>(ws + lay.colsum_off);
    a.ops.rowsum = reinterpret_cast<float*>(ws + lay.rowsum_off);
    if ((st = hip_status(launch_gate_scan(g, logf, gate2, gbase, a.gate_tot, s))) != ARP_OK)
      return st;
  }
  return hip_status(launch_backward_bf16(g, a, s));
}

arp_status arp_backward(const arp_desc* desc, const void* q, const void* k, const void* v,
                        const float* theta, const float* alibi, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, float* dtheta,
                        float* dphi, void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (gated(g)) return ARP_ERR_INVALID_ARG;  // the gates' input and gradient: arp_backward_ex
  return arp_backward_ex(desc, q, k, v, theta, alibi, nullptr, o, lse, dout, dq, dk, dv, dtheta,
                         dphi, nullptr, workspace, workspace_bytes, stream);
}

size_t arp_decode_workspace_bytes(const arp_desc* desc) {
  Geometry g;
  if (make_geometry(desc, &g) != ARP_OK || g.dtype != ARP_DTYPE_BF16) return 0;
  return align_up(decode_workspace_bytes(g));
}

arp_status arp_decode_prefill_ex(const arp_desc* desc, int32_t len, const void* k, const void* v,
                                 const float* phi, const float* theta, const float* logf,
                                 void* kcache, void* vcache, uint64_t* state, double* gcache,
                                 double* gstate, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (g.dtype != ARP_DTYPE_BF16) return ARP_ERR_UNSUPPORTED;
  if (len < 0 || len > g.L || kcache == nullptr || vcache == nullptr || state == nullptr)
    return ARP_ERR_INVALID_ARG;
  if (len > 0 && (k == nullptr || v == nullptr || phi == nullptr || (rotates(g) && theta == nullptr)))
    return ARP_ERR_INVALID_ARG;
  if (gated(g) && (gcache == nullptr || gstate == nullptr || (len > 0 && logf == nullptr)))
    return ARP_ERR_INVALID_ARG;
  if (!aligned16(kcache) || !aligned16(vcache) || !aligned16(state)) return ARP_ERR_ALIGNMENT;
  if (len > 0 && (!aligned16(k) || !aligned16(v) || !aligned16(phi) || (theta && !aligned16(theta))))
    return ARP_ERR_ALIGNMENT;
  if (gated(g) && (!aligned16(gcache) || !aligned16(gstate) || (len > 0 && !aligned16(logf))))
    return ARP_ERR_ALIGNMENT;
  return hip_status(launch_decode_prefill(
      g, len, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), phi, theta,
      static_cast<uint16_t*>(kcache), static_cast<uint16_t*>(vcache), state,
      gated(g) ? logf : nullptr, gated(g) ? gcache : nullptr, gated(g) ? gstate : nullptr,
      (hipStream_t)stream));
}

arp_status arp_decode_prefill(const arp_desc* desc, int32_t len, const void* k, const void* v,
                              const float* phi, const float* theta, void* kcache, void* vcache,
                              uint64_t* state, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (gated(g)) return ARP_ERR_INVALID_ARG;  // the gates: arp_decode_prefill_ex
  return arp_decode_prefill_ex(desc, len, k, v, phi, theta, nullptr, kcache, vcache, state,
                               nullptr, nullptr, stream);
}

arp_status arp_decode_step_ex(const arp_desc* desc, int32_t pos, const void* q, const void* k,
                              const void* v, const float* phi, const float* alibi,
                              const float* logf, uint64_t* state, float* theta, void* kcache,
                              void* vcache, double* gcache, double* gstate, void* o,
                              void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (g.dtype != ARP_DTYPE_BF16) return ARP_ERR_UNSUPPORTED;
  if (pos < 0 || pos >= g.L) return ARP_ERR_INVALID_ARG;
  const void* req[] = {q, k, v, phi, state, theta, kcache, vcache, o};
  for (const void* p : req)
    if (p == nullptr) return ARP_ERR_INVALID_ARG;
  if ((g.flags & ARP_ALIBI) && alibi == nullptr) return ARP_ERR_INVALID_ARG;
  if (gated(g) && (logf == nullptr || gcache == nullptr || gstate == nullptr))
    return ARP_ERR_INVALID_ARG;
  for (const void* p : req)
    if (!aligned16(p)) return ARP_ERR_ALIGNMENT;
  if (alibi && !aligned16(alibi)) return ARP_ERR_ALIGNMENT;
  if (gated(g) && (!aligned16(logf) || !aligned16(gcache) || !aligned16(gstate)))
    return ARP_ERR_ALIGNMENT;
  if ((st = check_buffer(workspace, workspace_bytes, align_up(decode_workspace_bytes(g)))) != ARP_OK)
    return st;
  DecodeArgs a{};
  a.pos = pos;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.phi = phi;
  a.alibi = alibi;
  a.state = state;
  a.theta = theta;
  a.kcache = static_cast<uint16_t*>(kcache);
  a.vcache = static_cast<uint16_t*>(vcache);
  a.o = static_cast<uint16_t*>(o);
  a.part = static_cast<float*>(workspace);
  if (gated(g)) {
    a.logf = logf;
    a.gcache = gcache;
    a.gstate = gstate;
  }
  return hip_status(launch_decode_step(g, a, (hipStream_t)stream));
}

arp_status arp_decode_step(const arp_desc* desc, int32_t pos, const void* q, const void* k,
                           const void* v, const float* phi, const float* alibi, uint64_t* state,
                           float* theta, void* kcache, void* vcache, void* o, void* workspace,
                           size_t workspace_bytes, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (gated(g)) return ARP_ERR_INVALID_ARG;  // the gates: arp_decode_step_ex
  return arp_decode_step_ex(desc, pos, q, k, v, phi, alibi, nullptr, state, theta, kcache, vcache,
                            nullptr, nullptr, o, workspace, workspace_bytes, stream);
}

arp_status arp_rotate(const arp_desc* desc, const void* x, const float* theta, float* out,
                      int inverse, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (x == nullptr || theta == nullptr || out == nullptr) return ARP_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(theta) || !aligned16(out)) return ARP_ERR_ALIGNMENT;
  return hip_status(launch_rotate_diag(g, x, theta, out, inverse, (hipStream_t)stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The no-alloc forward: arp_forward with its scan state and operand workspace
// in a library-owned device array instead of caller buffers, for callers that
// cannot allocate.  Host code never uses the array's name as an address: per
// device, the first call takes its device address with hipGetSymbolAddress
// and every later call uses that pointer.
// ---------------------------------------------------------------------------
namespace arp {
namespace {

constexpr size_t NOALLOC_STATE_BYTES = size_t(24) << 20;  // look-back status words
constexpr size_t NOALLOC_WS_BYTES = size_t(40) << 20;     // rotated bf16 operands
constexpr int NOALLOC_MAX_DEVICES = 64;

// One copy per GPU the library runs on, held until the process ends.
__device__ __align__(256) uint8_t scratch[NOALLOC_STATE_BYTES + NOALLOC_WS_BYTES];

// Zero fill of the scan-state region (a kernel, not a memset, so that a
// first call made under graph capture records a kernel node).
__global__ __launch_bounds__(256) void noalloc_clear_kernel(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

struct ScratchSlot {
  std::once_flag once;
  uint8_t* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[NOALLOC_MAX_DEVICES];

// The current device's scratch address; on the first call on a device, also
// clears the scan-state region on the caller's stream (the scan leaves the
// state ready for the next call from then on).
hipError_t scratch_on_device(hipStream_t stream, uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hipErrorInvalidDevice;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&] {
    void* p = nullptr;
    slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (slot.err != hipSuccess) return;
    slot.ptr = static_cast<uint8_t*>(p);
    hipLaunchKernelGGL(noalloc_clear_kernel, dim3(1024), dim3(256), 0, stream,
                       reinterpret_cast<uint4*>(slot.ptr), NOALLOC_STATE_BYTES / 16);
    slot.err = hipGetLastError();
  });
  if (slot.err != hipSuccess) return slot.err;
  *out = slot.ptr;
  return hipSuccess;
}

}  // namespace
}  // namespace arp

extern "C" arp_status arp_forward_noalloc(const arp_desc* desc, const void* q, const void* k,
                                          const void* v, const float* phi, const float* alibi,
                                          float* theta, void* o, void* stream) {
  Geometry g;
  arp_status st = make_geometry(desc, &g);
  if (st != ARP_OK) return st;
  if (gated(g)) return ARP_ERR_INVALID_ARG;  // as arp_forward
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || phi == nullptr ||
      theta == nullptr || ((g.flags & ARP_ALIBI) && alibi == nullptr))
    return ARP_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(phi) ||
      !aligned16(theta) || (alibi && !aligned16(alibi)))
    return ARP_ERR_ALIGNMENT;
  if (align_up(scan_state_bytes(g)) > NOALLOC_STATE_BYTES ||
      workspace_layout(g).total > NOALLOC_WS_BYTES)
    return ARP_ERR_SCRATCH;
  uint8_t* base = nullptr;
  if (scratch_on_device((hipStream_t)stream, &base) != hipSuccess) return ARP_ERR_HIP;
  return arp_forward(desc, q, k, v, phi, alibi, theta, o, base, NOALLOC_STATE_BYTES,
                     base + NOALLOC_STATE_BYTES, NOALLOC_WS_BYTES, stream);
}
