// Host-side checks of libarp's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_sanitizers.py links
// this file against a copy of the library whose api.hip host code carries the
// same instrumentation).  Every call either is host-only (descriptor checks,
// sizes, status strings, the AdaScale schedule) or fails validation before
// anything is enqueued, so no GPU is needed and no device address is ever
// dereferenced: the fake addresses below are never touched.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <limits>

#include "../../include/arp.h"

static int failures = 0;
#define EXPECT(cond)                                                               \
  do {                                                                             \
    if (!(cond)) {                                                                 \
      std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);       \
      ++failures;                                                                  \
    }                                                                              \
  } while (0)

static arp_desc desc(int32_t B, int32_t H, int32_t L, int32_t d, int32_t dtype, uint32_t flags) {
  arp_desc x;
  std::memset(&x, 0, sizeof x);
  x.batch = B;
  x.heads = H;
  x.seqlen = L;
  x.head_dim = d;
  x.dtype = dtype;
  x.flags = flags;
  return x;
}

static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

int main() {
  void* const A = fake(0x10000);   // 256-byte aligned, never dereferenced
  void* const M = fake(0x10004);   // misaligned
  const size_t big = size_t(1) << 40;

  EXPECT(arp_abi_version() == 2);
  for (int s = -3; s < 12; ++s) EXPECT(arp_status_string(s) != nullptr && std::strlen(arp_status_string(s)) > 0);

  // descriptors: every field at and beyond its limits
  const int32_t dims[] = {-1, 0, 2, 32, 63, 64, 96, 128, 256};
  const int32_t lens[] = {-5, 0, 1, 63, 64, 65, 16384, (1 << 24), (1 << 24) + 1,
                          std::numeric_limits<int32_t>::max()};
  for (int32_t d : dims)
    for (int32_t L : lens)
      for (int32_t dt = -1; dt <= 2; ++dt)
        for (uint32_t f : {0u, 1u, 3u, 0x7u, 0x20u, 0x41u, 0xFFu, 0x100u, 0xFFFFFFFFu}) {
          arp_desc x = desc(2, 3, L, d, dt, f);
          const arp_status st = arp_check(&x);
          EXPECT(st >= ARP_OK && st <= ARP_ERR_SCRATCH);
          // sizes are 0 exactly when the descriptor is rejected, and fit a size_t
          const size_t s1 = arp_scan_state_bytes(&x), s2 = arp_workspace_bytes(&x);
          const size_t s3 = arp_backward_workspace_bytes(&x), s4 = arp_decode_workspace_bytes(&x);
          if (st != ARP_OK) EXPECT(s1 == 0 && s2 == 0 && s3 == 0 && s4 == 0);
          else EXPECT(s1 > 0 && s1 % 256 == 0 && s2 % 256 == 0);
        }
  {
    arp_desc x = desc(std::numeric_limits<int32_t>::max(), std::numeric_limits<int32_t>::max(),
                      1 << 24, 128, ARP_DTYPE_BF16, ARP_ROTATE_QK | ARP_ROTATE_V | ARP_FORGET_GATE);
    (void)arp_check(&x);
    (void)arp_scan_state_bytes(&x);
    (void)arp_workspace_bytes(&x);
    (void)arp_backward_workspace_bytes(&x);
  }
  {
    arp_desc x = desc(2, 3, 100, 64, ARP_DTYPE_BF16, ARP_ROTATE_QK);
    x.scale = std::nanf("");
    EXPECT(arp_check(&x) == ARP_ERR_INVALID_ARG);
    x.scale = INFINITY;
    EXPECT(arp_check(&x) == ARP_ERR_INVALID_ARG);
    x.scale = 0.f;
    x.reserved = 1;
    EXPECT(arp_check(&x) == ARP_ERR_INVALID_ARG);
    x.reserved = 0;
    x.flags |= ARP_HEAD_SCALE;
    EXPECT(arp_check(&x) == ARP_ERR_INVALID_ARG);  // flag without the array
    x.head_scale = static_cast<const float*>(M);
    EXPECT(arp_check(&x) == ARP_ERR_ALIGNMENT);
    x.head_scale = static_cast<const float*>(A);
    EXPECT(arp_check(&x) == ARP_OK);
    x.flags &= ~ARP_HEAD_SCALE;
    EXPECT(arp_check(&x) == ARP_ERR_INVALID_ARG);  // array without the flag
    EXPECT(arp_check(nullptr) == ARP_ERR_INVALID_ARG);
  }

  // AdaScale schedule (host arrays)
  {
    float tau[5] = {1.f, 0.5f, 2.f, 1.f, 1.f}, gamma[5] = {0.f, 1.f, 2.f, -1.f, 30.f}, lam[5];
    EXPECT(arp_adascale_lambda(5, tau, gamma, 4096, 1024, lam) == ARP_OK);
    EXPECT(lam[0] == 1.f);
    EXPECT(std::fabs(lam[1] - 2.f * std::log(5.f)) < 1e-5f);
    EXPECT(arp_adascale_lambda(0, tau, gamma, 10, 10, lam) == ARP_ERR_INVALID_ARG);
    EXPECT(arp_adascale_lambda(5, nullptr, gamma, 10, 10, lam) == ARP_ERR_INVALID_ARG);
    EXPECT(arp_adascale_lambda(5, tau, gamma, 0, 10, lam) == ARP_ERR_INVALID_ARG);
    EXPECT(arp_adascale_lambda(5, tau, gamma, 10, 0, lam) == ARP_ERR_INVALID_ARG);
    float bad[2] = {0.f, -1.f};
    EXPECT(arp_adascale_lambda(2, bad, gamma, 10, 10, lam) == ARP_ERR_INVALID_ARG);
    EXPECT(arp_adascale_lambda(1, tau, gamma, std::numeric_limits<int64_t>::max(), 1, lam) == ARP_OK);
  }

  // entry points: null, misaligned and undersized arguments are rejected on the host
  {
    arp_desc x = desc(2, 8, 1000, 64, ARP_DTYPE_BF16, ARP_ROTATE_QK);
    const size_t st = arp_scan_state_bytes(&x), ws = arp_workspace_bytes(&x);
    float* const F = static_cast<float*>(A);
    float* const FM = static_cast<float*>(M);
    EXPECT(arp_angle_scan(&x, nullptr, F, A, st, nullptr) == ARP_ERR_INVALID_ARG);
    EXPECT(arp_angle_scan(&x, FM, F, A, st, nullptr) == ARP_ERR_ALIGNMENT);
    EXPECT(arp_angle_scan(&x, F, F, A, st - 1, nullptr) != ARP_OK);
    EXPECT(arp_angle_scan(&x, F, F, fake(0x10010), st, nullptr) == ARP_ERR_ALIGNMENT);
    EXPECT(arp_rotate_kv(&x, nullptr, A, F, A, ws, nullptr) == ARP_ERR_INVALID_ARG);
    EXPECT(arp_rotate_kv(&x, A, A, F, A, 8, nullptr) == ARP_ERR_WORKSPACE);
    EXPECT(arp_attn_rotated(&x, A, nullptr, F, nullptr, A, A, ws, nullptr) == ARP_ERR_INVALID_ARG);
    EXPECT(arp_attn_fwd(&x, A, A, M, F, nullptr, A, A, ws, nullptr) == ARP_ERR_ALIGNMENT);
    EXPECT(arp_forward(&x, A, A, A, F, F, F, A, A, st, A, 0, nullptr) != ARP_OK);  // alibi w/o flag
    EXPECT(arp_forward(&x, A, A, A, F, nullptr, F, A, A, st, A, 1, nullptr) == ARP_ERR_WORKSPACE);
    EXPECT(arp_forward_train(&x, A, A, A, F, nullptr, F, A, nullptr, A, st, A, ws, nullptr) ==
           ARP_ERR_INVALID_ARG);
    {
      arp_desc gx = x;
      gx.flags |= ARP_FORGET_GATE;
      const size_t gws = arp_workspace_bytes(&gx);
      EXPECT(gws > ws);  // the gate prefix, its tile bases and chunk totals
      EXPECT(arp_forward_ex(&gx, A, A, A, F, nullptr, nullptr, F, A, nullptr, A, st, A, gws,
                            nullptr) == ARP_ERR_INVALID_ARG);  // gated without logf
      EXPECT(arp_forward_ex(&gx, A, A, A, F, nullptr, FM, F, A, nullptr, A, st, A, gws, nullptr) ==
             ARP_ERR_ALIGNMENT);
      EXPECT(arp_forward_ex(&gx, A, A, A, F, nullptr, F, F, A, nullptr, A, st, A, ws, nullptr) ==
             ARP_ERR_WORKSPACE);
      EXPECT(arp_forward(&gx, A, A, A, F, nullptr, F, A, A, st, A, gws, nullptr) ==
             ARP_ERR_INVALID_ARG);  // the gate needs the _ex entry points
    }
    EXPECT(arp_backward(&x, A, A, A, F, nullptr, A, F, A, A, A, A, F, F, A, 1, nullptr) ==
           ARP_ERR_WORKSPACE);
    EXPECT(arp_backward(&x, A, A, A, F, nullptr, A, nullptr, A, A, A, A, F, F, A, big, nullptr) ==
           ARP_ERR_INVALID_ARG);
    EXPECT(arp_forward_noalloc(&x, A, A, A, F, nullptr, F, nullptr, nullptr) == ARP_ERR_INVALID_ARG);
    EXPECT(arp_rotate(&x, nullptr, F, F, 0, nullptr) == ARP_ERR_INVALID_ARG);
    uint64_t* const S = static_cast<uint64_t*>(A);
    EXPECT(arp_decode_prefill(&x, -1, A, A, F, F, A, A, S, nullptr) == ARP_ERR_INVALID_ARG);
    EXPECT(arp_decode_prefill(&x, 1001, A, A, F, F, A, A, S, nullptr) == ARP_ERR_INVALID_ARG);
    EXPECT(arp_decode_step(&x, 1000, A, A, A, F, nullptr, S, F, A, A, A, A, big, nullptr) ==
           ARP_ERR_INVALID_ARG);
    EXPECT(arp_decode_step(&x, -1, A, A, A, F, nullptr, S, F, A, A, A, A, big, nullptr) ==
           ARP_ERR_INVALID_ARG);
    float bound[1];
    (void)bound;
    EXPECT(arp_angle_scan_random(&x, 1, 2, nullptr, F, A, st, nullptr) == ARP_ERR_INVALID_ARG);
    EXPECT(arp_angle_scan_tokens(&x, static_cast<const int32_t*>(A), F, 0, F, A, st, nullptr) ==
           ARP_ERR_INVALID_ARG);
    EXPECT(arp_angle_scan_const(&x, nullptr, F, nullptr) == ARP_ERR_INVALID_ARG);
    EXPECT(arp_random_phi(&x, 1, 2, F, nullptr, nullptr) == ARP_ERR_INVALID_ARG);
    arp_desc bad = x;
    bad.head_dim = 96;
    EXPECT(arp_forward(&bad, A, A, A, F, nullptr, F, A, A, st, A, ws, nullptr) ==
           ARP_ERR_UNSUPPORTED);
  }
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi checks passed\n");
  return 0;
}
