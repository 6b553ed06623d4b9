// attn_f32.hip -- fp32 causal attention with accumulated rotations (gfx950).
//
// The fp32-I/O path: every product and sum in fp32, so outputs stay within
// ~1e-6 of the exact result.  A workgroup of 256 threads owns 256 / S
// queries; S adjacent lanes share one query and take every S-th key of each
// staged tile, each with its own online-softmax state (running maximum, sum,
// output accumulator), and the S states are merged with lane shuffles at the
// end.  S = 4 (64 queries per workgroup: each staged key serves 64 queries);
// grids of fewer 64-query workgroups than compute units take S = 32 (8
// queries per workgroup, eight times the workgroups, an eighth of the keys
// per lane): such launches are bound by the serial key walk of one lane, not
// by throughput.  64-key tiles of k and v are staged in LDS, each (key, pair)
// rotated by R(Theta_j) while staged (one sin/cos shared by k and v).  Dot
// products use four partial sums.  Online softmax in base 2 with an exact
// running maximum.
//
// Method: "Why Do Accumulated Transformations Extrapolate?" eq. (2) scores
// and softmax, eq. (4) transported values (un-rotated by R(Theta_i)^T in the
// epilogue), eq. (6)/(8) routed scores as <R(Theta_i) q_i, R(Theta_j) k_j>;
// rotation map from AdaRoPE Sec. 2.1 eq. (1).
#include "arp_device.hpp"
#include "arp_internal.hpp"

namespace arp {

namespace {

constexpr int F32_T = 256;  // threads per workgroup
constexpr int F32_K = 64;   // keys per staged tile

// F32_S: lanes (key subsets) per query; F32_T / F32_S queries per workgroup.
template <int D, int F32_S, bool ROT_QK, bool ROT_V, bool ALIBI>
__global__ __launch_bounds__(F32_T) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ theta, const float* __restrict__ alibi, float* __restrict__ o,
    float* __restrict__ lse, int L, int H, int Hphi, float qscale0,
    const float* __restrict__ hscale) {
  constexpr int P = D / 2;
  constexpr int F32_Q = F32_T / F32_S;
  static_assert(P % F32_S == 0, "each lane writes whole pairs");
  // Rows padded by 16 bytes: the F32_S lanes of a query read F32_S different
  // keys at once, and unpadded rows (256 or 512 bytes, a multiple of the bank
  // period) would put all of them in the same LDS banks.
  constexpr int ROW = D + 4;
  __shared__ __attribute__((aligned(16))) float sk[F32_K][ROW];
  __shared__ __attribute__((aligned(16))) float sv[F32_K][ROW];

  const int bh = blockIdx.y;
  const int b = bh / H, h = bh % H;
  const int g = (Hphi == 1) ? 0 : h;
  const int tid = threadIdx.x;
  const int sp = tid % F32_S;  // this lane's keys: j0 + sp, j0 + sp + F32_S, ... of each tile
  const int i = blockIdx.x * F32_Q + tid / F32_S;
  const bool valid = i < L;
  const int irow = valid ? i : L - 1;
  const float* th_base = theta + (size_t)(b * Hphi + g) * L * P;
  // scale * log2 e, times the head's query multiplier (AdaScale)
  const float qscale = hscale != nullptr ? qscale0 * hscale[h] : qscale0;

  float qv[D];
  const float* qrow = q + ((size_t)bh * L + irow) * D;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    float a = qrow[2 * p], c = qrow[2 * p + 1];
    if (ROT_QK) {
      float sn, cs;
      sincosf(th_base[(size_t)irow * P + p], &sn, &cs);
      rotate_pair(a, c, cs, sn);
    }
    qv[2 * p] = a * qscale;
    qv[2 * p + 1] = c * qscale;
  }
  const float slope2 = ALIBI ? alibi[h] * LOG2E : 0.f;

  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float m = -INFINITY, l = 0.f;

  // Key/value staging, software-pipelined: the raw k, v and angles of tile
  // n + 1 are loaded into registers (each thread IT (key, pair) items, pairs
  // fastest, so a wave reads whole rows) before tile n is computed; they are
  // rotated into LDS after it (one sin/cos per (key, pair), shared by k, v).
  constexpr int IT = F32_K * P / F32_T;
  static_assert(IT * F32_T == F32_K * P, "staging split");
  float2 rk[IT], rv[IT];
  float rt[IT];
  auto fetch = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int e = tid + it * F32_T;
      const int j = j0 + e / P, p = e % P;
      rk[it] = rv[it] = make_float2(0.f, 0.f);
      rt[it] = 0.f;
      if (j < L) {
        const size_t off = ((size_t)bh * L + j) * D + 2 * p;
        rk[it] = *reinterpret_cast<const float2*>(k + off);
        rv[it] = *reinterpret_cast<const float2*>(v + off);
        if (ROT_QK || ROT_V) rt[it] = th_base[(size_t)j * P + p];
      }
    }
  };
  auto commit = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int e = tid + it * F32_T;
      const int jj = e / P, p = e % P;
      float k0 = rk[it].x, k1 = rk[it].y, v0 = rv[it].x, v1 = rv[it].y;
      if (ROT_QK || ROT_V) {
        float sn, cs;
        sincosf(rt[it], &sn, &cs);
        if (ROT_QK) rotate_pair(k0, k1, cs, sn);
        if (ROT_V) rotate_pair(v0, v1, cs, sn);
      }
      *reinterpret_cast<float2*>(&sk[jj][2 * p]) = make_float2(k0, k1);
      *reinterpret_cast<float2*>(&sv[jj][2 * p]) = make_float2(v0, v1);
    }
  };

  const int i_last = min(L - 1, blockIdx.x * F32_Q + F32_Q - 1);
  fetch(0);
  for (int j0 = 0; j0 <= i_last; j0 += F32_K) {
    __syncthreads();  // every lane is done with the previous tile
    commit();
    __syncthreads();
    if (j0 + F32_K <= i_last) fetch(j0 + F32_K);
    const int jn = min(F32_K, i + 1 - j0);  // keys j <= i in this tile
    for (int jj = sp; jj < jn; jj += F32_S) {
      float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int d = 0; d < D; ++d) s4[d & 3] = fmaf(qv[d], sk[jj][d], s4[d & 3]);
      float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      if (ALIBI) s -= slope2 * (float)(i - (j0 + jj));
      if (s > m) {
        const float alpha = exp2f(m - s);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] *= alpha;
        m = s;
      }
      const float pexp = exp2f(s - m);
      l += pexp;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(pexp, sv[jj][d], acc[d]);
    }
  }
  // Merge the query's F32_S states (lanes F32_S qi .. F32_S qi + F32_S - 1).  A lane
  // that saw no key has m = -inf, l = 0 and acc = 0 and gets weight 0; key
  // j = i always exists, so the merged maximum is finite for a valid query.
#pragma unroll
  for (int off = 1; off < F32_S; off <<= 1) {
    const float m2 = __shfl_xor(m, off);
    const float l2 = __shfl_xor(l, off);
    const float mm = fmaxf(m, m2);
    const float wa = (m == -INFINITY) ? 0.f : exp2f(m - mm);
    const float wb = (m2 == -INFINITY) ? 0.f : exp2f(m2 - mm);
    l = l * wa + l2 * wb;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = acc[d] * wa + __shfl_xor(acc[d], off) * wb;
    m = mm;
  }
  if (!valid) return;
  // base-2 log-sum-exp of the row's scaled logits (the backward's statistic)
  if (lse != nullptr && sp == 0) lse[(size_t)bh * L + i] = m + log2f(l);
  const float inv = 1.f / l;
  float* orow = o + ((size_t)bh * L + i) * D;
  // each of the query's lanes writes P / F32_S of its pairs
#pragma unroll
  for (int p = 0; p < P; ++p) {
    if (p / (P / F32_S) != sp) continue;
    float a = acc[2 * p] * inv, c = acc[2 * p + 1] * inv;
    if (ROT_V) {
      float sn, cs;
      sincosf(th_base[(size_t)i * P + p], &sn, &cs);
      rotate_pair(a, c, cs, -sn);  // R(Theta_i)^T
    }
    orow[2 * p] = a;
    orow[2 * p + 1] = c;
  }
}

template <int D, int S>
hipError_t launch_f32_d(const Geometry& g, const float* q, const float* k, const float* v,
                        const float* theta, const float* alibi, float* o, float* lse,
                        hipStream_t stream) {
  constexpr int QPB = F32_T / S;
  dim3 grid((g.L + QPB - 1) / QPB, g.B * g.H);
  const float qscale = g.scale * LOG2E;
  const bool rqk = g.flags & ARP_ROTATE_QK, rv = g.flags & ARP_ROTATE_V, al = g.flags & ARP_ALIBI;
#define ARP_F32_LAUNCH(A, B, C)                                                                \
  hipLaunchKernelGGL((attn_f32_kernel<D, S, A, B, C>), grid, dim3(F32_T), 0, stream, q, k, v, \
                     theta, alibi, o, lse, g.L, g.H, g.Hphi, qscale, g.hscale)
  if (rqk) {
    if (rv) {
      if (al) ARP_F32_LAUNCH(true, true, true); else ARP_F32_LAUNCH(true, true, false);
    } else {
      if (al) ARP_F32_LAUNCH(true, false, true); else ARP_F32_LAUNCH(true, false, false);
    }
  } else {
    if (rv) {
      if (al) ARP_F32_LAUNCH(false, true, true); else ARP_F32_LAUNCH(false, true, false);
    } else {
      if (al) ARP_F32_LAUNCH(false, false, true); else ARP_F32_LAUNCH(false, false, false);
    }
  }
#undef ARP_F32_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const Geometry& g, const float* q, const float* k, const float* v,
                           const float* theta, const float* alibi, float* o, float* lse,
                           hipStream_t stream) {
  const long wg64 = (long)g.B * g.H * ((g.L + 63) / 64);
  if (wg64 < device_cus()) {
    if (g.D == 64) return launch_f32_d<64, 32>(g, q, k, v, theta, alibi, o, lse, stream);
    return launch_f32_d<128, 32>(g, q, k, v, theta, alibi, o, lse, stream);
  }
  if (g.D == 64) return launch_f32_d<64, 4>(g, q, k, v, theta, alibi, o, lse, stream);
  return launch_f32_d<128, 4>(g, q, k, v, theta, alibi, o, lse, stream);
}

}  // namespace arp
