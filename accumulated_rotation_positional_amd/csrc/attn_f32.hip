// attn_f32.hip -- fp32 causal attention with accumulated rotations (gfx950).
//
// The fp32-I/O path: every product and sum in fp32, so outputs stay within
// ~1e-6 of the exact result.  A workgroup of 256 threads owns 64 queries;
// four adjacent lanes share one query and take every fourth key of each
// staged tile, each with its own online-softmax state (running maximum, sum,
// output accumulator), and the four states are merged with lane shuffles at
// the end.  32-key tiles of k and v are staged in LDS, each (key, pair)
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

constexpr int F32_Q = 64;   // queries per workgroup: each staged key is used by 64 queries
constexpr int F32_S = 4;    // lanes (key subsets) per query
constexpr int F32_T = F32_Q * F32_S;
constexpr int F32_K = 32;   // keys per staged tile

template <int D, bool ROT_QK, bool ROT_V, bool ALIBI>
__global__ __launch_bounds__(F32_T) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ theta, const float* __restrict__ alibi, float* __restrict__ o,
    float* __restrict__ lse, int L, int H, int Hphi, float qscale0,
    const float* __restrict__ hscale) {
  constexpr int P = D / 2;
  __shared__ float sk[F32_K][D];
  __shared__ float sv[F32_K][D];

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

  const int i_last = min(L - 1, blockIdx.x * F32_Q + F32_Q - 1);
  for (int j0 = 0; j0 <= i_last; j0 += F32_K) {
    __syncthreads();
    // Stage and rotate keys/values j0 .. j0+F32_K-1 (one sin/cos per (key, pair)).
    for (int e = tid; e < F32_K * P; e += F32_T) {
      const int jj = e / P, p = e % P;
      const int j = j0 + jj;
      float k0 = 0.f, k1 = 0.f, v0 = 0.f, v1 = 0.f;
      if (j < L) {
        const size_t off = ((size_t)bh * L + j) * D + 2 * p;
        k0 = k[off];
        k1 = k[off + 1];
        v0 = v[off];
        v1 = v[off + 1];
        if (ROT_QK || ROT_V) {
          float sn, cs;
          sincosf(th_base[(size_t)j * P + p], &sn, &cs);
          if (ROT_QK) rotate_pair(k0, k1, cs, sn);
          if (ROT_V) rotate_pair(v0, v1, cs, sn);
        }
      }
      sk[jj][2 * p] = k0;
      sk[jj][2 * p + 1] = k1;
      sv[jj][2 * p] = v0;
      sv[jj][2 * p + 1] = v1;
    }
    __syncthreads();
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

template <int D>
hipError_t launch_f32_d(const Geometry& g, const float* q, const float* k, const float* v,
                        const float* theta, const float* alibi, float* o, float* lse,
                        hipStream_t stream) {
  dim3 grid((g.L + F32_Q - 1) / F32_Q, g.B * g.H);
  const float qscale = g.scale * LOG2E;
  const bool rqk = g.flags & ARP_ROTATE_QK, rv = g.flags & ARP_ROTATE_V, al = g.flags & ARP_ALIBI;
#define ARP_F32_LAUNCH(A, B, C)                                                                \
  hipLaunchKernelGGL((attn_f32_kernel<D, A, B, C>), grid, dim3(F32_T), 0, stream, q, k, v,    \
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
  if (g.D == 64) return launch_f32_d<64>(g, q, k, v, theta, alibi, o, lse, stream);
  return launch_f32_d<128>(g, q, k, v, theta, alibi, o, lse, stream);
}

}  // namespace arp
