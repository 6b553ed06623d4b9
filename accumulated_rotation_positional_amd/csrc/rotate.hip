// rotate.hip -- the rotation step on gfx950.
//
//   x~_t = R(Theta_t) x_t,  R(a) = [[cos a, -sin a], [sin a, cos a]] on (x[2p], x[2p+1])
//
// ("AdaRoPE: Not All Attention Heads Should Rotate and Scale Equally",
// Sec. 2.1 eq. (1); the RoPE decay-curve post's rope(): adjacent pairs, sine
// term negative in the first component.)
//
// rotate_kv_kernel: the pre-rotation pass in front of the bf16 attention
// kernel (which rotates q itself, in its prologue).  One workgroup handles
// 64 tokens x head_dim of one (batch, head):
//  * k (and v with value transport) and theta are read with 16-byte coalesced
//    loads (one chunk of 8 elements = 4 pairs per thread, with the matching
//    float4 of angles);
//  * sin/cos of the wrapped angle are computed once per (token, pair) and
//    shared by k and v, from the hardware sine and cosine of turns
//    (__sincosf: v_sin_f32 / v_cos_f32 of theta / 2 pi; absolute error below
//    3e-7 for angles in [-pi, pi), far below the bf16 rounding of k~);
//  * k~ and v~ are written row-major [Lp, D], the layout the attention
//    kernel stages into LDS (it reads the V^T operand with transpose reads);
//    without value transport v is not touched: the attention kernel reads
//    the caller's v;
//  * tokens in [L, Lp) are written as zeros (the attention kernel reads whole
//    tiles without bounds checks);
//  * the largest |k~| of the 64 keys (one attention key tile) is recorded, from
//    the stored bf16 values: the attention kernel bounds its logits with it.
#include "arp_device.hpp"
#include "arp_internal.hpp"

namespace arp {

namespace {

constexpr int ROT_TOKENS = 64;

template <int D>
__global__ __launch_bounds__(256) void rotate_kv_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ theta, uint16_t* __restrict__ kr, uint16_t* __restrict__ vr,
    float* __restrict__ kmax, int L, int Lp, int H, int Hphi, uint32_t flags) {
  constexpr int P = D / 2;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int ITER = ROT_TOKENS * CPR / 256;
  __shared__ uint32_t s_kmax2;  // max |k~|^2 of the tile, as the bits of a non-negative float
  static_assert(ROT_TOKENS == KEY_TILE, "one workgroup per attention key tile");

  const int bh = blockIdx.y;
  const int b = bh / H, h = bh % H;
  const int g = (Hphi == 1) ? 0 : h;
  const int t0 = blockIdx.x * ROT_TOKENS;
  const int tid = threadIdx.x;
  const bool rot_qk = (flags & ARP_ROTATE_QK) != 0;
  const bool rot_v = (flags & ARP_ROTATE_V) != 0;
  if (tid == 0) s_kmax2 = 0u;
  __syncthreads();

#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int idx = it * 256 + tid;
    const int r = idx / CPR, c = idx % CPR;
    const int tok = t0 + r;
    u32x4 ka = {0, 0, 0, 0}, va = {0, 0, 0, 0};
    if (tok < L) {
      const size_t off = ((size_t)bh * L + tok) * D + c * 8;
      ka = *reinterpret_cast<const u32x4*>(k + off);
      if (rot_v) va = *reinterpret_cast<const u32x4*>(v + off);
      float4 th = make_float4(0.f, 0.f, 0.f, 0.f);
      if (rot_qk || rot_v)
        th = *reinterpret_cast<const float4*>(theta + ((size_t)(b * Hphi + g) * L + tok) * P + c * 4);
      const float ang[4] = {th.x, th.y, th.z, th.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float sn, cs;
        __sincosf(ang[e], &sn, &cs);
        float k0 = lo_bf16(ka[e]), k1 = hi_bf16(ka[e]);
        if (rot_qk) rotate_pair(k0, k1, cs, sn);
        ka[e] = pack_bf16x2(k0, k1);
        if (rot_v) {
          float v0 = lo_bf16(va[e]), v1 = hi_bf16(va[e]);
          rotate_pair(v0, v1, cs, sn);
          va[e] = pack_bf16x2(v0, v1);
        }
      }
    }
    const size_t roff = ((size_t)bh * Lp + tok) * D + c * 8;
    *reinterpret_cast<u32x4*>(kr + roff) = ka;
    if (rot_v) *reinterpret_cast<u32x4*>(vr + roff) = va;
    // |k~|^2 of this row from the stored bf16 values (the CPR threads of a
    // row are consecutive lanes), then the tile maximum.
    float n2 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float k0 = lo_bf16(ka[e]), k1 = hi_bf16(ka[e]);
      n2 = fmaf(k0, k0, fmaf(k1, k1, n2));
    }
#pragma unroll
    for (int m = 1; m < CPR; m <<= 1) n2 += __shfl_xor(n2, m);
    if (c == 0) atomicMax(&s_kmax2, __float_as_uint(n2));
  }
  __syncthreads();
  if (tid == 0) kmax[(size_t)bh * (Lp / ROT_TOKENS) + blockIdx.x] = sqrtf(__uint_as_float(s_kmax2));
}

// Diagnostic rotation with fp32 output: one thread per (row, pair).
template <typename TIn>
__global__ __launch_bounds__(256) void rotate_diag_kernel(const TIn* __restrict__ x,
                                                          const float* __restrict__ theta,
                                                          float* __restrict__ out, long npairs_total,
                                                          int L, int H, int Hphi, int P, int inverse) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= npairs_total) return;
  const int p = (int)(i % P);
  const long row = i / P;  // (b*H + h)*L + t
  const int t = (int)(row % L);
  const long bh = row / L;
  const int h = (int)(bh % H), b = (int)(bh / H);
  const int g = (Hphi == 1) ? 0 : h;
  float a, bb;
  if constexpr (sizeof(TIn) == 4) {
    a = x[2 * i];
    bb = x[2 * i + 1];
  } else {
    a = bf16_bits_to_f32(x[2 * i]);
    bb = bf16_bits_to_f32(x[2 * i + 1]);
  }
  float sn, cs;
  sincosf(theta[((size_t)(b * Hphi + g) * L + t) * P + p], &sn, &cs);
  if (inverse) sn = -sn;
  rotate_pair(a, bb, cs, sn);
  out[2 * i] = a;
  out[2 * i + 1] = bb;
}

// Forget-gate prefix G_t = log2 e * sum_{s<=t} min(log f_s, 0) per (b, h), in
// chunks of GATE_CHUNK tokens: gate_totals sums each chunk (fp64), then
// gate_apply adds the totals of the earlier chunks to an in-chunk scan (fp64)
// and writes G in the tiled form the attention kernels read: per 64-token
// tile the fp64 prefix before it (gbase) and each token's fp32 offset from it
// (gate2), so G_i - G_j keeps its fp32 precision at any sequence length.
// Padded to Lp with the last value (padded keys only meet masked scores).
// Loads are coalesced; each thread then scans four consecutive tokens from
// LDS, and the 16 threads of a tile take its base from the first of them.
constexpr int GATE_THREADS = 256;
constexpr int GATE_PER_THREAD = GATE_CHUNK / GATE_THREADS;
static_assert(GATE_PER_THREAD == 4, "four consecutive tokens per thread");

__device__ __forceinline__ double block_sum_256(double x, double* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  const double t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(GATE_THREADS) void gate_totals_kernel(const float* __restrict__ logf,
                                                                   double* __restrict__ tot, int L,
                                                                   int nch) {
  __shared__ double red[4];
  const int c = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const float* src = logf + (size_t)bh * L;
  double x = 0.0;
#pragma unroll
  for (int e = 0; e < GATE_PER_THREAD; ++e) {
    const int t = c * GATE_CHUNK + e * GATE_THREADS + tid;
    if (t < L) x += (double)fminf(src[t], 0.f);
  }
  x = block_sum_256(x, red);
  if (tid == 0) tot[(size_t)bh * nch + c] = x;
}

__global__ __launch_bounds__(GATE_THREADS) void gate_apply_kernel(const float* __restrict__ logf,
                                                                  const double* __restrict__ tot,
                                                                  float* __restrict__ gate2,
                                                                  double* __restrict__ gbase, int L,
                                                                  int Lp, int nch) {
  static_assert(GATE_TILE == 16 * GATE_PER_THREAD, "a tile is 16 consecutive threads of a wave");
  __shared__ float sv[GATE_CHUNK];
  __shared__ double red[4], wsum[4];
  const int c = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  double carry = 0.0;  // the earlier chunks
  for (int i = tid; i < c; i += GATE_THREADS) carry += tot[(size_t)bh * nch + i];
  carry = block_sum_256(carry, red);
  const float* src = logf + (size_t)bh * L;
#pragma unroll
  for (int e = 0; e < GATE_PER_THREAD; ++e) {
    const int t = c * GATE_CHUNK + e * GATE_THREADS + tid;
    sv[e * GATE_THREADS + tid] = (t < L) ? fminf(src[t], 0.f) : 0.f;
  }
  __syncthreads();
  const float4 mine = *reinterpret_cast<const float4*>(sv + GATE_PER_THREAD * tid);
  double run[GATE_PER_THREAD];
  run[0] = (double)mine.x;
  run[1] = run[0] + (double)mine.y;
  run[2] = run[1] + (double)mine.z;
  run[3] = run[2] + (double)mine.w;
  double x = run[3];  // inclusive scan of the thread totals within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  double pre = carry + (x - run[3]);
  for (int i = 0; i < w; ++i) pre += wsum[i];
  const int t0 = c * GATE_CHUNK + GATE_PER_THREAD * tid;
  // the prefix before this thread's 64-token tile: the exclusive prefix of
  // the tile's first thread (lane 16 k of the wave)
  const double tile_pre = __shfl(pre, lane & ~15);
  if (t0 < Lp) {  // Lp is a multiple of 256, so all four tokens are below it
    constexpr double LOG2E_D = 1.4426950408889634;
    const double base = tile_pre * LOG2E_D;
    const float4 out = make_float4((float)((pre + run[0]) * LOG2E_D - base),
                                   (float)((pre + run[1]) * LOG2E_D - base),
                                   (float)((pre + run[2]) * LOG2E_D - base),
                                   (float)((pre + run[3]) * LOG2E_D - base));
    *reinterpret_cast<float4*>(gate2 + (size_t)bh * Lp + t0) = out;
    if ((lane & 15) == 0) gbase[(size_t)bh * (Lp / GATE_TILE) + t0 / GATE_TILE] = base;
  }
}

}  // namespace

hipError_t launch_gate_scan(const Geometry& g, const float* logf, float* gate2, double* gbase,
                            double* totals, hipStream_t stream) {
  const int nch = gate_chunks(g);
  const dim3 grid(nch, g.B * g.H);
  hipLaunchKernelGGL(gate_totals_kernel, grid, dim3(GATE_THREADS), 0, stream, logf, totals, g.L, nch);
  hipLaunchKernelGGL(gate_apply_kernel, grid, dim3(GATE_THREADS), 0, stream, logf, totals, gate2,
                     gbase, g.L, g.Lp, nch);
  return hipGetLastError();
}

hipError_t launch_rotate_kv(const Geometry& g, const void* k, const void* v, const float* theta,
                            uint16_t* kr, uint16_t* vr, float* kmax, hipStream_t stream) {
  dim3 grid(g.Lp / ROT_TOKENS, g.B * g.H);
  const auto* kb = static_cast<const uint16_t*>(k);
  const auto* vb = static_cast<const uint16_t*>(v);
  if (g.D == 64)
    hipLaunchKernelGGL((rotate_kv_kernel<64>), grid, dim3(256), 0, stream, kb, vb, theta, kr, vr,
                       kmax, g.L, g.Lp, g.H, g.Hphi, g.flags);
  else
    hipLaunchKernelGGL((rotate_kv_kernel<128>), grid, dim3(256), 0, stream, kb, vb, theta, kr, vr,
                       kmax, g.L, g.Lp, g.H, g.Hphi, g.flags);
  return hipGetLastError();
}

hipError_t launch_rotate_diag(const Geometry& g, const void* x, const float* theta, float* out,
                              int inverse, hipStream_t stream) {
  const long n = (long)g.B * g.H * g.L * g.P;
  dim3 grid((unsigned)((n + 255) / 256));
  if (g.dtype == ARP_DTYPE_F32)
    hipLaunchKernelGGL((rotate_diag_kernel<float>), grid, dim3(256), 0, stream,
                       static_cast<const float*>(x), theta, out, n, g.L, g.H, g.Hphi, g.P, inverse);
  else
    hipLaunchKernelGGL((rotate_diag_kernel<uint16_t>), grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), theta, out, n, g.L, g.H, g.Hphi, g.P,
                       inverse);
  return hipGetLastError();
}

}  // namespace arp
