// decode.hip -- token-by-token generation against a cache of pre-rotated
// keys and values, with the accumulated angle carried as a streaming state.
//
// Why no history is ever rewritten: a key rotated by its own accumulated angle
// Theta_j keeps that rotation forever; the route from j to a later query i is
// R(Theta_j - Theta_i) ("Why Do Accumulated Transformations Extrapolate?"
// Sec. 2.2 eq. (6)-(8) and Sec. 5), applied through the query's own rotation
// at query time.  So a decode step only has to
//   1. advance the angle state by the new token's steps phi_t (exact sums of
//      48-bit fixed-point turns, the same arithmetic as the full-sequence
//      scan, so Theta_t is bit-identical to the scan's),
//   2. rotate the new q, k, v by R(Theta_t) and append k~, v~ to the cache,
//   3. attend with q~_t over the cache positions 0..t (causal), and
//   4. un-rotate the output by R(Theta_t)^T when values are transported.
//
// Kernels of a step:
//   decode_attn     split over the keys: one workgroup per (256 keys, b, h);
//                   every workgroup forms the new token's angles (state +
//                   steps) and rotated query itself; the lanes holding row
//                   pos rotate the new key and value, use them from
//                   registers and append them to the caches; one lane group
//                   writes the angles out.  Each wave reads its 64 keys and
//                   values in whole-row, 1 KB-per-instruction loads, scores
//                   them, takes its own softmax maximum and sum and its P V;
//                   the four waves merge in LDS into one partial (m, l, acc)
//   decode_combine  one workgroup per (b, h): merges the partials, normalises,
//                   un-rotates, writes o, and advances the angle state.
// The attention pass is bound by HBM: it reads 2 * (t+1) * d bf16 per (b, h).
//
// Forget gates (ARP_FORGET_GATE): a third cache holds each key's gate prefix
// G_j = log2 e * sum_{s <= j} min(log f_s, 0) in fp64 (so G_t - G_j keeps fp32
// precision at any context length), and a per-(b, h) state the running sum of
// min(log f, 0) in fp64.  A step forms G_t from the state and the new token's
// gate, adds G_t - G_j (rounded once to fp32) to each score
// (the route's product of gates, PaTH reading notes Sec. 2.5), appends G_t
// to the gate cache, and the combine pass advances the state.
#include "angle_fixed.hpp"
#include "arp_device.hpp"
#include "arp_internal.hpp"

namespace arp {

namespace {

constexpr int DKC = 256;  // keys per workgroup of the attention pass

// ---------------------------------------------------------------------------
// prefill: cache rows [0, len) and the state after len tokens
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_fill_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ theta,
    uint16_t* __restrict__ kcache, uint16_t* __restrict__ vcache, int len, int Lmax, int H, int Hphi,
    uint32_t flags) {
  constexpr int P = D / 2, CPR = D / 8;
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh % H, g = (Hphi == 1) ? 0 : h;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int t = idx / CPR, c = idx % CPR;
  if (t >= len) return;
  const bool rqk = (flags & ARP_ROTATE_QK) != 0, rv = (flags & ARP_ROTATE_V) != 0;
  const size_t in = ((size_t)bh * len + t) * D + 8 * c;
  u32x4 wk = *reinterpret_cast<const u32x4*>(k + in);
  u32x4 wv = *reinterpret_cast<const u32x4*>(v + in);
  if (rqk || rv) {
    const float4 th = *reinterpret_cast<const float4*>(theta + ((size_t)(b * Hphi + g) * len + t) * P + 4 * c);
    const float ang[4] = {th.x, th.y, th.z, th.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float sn, cs;
      sincosf(ang[e], &sn, &cs);
      float k0 = lo_bf16(wk[e]), k1 = hi_bf16(wk[e]), v0 = lo_bf16(wv[e]), v1 = hi_bf16(wv[e]);
      if (rqk) rotate_pair(k0, k1, cs, sn);
      if (rv) rotate_pair(v0, v1, cs, sn);
      wk[e] = pack_bf16x2(k0, k1);
      wv[e] = pack_bf16x2(v0, v1);
    }
  }
  const size_t out = ((size_t)bh * Lmax + t) * D + 8 * c;
  *reinterpret_cast<u32x4*>(kcache + out) = wk;
  *reinterpret_cast<u32x4*>(vcache + out) = wv;
}

// state[b, g, p] = 2^47 + sum_{s < len} fixed(phi[b, g, s, p])   (mod 2^48)
template <int P>
__global__ __launch_bounds__(256) void decode_state_kernel(const float* __restrict__ phi,
                                                           uint64_t* __restrict__ state, int len) {
  constexpr int G = 256 / P;
  __shared__ uint64_t part[G][P];
  const int bg = blockIdx.x;
  const int p = threadIdx.x % P, rg = threadIdx.x / P;
  uint64_t acc = 0;
  for (int t = rg; t < len; t += G) acc += to_fixed(phi[((size_t)bg * len + t) * P + p]);
  part[rg][p] = acc;
  __syncthreads();
  if (rg == 0) {
    uint64_t s = FIXED_ZERO;
#pragma unroll
    for (int r = 0; r < G; ++r) s += part[r][p];
    state[(size_t)bg * P + p] = s & MASK48;
  }
}

// Gate prefix of the prompt: gcache[bh][t] = log2 e * sum_{s <= t} min(logf[bh][s], 0)
// (fp64) for t < len and gstate[bh] = the fp64 sum over the whole prompt.  One
// workgroup per (b, h) walks the prompt in chunks of 1024 tokens (four
// consecutive tokens per thread, an in-chunk scan in fp64 plus the carry).
__global__ __launch_bounds__(256) void decode_gate_fill_kernel(const float* __restrict__ logf,
                                                               double* __restrict__ gcache,
                                                               double* __restrict__ gstate, int len,
                                                               int Lmax) {
  __shared__ double wsum[4];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  constexpr double LOG2E_D = 1.4426950408889634;
  double carry = 0.0;
  for (int c0 = 0; c0 < len; c0 += 1024) {
    const int t0 = c0 + 4 * tid;
    double run[4];
    double acc = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (t0 + e < len) acc += (double)fminf(logf[(size_t)bh * len + t0 + e], 0.f);
      run[e] = acc;
    }
    double incl = acc;  // inclusive scan of the thread sums within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    double pre = carry + (incl - acc);
    for (int u = 0; u < w; ++u) pre += wsum[u];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (t0 + e < len) gcache[(size_t)bh * Lmax + t0 + e] = (pre + run[e]) * LOG2E_D;
    carry += (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    __syncthreads();  // wsum is rewritten by the next chunk
  }
  if (tid == 0) gstate[bh] = carry;
}

// ---------------------------------------------------------------------------
// step
// ---------------------------------------------------------------------------
// One partial per (256 keys, b, h): part = [m, l, acc[0..D)] in base-2 logits.
// Every load instruction of a wave reads whole consecutive cache rows (CPR
// lanes of 16 bytes per row, 1 KB per instruction): lane (r, c) holds chunk c
// of rows kw0 + RPI i + r.  Scores are reduced over the CPR lanes of a row;
// P V accumulates per lane and is reduced over the RPI row groups at the end.
template <int D, bool ALIBI, bool GATE>
__global__ __launch_bounds__(256) void decode_attn_kernel(
    const uint16_t* __restrict__ qin, const uint16_t* __restrict__ kin,
    const uint16_t* __restrict__ vin, const float* __restrict__ phi,
    const uint64_t* __restrict__ state, float* __restrict__ theta, uint16_t* __restrict__ kcache,
    uint16_t* __restrict__ vcache, const float* __restrict__ alibi, const float* __restrict__ logf,
    double* __restrict__ gcache, const double* __restrict__ gstate, float* __restrict__ part, int H,
    int Hphi, int Lmax, int pos, int nchunk, uint32_t flags, float qscale0,
    const float* __restrict__ hscale) {
  constexpr int CPR = D / 8;     // lanes per row
  constexpr int RPI = 64 / CPR;  // rows per load instruction
  constexpr int NI = 64 / RPI;   // instructions per 64 keys
  __shared__ float s_m[4], s_l[4];
  __shared__ float s_acc[4][D];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int b = bh / H, h = bh % H, g = (Hphi == 1) ? 0 : h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ch = lane % CPR, rg = lane / CPR;
  const int n = pos + 1;                // keys 0..pos
  const int kw0 = c * DKC + wave * 64;  // this wave's first key
  const float slope2 = ALIBI ? alibi[h] * LOG2E : 0.f;
  // scale * log2 e, times the head's query multiplier (AdaScale)
  const float qscale = hscale != nullptr ? qscale0 * hscale[h] : qscale0;
  // The new token's gate prefix G_t (every workgroup forms the same value;
  // the first one appends it to the gate cache).
  double gt = 0.0;
  if constexpr (GATE) {
    gt = (gstate[bh] + (double)fminf(logf[bh], 0.f)) * 1.4426950408889634;
    if (c == 0 && tid == 0) gcache[(size_t)bh * Lmax + pos] = gt;
  }

  // The new token's angles for this lane's four pairs 4 ch .. 4 ch + 3: the
  // state plus its steps (the scan's arithmetic, so bit-identical to it).
  float sn[4], cs[4];
  const size_t sbase = (size_t)(b * Hphi + g) * (D / 2) + 4 * ch;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint64_t cur = (flags & ARP_SCAN_EXCLUSIVE) ? state[sbase + e]
                                                      : state[sbase + e] + to_fixed(phi[sbase + e]);
    const float th = to_radians_offset(cur);
    // one writer per angle stream: the first chunk's row group 0 of wave 0
    if (c == 0 && wave == 0 && rg == 0 && (Hphi != 1 || h == 0)) theta[sbase + e] = th;
    sincosf(th, &sn[e], &cs[e]);
  }
  const bool rqk = (flags & ARP_ROTATE_QK) != 0, rv = (flags & ARP_ROTATE_V) != 0;
  // q~ as the products use it: rotated, scaled, rounded to bf16 like a cached key
  float qv[8];
  {
    const u32x4 w = *reinterpret_cast<const u32x4*>(qin + (size_t)bh * D + 8 * ch);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float q0 = lo_bf16(w[e]), q1 = hi_bf16(w[e]);
      if (rqk) rotate_pair(q0, q1, cs[e], sn[e]);
      const uint32_t r = pack_bf16x2(q0 * qscale, q1 * qscale);
      qv[2 * e] = lo_bf16(r);
      qv[2 * e + 1] = hi_bf16(r);
    }
  }
  // The new key and value, rotated, in the lanes that hold row pos: they
  // take part in this step from registers and are appended to the caches.
  const bool owner = (pos >= kw0) && (pos < kw0 + 64) && ((pos - kw0) % RPI == rg);
  u32x4 knew = {0, 0, 0, 0}, vnew = {0, 0, 0, 0};
  if (owner) {
    const u32x4 wk = *reinterpret_cast<const u32x4*>(kin + (size_t)bh * D + 8 * ch);
    const u32x4 wv = *reinterpret_cast<const u32x4*>(vin + (size_t)bh * D + 8 * ch);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float k0 = lo_bf16(wk[e]), k1 = hi_bf16(wk[e]), v0 = lo_bf16(wv[e]), v1 = hi_bf16(wv[e]);
      if (rqk) rotate_pair(k0, k1, cs[e], sn[e]);
      if (rv) rotate_pair(v0, v1, cs[e], sn[e]);
      knew[e] = pack_bf16x2(k0, k1);
      vnew[e] = pack_bf16x2(v0, v1);
    }
    const size_t out = ((size_t)bh * Lmax + pos) * D + 8 * ch;
    *reinterpret_cast<u32x4*>(kcache + out) = knew;
    *reinterpret_cast<u32x4*>(vcache + out) = vnew;
  }
  const uint16_t* kb = kcache + (size_t)bh * Lmax * D + 8 * ch;
  const uint16_t* vb = vcache + (size_t)bh * Lmax * D + 8 * ch;
  u32x4 kw[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = kw0 + RPI * i + rg;
    kw[i] = (row < pos) ? *reinterpret_cast<const u32x4*>(kb + (size_t)row * D)
                        : (row == pos ? knew : u32x4{0, 0, 0, 0});
  }
  // the rows' gate biases G_t - G_j (0 for row pos and beyond): lane l loads
  // the gate of the wave's row kw0 + l, and each lane takes its rows' gates
  // from the lanes that hold them
  // (G in fp64, its difference rounded once to fp32)
  float gb[NI];
  if constexpr (GATE) {
    const int mine = kw0 + lane;
    const double gl = (mine < pos) ? gcache[(size_t)bh * Lmax + mine] : gt;
#pragma unroll
    for (int i = 0; i < NI; ++i) gb[i] = (float)(gt - __shfl(gl, RPI * i + rg));
  }
  float sc[NI];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a = fmaf(lo_bf16(kw[i][e]), qv[2 * e], a);
      a = fmaf(hi_bf16(kw[i][e]), qv[2 * e + 1], a);
    }
#pragma unroll
    for (int mk = 1; mk < CPR; mk <<= 1) a += __shfl_xor(a, mk);
    const int row = kw0 + RPI * i + rg;
    if (ALIBI) a += slope2 * (float)(row - pos);
    if (GATE) a += gb[i];
    sc[i] = (row < n) ? a : -INFINITY;
    m = fmaxf(m, sc[i]);
  }
#pragma unroll
  for (int off = CPR; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
  // values of the same rows (issued before the exponentials)
  u32x4 vw[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = kw0 + RPI * i + rg;
    vw[i] = (row < pos) ? *reinterpret_cast<const u32x4*>(vb + (size_t)row * D)
                        : (row == pos ? vnew : u32x4{0, 0, 0, 0});
  }
  float l = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const float pr = (sc[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[i] - m);
    l += pr;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = fmaf(pr, lo_bf16(vw[i][e]), acc[2 * e]);
      acc[2 * e + 1] = fmaf(pr, hi_bf16(vw[i][e]), acc[2 * e + 1]);
    }
  }
  // over the row groups (each row's probability sits in its CPR lanes once per group)
#pragma unroll
  for (int off = CPR; off < 64; off <<= 1) {
    l += __shfl_xor(l, off);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
  }
  if (lane == 0) {
    s_m[wave] = m;
    s_l[wave] = l;
  }
  if (rg == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s_acc[wave][8 * ch + e] = acc[e];
  }
  __syncthreads();
  if (tid < D) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w]);
    float Ls = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (s_m[w] == -INFINITY) continue;
      const float f = __builtin_amdgcn_exp2f(s_m[w] - M);
      Ls = fmaf(s_l[w], f, Ls);
      A = fmaf(s_acc[w][tid], f, A);
    }
    float* dst = part + ((size_t)bh * nchunk + c) * (D + 2);
    if (tid == 0) {
      dst[0] = M;
      dst[1] = Ls;
    }
    dst[2 + tid] = A;
  }
}

// One workgroup per (b, h): thread (pair p, group cg) merges every G-th chunk
// of its pair in one pass, U chunks per trip with all their loads issued
// before any is used and the running sums rescaled once per trip to the
// trip's maximum; then the G groups are merged in LDS the same way.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const float* __restrict__ part, const float* __restrict__ theta, const float* __restrict__ phi,
    uint64_t* __restrict__ state, const float* __restrict__ logf, double* __restrict__ gstate,
    uint16_t* __restrict__ o, int H, int Hphi, int nchunk, uint32_t flags) {
  constexpr int P = D / 2, G = 256 / P;
  constexpr int U = 8;
  __shared__ float s_sum[G][P][4];
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H, g = (Hphi == 1) ? 0 : h;
  const int tid = threadIdx.x;
  const int p = tid % P, cg = tid / P;
  const float* src = part + (size_t)bh * nchunk * (D + 2);
  // the epilogue's own operands, loaded before the partials so that their
  // latency is not added after the merge (this workgroup is the only one that
  // writes the state and the gate state of its stream)
  const size_t sidx = (size_t)(b * Hphi + g) * P + p;
  const bool advance = cg == 0 && (Hphi != 1 || h == 0);
  const float th = (cg == 0 && (flags & ARP_ROTATE_V)) ? theta[sidx] : 0.f;
  const float ph = advance ? phi[sidx] : 0.f;
  const uint64_t st = advance ? state[sidx] : 0;
  const bool gadv = gstate != nullptr && tid == 0;
  const float lf = gadv ? logf[bh] : 0.f;
  const double gs = gadv ? gstate[bh] : 0.0;
  // every chunk holds at least one key, so its maximum is finite; a trip
  // always holds its first chunk (c0 < nchunk)
  float M = -INFINITY, Ls = 0.f, a0 = 0.f, a1 = 0.f;
  for (int c0 = cg; c0 < nchunk; c0 += U * G) {
    float mc[U], lc[U], x0[U], x1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float* pc = src + (size_t)min(c0 + u * G, nchunk - 1) * (D + 2);
      mc[u] = pc[0];
      lc[u] = pc[1];
      x0[u] = pc[2 + 2 * p];
      x1[u] = pc[3 + 2 * p];
    }
    float mt = M;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + u * G < nchunk) mt = fmaxf(mt, mc[u]);
    const float f0 = __builtin_amdgcn_exp2f(M - mt);  // 0 on the first trip (M = -inf)
    Ls *= f0;
    a0 *= f0;
    a1 *= f0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u * G >= nchunk) break;
      const float f = __builtin_amdgcn_exp2f(mc[u] - mt);
      Ls = fmaf(lc[u], f, Ls);
      a0 = fmaf(x0[u], f, a0);
      a1 = fmaf(x1[u], f, a1);
    }
    M = mt;
  }
  s_sum[cg][p][0] = M;
  s_sum[cg][p][1] = Ls;
  s_sum[cg][p][2] = a0;
  s_sum[cg][p][3] = a1;
  __syncthreads();
  if (cg != 0) return;
  // group 0 holds chunk 0, so the merged maximum is finite; a group with no
  // chunk (M = -inf) gets weight 0
#pragma unroll
  for (int r = 1; r < G; ++r) M = fmaxf(M, s_sum[r][p][0]);
  Ls = 0.f;
  a0 = 0.f;
  a1 = 0.f;
#pragma unroll
  for (int r = 0; r < G; ++r) {
    const float f = __builtin_amdgcn_exp2f(s_sum[r][p][0] - M);
    Ls = fmaf(s_sum[r][p][1], f, Ls);
    a0 = fmaf(s_sum[r][p][2], f, a0);
    a1 = fmaf(s_sum[r][p][3], f, a1);
  }
  const float inv = 1.f / Ls;
  float x0 = a0 * inv, x1 = a1 * inv;
  if (flags & ARP_ROTATE_V) {
    float sn, cs;
    sincosf(th, &sn, &cs);
    rotate_pair(x0, x1, cs, -sn);
  }
  *reinterpret_cast<uint32_t*>(o + (size_t)bh * D + 2 * p) = pack_bf16x2(x0, x1);
  // advance the state (one workgroup per angle stream; no other workgroup of
  // this kernel reads it)
  if (advance) state[sidx] = (st + to_fixed(ph)) & MASK48;
  // and the gate state (one workgroup per (b, h))
  if (gadv) gstate[bh] = gs + (double)fminf(lf, 0.f);
}

template <int D, bool ALIBI, bool GATE>
void launch_attn_step(const Geometry& g, const DecodeArgs& a, int nchunk, hipStream_t stream) {
  hipLaunchKernelGGL((decode_attn_kernel<D, ALIBI, GATE>), dim3(nchunk, g.B * g.H), dim3(256), 0,
                     stream, a.q, a.k, a.v, a.phi, a.state, a.theta, a.kcache, a.vcache, a.alibi,
                     a.logf, a.gcache, a.gstate, a.part, g.H, g.Hphi, g.L, a.pos, nchunk, g.flags,
                     g.scale * LOG2E, g.hscale);
}

template <int D>
hipError_t launch_step(const Geometry& g, const DecodeArgs& a, hipStream_t stream) {
  const int BH = g.B * g.H;
  const int nchunk = (a.pos + 1 + DKC - 1) / DKC;
  const bool al = (g.flags & ARP_ALIBI) != 0, gate = (g.flags & ARP_FORGET_GATE) != 0;
  if (al) {
    if (gate) launch_attn_step<D, true, true>(g, a, nchunk, stream);
    else launch_attn_step<D, true, false>(g, a, nchunk, stream);
  } else {
    if (gate) launch_attn_step<D, false, true>(g, a, nchunk, stream);
    else launch_attn_step<D, false, false>(g, a, nchunk, stream);
  }
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(BH), dim3(256), 0, stream, a.part, a.theta,
                     a.phi, a.state, gate ? a.logf : nullptr, gate ? a.gstate : nullptr, a.o, g.H,
                     g.Hphi, nchunk, g.flags);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(const Geometry& g) {
  const size_t nchunk = ((size_t)g.L + DKC - 1) / DKC;
  return (size_t)g.B * g.H * nchunk * (g.D + 2) * sizeof(float);
}

hipError_t launch_decode_prefill(const Geometry& g, int len, const uint16_t* k, const uint16_t* v,
                                 const float* phi, const float* theta, uint16_t* kcache,
                                 uint16_t* vcache, uint64_t* state, const float* logf,
                                 double* gcache, double* gstate, hipStream_t stream) {
  if (len > 0) {
    dim3 grid((unsigned)(((size_t)len * (g.D / 8) + 255) / 256), g.B * g.H);
    if (g.D == 64)
      hipLaunchKernelGGL((decode_fill_kernel<64>), grid, dim3(256), 0, stream, k, v, theta, kcache,
                         vcache, len, g.L, g.H, g.Hphi, g.flags);
    else
      hipLaunchKernelGGL((decode_fill_kernel<128>), grid, dim3(256), 0, stream, k, v, theta, kcache,
                         vcache, len, g.L, g.H, g.Hphi, g.flags);
  }
  if (g.P == 32)
    hipLaunchKernelGGL((decode_state_kernel<32>), dim3(g.B * g.Hphi), dim3(256), 0, stream, phi, state,
                       len);
  else
    hipLaunchKernelGGL((decode_state_kernel<64>), dim3(g.B * g.Hphi), dim3(256), 0, stream, phi, state,
                       len);
  if (g.flags & ARP_FORGET_GATE)
    hipLaunchKernelGGL(decode_gate_fill_kernel, dim3(g.B * g.H), dim3(256), 0, stream, logf, gcache,
                       gstate, len, g.L);
  return hipGetLastError();
}

hipError_t launch_decode_step(const Geometry& g, const DecodeArgs& a, hipStream_t stream) {
  return g.D == 64 ? launch_step<64>(g, a, stream) : launch_step<128>(g, a, stream);
}

}  // namespace arp
