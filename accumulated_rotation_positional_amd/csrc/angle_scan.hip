// angle_scan.hip -- accumulated rotation angles on gfx950.
//
//   theta[s, t, p] = wrap( sum_{u <= t} phi[s, u, p] )  in [-pi, pi)
//
// one independent segment per (batch, angle head) s and rotary pair p.
// ("Why Do Accumulated Transformations Extrapolate?", Sec. 5 "SO(2)
// notation": commuting block rotations accumulate by adding their angles;
// Sec. 2.2 eq. (6): the route from j to i holds steps j+1..i, hence the
// inclusive sum.)
//
// The kernel is HBM-bound (4 bytes read + 4 bytes written per element), so
// it is built like a copy: one read of phi, one write of theta, little
// arithmetic per element, and no memory fences.
//
// Number format.  Angles are accumulated as fixed-point turns with 48
// fractional bits, held in 64-bit integers: an angle a becomes
// round(frac(a / 2 pi) * 2^48).  Integer addition is exact and associative,
// so the result is the exact sum of the converted steps (each step is
// rounded once, by at most 2^-49 turn = 1.1e-14 rad), the reduction mod 2 pi
// is the wrap-around of the low 48 bits, and the result does not depend on
// the order in which partial sums are combined: runs are bit-reproducible.
// The conversion is a few fp64 operations: after subtracting the nearest
// whole turn, adding 24 = 1.5 * 2^4 pins the exponent, so the low 48
// mantissa bits of the sum are the wanted fraction.  The way back puts the
// 48 bits into a double of fixed exponent again, so every output is the
// correctly rounded fp32 of an exact fixed-point value.
//
// Work split.  A workgroup (256 threads) owns one chunk of CH consecutive
// tokens of one segment, all P pairs: each thread loads T consecutive token
// rows of 4 pairs (one float4 per row; a wave reads whole rows) and keeps
// them in registers.  Thread, wave and workgroup partial sums are combined
// with lane shuffles and one LDS exchange.
//
// Chunks are chained with decoupled look-back (Merrill & Garland,
// "Single-pass Parallel Prefix Scan with Decoupled Look-back", 2016): a
// chunk publishes its aggregate as soon as it has it, sums the published
// aggregates of its predecessors back to the nearest published inclusive
// prefix, and then publishes its own inclusive prefix.  Value and status
// share one 64-bit word (48 value bits, 2 status bits), so a single atomic
// load sees both and no fence is needed.  Chunks are numbered in launch
// order (blockIdx), with no ticket counter; a chunk that finds a predecessor
// still unpublished after a bounded number of polls reduces that
// predecessor's angles itself from phi ("decoupled fallback", Smith, Levien
// and Owens, 2025), so progress never depends on the order in which the
// hardware schedules workgroups, and every wait ends.
//
// State reuse without clearing kernels or fences.  The caller's state buffer
// holds a 256-byte header and two interleaved halves of 64-bit words
// (completion counters, then status words).  A call uses the half named by
// the header's parity (all zero on entry), clears the other half (which the
// previous call used) and, in its last workgroup to finish, flips the parity
// and records how many words it dirtied.  The next launch on the stream sees all of it at the kernel
// boundary.  A buffer zero-filled once therefore serves any number of calls
// of any size that fits it.
#include "angle_fixed.hpp"
#include "arp_device.hpp"
#include "arp_internal.hpp"

namespace arp {

namespace {

constexpr int SCAN_THREADS = 256;
// Polls of an unpublished word before its chunk is reduced from the source
// here.  A build with ARP_SCAN_FALLBACK_POLLS=0 is a test variant: it ignores
// every published word and reduces each predecessor chunk from the source, so
// that the fallback path (reduce_pair and its lane combine) produces every
// prefix; its angles must equal the normal build's bit for bit.
#ifndef ARP_SCAN_FALLBACK_POLLS
#define ARP_SCAN_FALLBACK_POLLS 256
#endif
constexpr int FALLBACK_POLLS = ARP_SCAN_FALLBACK_POLLS;
constexpr bool FROM_SOURCE = FALLBACK_POLLS == 0;
constexpr int GROUP = 16;            // workgroups per completion counter
constexpr uint64_t ST_AGG = 1, ST_INC = 2, ST_MASK = 3;

// Header of the state buffer, padded to 256 bytes so that every 128-byte
// cache line of the status words belongs to exactly one half (the halves are
// written by different kinds of store).  Read and written with agent-scope
// atomics only.
struct ScanHeader {
  uint32_t parity;     // half used by the next call
  uint32_t pad;
  uint32_t done[2];    // finished groups of workgroups of the call using each half
  uint64_t used[2];    // words dirtied by the last use of each half
  uint64_t reserved[28];
};
static_assert(sizeof(ScanHeader) == 256, "header size");

// Logical status word w of half h: halves interleave in blocks of 32 words,
// a layout that does not depend on the problem's shape.
__device__ __forceinline__ size_t phys_word(size_t w, uint32_t h) {
  return ((w >> 5) * 2 + h) * 32 + (w & 31);
}

__device__ __forceinline__ uint64_t shfl_up64(uint64_t v, int delta) {
  const uint32_t lo = __shfl_up((uint32_t)v, delta);
  const uint32_t hi = __shfl_up((uint32_t)(v >> 32), delta);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t peek(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish(uint64_t* p, uint64_t value, uint64_t status) {
  __hip_atomic_store(p, (value << 16) | status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- where the step angles come from --------------------------------------
// A source gives the angle of (segment s = b * Hphi + g, token, pair) one at a
// time (at), or T consecutive tokens x 4 pairs at once (rows; tbase is even,
// tokens past L may hold anything, the kernel zeroes them).

// phi [B * Hphi, L, P] in memory.
template <int P>
struct PhiTensor {
  const float* __restrict__ phi;
  int L;
  __device__ float at(int s, int tok, int p) const { return phi[((size_t)s * L + tok) * P + p]; }
  template <int T>
  __device__ void rows(int s, int tbase, int cq, float4 (&x)[T]) const {
    const float* sp = phi + (size_t)s * L * P;
    // Loads are unconditional (rows clamped into the segment) so that all T
    // of them are in flight at once.
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int tok = min(tbase + t, L - 1);
      x[t] = *reinterpret_cast<const float4*>(sp + (size_t)tok * P + cq * 4);
    }
  }
};

// Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): the block of four 64-bit words for counter c and
// key (k0, k1), in place.
// The 128-bit product of a and b from four 32 x 32 + 64 multiply-adds
// (v_mad_u64_u32), the partial products shared between the two halves:
// a b = a1 b1 2^64 + (a1 b0 + a0 b1) 2^32 + a0 b0.  No sum overflows 64 bits:
// (2^32 - 1)^2 + 2 (2^32 - 1) < 2^64.
__device__ __forceinline__ void mulhilo64(uint64_t a, uint64_t b, uint64_t& lo, uint64_t& hi) {
  const uint32_t a0 = (uint32_t)a, a1 = (uint32_t)(a >> 32);
  const uint32_t b0 = (uint32_t)b, b1 = (uint32_t)(b >> 32);
  const uint64_t p00 = (uint64_t)a0 * b0;
  const uint64_t t = (uint64_t)a1 * b0 + (p00 >> 32);
  const uint64_t u = (uint64_t)a0 * b1 + (uint32_t)t;
  hi = (uint64_t)a1 * b1 + ((t >> 32) + (u >> 32));
  lo = (u << 32) | (uint32_t)p00;
}

__device__ __forceinline__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t lo0, hi0, lo1, hi1;
    mulhilo64(M0, c[0], lo0, hi0);
    mulhilo64(M1, c[2], lo1, hi1);
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += W0;
    k1 += W1;
  }
}

// The random variant's steps ("Why Do Accumulated Transformations
// Extrapolate?", App. D "Model variants": independent per position and pair,
// uniform on (-f_b, f_b), redrawn every forward pass), generated where they
// are used.  One Philox block (key (seed, 0), counter (c, step, 0, 0)) covers
// tokens 2m, 2m+1 of pairs 4j..4j+3 of segment s, c = (s * ceil(L/2) + m) *
// P/4 + j; word p%4 serves pair p, its low 32 bits the even token and its high
// 32 bits the odd one; 32 bits w give phi = bound[g][p] * (2 w 2^-32 - 1),
// formed in fp64 and rounded once to fp32.
template <int P>
struct RandomAngles {
  const float* __restrict__ bound;  // [Hphi, P]
  uint64_t seed, step;
  int L, Hphi;
  __device__ void block(int s, int m, int j, uint64_t (&w)[4]) const {
    w[0] = ((uint64_t)s * (uint64_t)((L + 1) >> 1) + (uint64_t)m) * (uint64_t)(P / 4) + (uint64_t)j;
    w[1] = step;
    w[2] = 0;
    w[3] = 0;
    philox4x64_10(w, seed, 0);
  }
  __device__ static float draw(float b, uint32_t bits) {
#pragma clang fp contract(off)
    const double u = (double)bits * 0x1p-32;
    return (float)((double)b * (2.0 * u - 1.0));
  }
  __device__ float at(int s, int tok, int p) const {
    uint64_t w[4];
    block(s, tok >> 1, p >> 2, w);
    const uint64_t x = w[p & 3];
    return draw(bound[(s % Hphi) * P + p], (tok & 1) ? (uint32_t)(x >> 32) : (uint32_t)x);
  }
  template <int T>
  __device__ void rows(int s, int tbase, int cq, float4 (&x)[T]) const {
    static_assert(T % 2 == 0, "token pairs");
    const float4 b = *reinterpret_cast<const float4*>(bound + (s % Hphi) * P + cq * 4);
#pragma unroll
    for (int i = 0; i < T / 2; ++i) {
      uint64_t w[4];
      block(s, (tbase >> 1) + i, cq, w);
      x[2 * i] = make_float4(draw(b.x, (uint32_t)w[0]), draw(b.y, (uint32_t)w[1]),
                             draw(b.z, (uint32_t)w[2]), draw(b.w, (uint32_t)w[3]));
      x[2 * i + 1] = make_float4(draw(b.x, (uint32_t)(w[0] >> 32)), draw(b.y, (uint32_t)(w[1] >> 32)),
                                 draw(b.z, (uint32_t)(w[2] >> 32)), draw(b.w, (uint32_t)(w[3] >> 32)));
    }
  }
};

// The learned token-rotation variant's steps (same section: one angle vector
// per token identity): phi[b, g, t, p] = table[tokens[b, t], g, p], ids
// clamped into [0, V).
template <int P>
struct TokenTable {
  const int32_t* __restrict__ tokens;  // [B, L]
  const float* __restrict__ table;     // [V, Hphi, P]
  int L, Hphi, V;
  __device__ const float* entry(int s, int tok) const {
    const int v = tokens[(size_t)(s / Hphi) * L + tok];
    return table + ((size_t)min(max(v, 0), V - 1) * Hphi + (s % Hphi)) * P;
  }
  __device__ float at(int s, int tok, int p) const { return entry(s, tok)[p]; }
  template <int T>
  __device__ void rows(int s, int tbase, int cq, float4 (&x)[T]) const {
    const float* e[T];
#pragma unroll
    for (int t = 0; t < T; ++t) e[t] = entry(s, min(tbase + t, L - 1));
#pragma unroll
    for (int t = 0; t < T; ++t) x[t] = *reinterpret_cast<const float4*>(e[t] + cq * 4);
  }
};

// Sum of the converted angles of pair p over tokens t0, t0 + step, ... < t1,
// taken from the source (the fallback when a predecessor's aggregate is not
// yet published).
template <class Src>
__device__ uint64_t reduce_pair(const Src& src, int s, int p, int t0, int t1, int step) {
  uint64_t acc = 0;
  for (int t = t0; t < t1; t += step) acc += to_fixed(src.at(s, t, p));
  return acc;
}

// Look-back of one chunk, run by wave 0.  Lane l serves pair p = l % P and
// every K-th predecessor (K = 64 / P lanes per pair), W predecessors each per
// pass, so a pass reads K * W predecessors of every pair at once.  Returns
// the sum of the aggregates of chunks 0 .. chunk-1 of the segment for pair p
// (the same value on the K lanes of a pair).
template <int P, class Src>
__device__ uint64_t look_back(const uint64_t* __restrict__ wh, size_t wbase, uint32_t half,
                              int chunk, const Src& src, int seg, int L, int CH, int lane) {
  constexpr int K = 64 / P;
  constexpr int W = 8;
  constexpr int SPAN = K * W;  // predecessors per pass
  const int p = lane % P, k0 = lane / P;
  uint64_t acc = 0;
  int d = chunk - 1;  // nearest predecessor not yet accounted for
  int polls = 0;
  while (d >= 0) {
    // All W loads are issued unconditionally (indices clamped into the
    // segment) so that they are in flight together; words before the first
    // chunk are then replaced by a final prefix of zero.
    uint64_t wv[W];
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const int c = d - (k0 + K * i);
      wv[i] = peek(wh + phys_word(wbase + (size_t)max(c, 0) * P + p, half));
    }
#pragma unroll
    for (int i = 0; i < W; ++i)
      if (d - (k0 + K * i) < 0) wv[i] = ST_INC;
    // First predecessor (by distance) whose word is not an aggregate.
    int stop = SPAN;
#pragma unroll
    for (int i = W - 1; i >= 0; --i)
      if ((wv[i] & ST_MASK) != ST_AGG) stop = k0 + K * i;
    if (K == 2) stop = min(stop, __shfl_xor(stop, 32));
    if (FROM_SOURCE) stop = 0;
    uint64_t part = 0;
#pragma unroll
    for (int i = 0; i < W; ++i)
      if (k0 + K * i < stop) part += wv[i] >> 16;
    if (!FROM_SOURCE && stop < SPAN && (stop % K) == k0) {
      const uint64_t w = wv[stop / K];
      if ((w & ST_MASK) == ST_INC) part += (w >> 16) | (1ull << 62);  // mark: found final prefix
    }
    if (K == 2) {
      const uint32_t lo = __shfl_xor((uint32_t)part, 32), hi = __shfl_xor((uint32_t)(part >> 32), 32);
      part += ((uint64_t)hi << 32) | lo;
    }
    const bool found = (part >> 62) & 1;
    acc += part & ~(1ull << 62);
    if (found) break;
    if (stop == SPAN) {
      d -= SPAN;
      polls = 0;
      continue;
    }
    // Predecessor d - stop has published nothing yet: wait for it, or after
    // enough polls reduce its angles from phi here.
    d -= stop;
    if (stop > 0) polls = 0;
    if (++polls > FALLBACK_POLLS) {
      const int t0 = d * CH, t1 = min(t0 + CH, L);
      uint64_t r = reduce_pair(src, seg, p, t0 + k0, t1, K);
      if (K == 2) {
        const uint32_t lo = __shfl_xor((uint32_t)r, 32), hi = __shfl_xor((uint32_t)(r >> 32), 32);
        r += ((uint64_t)hi << 32) | lo;
      }
      acc += r;
      --d;
      polls = 0;
    } else {
      if (polls < 8) __builtin_amdgcn_s_sleep(1);
      else __builtin_amdgcn_s_sleep(8);
    }
  }
  return acc;
}

// The key rotation of the fused epilogue (kr == nullptr: none): the bf16
// k (and v) rows of the chunk's tokens for every head of the segment.
struct RotEpilogue {
  const uint16_t* __restrict__ k;
  const uint16_t* __restrict__ v;
  uint16_t* __restrict__ kr;
  uint16_t* __restrict__ vr;
  float* __restrict__ kmax;
  int H, Hphi, Lp;
  int rot_qk, rot_v;
};

template <int P, int T, int MINB, class Src>
__global__ __launch_bounds__(SCAN_THREADS, MINB) void angle_scan_kernel(
    Src src, float* __restrict__ theta, ScanHeader* __restrict__ hdr,
    uint64_t* __restrict__ words, int L, int nchunks, int exclusive, RotEpilogue rot) {
  constexpr int CPT = P / 4;              // threads per token row (4 pairs each)
  constexpr int RG = SCAN_THREADS / CPT;  // row groups per chunk
  constexpr int CH = RG * T;              // tokens per chunk
  constexpr int RGW = 64 / CPT;           // row groups per wave
  constexpr int NWAVE = SCAN_THREADS / 64;
  static_assert(P == 32 || P == 64, "P must be 32 or 64");

  __shared__ uint64_t s_wtot[NWAVE][P];  // per-wave totals
  __shared__ uint64_t s_carry[P];        // exclusive prefix of this chunk (+ 2^47)
  __shared__ uint32_t s_kmax2[4];        // fused rotation: max |k~|^2 per key tile of the chunk

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cq = tid % CPT;
  const int rg = tid / CPT;
  const int nblocks = gridDim.x;
  const int seg = blockIdx.x / nchunks;
  const int chunk = blockIdx.x % nchunks;
  const int tbase = chunk * CH + rg * T;

  // The header was last written by an earlier launch, so plain (cached)
  // loads see it; every workgroup reads it before it counts itself done.
  const uint32_t half = hdr->parity & 1u;
  const uint64_t stale = hdr->used[half ^ 1u];
  const int ngroups = (nblocks + GROUP - 1) / GROUP;

  // ---- T rows x 4 pairs of steps; thread totals of the converted angles ----
  // Rows past the end of the segment count as zero.
  float4 x[T];
  src.template rows<T>(seg, tbase, cq, x);
#pragma unroll
  for (int t = 0; t < T; ++t)
    if (tbase + t >= L) x[t] = make_float4(0.f, 0.f, 0.f, 0.f);
  uint64_t tot[4] = {0, 0, 0, 0};
#pragma unroll
  for (int t = 0; t < T; ++t) {
    tot[0] += to_fixed(x[t].x);
    tot[1] += to_fixed(x[t].y);
    tot[2] += to_fixed(x[t].z);
    tot[3] += to_fixed(x[t].w);
  }

  // ---- exclusive prefix of this thread within the chunk ----
  // Inclusive scan over the wave's row groups (lanes CPT apart), then the
  // totals of the earlier waves from LDS.
  uint64_t pre[4];
  const int rgw = lane / CPT;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint64_t v = tot[c];
#pragma unroll
    for (int off = 1; off < RGW; off <<= 1) {
      const uint64_t u = shfl_up64(v, off * CPT);
      if (rgw >= off) v += u;
    }
    pre[c] = v - tot[c];
    if (rgw == RGW - 1) s_wtot[wave][cq * 4 + c] = v;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 4; ++c)
    for (int w = 0; w < wave; ++w) pre[c] += s_wtot[w][cq * 4 + c];

  // ---- publish the aggregate, look back, publish the inclusive prefix ----
  const size_t wbase = (size_t)ngroups + ((size_t)seg * nchunks) * P;
  if (wave == 0) {
    const int p = lane % P;
    uint64_t agg = 0;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) agg += s_wtot[w][p];
    uint64_t* my = words + phys_word(wbase + (size_t)chunk * P + p, half);
    if (lane < P) publish(my, agg, chunk == 0 ? ST_INC : ST_AGG);
    uint64_t acc = 0;
    if (chunk > 0) {
      acc = look_back<P>(words, wbase, half, chunk, src, seg, L, CH, lane);
      if (lane < P) publish(my, acc + agg, ST_INC);
    }
    if (lane < P) s_carry[p] = acc + FIXED_ZERO;  // turns [0,1) into [-1/2,1/2) below
  }
  __syncthreads();

  // ---- outputs: running angle from the thread's first row ----
  // The steps are converted again from the raw angles rather than kept from
  // the first pass: holding T x 4 64-bit values live across the look-back
  // would cut the number of resident workgroups by up to four.  The empty asm
  // hides the equality from the compiler so that it cannot merge the two
  // conversions.
#pragma unroll
  for (int t = 0; t < T; ++t) asm volatile("" : "+v"(x[t].x), "+v"(x[t].y), "+v"(x[t].z), "+v"(x[t].w));
  float* seg_theta = theta + (size_t)seg * L * P;
  uint64_t run[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) run[c] = pre[c] + s_carry[cq * 4 + c];
  float ang[T][4];  // the thread's angles, for the fused key rotation
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const float xs[4] = {x[t].x, x[t].y, x[t].z, x[t].w};
    float out[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint64_t step = to_fixed(xs[c]);
      if (exclusive) {
        out[c] = to_radians_offset(run[c]);
        run[c] += step;
      } else {
        run[c] += step;
        out[c] = to_radians_offset(run[c]);
      }
      ang[t][c] = out[c];
    }
    const int tok = tbase + t;
    if (tok < L)
      // Streaming store: theta is not read again by this kernel, and keeping
      // it out of the caches measured 5-15% faster than a plain store.
      __builtin_nontemporal_store(f32x4{out[0], out[1], out[2], out[3]},
                                  reinterpret_cast<f32x4*>(seg_theta + (size_t)tok * P + cq * 4));
  }

  // ---- fused key rotation: the pre-rotation pass of these tokens ----
  // Thread (row group rg, chunk cq) owns 16 bytes (4 pairs) of T consecutive
  // rows, which lie in one 64-key tile (T divides 64); the arithmetic is the
  // pass's (rotate.hip), operation for operation, so k~, v~ and the tile
  // maxima are bit-identical to it: hardware sin/cos of the angle, fp32
  // rotation rounded to bf16, |k~|^2 from the stored values summed over the
  // row's lanes in the same butterfly order.
  if constexpr (64 % T == 0 && CH % 64 == 0 && CH / 64 <= 4) {  // plans of whole key tiles
   if (rot.kr != nullptr) {
    constexpr int D = 2 * P;
    const int nh = rot.Hphi == 1 ? rot.H : 1;
    const int bh0 = (seg / rot.Hphi) * rot.H + (rot.Hphi == 1 ? 0 : seg % rot.Hphi);
    const int tile = (rg * T) / 64;  // key tile of this thread's rows within the chunk
    for (int hh = 0; hh < nh; ++hh) {
      const int bh = bh0 + hh;
      if (tid < 4) s_kmax2[tid] = 0u;
      __syncthreads();
      uint32_t n2max = 0u;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int tok = tbase + t;  // the same on the CPT lanes of a row
        if (tok >= rot.Lp) break;
        u32x4 ka = {0, 0, 0, 0}, va = {0, 0, 0, 0};
        if (tok < L) {
          const size_t off = ((size_t)bh * L + tok) * D + cq * 8;
          ka = *reinterpret_cast<const u32x4*>(rot.k + off);
          if (rot.rot_v) va = *reinterpret_cast<const u32x4*>(rot.v + off);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float sn, cs;
            __sincosf(ang[t][e], &sn, &cs);
            float k0 = lo_bf16(ka[e]), k1 = hi_bf16(ka[e]);
            if (rot.rot_qk) rotate_pair(k0, k1, cs, sn);
            ka[e] = pack_bf16x2(k0, k1);
            if (rot.rot_v) {
              float v0 = lo_bf16(va[e]), v1 = hi_bf16(va[e]);
              rotate_pair(v0, v1, cs, sn);
              va[e] = pack_bf16x2(v0, v1);
            }
          }
        }
        const size_t roff = ((size_t)bh * rot.Lp + tok) * D + cq * 8;
        *reinterpret_cast<u32x4*>(rot.kr + roff) = ka;
        if (rot.rot_v) *reinterpret_cast<u32x4*>(rot.vr + roff) = va;
        float n2 = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float k0 = lo_bf16(ka[e]), k1 = hi_bf16(ka[e]);
          n2 = fmaf(k0, k0, fmaf(k1, k1, n2));
        }
#pragma unroll
        for (int m = 1; m < CPT; m <<= 1) n2 += __shfl_xor(n2, m);
        n2max = max(n2max, __float_as_uint(n2));  // non-negative floats order as their bits
      }
      if (cq == 0 && n2max != 0u) atomicMax(&s_kmax2[tile], n2max);
      __syncthreads();
      const int t0 = chunk * CH / 64;  // the chunk's first key tile
      if (tid < CH / 64 && t0 + tid < rot.Lp / 64)
        rot.kmax[(size_t)bh * (rot.Lp / 64) + t0 + tid] = sqrtf(__uint_as_float(s_kmax2[tid]));
    }
   }
  }

  // ---- state upkeep: clear this block's share of the other half ----
  {
    const uint64_t per = (stale + nblocks - 1) / nblocks;
    const uint64_t w0 = per * blockIdx.x;
    const uint64_t w1 = min(stale, w0 + per);
    for (uint64_t w = w0 + tid; w < w1; w += SCAN_THREADS) words[phys_word(w, half ^ 1u)] = 0;
  }
  __syncthreads();  // every thread of the block is past its last use of the state

  // Completion count in two levels (a counter per GROUP workgroups, then one
  // for the groups), so that no single address takes an atomic from every
  // workgroup.  The workgroup that completes the last group hands the state
  // to the next call: every other workgroup has read the header and finished
  // with the status words by then, and the next launch sees these header
  // fields at the kernel boundary.
  if (tid == 0) {
    const int grp = blockIdx.x / GROUP;
    const uint32_t gsize = (uint32_t)min(GROUP, nblocks - grp * GROUP);
    uint64_t* gc = words + phys_word((size_t)grp, half);
    const uint64_t pg =
        __hip_atomic_fetch_add(gc, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (pg == gsize - 1) {
      const uint32_t pd =
          __hip_atomic_fetch_add(&hdr->done[half], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (pd == (uint32_t)(ngroups - 1)) {
        __hip_atomic_store(&hdr->done[half], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&hdr->used[half], (uint64_t)ngroups + (uint64_t)nblocks * P,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&hdr->used[half ^ 1u], (uint64_t)0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&hdr->parity, half ^ 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

constexpr int rows_per_group(int P) { return SCAN_THREADS / (P / 4); }

}  // namespace

ScanPlan scan_plan(const Geometry& g, bool rotating) {
  // Rows per thread on large grids: 10, built for four workgroups per CU
  // (120 registers, no spills), so that three other workgroups stream while
  // one waits in its look-back.  Measured on 4 x 32 x 8192 x 64 (537 MB):
  // 10 rows 106 us, 12 rows 106 us (2 spilled registers), 16 rows at three
  // workgroups per CU 113 us, 16 rows at four (17 spilled) slower still,
  // 8 rows 114 us, 32 rows 124 us, 4 rows 142 us; 4 x 32 x 16384 x 32:
  // 10 rows 105 us, 8 rows 109 us.  Grids of at most 1024 16-row chunks take
  // 8 rows (2 x 8 x 16384 x 32: 21.6 us), smaller problems 4 rows so that the
  // grid still covers the chip.
  const long nseg = (long)g.B * g.Hphi;
  const int rg = rows_per_group(g.P);
  auto blocks = [&](int T) { return nseg * ((g.L + (long)rg * T - 1) / ((long)rg * T)); };
  int T = 4, minb = 1;
  if (blocks(16) > 1024 && !rotating) {
    T = 10;
    minb = 4;
  } else if (blocks(8) >= 512) {
    T = 8;  // (also where a rotating scan would take 10: its chunks hold whole key tiles)
  }
  ScanPlan sp;
  sp.rows_per_thread = T;
  sp.min_blocks = minb;
  sp.chunk = rg * T;
  sp.nchunks = (g.L + sp.chunk - 1) / sp.chunk;
  return sp;
}

size_t scan_state_bytes(const Geometry& g) {
  // Sized for the smallest chunk any plan uses, so the bound holds whatever
  // rows-per-thread the plan picks.
  const size_t min_chunk = (size_t)rows_per_group(g.P) * 4;
  const size_t nchunks = (g.L + min_chunk - 1) / min_chunk;
  const size_t nblocks = (size_t)g.B * g.Hphi * nchunks;
  const size_t words = (nblocks + GROUP - 1) / GROUP + nblocks * g.P;  // counters + status
  const size_t blocks = (words + 31) / 32;  // both halves, 32-word blocks
  const size_t bytes = sizeof(ScanHeader) + blocks * 2 * 32 * sizeof(uint64_t);
  return (bytes + 255) & ~(size_t)255;
}

namespace {

template <int P, class Src>
hipError_t launch_scan(const Geometry& g, const Src& src, float* theta, void* scan_state,
                       hipStream_t stream, const RotEpilogue& rot = RotEpilogue{}) {
  const ScanPlan sp = scan_plan(g, rot.kr != nullptr);
  const long nblocks = (long)g.B * g.Hphi * sp.nchunks;
  auto* hdr = reinterpret_cast<ScanHeader*>(scan_state);
  auto* words = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(scan_state) + sizeof(ScanHeader));
  const int excl = (g.flags & ARP_SCAN_EXCLUSIVE) ? 1 : 0;
  if (nblocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)nblocks);
  dim3 block(SCAN_THREADS);
#define ARP_SCAN_LAUNCH(TT, MB)                                                               \
  hipLaunchKernelGGL((angle_scan_kernel<P, TT, MB, Src>), grid, block, 0, stream, src, theta, hdr, \
                     words, g.L, sp.nchunks, excl, rot)
  if (sp.rows_per_thread == 10) {
    ARP_SCAN_LAUNCH(10, 4);
  } else if (sp.rows_per_thread == 8) {
    ARP_SCAN_LAUNCH(8, 1);
  } else {
    ARP_SCAN_LAUNCH(4, 1);
  }
#undef ARP_SCAN_LAUNCH
  return hipGetLastError();
}

// phi of the random variant written out: one thread per Philox block (two
// tokens x four pairs; consecutive threads take consecutive pair groups).
template <int P>
__global__ __launch_bounds__(256) void random_phi_kernel(RandomAngles<P> src, float* __restrict__ phi,
                                                         long nseg) {
  constexpr int J = P / 4;
  const long half = (src.L + 1) >> 1;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= nseg * half * J) return;
  const int j = (int)(i % J);
  const long sm = i / J;
  const int m = (int)(sm % half);
  const int seg = (int)(sm / half);
  float4 x[2];
  src.template rows<2>(seg, 2 * m, j, x);
  float* row = phi + ((size_t)seg * src.L + 2 * m) * P + 4 * j;
  *reinterpret_cast<float4*>(row) = x[0];
  if (2 * m + 1 < src.L) *reinterpret_cast<float4*>(row + P) = x[1];
}

// Constant steps need no scan: the sum of n copies of one fixed-point step is
// n times it, mod 2^48 -- the very integer the scan would reach, so the result
// is bit-identical to scanning the broadcast steps.  One thread per token and
// four pairs, consecutive threads along the row.
template <int P>
__global__ __launch_bounds__(256) void const_angles_kernel(const float* __restrict__ freq,
                                                           float* __restrict__ theta, long n, int L,
                                                           int Hphi, int exclusive) {
  constexpr int J = P / 4;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int j = (int)(i % J);
  const long st = i / J;  // segment * L + token
  const int t = (int)(st % L);
  const int g = (int)((st / L) % Hphi);
  const float4 f = *reinterpret_cast<const float4*>(freq + g * P + 4 * j);
  const uint64_t count = (uint64_t)(exclusive ? t : t + 1);
  const float fx[4] = {f.x, f.y, f.z, f.w};
  float out[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) out[c] = to_radians_offset(FIXED_ZERO + count * to_fixed(fx[c]));
  __builtin_nontemporal_store(f32x4{out[0], out[1], out[2], out[3]},
                              reinterpret_cast<f32x4*>(theta + st * P + 4 * j));
}

}  // namespace

hipError_t launch_angle_scan(const Geometry& g, const float* phi, float* theta, void* scan_state,
                             hipStream_t stream) {
  if (g.P == 32) return launch_scan<32>(g, PhiTensor<32>{phi, g.L}, theta, scan_state, stream);
  return launch_scan<64>(g, PhiTensor<64>{phi, g.L}, theta, scan_state, stream);
}

hipError_t launch_angle_scan_rotate(const Geometry& g, const float* phi, float* theta,
                                    void* scan_state, const KeyRotation& kr, hipStream_t stream) {
  const ScanPlan sp = scan_plan(g, true);
  if (sp.chunk % KEY_TILE != 0 || sp.chunk / KEY_TILE > 4 || KEY_TILE % sp.rows_per_thread != 0) {
    const hipError_t e = launch_angle_scan(g, phi, theta, scan_state, stream);
    if (e != hipSuccess) return e;
    return launch_rotate_kv(g, kr.k, kr.v, theta, kr.kr, kr.vr, kr.kmax, stream);
  }
  const RotEpilogue rot{static_cast<const uint16_t*>(kr.k), static_cast<const uint16_t*>(kr.v),
                        kr.kr, kr.vr, kr.kmax, g.H, g.Hphi, g.Lp,
                        (g.flags & ARP_ROTATE_QK) ? 1 : 0, (g.flags & ARP_ROTATE_V) ? 1 : 0};
  if (g.P == 32) return launch_scan<32>(g, PhiTensor<32>{phi, g.L}, theta, scan_state, stream, rot);
  return launch_scan<64>(g, PhiTensor<64>{phi, g.L}, theta, scan_state, stream, rot);
}

hipError_t launch_angle_scan_random(const Geometry& g, uint64_t seed, uint64_t step,
                                    const float* bound, float* theta, void* scan_state,
                                    hipStream_t stream) {
  if (g.P == 32)
    return launch_scan<32>(g, RandomAngles<32>{bound, seed, step, g.L, g.Hphi}, theta, scan_state,
                           stream);
  return launch_scan<64>(g, RandomAngles<64>{bound, seed, step, g.L, g.Hphi}, theta, scan_state,
                         stream);
}

hipError_t launch_angle_scan_tokens(const Geometry& g, const int32_t* tokens, const float* table,
                                    int vocab, float* theta, void* scan_state, hipStream_t stream) {
  if (g.P == 32)
    return launch_scan<32>(g, TokenTable<32>{tokens, table, g.L, g.Hphi, vocab}, theta, scan_state,
                           stream);
  return launch_scan<64>(g, TokenTable<64>{tokens, table, g.L, g.Hphi, vocab}, theta, scan_state,
                         stream);
}

hipError_t launch_angle_scan_const(const Geometry& g, const float* freq, float* theta,
                                   hipStream_t stream) {
  const long n = (long)g.B * g.Hphi * g.L * (g.P / 4);
  if (n == 0) return hipSuccess;
  const long blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const int excl = (g.flags & ARP_SCAN_EXCLUSIVE) ? 1 : 0;
  if (g.P == 32)
    hipLaunchKernelGGL(const_angles_kernel<32>, dim3((unsigned)blocks), dim3(256), 0, stream, freq,
                       theta, n, g.L, g.Hphi, excl);
  else
    hipLaunchKernelGGL(const_angles_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, freq,
                       theta, n, g.L, g.Hphi, excl);
  return hipGetLastError();
}

hipError_t launch_random_phi(const Geometry& g, uint64_t seed, uint64_t step, const float* bound,
                             float* phi, hipStream_t stream) {
  const long nseg = (long)g.B * g.Hphi;
  const long n = nseg * ((g.L + 1) / 2) * (g.P / 4);
  if (n == 0) return hipSuccess;
  const long blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (g.P == 32)
    hipLaunchKernelGGL(random_phi_kernel<32>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       RandomAngles<32>{bound, seed, step, g.L, g.Hphi}, phi, nseg);
  else
    hipLaunchKernelGGL(random_phi_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       RandomAngles<64>{bound, seed, step, g.L, g.Hphi}, phi, nseg);
  return hipGetLastError();
}

}  // namespace arp
