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
// Design (HBM-bound; 4 bytes read + 4 bytes written per element):
//  * A workgroup (256 threads) owns one chunk of CH consecutive tokens of one
//    segment, all P pairs.  Each thread loads float4s (4 adjacent pairs) of
//    T consecutive tokens -- a wave reads whole 128/256-byte rows -- and keeps
//    them in registers, so phi is read from HBM exactly once.
//  * Angles are accumulated as 64-bit fixed-point turns: an angle a maps to
//    the integer round(frac(a / 2 pi) * 2^63) * 2 (mod 2^64), whose signed
//    value spans [-pi, pi).  Integer addition mod 2^64 is exact and
//    associative, so (i) the sum is the exact sum of the converted steps --
//    no drift with the sequence length (a plain fp32 running sum of 32K
//    angles drifts by ~1e-3 rad), (ii) the reduction mod 2 pi is the
//    overflow itself, and (iii) the result does not depend on the order in
//    which chunk totals are combined: runs are bit-reproducible.  Each step's
//    conversion (in fp64) is accurate to ~4e-16 rad.
//  * Chunks are chained with decoupled look-back (Merrill & Garland,
//    "Single-pass Parallel Prefix Scan with Decoupled Look-back", 2016): a
//    chunk publishes its aggregate at once, then sums its predecessors'
//    published aggregates, back to the nearest published inclusive prefix.
//    All 256 threads take part: each pass reads a window of 16-32
//    predecessors per pair in parallel, so the look-back costs a pass or
//    two of memory latency instead of one round trip per predecessor.
//    Fixed-point values are even, so the low bit of each published 64-bit
//    word is free to be the "ready" tag (zeroed memory = not ready): one
//    atomic load sees value and flag together and no fence is needed.
//  * Chunk order comes from a per-segment ticket (atomic counter), so a
//    chunk only ever waits on chunks that were already running.
//  * The last chunk of a segment to finish clears that segment's state, so
//    the state buffer is zero again for the next call on the stream.
//  * Every wait is bounded; a chunk that gives up writes NaN angles.
#include "arp_device.hpp"
#include "arp_internal.hpp"

namespace arp {

namespace {

constexpr int SCAN_THREADS = 256;
constexpr uint32_t SPIN_LIMIT = 1u << 22;  // look-back passes before giving up
constexpr int LB_R = 4;                    // predecessors per look-back slot
constexpr int LB_ALL = 0, LB_FOUND = 1, LB_BLOCKED = 2;

// Angle (radians, fp32) -> even 64-bit fixed-point turns.  frac() is taken
// in fp64, exact for |a| < 2^50 turns.
__device__ __forceinline__ uint64_t to_turns(float a) {
  const double t = (double)a * 0.15915494309189533577;  // 1 / (2 pi)
  const double f = t - rint(t);                           // [-0.5, 0.5]
  return ((uint64_t)(int64_t)rint(f * 9223372036854775808.0)) << 1;
}
// Fixed-point turns -> radians in [-pi, pi) (then rounded to fp32).
__device__ __forceinline__ float to_radians(uint64_t u) {
  return (float)((double)(int64_t)u * 3.4061215800865545e-19);  // 2 pi / 2^64
}
__device__ __forceinline__ void publish(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v | 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t peek(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool is_ready(uint64_t w) { return (w & 1u) != 0; }
__device__ __forceinline__ uint64_t value_of(uint64_t w) { return w & ~(uint64_t)1; }

// hdr: 4 words per segment {ticket, done, failed, unused}.
// words: per segment [nchunks][P][2] (aggregate, inclusive prefix).
template <int P, int T>
__global__ __launch_bounds__(SCAN_THREADS) void angle_scan_kernel(
    const float* __restrict__ phi, float* __restrict__ theta, uint32_t* __restrict__ hdr,
    uint64_t* __restrict__ words, int L, int nchunks, int exclusive) {
  constexpr int CPT = P / 4;              // threads per token row
  constexpr int RG = SCAN_THREADS / CPT;  // row groups per chunk
  constexpr int CH = RG * T;              // tokens per chunk
  static_assert(P % 4 == 0 && SCAN_THREADS % CPT == 0 && P <= 64, "P must be 32 or 64");

  constexpr int SLOTS = SCAN_THREADS / P;  // look-back slots per pair
  __shared__ int s_chunk;
  __shared__ int s_last;
  __shared__ int s_fail;
  __shared__ uint64_t s_tot[RG * P];
  __shared__ uint64_t s_pre[P];   // exclusive prefix of this chunk, per pair
  __shared__ uint64_t s_agg[P];   // aggregate of this chunk, per pair
  __shared__ int s_chi[P];        // next predecessor to examine, per pair
  __shared__ int s_done[P];
  __shared__ uint64_t s_part[SLOTS * P];
  __shared__ int s_stat[SLOTS * P];

  const int seg = blockIdx.y;
  const int tid = threadIdx.x;
  const int cq = tid % CPT;
  const int rg = tid / CPT;
  uint32_t* h = hdr + 4 * seg;
  uint64_t* wseg = words + (size_t)seg * nchunks * P * 2;

  if (tid == 0) {
    s_chunk = (int)atomicAdd(&h[0], 1u);
    s_fail = 0;
  }
  __syncthreads();
  const int chunk = s_chunk;
  const int tbase = chunk * CH + rg * T;

  // Load this thread's T x 4 step angles (one HBM read of phi).
  const float* src = phi + (size_t)seg * L * P + cq * 4;
  float4 x[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int tok = tbase + t;
    x[t] = (tok < L) ? *reinterpret_cast<const float4*>(src + (size_t)tok * P)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  // Thread totals.
  uint64_t tot[4] = {0, 0, 0, 0};
#pragma unroll
  for (int t = 0; t < T; ++t) {
    tot[0] += to_turns(x[t].x);
    tot[1] += to_turns(x[t].y);
    tot[2] += to_turns(x[t].z);
    tot[3] += to_turns(x[t].w);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) s_tot[rg * P + cq * 4 + c] = tot[c];
  __syncthreads();

  // One thread per pair (all in wave 0): exclusive scan over the row groups
  // and publication of the chunk aggregate (the inclusive prefix for chunk 0).
  if (tid < P) {
    uint64_t run = 0;
    for (int r = 0; r < RG; ++r) {
      const uint64_t v = s_tot[r * P + tid];
      s_tot[r * P + tid] = run;
      run += v;
    }
    s_agg[tid] = run;
    publish(&wseg[((size_t)chunk * P + tid) * 2 + (chunk == 0 ? 1 : 0)], run);
    s_pre[tid] = 0;
    s_chi[tid] = chunk - 1;
    s_done[tid] = (chunk == 0);
  }
  __syncthreads();

  // Look-back over earlier chunks with every thread: per pair, SLOTS slots of
  // LB_R consecutive predecessors each, i.e. SLOTS * LB_R predecessors per
  // pass, loaded in parallel.  A pass stops at the nearest published inclusive
  // prefix (done), or at the first predecessor whose aggregate is not yet
  // published (retry from there).
  if (chunk > 0) {
    const int p = tid % P, slot = tid / P;
    uint32_t passes = 0;
    bool all_done = false;
    while (!all_done) {
      uint64_t part = 0;
      int stat = LB_ALL, used = LB_R;
      if (!s_done[p]) {
        const int c0 = s_chi[p] - slot * LB_R;
        uint64_t wi[LB_R], wa[LB_R];
#pragma unroll
        for (int r = 0; r < LB_R; ++r) {
          const int c = c0 - r;
          wi[r] = (c >= 0) ? peek(&wseg[((size_t)c * P + p) * 2 + 1]) : 0;
          wa[r] = (c >= 0) ? peek(&wseg[((size_t)c * P + p) * 2 + 0]) : 0;
        }
#pragma unroll
        for (int r = 0; r < LB_R; ++r) {
          if (stat != LB_ALL) break;
          const int c = c0 - r;
          if (c < 0) {
            stat = LB_FOUND;
            used = r;
          } else if (is_ready(wi[r])) {
            part += value_of(wi[r]);
            stat = LB_FOUND;
            used = r + 1;
          } else if (is_ready(wa[r])) {
            part += value_of(wa[r]);
          } else {
            stat = LB_BLOCKED;
            used = r;
          }
        }
      }
      s_part[slot * P + p] = part;
      s_stat[slot * P + p] = stat | (used << 2);
      __syncthreads();
      int blocked = 0;
      if (tid < P && !s_done[tid]) {
        uint64_t acc = s_pre[tid];
        int chi = s_chi[tid];
        int done = 0;
        for (int sl = 0; sl < SLOTS; ++sl) {
          const int st = s_stat[sl * P + tid];
          acc += s_part[sl * P + tid];
          if ((st & 3) == LB_FOUND) {
            done = 1;
            break;
          }
          if ((st & 3) == LB_BLOCKED) {
            chi -= sl * LB_R + (st >> 2);
            blocked = 1;
            break;
          }
          if (sl == SLOTS - 1) chi -= SLOTS * LB_R;
        }
        if (!done && ++passes > SPIN_LIMIT) {
          // give up: this segment's angles read NaN (flag seen by later chunks)
          s_fail = 1;
          __hip_atomic_store(&h[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          done = 1;
        }
        s_pre[tid] = acc;
        s_chi[tid] = chi;
        s_done[tid] = done;
      }
      if (__syncthreads_or(blocked)) __builtin_amdgcn_s_sleep(2);
      all_done = __syncthreads_and(tid < P ? s_done[tid] : 1);
    }
  }

  // Publish this chunk's inclusive prefix; lane 0 of the same wave then counts
  // the chunk as finished (its release covers the wave's publications).
  if (tid < P) {
    if (chunk > 0) publish(&wseg[((size_t)chunk * P + tid) * 2 + 1], s_pre[tid] + s_agg[tid]);
    if (tid == 0) {
      uint32_t prev = __hip_atomic_fetch_add(&h[1], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (prev == (uint32_t)(nchunks - 1));
    }
  }
  __syncthreads();

  // Second pass over the registers: running angle from the thread's start.
  uint64_t run[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) run[c] = s_pre[cq * 4 + c] + s_tot[rg * P + cq * 4 + c];
  const bool fail =
      s_fail != 0 || __hip_atomic_load(&h[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
  float* dst = theta + (size_t)seg * L * P + cq * 4;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const float xs[4] = {x[t].x, x[t].y, x[t].z, x[t].w};
    float out[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint64_t step = to_turns(xs[c]);
      if (exclusive) {
        out[c] = to_radians(run[c]);
        run[c] += step;
      } else {
        run[c] += step;
        out[c] = to_radians(run[c]);
      }
      if (fail) out[c] = __builtin_nanf("");
    }
    const int tok = tbase + t;
    if (tok < L)
      *reinterpret_cast<float4*>(dst + (size_t)tok * P) = make_float4(out[0], out[1], out[2], out[3]);
  }

  // The last chunk of the segment leaves the state zeroed for the next call.
  if (s_last) {
    for (int i = tid; i < nchunks * P * 2; i += SCAN_THREADS) wseg[i] = 0;
    if (tid == 0) {
      h[0] = 0;
      h[1] = 0;
      h[2] = 0;
    }
  }
}

constexpr int rows_per_group(int P) { return SCAN_THREADS / (P / 4); }

}  // namespace

ScanPlan scan_plan(const Geometry& g) {
  const int rg = rows_per_group(g.P);
  const long nseg = (long)g.B * g.Hphi;
  int T = 4;
  for (int cand : {16, 8}) {
    const long nch = (g.L + (long)rg * cand - 1) / ((long)rg * cand);
    if (nseg * nch >= 1024) {
      T = cand;
      break;
    }
  }
  ScanPlan sp;
  sp.rows_per_thread = T;
  sp.chunk = rg * T;
  sp.nchunks = (g.L + sp.chunk - 1) / sp.chunk;
  return sp;
}

size_t scan_state_bytes(const Geometry& g) {
  const size_t nseg = (size_t)g.B * g.Hphi;
  const size_t min_chunk = (size_t)rows_per_group(g.P) * 4;
  const size_t nchunks_max = (g.L + min_chunk - 1) / min_chunk;
  size_t bytes = nseg * 16 + nseg * nchunks_max * g.P * 2 * sizeof(uint64_t);
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_angle_scan(const Geometry& g, const float* phi, float* theta, void* scan_state,
                             hipStream_t stream) {
  const ScanPlan sp = scan_plan(g);
  const int nseg = g.B * g.Hphi;
  uint32_t* hdr = reinterpret_cast<uint32_t*>(scan_state);
  uint64_t* words = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(scan_state) + (size_t)nseg * 16);
  const int excl = (g.flags & ARP_SCAN_EXCLUSIVE) ? 1 : 0;
  dim3 grid(sp.nchunks, nseg);
  dim3 block(SCAN_THREADS);
#define ARP_SCAN_LAUNCH(PP, TT)                                                                   \
  hipLaunchKernelGGL((angle_scan_kernel<PP, TT>), grid, block, 0, stream, phi, theta, hdr, words, \
                     g.L, sp.nchunks, excl)
  if (g.P == 32) {
    if (sp.rows_per_thread == 16) ARP_SCAN_LAUNCH(32, 16);
    else if (sp.rows_per_thread == 8) ARP_SCAN_LAUNCH(32, 8);
    else ARP_SCAN_LAUNCH(32, 4);
  } else {
    if (sp.rows_per_thread == 16) ARP_SCAN_LAUNCH(64, 16);
    else if (sp.rows_per_thread == 8) ARP_SCAN_LAUNCH(64, 8);
    else ARP_SCAN_LAUNCH(64, 4);
  }
#undef ARP_SCAN_LAUNCH
  return hipGetLastError();
}

}  // namespace arp
