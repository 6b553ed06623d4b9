// attn_bwd.hip -- gradients of causal attention with accumulated SO(2)
// rotations (bf16 operands, fp32 accumulation) on the gfx950 matrix cores.
//
// The forward ("Why Do Accumulated Transformations Extrapolate?" eq. (2)-(4),
// with q~ = R(Theta) q etc. as in "AdaRoPE" Sec. 2.1 eq. (1)) differentiated:
//   do~_i = R(Theta_i) dO_i (value transport) or dO_i
//   D_i   = <do~_i, o~_i>,  o~_i = R(Theta_i) o_i (value transport) or o_i
//   P_ij  = 2^(s2_ij - lse2_i)                   (base-2 logits of the forward)
//   dS_ij = P_ij (<do~_i, v~_j> - D_i)
//   dq~_i = scale sum_j dS_ij k~_j,  dk~_j = scale sum_i dS_ij q~_i,
//   dv~_j = sum_i P_ij do~_i
//   dx = R(Theta)^T dx~ for every rotated x, and per pair
//   dTheta_t = <dq~_t, J q~_t> + <dk~_t, J k~_t> + <dv~_t, J v~_t> - <do~_t, J o~_t>
//   (J = [[0, -1], [1, 0]]; each term only when that tensor is rotated)
//   dphi_s = sum_{t >= s} dTheta_t (t > s for the exclusive scan), summed over
//   the heads that share one angle stream.
//
// Kernels, in stream order:
//  1. bwd_prep: one pass over q, k, v, o, dO and Theta per 64-token tile:
//     the bf16 operands (q~ scaled by scale log2 e, k~, v~, do~ row-major;
//     q~^T, k~^T, do~^T transposed through LDS), per-row -lse (padded with
//     -inf) and -D, and dTheta initialised with the value-transport term.
//  2. bwd_dkdv: key-stationary; a lane owns one key.  Per 32-query block:
//       S    = Q~ K~^T   - lse   (A: q~ rows from LDS, B: k~ row in registers)
//       dP'  = dO~ V~^T  - D     (A: do~ rows from LDS, B: v~ row in registers)
//       dS   = P * dP'
//       dV^T += dO~^T P,  dK^T += Q~^T dS   (A: transposed tiles from LDS)
//     The query rows sit in LDS in the swap_bits23 order, so the S and dP'
//     accumulators are directly the B operands of the dV^T / dK^T products.
//  3. bwd_dq: query-stationary (the forward's orientation); a lane owns one
//     query.  Per 64-key tile: S^T = K~ Q~^T - lse, dP'^T = V~ dO~^T - D,
//     dS^T = P^T * dP'^T, dQ^T += K~^T dS^T.
//  Both kernels end with the un-rotation of their gradients and add their
//  <dx~, J x~> terms to dTheta (each (t, p) owned by one lane).
//  4. reverse scan of dTheta into dphi: chunk totals, then the in-chunk
//     suffix sums plus the totals of the later chunks.
// With forget gates the logits carry G_i - G_j (G = log2 e times the prefix
// sums of log f, from the forward's gate pass): G_i rides in the -lse
// statistic, -G_j is added per key.  The dK/dV pass sums each key's column
// of dS and the dQ pass each query's row, and
//  5. dlogf_s = sum_{t < s} (column sum_t - row sum_t), the sum of dS over
//     the rectangle j < s <= i (the rows of dS sum to zero).
#include <type_traits>

#include "arp_device.hpp"
#include "arp_internal.hpp"
#include "mfma_tile.hpp"

namespace arp {

namespace {

constexpr int TILE = 64;  // tokens per tile (queries or keys)
// With a distance bias, a (query tile, key range) block whose base-2
// log-probabilities s_ij - lse_i are all below -ZGAP_B has probabilities
// 2^(s - lse) < 2^-160, below fp32's smallest subnormal: all exactly zero, so
// P, dS and every contribution of the block to dK, dV and dQ are exactly
// zero and the block can be left out without changing a bit.  The bound is
//   |q~s_i| |k~_j| + slope2 (j - i) - lse_i
//     <= max_i |q~s_i| * max_j |k~_j| + max_j slope2 j + max_i (-lse_i - slope2 i)
// (Cauchy-Schwarz; the per-tile maxima come from the prep pass).
constexpr float ZGAP_B = 160.0f;

// ---------------------------------------------------------------------------
// 1. prep
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
    const float* __restrict__ theta, const float* __restrict__ lse, const float* __restrict__ alibi,
    BwdOperands ops, float* __restrict__ dtheta, int L, int Lp, int H, int Hphi, uint32_t flags,
    float qscale0, const float* __restrict__ hscale) {
  constexpr int P = D / 2;
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  constexpr int ITER = TILE * CPR / 256;
  constexpr int TS = TILE + 8;  // padded LDS row of a transposed tile (elements)
  __shared__ __attribute__((aligned(16))) uint16_t s_t[3][D * TS];
  // tile maxima of |q~s|^2, |k~|^2 (bits of non-negative floats) and of -lse_i - slope2 i
  __shared__ uint32_t s_n2[2];
  __shared__ float s_c[TILE];
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh % H;
  const int g = (Hphi == 1) ? 0 : h;
  const int t0 = blockIdx.x * TILE;
  const int tid = threadIdx.x;
  const bool rqk = (flags & ARP_ROTATE_QK) != 0, rv = (flags & ARP_ROTATE_V) != 0;
  const size_t rm = (size_t)bh * Lp * D;  // row-major block of this head
  float* stats = ops.stats + ((size_t)bh * (Lp / TILE) + blockIdx.x) * (2 * TILE);
  const float slope2 = (flags & ARP_ALIBI) ? alibi[h] * LOG2E : 0.f;
  // q~s = q~ scale log2 e, times the head's query multiplier (AdaScale)
  const float qscale = hscale != nullptr ? qscale0 * hscale[h] : qscale0;
  if (tid < 2) s_n2[tid] = 0u;
  __syncthreads();

#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int idx = it * 256 + tid;
    const int r = idx / CPR, c = idx % CPR;
    const int tok = t0 + r;
    u32x4 wq = {0, 0, 0, 0}, wk = wq, wv = wq, wd = wq;
    float dsum = 0.f;
    if (tok < L) {
      const size_t off = ((size_t)bh * L + tok) * D + c * 8;
      const u32x4 xq = *reinterpret_cast<const u32x4*>(q + off);
      const u32x4 xk = *reinterpret_cast<const u32x4*>(k + off);
      const u32x4 xv = *reinterpret_cast<const u32x4*>(v + off);
      const u32x4 xo = *reinterpret_cast<const u32x4*>(o + off);
      const u32x4 xd = *reinterpret_cast<const u32x4*>(dout + off);
      float4 th = make_float4(0.f, 0.f, 0.f, 0.f);
      if (rqk || rv)
        th = *reinterpret_cast<const float4*>(theta + ((size_t)(b * Hphi + g) * L + tok) * P + c * 4);
      const float ang[4] = {th.x, th.y, th.z, th.w};
      float dth[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float sn, cs;
        sincosf(ang[e], &sn, &cs);
        float q0 = lo_bf16(xq[e]), q1 = hi_bf16(xq[e]);
        float k0 = lo_bf16(xk[e]), k1 = hi_bf16(xk[e]);
        float v0 = lo_bf16(xv[e]), v1 = hi_bf16(xv[e]);
        float o0 = lo_bf16(xo[e]), o1 = hi_bf16(xo[e]);
        float d0 = lo_bf16(xd[e]), d1 = hi_bf16(xd[e]);
        if (rqk) {
          rotate_pair(q0, q1, cs, sn);
          rotate_pair(k0, k1, cs, sn);
        }
        if (rv) {
          rotate_pair(v0, v1, cs, sn);
          rotate_pair(o0, o1, cs, sn);
          rotate_pair(d0, d1, cs, sn);
        }
        wq[e] = pack_bf16x2(q0 * qscale, q1 * qscale);
        wk[e] = pack_bf16x2(k0, k1);
        wv[e] = pack_bf16x2(v0, v1);
        wd[e] = pack_bf16x2(d0, d1);
        // D and the transport term from the bf16 do~ the products use, so
        // that sum_j dS_ij = 0 and sum_t dTheta_t = 0 hold for the computed
        // gradients as they do for the exact ones
        d0 = lo_bf16(wd[e]);
        d1 = hi_bf16(wd[e]);
        dsum = fmaf(d0, o0, fmaf(d1, o1, dsum));
        // value transport: -<do~, J o~> = d0 o1 - d1 o0
        dth[e] = rv ? (d0 * o1 - d1 * o0) : 0.f;
      }
      *reinterpret_cast<float4*>(dtheta + ((size_t)bh * L + tok) * P + c * 4) =
          make_float4(dth[0], dth[1], dth[2], dth[3]);
    }
    const size_t roff = rm + (size_t)tok * D + c * 8;
    *reinterpret_cast<u32x4*>(ops.qs + roff) = wq;
    *reinterpret_cast<u32x4*>(ops.k + roff) = wk;
    *reinterpret_cast<u32x4*>(ops.v + roff) = wv;
    *reinterpret_cast<u32x4*>(ops.dout + roff) = wd;
    // D_i and the row norms of the bf16 operands: the CPR threads of a row
    // are consecutive lanes
    float qn2 = 0.f, kn2 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qn2 = fmaf(lo_bf16(wq[e]), lo_bf16(wq[e]), fmaf(hi_bf16(wq[e]), hi_bf16(wq[e]), qn2));
      kn2 = fmaf(lo_bf16(wk[e]), lo_bf16(wk[e]), fmaf(hi_bf16(wk[e]), hi_bf16(wk[e]), kn2));
    }
#pragma unroll
    for (int m = 1; m < CPR; m <<= 1) {
      dsum += __shfl_xor(dsum, m);
      qn2 += __shfl_xor(qn2, m);
      kn2 += __shfl_xor(kn2, m);
    }
    if (c == 0) {
      const float nl = (tok < L) ? -lse[(size_t)bh * L + tok] : -INFINITY;
      // the query's gate offset within its 64-token tile joins -lse_i (the
      // tile base difference is added per block; the walk bounds below leave
      // the gates out: G_i - G_j <= 0 for j <= i, so they stay upper bounds)
      stats[r] = (ops.gate2 != nullptr && tok < L) ? nl + ops.gate2[(size_t)bh * Lp + tok] : nl;
      stats[TILE + r] = (tok < L) ? -dsum : 0.f;
      s_c[r] = nl - slope2 * (float)tok;
      atomicMax(&s_n2[0], __float_as_uint(qn2));
      atomicMax(&s_n2[1], __float_as_uint(kn2));
    }
    const u32x4* src[3] = {&wq, &wk, &wd};
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_t[a][(c * 8 + 2 * e) * TS + r] = (uint16_t)((*src[a])[e] & 0xFFFFu);
        s_t[a][(c * 8 + 2 * e + 1) * TS + r] = (uint16_t)((*src[a])[e] >> 16);
      }
  }
  __syncthreads();
  // The tile's bound statistics (used by the gradient kernels to start their
  // walks at the first tile that can hold a nonzero probability).  The norms
  // carry a margin for the fp32 accumulation of the products they bound.
  if (tid < 64) {
    float cm = s_c[tid];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
    if (tid == 0) {
      const f32x4 ts = {sqrtf(__uint_as_float(s_n2[0])) * (1.f + 1e-3f),
                        sqrtf(__uint_as_float(s_n2[1])) * (1.f + 1e-3f), cm, 0.f};
      *reinterpret_cast<f32x4*>(ops.tstat + ((size_t)bh * (Lp / TILE) + blockIdx.x) * 4) = ts;
    }
  }
  uint16_t* dstT[3] = {ops.qsT, ops.kT, ops.doutT};
  const size_t tb = (size_t)bh * D * Lp;
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int it = 0; it < D * 8 / 256; ++it) {
      const int idx = it * 256 + tid;
      const int drow = idx / 8, cc = idx % 8;
      const u32x4 w = *reinterpret_cast<const u32x4*>(&s_t[a][drow * TS + cc * 8]);
      *reinterpret_cast<u32x4*>(dstT[a] + tb + (size_t)drow * Lp + t0 + cc * 8) = w;
    }
}

// Direct global -> LDS copy of one 64-row tile, rows row-major [64][D] bf16,
// stored with rows in the swap_bits23 order and 16-byte chunks swizzled.
template <int D, int NW>
__device__ __forceinline__ void load_rows_tile(const uint16_t* base, int r0, uint8_t* lds, int wave,
                                               int lane) {
  constexpr int ROWB = D * 2, BYTES = TILE * ROWB, PER = BYTES / (1024 * NW);
  static_assert(PER * 1024 * NW == BYTES, "row tile split");
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int p0 = (wave * PER + i) * 1024;
    const int p = p0 + 16 * lane;
    const int row = p / ROWB, cs = (p % ROWB) / 16;
    const int c = cs ^ swz<ROWB>(row);
    const uint16_t* src = base + (size_t)(r0 + swap_bits23(row)) * D + 8 * c;
    __builtin_amdgcn_global_load_lds((global_void_ptr)src, (lds_void_ptr)(lds + p0), 16, 0, 0);
  }
}
// Same for a transposed tile [D][64] of a [D][Lp] block (columns c0 .. c0+63).
template <int D, int NW>
__device__ __forceinline__ void load_cols_tile(const uint16_t* base, int Lp, int c0, uint8_t* lds,
                                               int wave, int lane) {
  constexpr int ROWB = TILE * 2, BYTES = D * ROWB, PER = BYTES / (1024 * NW);
  static_assert(PER * 1024 * NW == BYTES, "column tile split");
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int p0 = (wave * PER + i) * 1024;
    const int p = p0 + 16 * lane;
    const int row = p / ROWB, cs = (p % ROWB) / 16;
    const int c = cs ^ swz<ROWB>(row);
    const uint16_t* src = base + (size_t)row * Lp + c0 + 8 * c;
    __builtin_amdgcn_global_load_lds((global_void_ptr)src, (lds_void_ptr)(lds + p0), 16, 0, 0);
  }
}
// A operand (16 bytes) of a row tile: row `row`, chunk ch.
template <int ROWB>
__device__ __forceinline__ bf16x8 lds_op(const uint8_t* t, int row, int ch) {
  return *reinterpret_cast<const bf16x8*>(t + row * ROWB + ((ch ^ swz<ROWB>(row)) << 4));
}

// Epilogue helper: gradient rows of rotated tensors.  acc[db][r] holds
// dx~[d] / mul for d = 32 db + 8 (r / 4) + 4 hf + r % 4 of this lane's token;
// xr is the bf16 operand row the products used (x~ times xmul), th the
// token's angles.  Writes dx = R^T dx~ (or dx~) as bf16; when rot, adds
// <dx~, J x~> to dth (per pair), with the same x~ the products used, so that
// the sum over tokens cancels as it does for the exact gradient.
template <int DB>
__device__ __forceinline__ void grad_rows(const f32x16 (&acc)[DB], float mul, const uint16_t* xr,
                                          float xmul, const float* th, bool rot, uint16_t* out,
                                          float* dth, int hf) {
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * db + 8 * j + 4 * hf;
      float g0 = acc[db][4 * j + 0] * mul, g1 = acc[db][4 * j + 1] * mul;
      float g2 = acc[db][4 * j + 2] * mul, g3 = acc[db][4 * j + 3] * mul;
      if (rot) {
        const u32x2 xw = *reinterpret_cast<const u32x2*>(xr + d0);
        const float2 a = *reinterpret_cast<const float2*>(th + d0 / 2);
        float s0, c0, s1, c1;
        sincosf(a.x, &s0, &c0);
        sincosf(a.y, &s1, &c1);
        const float x0 = lo_bf16(xw[0]) * xmul, x1 = hi_bf16(xw[0]) * xmul;
        const float x2 = lo_bf16(xw[1]) * xmul, x3 = hi_bf16(xw[1]) * xmul;
        float2 acc_th = *reinterpret_cast<float2*>(dth + d0 / 2);
        acc_th.x += -g0 * x1 + g1 * x0;
        acc_th.y += -g2 * x3 + g3 * x2;
        *reinterpret_cast<float2*>(dth + d0 / 2) = acc_th;
        rotate_pair(g0, g1, c0, -s0);
        rotate_pair(g2, g3, c1, -s1);
      }
      u32x2 w = {pack_bf16x2(g0, g1), pack_bf16x2(g2, g3)};
      *reinterpret_cast<u32x2*>(out + d0) = w;
    }
}

// ---------------------------------------------------------------------------
// 2. dK, dV (key-stationary)
// ---------------------------------------------------------------------------
// Biased launches: groups of BWD_GROUP adjacent blocks of one head, dealt
// round-robin over the XCDs (blockIdx % 8) in dispatch order, the heads rotated
// from round to round (the forward's spread order): a group runs together on
// one XCD and shares its walks' operand tiles in L2, while heads whose walks
// stop at different depths are spread over the XCDs.  r: the block's rank from
// the longest walk; false for a slot past the last block.
constexpr int BWD_GROUP = 4;
__device__ __forceinline__ bool spread_slot(int slot, int nbh, int nblk, int& bh, int& r) {
  const int x = slot % 8, m = slot / 8;
  const int gi = (m / BWD_GROUP) * 8 + x;
  const int rnd = gi / nbh;
  bh = (gi % nbh + rnd) % nbh;
  r = rnd * BWD_GROUP + m % BWD_GROUP;
  return r < nblk;
}

// The dK/dV of one block of BK = 32 NW keys (kt) of head bh, walking the
// query tiles from the last one down (ascending = false) or from the block's
// diagonal up (ascending = true).
template <int D, int NW, bool ALIBI, bool GATE>
__device__ __forceinline__ void dkdv_block(
    uint8_t* smem, const BwdOperands& ops, const float* __restrict__ theta,
    const float* __restrict__ alibi, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    float* __restrict__ dtheta, int L, int Lp, int H, int Hphi, uint32_t flags, int kt, int bh,
    bool ascending) {
  constexpr int BK = 32 * NW;  // keys per workgroup
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int ROWB = D * 2, RT = TILE * ROWB;     // row tile bytes
  constexpr int COLB = TILE * 2, CT = D * COLB;     // column tile bytes
  // + with gates the query tile's fp64 gate base (padded to keep stages on
  // 256-byte boundaries, the LDS bank period)
  constexpr int STAGE = 2 * RT + 2 * CT + 2 * TILE * 4 + (GATE ? 256 : 0);
  const int K0 = kt * BK;
  const int b = bh / H, h = bh % H;
  const int g = (Hphi == 1) ? 0 : h;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, hf = lane >> 5;
  const int kw = K0 + 32 * wave;  // this wave's first key
  const int j = kw + ln;          // this lane's key
  const int first_tile = K0 / TILE;
  const int last_tile = (L - 1) / TILE;
  const size_t rm = (size_t)bh * Lp * D, tb = (size_t)bh * D * Lp;
  const float* stats_bh = ops.stats + (size_t)bh * (Lp / TILE) * (2 * TILE);

  auto issue = [&](int t, uint8_t* st) __attribute__((always_inline)) {
    load_rows_tile<D, NW>(ops.qs + rm, t * TILE, st, wave, lane);
    load_rows_tile<D, NW>(ops.dout + rm, t * TILE, st + RT, wave, lane);
    load_cols_tile<D, NW>(ops.qsT + tb, Lp, t * TILE, st + 2 * RT, wave, lane);
    load_cols_tile<D, NW>(ops.doutT + tb, Lp, t * TILE, st + 2 * RT + CT, wave, lane);
    if (wave == 0 && lane < 32)
      __builtin_amdgcn_global_load_lds((global_void_ptr)(stats_bh + (size_t)t * 2 * TILE + 4 * lane),
                                       (lds_void_ptr)(st + 2 * RT + 2 * CT), 16, 0, 0);
    if (GATE && wave == 0 && lane < 2)  // one 4-byte half per lane (lane l lands at 4 l)
      __builtin_amdgcn_global_load_lds(
          (global_void_ptr)(reinterpret_cast<const uint32_t*>(ops.gbase + (size_t)bh * (Lp / TILE) + t) +
                            lane),
          (lds_void_ptr)(st + 2 * RT + 2 * CT + 2 * TILE * 4), 4, 0, 0);
  };

  // B operands: this lane's key row of k~ and v~ (d = 16 ks + 8 hf .. +7)
  bf16x8 kop[KS], vop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const size_t off = rm + (size_t)min(j, Lp - 1) * D + 16 * ks + 8 * hf;
    kop[ks] = *reinterpret_cast<const bf16x8*>(ops.k + off);
    vop[ks] = *reinterpret_cast<const bf16x8*>(ops.v + off);
  }
  f32x16 dkt[DB], dvt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dkt[db][r] = dvt[db][r] = 0.f;
  const float slope2 = ALIBI ? alibi[h] * LOG2E : 0.f;
  // the key's gate offset within its 64-token tile, subtracted from every
  // logit of its column with the (query tile, key tile) base difference
  const float gj = GATE ? ops.gate2[(size_t)bh * Lp + min(j, Lp - 1)] : 0.f;
  // the wave's keys share a tile
  const double gbase_k = GATE ? ops.gbase[(size_t)bh * (Lp / TILE) + min(kw / TILE, Lp / TILE - 1)]
                              : 0.0;
  float csum = 0.f;  // sum of dS over this lane's part of the key's column

  // Query tiles from the last one down: the workgroups that run at the same
  // time on an XCD (keys of the same heads) then stream the same query tiles
  // together, which keeps them in L2 (from its own diagonal upwards, each
  // workgroup would start at a different tile).  With a distance bias the
  // walk starts at the last query tile that can hold a nonzero probability
  // for these keys (every wave finds the same tile).
  int t_hi = last_tile;
  if constexpr (ALIBI) {
    const float* ts = ops.tstat + (size_t)bh * (Lp / TILE) * 4;
    const int j_hi = min(K0 + BK, L) - 1;
    float kwn = 0.f;
    for (int u = K0 / TILE; u <= j_hi / TILE; ++u) kwn = fmaxf(kwn, ts[4 * u + 1]);
    const float jb = fmaxf(slope2 * (float)K0, slope2 * (float)j_hi);
    t_hi = first_tile - 1;
    for (int base = last_tile; base >= first_tile; base -= 64) {
      const int t = base - lane;
      bool alive = false;
      if (t >= first_tile) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(ts + 4 * t);
        alive = fmaf(v[0], kwn, jb + v[2]) >= -ZGAP_B;
      }
      const uint64_t m = __ballot(alive);
      if (m != 0) {
        t_hi = base - (__ffsll((unsigned long long)m) - 1);
        break;
      }
    }
  }
  const int nsteps = t_hi - first_tile + 1;
  auto tile_of = [&](int n) { return ascending ? first_tile + n : t_hi - n; };
  if (nsteps > 0) issue(tile_of(0), smem);
  for (int n = 0; n < nsteps; ++n) {
    const int t = tile_of(n);
    uint8_t* st = smem + (n & 1) * STAGE;
    wait_loads<0>();
    __builtin_amdgcn_s_barrier();
    if (n + 1 < nsteps) issue(tile_of(n + 1), smem + ((n + 1) & 1) * STAGE);
    const uint8_t* tq = st;
    const uint8_t* tdo = st + RT;
    const uint8_t* tqT = st + 2 * RT;
    const uint8_t* tdoT = st + 2 * RT + CT;
    const float* sl = reinterpret_cast<const float*>(st + 2 * RT + 2 * CT);
    // G_i - G_j = fp32(gbase[t] - gbase[key tile]) + offset_i - offset_j
    // (the query tile's base came into LDS with its statistics)
    const float dg =
        GATE ? (float)(*reinterpret_cast<const double*>(st + 2 * RT + 2 * CT + 2 * TILE * 4) - gbase_k) - gj
             : 0.f;
    // The parts of one 32-query block qb of the tile: the accumulator inputs
    // -lse and -D of this lane's rows, S and dP' (first products), P and dS
    // (bf16 B operands), then dV and dK.
    auto first_products = [&](int qb, f32x16& sv, f32x16& dpv) __attribute__((always_inline)) {
      f32x16 cl, cd;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int ro = 32 * qb + 16 * h2 + 8 * hf;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(sl + ro);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(sl + ro + 4);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(sl + TILE + ro);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(sl + TILE + ro + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          cl[8 * h2 + e] = l0[e];
          cl[8 * h2 + 4 + e] = l1[e];
          cd[8 * h2 + e] = d0[e];
          cd[8 * h2 + 4 + e] = d1[e];
        }
      }
      if constexpr (GATE) {
#pragma unroll
        for (int r = 0; r < 16; ++r) cl[r] += dg;
      }
      sv = cl;
      dpv = cd;
      // every LDS operand of the block is read before its first product:
      // left to itself the compiler reads each one just before its product
      // and waits for it there, which at one wave per SIMD (d = 128) leaves
      // the matrix core idle for the LDS latency at every product
      bf16x8 qa[KS], da[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qa[ks] = lds_op<ROWB>(tq, 32 * qb + ln, 2 * ks + hf);
        da[ks] = lds_op<ROWB>(tdo, 32 * qb + ln, 2 * ks + hf);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sv = mfma32(qa[ks], kop[ks], sv);
        dpv = mfma32(da[ks], vop[ks], dpv);
      }
    };
    auto probabilities = [&](const f32x16& sv, const f32x16& dpv, bf16x8 (&pop)[2],
                             bf16x8 (&dsop)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        uint32_t wp[4], wd[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) x[u] = __builtin_amdgcn_exp2f(sv[8 * h2 + 2 * e + u]);
          wp[e] = pack_bf16x2(x[0], x[1]);
          const float ds0 = x[0] * dpv[8 * h2 + 2 * e], ds1 = x[1] * dpv[8 * h2 + 2 * e + 1];
          wd[e] = pack_bf16x2(ds0, ds1);
          if (GATE) csum += ds0 + ds1;
        }
        u32x4 a = {wp[0], wp[1], wp[2], wp[3]}, c = {wd[0], wd[1], wd[2], wd[3]};
        pop[h2] = __builtin_bit_cast(bf16x8, a);
        dsop[h2] = __builtin_bit_cast(bf16x8, c);
      }
    };
    auto second_products = [&](int qb, const bf16x8 (&pop)[2], const bf16x8 (&dsop)[2])
        __attribute__((always_inline)) {
      bf16x8 oa[DB][2], qa[DB][2];  // operands first, as in first_products
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int ch = 4 * qb + 2 * h2 + hf;
          oa[db][h2] = lds_op<COLB>(tdoT, 32 * db + ln, ch);
          qa[db][h2] = lds_op<COLB>(tqT, 32 * db + ln, ch);
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          dvt[db] = mfma32(oa[db][h2], pop[h2], dvt[db]);
          dkt[db] = mfma32(qa[db][h2], dsop[h2], dkt[db]);
        }
    };
    if (t * TILE >= kw + 32) {
      // Every query of the tile follows every key of the wave: no block is
      // skipped and none is masked.  Both blocks' first products come first,
      // with no branch between them and the softmax, so that the second
      // block's products can overlap the first block's exponentials (the
      // same accumulation order as below: identical results).
      f32x16 s0, dp0, s1, dp1;
      bf16x8 p0[2], ds0[2], p1[2], ds1[2];
      first_products(0, s0, dp0);
      first_products(1, s1, dp1);
      if (ALIBI) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i0 = t * TILE + 16 * (r >> 3) + 8 * hf + (r & 7);  // query of element r, block 0
          s0[r] = fmaf(slope2, (float)(j - i0), s0[r]);
          s1[r] = fmaf(slope2, (float)(j - (i0 + 32)), s1[r]);
        }
      }
      probabilities(s0, dp0, p0, ds0);
      second_products(0, p0, ds0);
      probabilities(s1, dp1, p1, ds1);
      second_products(1, p1, ds1);
      continue;
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qbase = t * TILE + 32 * qb;
      if (qbase + 31 < kw) continue;  // every query of the block precedes every key of the wave
      f32x16 sv, dpv;
      first_products(qb, sv, dpv);
      if (ALIBI || qbase == kw) {  // distance bias; the causal mask on the diagonal block
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = qbase + 16 * (r >> 3) + 8 * hf + (r & 7);  // query of element r
          if (ALIBI) sv[r] = fmaf(slope2, (float)(j - i), sv[r]);
          if (qbase == kw && j > i) sv[r] = -INFINITY;
        }
      }
      bf16x8 pop[2], dsop[2];
      probabilities(sv, dpv, pop, dsop);
      second_products(qb, pop, dsop);
    }
  }

  if constexpr (GATE) {  // lanes ln and ln + 32 hold the two halves of the column
    csum += __shfl_xor(csum, 32);
    if (hf == 0 && j < L) ops.colsum[(size_t)bh * Lp + j] = csum;
  }
  if (j >= L) return;
  const size_t row = ((size_t)bh * L + j) * D;
  const uint16_t* oprow = ops.k + rm + (size_t)j * D;
  const float* th = theta + ((size_t)(b * Hphi + g) * L + j) * (D / 2);
  float* dth = dtheta + ((size_t)bh * L + j) * (D / 2);
  // dk~ = scale sum dS q~ = ln 2 * (Q~s^T dS) since q~s carries scale log2 e
  grad_rows<DB>(dkt, 0.69314718055994531f, oprow, 1.f, th, (flags & ARP_ROTATE_QK) != 0,
                dk + row, dth, hf);
  grad_rows<DB>(dvt, 1.f, ops.v + rm + (size_t)j * D, 1.f, th, (flags & ARP_ROTATE_V) != 0,
                dv + row, dth, hf);
}

template <int D, int NW, bool ALIBI, bool GATE>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dkdv_kernel(
    BwdOperands ops, const float* __restrict__ theta, const float* __restrict__ alibi,
    uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, float* __restrict__ dtheta, int L, int Lp, int H, int Hphi, int nkt,
    int total_tiles, uint32_t flags, int paired) {
  constexpr int ROWB = D * 2, RT = TILE * ROWB, COLB = TILE * 2, CT = D * COLB;
  constexpr int STAGE = 2 * RT + 2 * CT + 2 * TILE * 4 + (GATE ? 256 : 0);  // as in dkdv_block
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

  // Unbiased: each XCD (blockIdx % 8) gets whole heads, so their key
  // workgroups share the streamed query tiles in its L2.  Paired (grids that
  // still fill the chip with half the workgroups): workgroup c of a head
  // takes key block c, walking the query tiles down from the last, then key
  // block nkt - 1 - c, walking up from its diagonal.  Every workgroup then
  // does the same work (nkt + 1 tiles' worth), and at any moment the
  // workgroups of a head are on one of only two query tiles (the last tile
  // minus the steps taken, or the steps taken minus the offset of the second
  // block), so each tile streams through the XCD's L2 about twice instead of
  // once per key block.  With a distance bias the work per head differs
  // widely (a steep slope leaves most query tiles out), so the key blocks are
  // dealt out across the XCDs in groups instead (spread_slot), the longest
  // query ranges (small kt) first.
  if constexpr (ALIBI) {
    int bh, kt;
    if (!spread_slot((int)blockIdx.x, total_tiles / nkt, nkt, bh, kt)) return;
    dkdv_block<D, NW, ALIBI, GATE>(smem, ops, theta, alibi, dk, dv, dtheta, L, Lp, H, Hphi, flags,
                                   kt, bh, false);
    return;
  }
  const int per = (total_tiles + 7) / 8;
  const int logical = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (logical >= total_tiles) return;
  if (paired) {
    const int npk = (nkt + 1) / 2;  // workgroups per head
    const int bh = logical / npk, c = logical % npk;
    dkdv_block<D, NW, ALIBI, GATE>(smem, ops, theta, alibi, dk, dv, dtheta, L, Lp, H, Hphi, flags,
                                   c, bh, false);
    if (nkt - 1 - c != c) {
      __syncthreads();  // every wave is done with the LDS stages before they are refilled
      dkdv_block<D, NW, ALIBI, GATE>(smem, ops, theta, alibi, dk, dv, dtheta, L, Lp, H, Hphi,
                                     flags, nkt - 1 - c, bh, true);
    }
    return;
  }
  dkdv_block<D, NW, ALIBI, GATE>(smem, ops, theta, alibi, dk, dv, dtheta, L, Lp, H, Hphi, flags,
                                 logical % nkt, logical / nkt, false);
}

// ---------------------------------------------------------------------------
// 3. dQ (query-stationary)
// ---------------------------------------------------------------------------
template <int D, int NW, bool ALIBI, bool GATE, bool PAIR>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dq_kernel(
    BwdOperands ops, const float* __restrict__ theta, const float* __restrict__ alibi,
    uint16_t* __restrict__ dq, float* __restrict__ dtheta, int L, int Lp, int H, int Hphi, int nqt,
    int total_tiles, uint32_t flags, float scale0, const float* __restrict__ hscale) {
  static_assert(!PAIR || !ALIBI, "pairs are for unbiased walks");
  constexpr int BM = 32 * NW;
  constexpr int KS = D / 16, DB = D / 32, KB = 2, KS2 = 4;
  constexpr int ROWB = D * 2, RT = TILE * ROWB;
  constexpr int COLB = TILE * 2, CT = D * COLB;
  // + the tile's key gates and base (padded to a 256-byte multiple)
  constexpr int STAGE = 2 * RT + CT + (GATE ? TILE * 4 + 256 : 0);
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

  // Workgroup order as in the dK/dV pass: whole heads per XCD unbiased,
  // groups of query blocks dealt out across the XCDs with a distance bias
  // (spread_slot); longest first.  PAIR (unbiased grids whose pairs still
  // fill every CU): a workgroup takes the c-th longest and the c-th shortest
  // block of its XCD's share one after the other, so every workgroup has the
  // same work (8 x 8 heads at 2048 tokens, d = 64: backward 0.269 -> 0.249
  // ms; 2 x 16 at 4096, d = 128: 0.792 -> 0.738 ms; extrap_16k unchanged).
  // It is an instantiation of its own, so the unpaired walk keeps its
  // register allocation.
  //
  // One query block (bh, qt):
  auto run = [&](int bh, int qt) __attribute__((always_inline)) {
    const int q0 = qt * BM;
    const int b = bh / H, h = bh % H;
    const int g = (Hphi == 1) ? 0 : h;
    // the logit scale of this head: scale times its query multiplier (AdaScale),
    // so dq = lambda_h dq' where q' = lambda_h q
    const float scale = hscale != nullptr ? scale0 * hscale[h] : scale0;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 31, hf = lane >> 5;
    const int qw = q0 + 32 * wave;
    const int i = qw + ln;  // this lane's query
    const int last_tile = min(q0 + BM - 1, L - 1) / TILE;
    const int last_w = (qw < L) ? min(qw + 31, L - 1) / TILE : -1;
    const size_t rm = (size_t)bh * Lp * D, tb = (size_t)bh * D * Lp;

    auto issue = [&](int t, uint8_t* st) __attribute__((always_inline)) {
      load_rows_tile<D, NW>(ops.k + rm, t * TILE, st, wave, lane);
      load_rows_tile<D, NW>(ops.v + rm, t * TILE, st + RT, wave, lane);
      load_cols_tile<D, NW>(ops.kT + tb, Lp, t * TILE, st + 2 * RT, wave, lane);
      if (GATE && wave == 0 && lane < TILE / 4)
        __builtin_amdgcn_global_load_lds(
            (global_void_ptr)(ops.gate2 + (size_t)bh * Lp + (size_t)t * TILE + 4 * lane),
            (lds_void_ptr)(st + 2 * RT + CT), 16, 0, 0);
      if (GATE && wave == 0 && lane < 2)  // the key tile's base, one 4-byte half per lane
        __builtin_amdgcn_global_load_lds(
            (global_void_ptr)(reinterpret_cast<const uint32_t*>(ops.gbase + (size_t)bh * (Lp / TILE) + t) +
                              lane),
            (lds_void_ptr)(st + 2 * RT + CT + TILE * 4), 4, 0, 0);
    };

    bf16x8 qop[KS], doop[KS];
    const int ic = min(i, Lp - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const size_t off = rm + (size_t)ic * D + 16 * ks + 8 * hf;
      qop[ks] = *reinterpret_cast<const bf16x8*>(ops.qs + off);
      doop[ks] = *reinterpret_cast<const bf16x8*>(ops.dout + off);
    }
    const float* srow = ops.stats + ((size_t)bh * (Lp / TILE) + ic / TILE) * (2 * TILE);
    const float nl = srow[ic % TILE], nd = srow[TILE + ic % TILE];
    f32x16 cl, cd, dqt[DB];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      cl[r] = nl;
      cd[r] = nd;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dqt[db][r] = 0.f;
    const float slope2 = ALIBI ? alibi[h] * LOG2E : 0.f;
    float rsum = 0.f;  // sum of dS over this lane's part of the query's row
    // the gate base of the wave's query tile (its 32 queries share one)
    const double gbase_q = GATE ? ops.gbase[(size_t)bh * (Lp / TILE) + min(qw / TILE, Lp / TILE - 1)]
                                : 0.0;

    // With a distance bias the walk starts at the first key tile that can
    // hold a nonzero probability for these queries (every wave finds the same
    // tile).
    int n_lo = 0;
    if constexpr (ALIBI) {
      const float* ts = ops.tstat + (size_t)bh * (Lp / TILE) * 4;
      float qwn = 0.f, cw = -INFINITY;
      for (int u = q0 / TILE; u <= last_tile; ++u) {
        qwn = fmaxf(qwn, ts[4 * u]);
        cw = fmaxf(cw, ts[4 * u + 2]);
      }
      n_lo = last_tile + 1;
      for (int base = 0; base <= last_tile; base += 64) {
        const int n = base + lane;
        bool alive = false;
        if (n <= last_tile) {
          const float jb = fmaxf(slope2 * (float)(n * TILE), slope2 * (float)(n * TILE + TILE - 1));
          alive = fmaf(qwn, ts[4 * n + 1], jb + cw) >= -ZGAP_B;
        }
        const uint64_t m = __ballot(alive);
        if (m != 0) {
          n_lo = base + (__ffsll((unsigned long long)m) - 1);
          break;
        }
      }
    }
    if (n_lo <= last_tile) issue(n_lo, smem);
    for (int n = n_lo; n <= last_tile; ++n) {
      uint8_t* st = smem + ((n - n_lo) & 1) * STAGE;
      wait_loads<0>();
      __builtin_amdgcn_s_barrier();
      if (n + 1 <= last_tile) issue(n + 1, smem + ((n - n_lo + 1) & 1) * STAGE);
      if (n > last_w) continue;
      const uint8_t* tk = st;
      const uint8_t* tv = st + RT;
      const uint8_t* tkT = st + 2 * RT;
      const bool diag = (n == last_w);
      // with gates: the (query tile, key tile) base difference joins -lse_i +
      // the query's offset; the key offsets are subtracted per element below
      f32x16 clt = cl;
      if constexpr (GATE) {
        const float dt =
            (float)(gbase_q - *reinterpret_cast<const double*>(st + 2 * RT + CT + TILE * 4));
#pragma unroll
        for (int r = 0; r < 16; ++r) clt[r] += dt;
      }
      // S^T and dP'^T of the keys 32 kb .. 32 kb + 31 of the tile, then their
      // dS^T (the B operands of dQ^T += K~^T dS^T)
      auto first_products = [&](int kb, f32x16& sv, f32x16& dpv) __attribute__((always_inline)) {
        sv = clt;
        dpv = cd;
        if constexpr (GATE) {  // minus the offset of the key of each element
          const float* gp = reinterpret_cast<const float*>(st + 2 * RT + CT) + 32 * kb + 8 * hf;
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const f32x4 ga = *reinterpret_cast<const f32x4*>(gp + 16 * h2);
            const f32x4 gb = *reinterpret_cast<const f32x4*>(gp + 16 * h2 + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sv[8 * h2 + e] -= ga[e];
              sv[8 * h2 + 4 + e] -= gb[e];
            }
          }
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          sv = mfma32(lds_op<ROWB>(tk, 32 * kb + ln, 2 * ks + hf), qop[ks], sv);
          dpv = mfma32(lds_op<ROWB>(tv, 32 * kb + ln, 2 * ks + hf), doop[ks], dpv);
        }
      };
      // the distance bias (and on the diagonal tile the causal mask)
      auto bias = [&](int kb, f32x16& sv, bool mask) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jj = n * TILE + 32 * kb + 16 * (r >> 3) + 8 * hf + (r & 7);  // key of element r
          if (ALIBI) sv[r] = fmaf(slope2, (float)(jj - i), sv[r]);
          if (mask && jj > i) sv[r] = -INFINITY;
        }
      };
      bf16x8 dsop[KS2];
      auto scores = [&](int kb, const f32x16& sv, const f32x16& dpv) __attribute__((always_inline)) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          uint32_t wd[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float x[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int r = 8 * h2 + 2 * e + u;
              x[u] = __builtin_amdgcn_exp2f(sv[r]) * dpv[r];
            }
            if (GATE) rsum += x[0] + x[1];
            wd[e] = pack_bf16x2(x[0], x[1]);
          }
          u32x4 c = {wd[0], wd[1], wd[2], wd[3]};
          dsop[2 * kb + h2] = __builtin_bit_cast(bf16x8, c);
        }
      };
      if (!diag && D == 64) {
        // No mask: both key blocks' products first, with no branch before the
        // exponentials, so that the second block's products can overlap the
        // first block's (same accumulation order: identical results).  At
        // d = 128 the two blocks' S and dP' would not fit beside the second
        // wave of the SIMD.
        f32x16 s0, dp0, s1, dp1;
        first_products(0, s0, dp0);
        first_products(1, s1, dp1);
        if (ALIBI) {
          bias(0, s0, false);
          bias(1, s1, false);
        }
        scores(0, s0, dp0);
        scores(1, s1, dp1);
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          f32x16 sv, dpv;
          first_products(kb, sv, dpv);
          bias(kb, sv, true);
          scores(kb, sv, dpv);
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int ks2 = 0; ks2 < KS2; ++ks2)
          dqt[db] = mfma32(lds_op<COLB>(tkT, 32 * db + ln, 2 * ks2 + hf), dsop[ks2], dqt[db]);
    }

    if constexpr (GATE) {  // lanes ln and ln + 32 hold the two halves of the row
      rsum += __shfl_xor(rsum, 32);
      if (hf == 0 && i < L) ops.rowsum[(size_t)bh * Lp + i] = rsum;
    }
    if (i >= L) return;
    const size_t row = ((size_t)bh * L + i) * D;
    const float* th = theta + ((size_t)(b * Hphi + g) * L + i) * (D / 2);
    float* dth = dtheta + ((size_t)bh * L + i) * (D / 2);
    // dq~ = scale lambda_h sum dS k~ (the gradient of the unscaled q~), and
    // q~ = q~s / (scale lambda_h log2 e): their product, the dTheta term, is
    // that of the scaled query
    grad_rows<DB>(dqt, scale, ops.qs + rm + (size_t)i * D, 1.f / (scale * LOG2E), th,
                  (flags & ARP_ROTATE_QK) != 0, dq + row, dth, hf);
  };
  if constexpr (ALIBI) {
    int bh, r;
    if (!spread_slot((int)blockIdx.x, total_tiles / nqt, nqt, bh, r)) return;
    run(bh, nqt - 1 - r);
    return;
  }
  const int per = (total_tiles + 7) / 8;
  if constexpr (PAIR) {
    // the c-th longest and the c-th shortest block of the XCD's share
    const int x = (int)(blockIdx.x % 8), c = (int)(blockIdx.x / 8);
    const int l1 = x * per + c, l2 = x * per + per - 1 - c;
    run(l1 / nqt, nqt - 1 - l1 % nqt);
    __syncthreads();  // every wave is done with the LDS stages before they are refilled
    run(l2 / nqt, nqt - 1 - l2 % nqt);
    return;
  }
  const int logical = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (logical >= total_tiles) return;
  run(logical / nqt, nqt - 1 - logical % nqt);
}

// ---------------------------------------------------------------------------
// 4. reverse scan: dphi[b, g, s, p] = sum_{h in g} sum_{t >= s} dTheta[b, h, t, p]
// ---------------------------------------------------------------------------
constexpr int RCH = 256;  // tokens per chunk

// Thread layout of both passes: lane group c4 (P / 4 lanes per token) holds
// four consecutive pairs 4 c4 .. 4 c4 + 3 (16-byte loads and stores), row
// group rg = tid / (P / 4) a set of the chunk's tokens.
template <int P>
struct RscanLayout {
  static constexpr int C4 = P / 4;      // lanes per token
  static constexpr int G = 256 / C4;    // row groups
  static constexpr int R = RCH / G;     // tokens per thread in the apply pass
};

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// chunk totals (summed over the heads of the stream)
template <int P>
__global__ __launch_bounds__(256) void rscan_totals_kernel(const float* __restrict__ dtheta,
                                                           float* __restrict__ totals, int L,
                                                           int H, int Hphi, int nch) {
  using Y = RscanLayout<P>;
  __shared__ float4 part[Y::G][Y::C4];
  const int c = blockIdx.x, bg = blockIdx.y;
  const int b = bg / Hphi, gg = bg % Hphi;
  const int c4 = threadIdx.x % Y::C4, rg = threadIdx.x / Y::C4;
  const int hn = (Hphi == 1) ? H : 1;
  const int tend = min(L, (c + 1) * RCH);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int hh = 0; hh < hn; ++hh) {
    const int h = (Hphi == 1) ? hh : gg;
    const float4* src = reinterpret_cast<const float4*>(dtheta + ((size_t)(b * H + h) * L) * P) + c4;
    // the thread's tokens c RCH + rg + G u, all loads in flight together
    float4 x[Y::R];
#pragma unroll
    for (int u = 0; u < Y::R; ++u) {
      const int t = c * RCH + rg + Y::G * u;
      x[u] = (t < tend) ? src[(size_t)t * Y::C4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < Y::R; ++u) acc = add4(acc, x[u]);
  }
  part[rg][c4] = acc;
  __syncthreads();
  if (rg == 0) {
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int r = 0; r < Y::G; ++r) t = add4(t, part[r][c4]);
    reinterpret_cast<float4*>(totals + ((size_t)bg * nch + c) * P)[c4] = t;
  }
}

// In-chunk suffix sums plus the totals of every later chunk (read directly:
// a few 16-byte loads per thread, no separate pass).
template <int P>
__global__ __launch_bounds__(256) void rscan_apply_kernel(const float* __restrict__ dtheta,
                                                          const float* __restrict__ totals,
                                                          float* __restrict__ dphi, int L, int H,
                                                          int Hphi, int nch, int exclusive) {
  using Y = RscanLayout<P>;
  constexpr int R = Y::R;  // each thread: R consecutive tokens of four pairs
  __shared__ float4 run_tot[Y::G][Y::C4];
  const int c = blockIdx.x, bg = blockIdx.y;
  const int b = bg / Hphi, gg = bg % Hphi;
  const int c4 = threadIdx.x % Y::C4, rg = threadIdx.x / Y::C4;
  const int hn = (Hphi == 1) ? H : 1;
  const int t0 = c * RCH + rg * R;
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 x[R];
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = z;
  for (int hh = 0; hh < hn; ++hh) {
    const int h = (Hphi == 1) ? hh : gg;
    const float4* src = reinterpret_cast<const float4*>(dtheta + ((size_t)(b * H + h) * L) * P) + c4;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (t0 + r < L) x[r] = add4(x[r], src[(size_t)(t0 + r) * Y::C4]);
  }
  float4 tot = z;
#pragma unroll
  for (int r = 0; r < R; ++r) tot = add4(tot, x[r]);
  // chunks after this one: the G row groups of a pair set split them
  float4 later = z;
  const float4* tsrc = reinterpret_cast<const float4*>(totals + (size_t)bg * nch * P) + c4;
  for (int c2 = c + 1 + rg; c2 < nch; c2 += Y::G) later = add4(later, tsrc[(size_t)c2 * Y::C4]);
  run_tot[rg][c4] = later;
  __syncthreads();
  float4 off = z;
#pragma unroll
  for (int r2 = 0; r2 < Y::G; ++r2) off = add4(off, run_tot[r2][c4]);
  __syncthreads();
  run_tot[rg][c4] = tot;
  __syncthreads();
  for (int r2 = rg + 1; r2 < Y::G; ++r2) off = add4(off, run_tot[r2][c4]);
  float4* dst = reinterpret_cast<float4*>(dphi + ((size_t)bg * L) * P) + c4;
  float4 run = off;
#pragma unroll
  for (int r = R - 1; r >= 0; --r) {
    if (!exclusive) run = add4(run, x[r]);
    if (t0 + r < L) dst[(size_t)(t0 + r) * Y::C4] = run;
    if (exclusive) run = add4(run, x[r]);
  }
}

// ---------------------------------------------------------------------------
// 5. gate gradient: dlogf[bh, s] = sum_{t < s} (colsum_t - rowsum_t) (fp64
// sums), 0 where log f_s > 0 (the forward takes such gates as 1).  Chunks of
// 1024 tokens, four consecutive tokens per thread: the first kernel sums each
// chunk, the second adds the sums of the earlier chunks to an in-chunk
// exclusive scan.
// ---------------------------------------------------------------------------
constexpr int GG_THREADS = 256, GG_CHUNK = 4 * GG_THREADS;

// The thread's four differences colsum - rowsum (0 past L).
__device__ __forceinline__ void gate_diffs(const float* __restrict__ colsum,
                                           const float* __restrict__ rowsum, int bh, int t0, int L,
                                           int Lp, double (&x)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = 0.0;
  if (t0 >= Lp) return;  // Lp is a multiple of 256: all four tokens are below it
  const float4 cs = *reinterpret_cast<const float4*>(colsum + (size_t)bh * Lp + t0);
  const float4 rs = *reinterpret_cast<const float4*>(rowsum + (size_t)bh * Lp + t0);
  const float cv[4] = {cs.x, cs.y, cs.z, cs.w}, rv[4] = {rs.x, rs.y, rs.z, rs.w};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (t0 + e < L) x[e] = (double)cv[e] - (double)rv[e];
}

__device__ __forceinline__ double block_sum_gg(double x, double* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int u = 0; u < GG_THREADS / 64; ++u) t += red[u];
  return t;
}

__global__ __launch_bounds__(GG_THREADS) void bwd_gate_tot_kernel(
    const float* __restrict__ colsum, const float* __restrict__ rowsum, double* __restrict__ tot,
    int L, int Lp, int nch) {
  __shared__ double red[GG_THREADS / 64];
  const int c = blockIdx.x, bh = blockIdx.y;
  double x[4];
  gate_diffs(colsum, rowsum, bh, c * GG_CHUNK + 4 * threadIdx.x, L, Lp, x);
  const double t = block_sum_gg((x[0] + x[1]) + (x[2] + x[3]), red);
  if (threadIdx.x == 0) tot[(size_t)bh * nch + c] = t;
}

__global__ __launch_bounds__(GG_THREADS) void bwd_gate_grad_kernel(
    const float* __restrict__ colsum, const float* __restrict__ rowsum,
    const double* __restrict__ tot, const float* __restrict__ logf, float* __restrict__ dlogf,
    int L, int Lp, int nch) {
  __shared__ double red[GG_THREADS / 64], wsum[GG_THREADS / 64];
  const int c = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  double carry = 0.0;  // the earlier chunks
  for (int u = tid; u < c; u += GG_THREADS) carry += tot[(size_t)bh * nch + u];
  carry = block_sum_gg(carry, red);
  const int t0 = c * GG_CHUNK + 4 * tid;
  double x[4];
  gate_diffs(colsum, rowsum, bh, t0, L, Lp, x);
  const double mine = (x[0] + x[1]) + (x[2] + x[3]);
  double incl = mine;  // inclusive scan of the thread sums within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  double pre = carry + (incl - mine);
  for (int u = 0; u < w; ++u) pre += wsum[u];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = t0 + e;
    if (t < L) {
      const float lf = logf[(size_t)bh * L + t];
      dlogf[(size_t)bh * L + t] = (lf <= 0.f) ? (float)pre : 0.f;
    }
    pre += x[e];
  }
}

template <int D, int NW, bool ALIBI, bool GATE>
hipError_t launch_bwd_grads(const Geometry& g, const BwdArgs& a, hipStream_t stream) {
  const uint32_t fl = g.flags;
  {
    const int nkt = (g.L + 32 * NW - 1) / (32 * NW);
    // key blocks paired when half as many workgroups still fill every CU
    const long pairs = (long)g.B * g.H * ((nkt + 1) / 2);
    const int paired = (!ALIBI && pairs >= device_cus()) ? 1 : 0;
    const int total = paired ? (int)pairs : g.B * g.H * nkt;
    const long groups = (long)g.B * g.H * ((nkt + BWD_GROUP - 1) / BWD_GROUP);
    const int grid = ALIBI ? (int)(((groups + 7) / 8) * 8 * BWD_GROUP) : ((total + 7) / 8) * 8;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, ALIBI, GATE>), dim3(grid), dim3(NW * 64), 0, stream,
                       a.ops, a.theta, a.alibi, a.dk, a.dv, a.dtheta, g.L, g.Lp, g.H, g.Hphi, nkt,
                       total, fl, paired);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    // dQ runs 8 waves (two per SIMD) at both head dims: at d = 128 its
    // registers fit two waves per SIMD when the key blocks are taken one at a
    // time, which beats one wave per SIMD with both blocks in flight
    // (rope_8k_d128 backward 10.87 -> 9.42 ms, gradients bit-identical)
    constexpr int NQ = 8;
    const int nqt = (g.L + 32 * NQ - 1) / (32 * NQ);
    const int total = g.B * g.H * nqt;
    const long groups = (long)g.B * g.H * ((nqt + BWD_GROUP - 1) / BWD_GROUP);
    const bool paired = !ALIBI && total % 16 == 0 && total / 2 >= device_cus();
    const int grid = ALIBI ? (int)(((groups + 7) / 8) * 8 * BWD_GROUP)
                     : paired ? total / 2 : ((total + 7) / 8) * 8;
    if (paired)
      hipLaunchKernelGGL((bwd_dq_kernel<D, NQ, ALIBI, GATE, !ALIBI>), dim3(grid), dim3(NQ * 64), 0,
                         stream, a.ops, a.theta, a.alibi, a.dq, a.dtheta, g.L, g.Lp, g.H, g.Hphi,
                         nqt, total, fl, g.scale, g.hscale);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, NQ, ALIBI, GATE, false>), dim3(grid), dim3(NQ * 64), 0,
                         stream, a.ops, a.theta, a.alibi, a.dq, a.dtheta, g.L, g.Lp, g.H, g.Hphi,
                         nqt, total, fl, g.scale, g.hscale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if constexpr (GATE) {
    // the chunk sums reuse the gate prefix's totals (read by then); both
    // have ceil(Lp / 1024) chunks per (b, h)
    static_assert(GG_CHUNK == GATE_CHUNK, "one chunk size for both gate scans");
    const int nch = gate_chunks(g);
    const dim3 grid(nch, g.B * g.H);
    hipLaunchKernelGGL(bwd_gate_tot_kernel, grid, dim3(GG_THREADS), 0, stream, a.ops.colsum,
                       a.ops.rowsum, a.gate_tot, g.L, g.Lp, nch);
    hipLaunchKernelGGL(bwd_gate_grad_kernel, grid, dim3(GG_THREADS), 0, stream, a.ops.colsum,
                       a.ops.rowsum, a.gate_tot, a.logf, a.dlogf, g.L, g.Lp, nch);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int D, int NW>
hipError_t launch_bwd_d(const Geometry& g, const BwdArgs& a, hipStream_t stream) {
  const uint32_t fl = g.flags;
  const bool al = (fl & ARP_ALIBI) != 0;
  {
    dim3 grid(g.Lp / TILE, g.B * g.H);
    hipLaunchKernelGGL((bwd_prep_kernel<D>), grid, dim3(256), 0, stream, a.q, a.k, a.v, a.o, a.dout,
                       a.theta, a.lse, a.alibi, a.ops, a.dtheta, g.L, g.Lp, g.H, g.Hphi, fl,
                       g.scale * LOG2E, g.hscale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool gate = a.ops.gate2 != nullptr;
  if (al) return gate ? launch_bwd_grads<D, NW, true, true>(g, a, stream)
                      : launch_bwd_grads<D, NW, true, false>(g, a, stream);
  return gate ? launch_bwd_grads<D, NW, false, true>(g, a, stream)
              : launch_bwd_grads<D, NW, false, false>(g, a, stream);
}

template <int P>
hipError_t launch_rscan(const Geometry& g, const float* dtheta, float* totals, float* dphi,
                        hipStream_t stream) {
  const int nch = (g.L + RCH - 1) / RCH;
  const int nseg = g.B * g.Hphi;
  hipLaunchKernelGGL((rscan_totals_kernel<P>), dim3(nch, nseg), dim3(256), 0, stream, dtheta,
                     totals, g.L, g.H, g.Hphi, nch);
  hipLaunchKernelGGL((rscan_apply_kernel<P>), dim3(nch, nseg), dim3(256), 0, stream, dtheta,
                     totals, dphi, g.L, g.H, g.Hphi, nch, (g.flags & ARP_SCAN_EXCLUSIVE) ? 1 : 0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 6. fp32 I/O: the same gradients with plain FMAs (no matrix cores), for the
// small fp32 problems.  Four lanes per row, each holding a quarter of the
// head dimension; dot products are reduced over the four lanes.
// ---------------------------------------------------------------------------
constexpr int F32B_ROWS = 64;  // rows (queries or keys) per workgroup
constexpr int F32B_T = 32;     // rows per staged LDS tile

// Rotated operands, -lse, -D and dTheta's transport term: one thread per
// (token, pair); the P threads of a token are consecutive lanes.
template <int D>
__global__ __launch_bounds__(256) void bwd_f32_prep_kernel(BwdF32Args a, int L, int H, int Hphi,
                                                           uint32_t flags, float qscale0,
                                                           const float* __restrict__ hscale) {
  constexpr int P = D / 2;
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh % H, g = (Hphi == 1) ? 0 : h;
  const float qscale = hscale != nullptr ? qscale0 * hscale[h] : qscale0;  // AdaScale
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int t = idx / P, p = idx % P;
  const bool ok = t < L;
  const bool rqk = (flags & ARP_ROTATE_QK) != 0, rv = (flags & ARP_ROTATE_V) != 0;
  float dsum = 0.f;
  if (ok) {
    const size_t off = ((size_t)bh * L + t) * D + 2 * p;
    float q0 = a.q[off], q1 = a.q[off + 1], k0 = a.k[off], k1 = a.k[off + 1];
    float v0 = a.v[off], v1 = a.v[off + 1], o0 = a.o[off], o1 = a.o[off + 1];
    float d0 = a.dout[off], d1 = a.dout[off + 1];
    if (rqk || rv) {
      float sn, cs;
      sincosf(a.theta[((size_t)(b * Hphi + g) * L + t) * P + p], &sn, &cs);
      if (rqk) {
        rotate_pair(q0, q1, cs, sn);
        rotate_pair(k0, k1, cs, sn);
      }
      if (rv) {
        rotate_pair(v0, v1, cs, sn);
        rotate_pair(o0, o1, cs, sn);
        rotate_pair(d0, d1, cs, sn);
      }
    }
    a.qs[off] = q0 * qscale;
    a.qs[off + 1] = q1 * qscale;
    a.kr[off] = k0;
    a.kr[off + 1] = k1;
    a.vr[off] = v0;
    a.vr[off + 1] = v1;
    a.dor[off] = d0;
    a.dor[off + 1] = d1;
    dsum = fmaf(d0, o0, d1 * o1);
    // value transport: -<do~, J o~> = d0 o1 - d1 o0
    a.dtheta[((size_t)bh * L + t) * P + p] = rv ? (d0 * o1 - d1 * o0) : 0.f;
  }
#pragma unroll
  for (int m = 1; m < P; m <<= 1) dsum += __shfl_xor(dsum, m);
  if (ok && p == 0) {
    a.nd[(size_t)bh * L + t] = -dsum;
    a.nl[(size_t)bh * L + t] = -a.lse[(size_t)bh * L + t];
  }
}

// <a, J x> per pair for this lane's dims, added to dth; then g <- R(theta)^T g.
template <int DQ>
__device__ __forceinline__ void f32_grad_out(float (&gr)[DQ], const float (&x)[DQ], float xmul,
                                             const float* th, bool rot, float* dth, float* out) {
#pragma unroll
  for (int e = 0; e < DQ; e += 2) {
    float g0 = gr[e], g1 = gr[e + 1];
    if (rot) {
      const float x0 = x[e] * xmul, x1 = x[e + 1] * xmul;
      dth[e / 2] += -g0 * x1 + g1 * x0;
      float sn, cs;
      sincosf(th[e / 2], &sn, &cs);
      rotate_pair(g0, g1, cs, -sn);
    }
    out[e] = g0;
    out[e + 1] = g1;
  }
}

// dK, dV: a workgroup owns 64 keys and walks the query tiles from its first
// key to the end.
template <int D, bool ALIBI>
__global__ __launch_bounds__(256) void bwd_f32_dkdv_kernel(BwdF32Args a, int L, int H, int Hphi,
                                                           uint32_t flags) {
  constexpr int DQ = D / 4, P = D / 2;
  __shared__ float sq[F32B_T][D], sdo[F32B_T][D], snl[F32B_T], snd[F32B_T];
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh % H, g = (Hphi == 1) ? 0 : h;
  const int tid = threadIdx.x, sp = tid & 3;
  const int j = blockIdx.x * F32B_ROWS + tid / 4;
  const int jc = min(j, L - 1);
  const int d0 = sp * DQ;
  float kv[DQ], vv[DQ], dk[DQ], dv[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    kv[e] = a.kr[((size_t)bh * L + jc) * D + d0 + e];
    vv[e] = a.vr[((size_t)bh * L + jc) * D + d0 + e];
    dk[e] = dv[e] = 0.f;
  }
  const float slope2 = ALIBI ? a.alibi[h] * LOG2E : 0.f;
  const int jfirst = blockIdx.x * F32B_ROWS;
  for (int i0 = (jfirst / F32B_T) * F32B_T; i0 < L; i0 += F32B_T) {
    __syncthreads();
    for (int e = tid; e < F32B_T * D; e += 256) {
      const int r = e / D, c = e % D, i = i0 + r;
      sq[r][c] = (i < L) ? a.qs[((size_t)bh * L + i) * D + c] : 0.f;
      sdo[r][c] = (i < L) ? a.dor[((size_t)bh * L + i) * D + c] : 0.f;
    }
    if (tid < F32B_T) {
      const int i = i0 + tid;
      snl[tid] = (i < L) ? a.nl[(size_t)bh * L + i] : -INFINITY;
      snd[tid] = (i < L) ? a.nd[(size_t)bh * L + i] : 0.f;
    }
    __syncthreads();
    // queries i >= j of the tile (the four lanes of a key share the bounds)
    const int ibeg = max(0, j - i0), iend = min(F32B_T, L - i0);
    for (int r = ibeg; r < iend; ++r) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < DQ; ++e) {
        s = fmaf(kv[e], sq[r][d0 + e], s);
        dp = fmaf(vv[e], sdo[r][d0 + e], dp);
      }
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      dp += __shfl_xor(dp, 1);
      dp += __shfl_xor(dp, 2);
      s += snl[r];
      if (ALIBI) s += slope2 * (float)(j - (i0 + r));
      const float pr = exp2f(s);
      const float ds = pr * (dp + snd[r]);
#pragma unroll
      for (int e = 0; e < DQ; ++e) {
        dk[e] = fmaf(ds, sq[r][d0 + e], dk[e]);
        dv[e] = fmaf(pr, sdo[r][d0 + e], dv[e]);
      }
    }
  }
  if (j >= L) return;
  // dk~ = scale sum dS q~ = ln 2 sum dS q~s (q~s carries scale log2 e)
#pragma unroll
  for (int e = 0; e < DQ; ++e) dk[e] *= 0.69314718055994531f;
  const float* th = a.theta + ((size_t)(b * Hphi + g) * L + j) * P + d0 / 2;
  float* dth = a.dtheta + ((size_t)bh * L + j) * P + d0 / 2;
  const size_t row = ((size_t)bh * L + j) * D + d0;
  f32_grad_out<DQ>(dk, kv, 1.f, th, (flags & ARP_ROTATE_QK) != 0, dth, a.dk + row);
  f32_grad_out<DQ>(dv, vv, 1.f, th, (flags & ARP_ROTATE_V) != 0, dth, a.dv + row);
}

// dQ: a workgroup owns 64 queries and walks the key tiles up to its last query.
template <int D, bool ALIBI>
__global__ __launch_bounds__(256) void bwd_f32_dq_kernel(BwdF32Args a, int L, int H, int Hphi,
                                                         uint32_t flags, float scale0,
                                                         const float* __restrict__ hscale) {
  constexpr int DQ = D / 4, P = D / 2;
  __shared__ float sk[F32B_T][D], sv[F32B_T][D];
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh % H, g = (Hphi == 1) ? 0 : h;
  // scale times the head's query multiplier (AdaScale): dq = lambda_h dq'
  const float scale = hscale != nullptr ? scale0 * hscale[h] : scale0;
  const int tid = threadIdx.x, sp = tid & 3;
  const int i = blockIdx.x * F32B_ROWS + tid / 4;
  const int ic = min(i, L - 1);
  const int d0 = sp * DQ;
  float qv[DQ], dov[DQ], dq[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    qv[e] = a.qs[((size_t)bh * L + ic) * D + d0 + e];
    dov[e] = a.dor[((size_t)bh * L + ic) * D + d0 + e];
    dq[e] = 0.f;
  }
  const float nl = a.nl[(size_t)bh * L + ic], nd = a.nd[(size_t)bh * L + ic];
  const float slope2 = ALIBI ? a.alibi[h] * LOG2E : 0.f;
  const int i_last = min(L - 1, blockIdx.x * F32B_ROWS + F32B_ROWS - 1);
  for (int j0 = 0; j0 <= i_last; j0 += F32B_T) {
    __syncthreads();
    for (int e = tid; e < F32B_T * D; e += 256) {
      const int r = e / D, c = e % D, jj = j0 + r;
      sk[r][c] = (jj < L) ? a.kr[((size_t)bh * L + jj) * D + c] : 0.f;
      sv[r][c] = (jj < L) ? a.vr[((size_t)bh * L + jj) * D + c] : 0.f;
    }
    __syncthreads();
    // keys j <= i of the tile (the four lanes of a query share the bound)
    const int jn = min(F32B_T, ic + 1 - j0);
    for (int r = 0; r < jn; ++r) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < DQ; ++e) {
        s = fmaf(qv[e], sk[r][d0 + e], s);
        dp = fmaf(dov[e], sv[r][d0 + e], dp);
      }
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      dp += __shfl_xor(dp, 1);
      dp += __shfl_xor(dp, 2);
      s += nl;
      if (ALIBI) s += slope2 * (float)((j0 + r) - ic);
      const float ds = exp2f(s) * (dp + nd);
#pragma unroll
      for (int e = 0; e < DQ; ++e) dq[e] = fmaf(ds, sk[r][d0 + e], dq[e]);
    }
  }
  if (i >= L) return;
#pragma unroll
  for (int e = 0; e < DQ; ++e) dq[e] *= scale;  // dq~ = scale sum dS k~
  const float* th = a.theta + ((size_t)(b * Hphi + g) * L + i) * P + d0 / 2;
  float* dth = a.dtheta + ((size_t)bh * L + i) * P + d0 / 2;
  // q~ = q~s / (scale log2 e)
  f32_grad_out<DQ>(dq, qv, 1.f / (scale * LOG2E), th, (flags & ARP_ROTATE_QK) != 0, dth,
                   a.dq + ((size_t)bh * L + i) * D + d0);
}

template <int D>
hipError_t launch_bwd_f32_d(const Geometry& g, const BwdF32Args& a, hipStream_t stream) {
  constexpr int P = D / 2;
  const int BH = g.B * g.H;
  const bool al = (g.flags & ARP_ALIBI) != 0;
  hipLaunchKernelGGL((bwd_f32_prep_kernel<D>), dim3((g.L * P + 255) / 256, BH), dim3(256), 0,
                     stream, a, g.L, g.H, g.Hphi, g.flags, g.scale * LOG2E, g.hscale);
  const dim3 grid((g.L + F32B_ROWS - 1) / F32B_ROWS, BH);
  if (al) {
    hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D, true>), grid, dim3(256), 0, stream, a, g.L, g.H,
                       g.Hphi, g.flags);
    hipLaunchKernelGGL((bwd_f32_dq_kernel<D, true>), grid, dim3(256), 0, stream, a, g.L, g.H,
                       g.Hphi, g.flags, g.scale, g.hscale);
  } else {
    hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D, false>), grid, dim3(256), 0, stream, a, g.L, g.H,
                       g.Hphi, g.flags);
    hipLaunchKernelGGL((bwd_f32_dq_kernel<D, false>), grid, dim3(256), 0, stream, a, g.L, g.H,
                       g.Hphi, g.flags, g.scale, g.hscale);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_f32(const Geometry& g, const BwdF32Args& a, hipStream_t stream) {
  hipError_t e = (g.D == 64) ? launch_bwd_f32_d<64>(g, a, stream) : launch_bwd_f32_d<128>(g, a, stream);
  if (e != hipSuccess) return e;
  return (g.P == 32) ? launch_rscan<32>(g, a.dtheta, a.totals, a.dphi, stream)
                     : launch_rscan<64>(g, a.dtheta, a.totals, a.dphi, stream);
}

hipError_t launch_backward_bf16(const Geometry& g, const BwdArgs& a, hipStream_t stream) {
  hipError_t e = (g.D == 64) ? launch_bwd_d<64, 8>(g, a, stream) : launch_bwd_d<128, 4>(g, a, stream);
  if (e != hipSuccess) return e;
  return (g.P == 32) ? launch_rscan<32>(g, a.dtheta, a.totals, a.dphi, stream)
                     : launch_rscan<64>(g, a.dtheta, a.totals, a.dphi, stream);
}

}  // namespace arp
