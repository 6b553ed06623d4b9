// attn_bf16.hip -- causal attention over rotated bf16 operands, on the gfx950
// matrix cores.
//
//   s_ij  = <q~_i, k~_j> (q~ already carries scale * log2 e)  [- m_h log2e (i-j)]
//   o~_i  = sum_{j<=i} 2^(s_ij - M_i) v~_j / sum_{j<=i} 2^(s_ij - M_i)
//   o_i   = R(Theta_i)^T o~_i  (value transport)  or  o~_i
//
// ("Why Do Accumulated Transformations Extrapolate?" eq. (2)-(4), (8), (11);
// the distance bias is the far-mass control its Sec. 4 names.)
//
// Work decomposition
//  * A workgroup owns BM = NW * QPW consecutive queries of one (batch, head)
//    and walks the key tiles j0 = 0, BN, 2BN, ... up to its last query.
//    Each of its NW waves owns QPW queries; a wave skips tiles past its own
//    last query and masks only the tile that crosses its diagonal.
//  * Both products put the query on the matrix-core N axis, so one lane owns
//    one query and the softmax row statistics are per lane:
//      S^T [keys x queries] = K~ [keys x D] . Q~^T          (v_mfma_f32_32x32x16_bf16)
//      O^T [D x queries]   += V~^T [D x keys] . P^T         (same instruction)
//    The row maximum needs one cross-lane exchange (lane ^ 32) per tile.
//  * K~ rows are stored in LDS in an order (bits 2 and 3 of the row index
//    swapped) that makes the S^T accumulator layout coincide with the P^T
//    operand layout: a lane's 8 consecutive accumulator values are its 8
//    consecutive keys, so P^T is built with no data movement.
//  * Q~ stays in registers for the whole key loop.  K~ and V~^T tiles are
//    double-buffered in LDS with an XOR swizzle of 16-byte chunks (no bank
//    conflicts on the 128-bit reads); the next tile's global loads are in
//    flight while the current tile is computed; one barrier per tile.
//  * The running max is subtracted inside the matrix-core product (the
//    accumulator is initialised to -m), and it is only raised when a row's
//    tile maximum exceeds it by more than TAU = 8 (so 2^(s-m) <= 256): most
//    tiles need no rescale of the output accumulator.  Row sums are formed
//    from the bf16 probabilities with v_dot2_f32_bf16 (two per instruction).
//  * Workgroups are numbered so that each XCD (blockIdx % 8) gets whole heads
//    (its L2 then holds that head's K/V), longest query tiles first.
#include "arp_device.hpp"
#include "arp_internal.hpp"

namespace arp {

namespace {

constexpr int BN = 64;        // keys per tile
constexpr float TAU = 8.0f;   // lazy-rescale threshold (base-2 logits)

__device__ __forceinline__ int swap_bits23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D, int QPW, int NW, bool ALIBI, bool ROTV>
__global__ __launch_bounds__(NW * 64, 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kr,
    const uint16_t* __restrict__ vt, const float* __restrict__ theta,
    const float* __restrict__ alibi, uint16_t* __restrict__ o, int L, int Lp, int H, int Hphi,
    int nqt, int total_tiles) {
  constexpr int NT = NW * 64;
  constexpr int BM = QPW * NW;
  constexpr int QB = QPW / 32;         // 32-query blocks per wave
  constexpr int KS = D / 16;           // k-steps of S^T (16 of D each)
  constexpr int DB = D / 32;           // 32-row blocks of O^T
  constexpr int KB = BN / 32;          // 32-key blocks of S^T
  constexpr int KS2 = BN / 16;         // k-steps of O^T (16 keys each)
  constexpr int KROW = D * 2;          // bytes per K~ row in LDS
  constexpr int KTILE = BN * KROW;
  constexpr int VROW = BN * 2;         // bytes per V~^T row in LDS
  constexpr int VTILE = D * VROW;
  constexpr int STAGE = KTILE + VTILE;
  constexpr int KCH = D / 8;           // 16-byte chunks per K~ row
  constexpr int NKL = BN * KCH / NT;   // K chunks each thread stages
  constexpr int NVL = D * (BN / 8) / NT;
  static_assert(NKL * NT == BN * KCH && NVL * NT == D * (BN / 8), "staging split");
  static_assert(QPW % 32 == 0 && BN == 64, "tile shape");

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  // ---- which tile: XCD-aware, heads grouped per XCD, longest tiles first ----
  const int per = (total_tiles + 7) / 8;
  const int logical = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (logical >= total_tiles) return;
  const int bh = logical / nqt;
  const int qt = nqt - 1 - logical % nqt;
  const int q0 = qt * BM;
  const int b = bh / H, h = bh % H;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, hf = lane >> 5;
  const int qw = q0 + wave * QPW;  // first query of this wave
  const int last_tile = min(q0 + BM - 1, L - 1) / BN;
  const int last_tile_w = min(qw + QPW - 1, L - 1) / BN;

  // ---- Q~ operand: lane (ln, hf) holds query qw+32qb+ln, d = 16ks+8hf..+7 ----
  bf16x8 qop[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[qb][ks] = *reinterpret_cast<const bf16x8*>(
          qr + ((size_t)bh * Lp + qw + 32 * qb + ln) * D + 16 * ks + 8 * hf);

  f32x16 oacc[DB][QB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][qb][r] = 0.f;
  float mrun[QB], lsum[QB];
  f32x16 cneg[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mrun[qb] = 0.f;
    lsum[qb] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) cneg[qb][r] = 0.f;
  }
  const float slope2 = ALIBI ? alibi[h] * LOG2E : 0.f;

  // ---- staging: global -> registers -> LDS (swizzled) ----
  const uint16_t* kbase = kr + (size_t)bh * Lp * D;
  const uint16_t* vbase = vt + (size_t)bh * D * Lp;
  u32x4 kreg[NKL], vreg[NVL];
  auto stage_load = [&](int tile) {
    const int j0 = tile * BN;
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const int idx = i * NT + tid;
      const int r = idx / KCH, c = idx % KCH;
      kreg[i] = *reinterpret_cast<const u32x4*>(kbase + (size_t)(j0 + r) * D + 8 * c);
    }
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      const int idx = i * NT + tid;
      const int drow = idx / (BN / 8), c = idx % (BN / 8);
      vreg[i] = *reinterpret_cast<const u32x4*>(vbase + (size_t)drow * Lp + j0 + 8 * c);
    }
  };
  auto stage_store = [&](int buf) {
    uint8_t* base = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const int idx = i * NT + tid;
      const int r = idx / KCH, c = idx % KCH;
      const int row = (r & ~31) | swap_bits23(r & 31);
      *reinterpret_cast<u32x4*>(base + row * KROW + ((c ^ (row & 7)) << 4)) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      const int idx = i * NT + tid;
      const int drow = idx / (BN / 8), c = idx % (BN / 8);
      *reinterpret_cast<u32x4*>(base + KTILE + drow * VROW + ((c ^ (drow & 7)) << 4)) = vreg[i];
    }
  };

  stage_load(0);
  stage_store(0);
  __syncthreads();

  for (int n = 0; n <= last_tile; ++n) {
    const int cur = n & 1;
    if (n < last_tile) stage_load(n + 1);
    if (n <= last_tile_w) {
      const uint8_t* kt = smem + cur * STAGE;
      const uint8_t* vtile = kt + KTILE;
      const int j0 = n * BN;

      // S^T - m = K~ Q~^T + cneg
      f32x16 s[KB][QB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int row = 32 * kb + ln;
        bf16x8 ka[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          ka[ks] = *reinterpret_cast<const bf16x8*>(kt + row * KROW + (((2 * ks + hf) ^ (ln & 7)) << 4));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          s[kb][qb] = mfma32(ka[0], qop[qb][0], cneg[qb]);
#pragma unroll
          for (int ks = 1; ks < KS; ++ks) s[kb][qb] = mfma32(ka[ks], qop[qb][ks], s[kb][qb]);
        }
      }

      // Element r of s[kb][qb] on this lane is key j0 + koff(kb, r) + 8 hf,
      // koff = 32 kb + 16 (r>>3) + 4 ((r>>2)&1) + (r&3); query qw + 32 qb + ln.
      const bool diag = (j0 + BN - 1 > qw);
      if (ALIBI || diag) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int base = j0 + 8 * hf - (qw + 32 * qb + ln);  // key - query minus koff
          const float fb = slope2 * (float)base;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int koff = 32 * kb + 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3);
              float x = s[kb][qb][r];
              if (ALIBI) x += fmaf(slope2, (float)koff, fb);
              if (diag && koff + base > 0) x = -INFINITY;
              s[kb][qb][r] = x;
            }
        }
      }

      // Row maxima of the shifted logits (both lane halves).
      float mx[QB];
      bool need = (n == 0);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float t = s[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = (kb == 0 ? 1 : 0); r < 16; r += 2) {
            if (r + 1 < 16) t = fmaxf(t, fmaxf(s[kb][qb][r], s[kb][qb][r + 1]));
            else t = fmaxf(t, s[kb][qb][r]);
          }
        t = fmaxf(t, __shfl_xor(t, 32));
        mx[qb] = t;
        need |= (t > TAU);
      }
      if (__any(need)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float delta = (n == 0) ? mx[qb] : fmaxf(mx[qb], 0.f);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][qb][r] -= delta;
          if (n != 0) {
            const float alpha = __builtin_amdgcn_exp2f(-delta);
            lsum[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
              for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha;
          }
          mrun[qb] += delta;
#pragma unroll
          for (int r = 0; r < 16; ++r) cneg[qb][r] = -mrun[qb];
        }
      }

      // P = 2^(s - m) in bf16, row sums, then O^T += V~^T P^T.
      bf16x8 pop[KS2][QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int ks2 = 0; ks2 < KS2; ++ks2) {
          const int kb = ks2 >> 1, r0 = 8 * (ks2 & 1);
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(s[kb][qb][r0 + 2 * e]);
            const float p1 = __builtin_amdgcn_exp2f(s[kb][qb][r0 + 2 * e + 1]);
            w[e] = pack_bf16x2(p0, p1);
            lsum[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]),
                                                       __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                                       lsum[qb], false);
          }
          u32x4 wv = {w[0], w[1], w[2], w[3]};
          pop[ks2][qb] = __builtin_bit_cast(bf16x8, wv);
        }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = 32 * db + ln;
#pragma unroll
        for (int ks2 = 0; ks2 < KS2; ++ks2) {
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(
              vtile + row * VROW + (((2 * ks2 + hf) ^ (ln & 7)) << 4));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = mfma32(va, pop[ks2][qb], oacc[db][qb]);
        }
      }
    }
    if (n < last_tile) stage_store(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, value-transport un-rotation, store bf16 ----
  const int g = (Hphi == 1) ? 0 : h;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int i = qw + 32 * qb + ln;
    const float ltot = lsum[qb] + __shfl_xor(lsum[qb], 32);
    if (i >= L) continue;
    const float inv = 1.f / ltot;
    const float* th = theta + ((size_t)(b * Hphi + g) * L + i) * (D / 2);
    uint16_t* orow = o + ((size_t)bh * L + i) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // rows 32db + 8j + 4hf + {0..3}: two rotary pairs
        const int d0 = 32 * db + 8 * j + 4 * hf;
        float x0 = oacc[db][qb][4 * j + 0] * inv, x1 = oacc[db][qb][4 * j + 1] * inv;
        float x2 = oacc[db][qb][4 * j + 2] * inv, x3 = oacc[db][qb][4 * j + 3] * inv;
        if (ROTV) {
          const float2 a = *reinterpret_cast<const float2*>(th + d0 / 2);
          float s0, c0, s1, c1;
          sincosf(a.x, &s0, &c0);
          sincosf(a.y, &s1, &c1);
          rotate_pair(x0, x1, c0, -s0);
          rotate_pair(x2, x3, c1, -s1);
        }
        u32x2 w = {pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
  }
}

template <int D, int QPW, int NW>
hipError_t launch_bf16_cfg(const Geometry& g, const uint16_t* qr, const uint16_t* kr,
                           const uint16_t* vt, const float* theta, const float* alibi, uint16_t* o,
                           hipStream_t stream) {
  constexpr int BM = QPW * NW;
  const int nqt = (g.L + BM - 1) / BM;
  const int total = g.B * g.H * nqt;
  const int grid = ((total + 7) / 8) * 8;
  const bool al = g.flags & ARP_ALIBI, rv = g.flags & ARP_ROTATE_V;
#define ARP_BF16_LAUNCH(A, R)                                                                 \
  hipLaunchKernelGGL((attn_bf16_kernel<D, QPW, NW, A, R>), dim3(grid), dim3(NW * 64), 0,     \
                     stream, qr, kr, vt, theta, alibi, o, g.L, g.Lp, g.H, g.Hphi, nqt, total)
  if (al) {
    if (rv) ARP_BF16_LAUNCH(true, true); else ARP_BF16_LAUNCH(true, false);
  } else {
    if (rv) ARP_BF16_LAUNCH(false, true); else ARP_BF16_LAUNCH(false, false);
  }
#undef ARP_BF16_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16_rotated(const Geometry& g, const uint16_t* qr, const uint16_t* kr,
                                    const uint16_t* vt, const float* theta, const float* alibi,
                                    uint16_t* o, hipStream_t stream) {
  if (g.D == 64) return launch_bf16_cfg<64, 64, 4>(g, qr, kr, vt, theta, alibi, o, stream);
  return launch_bf16_cfg<128, 32, 4>(g, qr, kr, vt, theta, alibi, o, stream);
}

hipError_t launch_attn_bf16_fused(const Geometry&, const uint16_t*, const uint16_t*,
                                  const uint16_t*, const float*, const float*, uint16_t*,
                                  hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace arp
