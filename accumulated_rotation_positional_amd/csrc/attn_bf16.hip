// attn_bf16.hip -- causal attention over rotated bf16 operands, on the gfx950
// matrix cores.
//
//   s_ij  = <q~_i, k~_j> (q~ already carries scale * log2 e)  [+ m_h log2e (j - i)]
//   o~_i  = sum_{j<=i} 2^(s_ij - M_i) v~_j / sum_{j<=i} 2^(s_ij - M_i)
//   o_i   = R(Theta_i)^T o~_i  (value transport)  or  o~_i
//
// ("Why Do Accumulated Transformations Extrapolate?" eq. (2)-(4), (8), (11);
// the distance bias is the far-mass control its Sec. 4 names.)
//
// Work decomposition
//  * A workgroup owns BM = NW * QPW consecutive queries of one (batch, head)
//    and walks the key tiles j0 = 0, BN, 2BN, ... up to its last query (with
//    a distance or gate bias: from its last query back to key 0, stopping
//    once every remaining probability is exactly zero).  Each of its NW
//    waves owns QPW queries; a wave skips the tiles past its own last query
//    and masks only the tile that holds its diagonal.
//  * Both products put the query on the matrix-core N axis, so one lane owns
//    one query and the softmax row statistics are per lane:
//      S^T [keys x queries] = K~ [keys x D] . Q~^T          (v_mfma_f32_32x32x16_bf16)
//      O^T [D x queries]   += V~^T [D x keys] . P^T         (same instruction)
//    A row maximum needs one exchange between the two half-waves.
//  * K~ rows sit in LDS in an order (bits 2 and 3 of the row index swapped)
//    that makes the S^T accumulator layout coincide with the P^T operand
//    layout: a lane's 8 consecutive accumulator values are its 8 consecutive
//    keys, so P^T is built in registers with no data movement.
//  * K~ and V tiles go from global memory straight into LDS
//    (global_load_lds_dwordx4, no staging registers) through a ring of NST
//    stages: the loads of the next NST-1 tiles are in flight while a tile is
//    computed; one barrier per tile.  The LDS layout XOR-swizzles 16-byte chunks (no bank
//    conflicts on the 128-bit operand reads); since a direct load writes lane
//    l's 16 bytes to position 16 l, the swizzle is applied to the global
//    addresses instead.  V rows stay in their natural [key, d] layout (the
//    caller's v, or the rotation pass's v~ with value transport); the P V
//    product's V^T operand is read from them with LDS transpose reads
//    (ds_read_b64_tr_b16: each group of 16 lanes names a 16 x 4 block of
//    16-bit elements, four consecutive d of four keys per lane, and lane i
//    receives d = i of the four keys).
//  * q is rotated, scaled by scale * log2 e (and the head's query multiplier)
//    and rounded to bf16 in the prologue; the rotation pass only writes k~
//    (and v~ with value transport).  Every sin/cos here (q, the fused
//    staging, the value-transport epilogue) is the hardware sine and cosine
//    of turns (__sincosf), absolute error below 3e-7 on the scan's [-pi, pi).
//  * The running maximum is subtracted inside the matrix-core product (the
//    accumulator input is -m, kept in registers; on the biased walk it also
//    carries each logit's distance bias), and it is only raised when
//    a row's tile maximum exceeds it by more than TAU = 8 (so 2^(s-m) <= 256):
//    most tiles need no rescale of the output accumulator.  Row sums are
//    formed from the bf16 probabilities with v_dot2_f32_bf16.
//  * Workgroups are numbered so that each XCD (blockIdx % 8) gets whole
//    heads (its L2 then holds that head's K/V), longest query tiles first;
//    with a bias, whose early stop makes the work per head uneven, they are
//    spread across the XCDs instead.
#include "arp_device.hpp"
#include "arp_internal.hpp"
#include "mfma_tile.hpp"

namespace arp {

namespace {

constexpr int BN = KEY_TILE;  // keys per tile
constexpr float TAU = 8.0f;   // lazy-rescale threshold (base-2 logits)
// A tile whose logits all lie more than ZGAP below the running maximum has
// probabilities 2^(s - m) < 2^-160, below fp32's smallest subnormal (2^-149):
// every one of them is exactly zero, so skipping the tile changes no bit.
constexpr float ZGAP = 160.0f;
// Adjacent query tiles of one head that a biased launch places on one XCD at
// the same time (they share key/value tiles in its L2): 8 at d = 64, 4 at d =
// 128, where a tile's K/V walk holds twice the bytes (4 x 8 heads at 8192
// tokens with ALiBi: 436 us with groups of 8, 398 us with 4; at d = 64 groups
// of 4 or 16 were no faster).
template <int D>
constexpr int spread_group() { return D == 64 ? 8 : 4; }

// qr is the raw q ([B, H, L, D]), rotated and scaled in the prologue.
// FUSED = false: k~ (L padded to Lp) comes pre-rotated from the rotation pass,
// V rows come from vt ([B*H, vrows, D]: the pass's v~ with vrows = Lp, or the
// caller's v with vrows = L, rows past vrows - 1 read as row vrows - 1 -- their
// probabilities are zero), both tiles load straight into LDS, and the per-tile
// key-norm maxima kmax bound the logits.
// FUSED = true: kr, vt are the raw k, v ([B, H, L, D]); each K/V tile is
// rotated while it is staged through registers into LDS (sin/cos once per
// (key, pair), shared by k and v) in the layout the direct loads give the
// pre-rotated rows; row maxima are always taken exactly.
// BIAS: bit 0 the distance bias -m_h (i - j), bit 1 the forget-gate bias
// G_i - G_j, with G = log2 e * (prefix sums of log f) from the gate pass
// (non-increasing, so the bias never raises a score), read in its tiled
// form: gate2 [B*H, Lp] the offset of G_t within its 64-token tile, gbase
// [B*H, Lp/64] (fp64) the prefix before each tile, so G_i - G_j =
// D + gate2[i] - gate2[j] with D = fp32(gbase[i/64] - gbase[j/64]) formed once
// per (wave, key tile).
// One query tile (logical index `logical`, mapped to (head, query tile) below)
// with the workgroup's LDS ring smem.
template <int D, int QPW, int NW, int NST, int MINB, bool FUSED, int BIAS, bool ROTV>
__device__ __forceinline__ void attn_tile(
    int logical, uint8_t* smem, const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kr,
    const uint16_t* __restrict__ vt, const float* __restrict__ kmax,
    const float* __restrict__ theta, const float* __restrict__ alibi,
    const float* __restrict__ gate2, const double* __restrict__ gbase, uint16_t* __restrict__ o,
    float* __restrict__ lse, int L, int Lp, int vrows, int H, int Hphi, int nqt, int total_tiles,
    int rot_qk, float qscale0, const float* __restrict__ hscale) {
  constexpr bool ALIBI = (BIAS & 1) != 0;
  constexpr bool FORGET = (BIAS & 2) != 0;
  static_assert(!(FUSED && FORGET), "the gate bias needs the pre-rotation path");
  constexpr int BM = QPW * NW;
  constexpr int QB = QPW / 32;         // 32-query blocks per wave
  constexpr int KS = D / 16;           // k-steps of S^T (16 of D each)
  constexpr int DB = D / 32;           // 32-row blocks of O^T
  constexpr int KB = BN / 32;          // 32-key blocks of S^T
  constexpr int KS2 = BN / 16;         // k-steps of O^T (16 keys each)
  constexpr int KROW = D * 2;          // bytes per K~ row in LDS
  constexpr int KTILE = BN * KROW;
  constexpr int VTILE = BN * KROW;     // the natural V rows
  constexpr int KLD = KTILE / (1024 * NW);  // 1 KB direct loads per wave per tile
  constexpr int VLD = VTILE / (1024 * NW);
  static_assert(KLD * 1024 * NW == KTILE && VLD * 1024 * NW == VTILE, "staging split");
  static_assert(QPW % 32 == 0 && BN == 64, "tile shape");
  static_assert(NST == 2 || NST == 3, "load-wait counts are written for 2 or 3 stages");
  static_assert(!FUSED || NST == 2, "register staging uses two stages");
  constexpr int P = D / 2;
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int IPT = BN * CPR / NT;      // fused staging: (key, chunk) items per thread
  static_assert(!FUSED || IPT * NT == BN * CPR, "fused staging split");

  // the tile's 64 key gate offsets (fp32) and its fp64 gate base, padded so
  // that every stage starts on a 256-byte boundary (the LDS bank period)
  constexpr int GTILE = FORGET ? BN * 4 + 256 : 0;
  constexpr int STAGE = KTILE + VTILE + GTILE;

  // ---- which tile (the logical order is set by the kernel below) ----
  constexpr bool SPREAD = (BIAS != 0) && !FUSED;
  const int nbh = total_tiles / nqt;
  int bh, qt;
  if constexpr (SPREAD) {
    // Spread: groups of SG adjacent query tiles of one head, dealt
    // round-robin over the XCDs (blockIdx % 8) in dispatch order, so that a
    // group's workgroups run at the same time on one XCD and share the key
    // and value tiles of their overlapping walks in its L2, while the heads
    // (whose walks stop at different depths) are spread over the XCDs.  Round
    // r deals the r-th group from the end of every head, rotated by r so that
    // a head does not stay on one XCD from round to round.
    const int x = logical % 8, m = logical / 8;
    constexpr int SG = spread_group<D>();
    const int gi = (m / SG) * 8 + x;
    const int rnd = gi / nbh;
    bh = (gi % nbh + rnd) % nbh;
    qt = nqt - 1 - (rnd * SG + m % SG);
    if (qt < 0) return;
  } else {
    if (logical >= total_tiles) return;
    bh = logical / nqt;
    qt = nqt - 1 - logical % nqt;
  }
  const int q0 = qt * BM;
  const int b = bh / H, h = bh % H;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, hf = lane >> 5;
  const int qw = q0 + wave * QPW;  // first query of this wave
  const int last_tile = min(q0 + BM - 1, L - 1) / BN;
  const int last_w = (qw < L) ? min(qw + QPW - 1, L - 1) / BN : -1;
  // With a bias the key tiles are walked from the diagonal back to key 0:
  // both biases only fall with the distance (the gate prefix never rises), so
  // the first tile holds every row's largest biases, later tiles rarely raise
  // the running maximum, and once a bound on every remaining logit is ZGAP
  // below it the wave is done.  Unbiased attention walks forward, so the
  // workgroups of a head stream the same tiles through L2 together.
  constexpr bool DESC = (BIAS != 0) && !FUSED;
  // The unbiased walk at d = 128 splits off its tiles that need no maxima
  // (the key loop below); measured 1-2% faster there, and 1% slower at d = 64.
  constexpr bool SPLIT = !DESC && !FUSED && D == 128;
  auto tile_at = [&](int step) { return DESC ? last_tile - step : step; };

  // ---- direct global -> LDS loads of one K~ / V tile ----
  const uint16_t* kbase = kr + (size_t)bh * Lp * D;
  const uint16_t* vbase = vt + (size_t)bh * vrows * D;
  auto issue = [&](int tile, uint8_t* stage) __attribute__((always_inline)) {
    const int j0 = tile * BN;
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int p0 = (wave * KLD + i) * 1024;
      const int p = p0 + 16 * lane;
      const int row = p / KROW, cs = (p % KROW) / 16;
      const int c = cs ^ swz<KROW>(row);
      const uint16_t* src = kbase + (size_t)(j0 + swap_bits23(row)) * D + 8 * c;
      __builtin_amdgcn_global_load_lds((global_void_ptr)src, (lds_void_ptr)(stage + p0), 16, 0, 0);
    }
    // V rows in key order (rows past the source are clamped)
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int p0 = (wave * VLD + i) * 1024;
      const int p = p0 + 16 * lane;
      const int row = p / KROW, cs = (p % KROW) / 16;
      const int c = cs ^ swzv<KROW>(row);
      const uint16_t* src = vbase + (size_t)min(j0 + row, vrows - 1) * D + 8 * c;
      __builtin_amdgcn_global_load_lds((global_void_ptr)src, (lds_void_ptr)(stage + KTILE + p0), 16,
                                       0, 0);
    }
    if constexpr (FORGET) {
      if (wave == 0 && lane < BN / 4)
        __builtin_amdgcn_global_load_lds((global_void_ptr)(gate2 + (size_t)bh * Lp + j0 + 4 * lane),
                                         (lds_void_ptr)(stage + KTILE + VTILE), 16, 0, 0);
      // the tile's base, one 4-byte half per lane (lane l lands at 4 l)
      if (wave == 0 && lane < 2)
        __builtin_amdgcn_global_load_lds(
            (global_void_ptr)(reinterpret_cast<const uint32_t*>(gbase + (size_t)bh * (Lp / BN) + tile) +
                              lane),
            (lds_void_ptr)(stage + KTILE + VTILE + BN * 4), 4, 0, 0);
    }
  };
  // ---- fused staging: raw k, v and angles of one tile -> registers -> rotated into LDS ----
  // Item = (key kk of the tile, 16-byte chunk c of its row: four pairs); the
  // CPR lanes of a key are adjacent, so each load instruction reads whole
  // rows of k, v and theta.  The rotated rows land in the layout the direct
  // loads give the pre-rotated operands (K~ rows in swap_bits23 order,
  // chunks swizzled; natural V rows with the V swizzle), so the products
  // are the same code.
  const int g = (Hphi == 1) ? 0 : h;
  const float* th_bh = theta + (size_t)(b * Hphi + g) * L * P;
  u32x4 kreg[IPT > 0 ? IPT : 1], vreg[IPT > 0 ? IPT : 1];
  float4 treg[IPT > 0 ? IPT : 1];
  auto fetch = [&](int tile) __attribute__((always_inline)) {
    const uint16_t* kb = kr + (size_t)bh * L * D;
    const uint16_t* vb = vt + (size_t)bh * L * D;
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int it = tid + i * NT;
      const int kk = it / CPR, c = it % CPR;
      const int key = min(tile * BN + kk, L - 1);  // rows past L are masked anyway
      kreg[i] = *reinterpret_cast<const u32x4*>(kb + (size_t)key * D + 8 * c);
      vreg[i] = *reinterpret_cast<const u32x4*>(vb + (size_t)key * D + 8 * c);
      treg[i] = (rot_qk || ROTV) ? *reinterpret_cast<const float4*>(th_bh + (size_t)key * P + 4 * c)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto commit = [&](uint8_t* stage) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int it = tid + i * NT;
      const int kk = it / CPR, c = it % CPR;
      const float ang[4] = {treg[i].x, treg[i].y, treg[i].z, treg[i].w};
      u32x4 kw, vw;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float sn, cs;
        __sincosf(ang[e], &sn, &cs);
        float k0 = lo_bf16(kreg[i][e]), k1 = hi_bf16(kreg[i][e]);
        float v0 = lo_bf16(vreg[i][e]), v1 = hi_bf16(vreg[i][e]);
        if (rot_qk) rotate_pair(k0, k1, cs, sn);
        if (ROTV) rotate_pair(v0, v1, cs, sn);
        kw[e] = pack_bf16x2(k0, k1);
        vw[e] = pack_bf16x2(v0, v1);
      }
      const int row = swap_bits23(kk);  // LDS row holding this key
      *reinterpret_cast<u32x4*>(stage + row * KROW + ((c ^ swz<KROW>(row)) << 4)) = kw;
      *reinterpret_cast<u32x4*>(stage + KTILE + kk * KROW + ((c ^ swzv<KROW>(kk)) << 4)) = vw;
    }
  };

  // ---- Q~ operand: lane (ln, hf) holds query qw+32qb+ln, d = 16ks+8hf..+7,
  // rotated and multiplied by scale * log2 e and the head's query multiplier
  // here, then rounded to bf16 ----
  const float qscale = hscale != nullptr ? qscale0 * hscale[h] : qscale0;
  // The angles of the wave's queries are staged through LDS (the space of the
  // tile ring, before its first load): a lane needs 16 bytes every 32 of its
  // query's angle row, and reading them straight from global memory touches
  // QPW rows per instruction, which the L1 cannot hold across the KS
  // instructions.  Rows are loaded whole and coalesced (C4 16-byte chunks per
  // row, 64 / C4 rows per instruction), their chunks XOR-swizzled so that the
  // column reads are conflict-free.
  constexpr int TROW = P * 4;  // bytes per angle row
  constexpr int C4 = P / 4;
  // Where the LDS holds them both (one workgroup's share of the CU's 160 KB),
  // the angle rows have their own region after the ring, and the first tiles
  // are already in flight while they are staged; otherwise they use the
  // ring's space first.
  constexpr int RINGB = NST * STAGE, TSTAGEB = NW * QPW * TROW;
  constexpr bool TSEP = !FUSED && RINGB + TSTAGEB <= 163840 / MINB;
  uint8_t* const tw = smem + (TSEP ? RINGB : 0) + wave * QPW * TROW;
  if constexpr (TSEP) {
#pragma unroll
    for (int t = 0; t < NST - 1; ++t)
      if (t <= last_tile) issue(tile_at(t), smem + t * STAGE);
  }
  // the raw query words first, so that their loads and the angle rows' are in
  // flight together
  u32x4 qraw[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qraw[qb][ks] = *reinterpret_cast<const u32x4*>(
          qr + ((size_t)bh * L + min(qw + 32 * qb + ln, L - 1)) * D + 16 * ks + 8 * hf);
  // the per-tile key-norm maxima of the wave's first 256 key tiles, loaded
  // with the query words so that their latency overlaps (reduced to kglob
  // below)
  const float* kmax_bh = FUSED ? nullptr : kmax + (size_t)bh * (Lp / BN);
  float kpre[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (!FUSED) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (lane + 64 * u <= last_w) kpre[u] = kmax_bh[lane + 64 * u];
  }
  if constexpr (!FUSED) {
    if (rot_qk) {
#pragma unroll
      for (int r0 = 0; r0 < QPW; r0 += 64 / C4) {
        const int row = r0 + lane / C4, c = lane % C4;
        const float4 x = *reinterpret_cast<const float4*>(th_bh + (size_t)min(qw + row, L - 1) * P + 4 * c);
        *reinterpret_cast<float4*>(tw + row * TROW + ((c ^ swz<TROW>(row)) << 4)) = x;
      }
    }
    // a wave reads only the rows it wrote (LDS operations of a wave complete
    // in order); a shared region also waits for every wave before the ring
    if constexpr (TSEP) __builtin_amdgcn_wave_barrier();
    else __syncthreads();
  }
  bf16x8 qop[QB][KS];
  {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int i = min(qw + 32 * qb + ln, L - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 w = qraw[qb][ks];
        const int trow = 32 * qb + ln;
        const float4 a =
            !rot_qk ? make_float4(0.f, 0.f, 0.f, 0.f)
            : FUSED ? *reinterpret_cast<const float4*>(th_bh + (size_t)i * P + 8 * ks + 4 * hf)
                    : *reinterpret_cast<const float4*>(tw + trow * TROW +
                                                       (((2 * ks + hf) ^ swz<TROW>(trow)) << 4));
        const float ang[4] = {a.x, a.y, a.z, a.w};
        u32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float sn, cs;
          __sincosf(ang[e], &sn, &cs);
          float x0 = lo_bf16(w[e]), x1 = hi_bf16(w[e]);
          if (rot_qk) rotate_pair(x0, x1, cs, sn);
          r[e] = pack_bf16x2(x0 * qscale, x1 * qscale);
        }
        qop[qb][ks] = __builtin_bit_cast(bf16x8, r);
      }
    }
  }

  if constexpr (!FUSED && !TSEP) __syncthreads();  // every wave has its angles before the ring is loaded

  // |q~_i| of this lane's queries (both half-waves hold half of each row).
  float qn[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float n2 = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) n2 = fmaf((float)qop[qb][ks][e], (float)qop[qb][ks][e], n2);
    qn[qb] = sqrtf(halves_sum(n2)) * (1.f + 1e-4f);  // margin for the fp32 accumulation
  }

  // First tiles in flight before the loop: NST-1 direct loads, or tile 0
  // staged and rotated.
  if constexpr (!FUSED) {
    if constexpr (!TSEP) {
#pragma unroll
      for (int t = 0; t < NST - 1; ++t)
        if (t <= last_tile) issue(tile_at(t), smem + t * STAGE);
    }
  } else {
    fetch(0);
    commit(smem);
    __syncthreads();
  }

  f32x16 oacc[DB][QB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][qb][r] = 0.f;
  const float slope2 = ALIBI ? alibi[h] * LOG2E : 0.f;
  float gq[QB];    // the forget-gate offset of this lane's queries within their tile
  double gqb[QB];  // and that tile's base (the rows of block qb share one tile)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    gq[qb] = FORGET ? gate2[(size_t)bh * Lp + min(qw + 32 * qb + ln, Lp - 1)] : 0.f;
    gqb[qb] = FORGET ? gbase[(size_t)bh * (Lp / BN) + min((qw + 32 * qb) / BN, Lp / BN - 1)] : 0.0;
  }
  // The accumulator input of Q K^T: -m, plus with a gate bias the query's
  // gate offset and the tile base difference D (so only the key's offset is
  // left to subtract per logit; set per key tile in the walk below).
  float mrun[QB], lsum[QB];
  f32x16 cneg[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mrun[qb] = 0.f;
    lsum[qb] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) cneg[qb][r] = gq[qb];
  }

  // The largest key norm of the wave's tiles (kglob).  Unbiased walk: once
  // |q~_i| kglob lies within TAU of every row's running maximum (after the
  // first tile, on typical inputs), no later tile can need a rescale, since
  // the running maximum never falls: the per-tile bound (a load of that tile's
  // norm, waited on between Q K^T and the softmax) is then skipped for good.
  // Biased walk: a bound on the logits of the tile in flight (tb), and
  // per-wave "done" flags, kept per step parity so that a flag set in step n
  // is read in step n+1 after the barrier and no wave writes that parity
  // before every wave has read it.  A wave with no query below L is done from
  // the start.
  float tb[QB];
  float kglob = 0.f;
  bool nb_safe = false;  // wave-uniform
  __shared__ int wdone[2][DESC ? NW : 1];
  bool wave_done = false;
  if constexpr (!FUSED) {
    kglob = fmaxf(fmaxf(kpre[0], kpre[1]), fmaxf(kpre[2], kpre[3]));
    // walks of more than 256 key tiles: four loads in flight per trip
    for (int c0 = lane + 256; c0 <= last_w; c0 += 256) {
      float km4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) km4[u] = kmax_bh[min(c0 + 64 * u, last_w)];
      kglob = fmaxf(kglob, fmaxf(fmaxf(km4[0], km4[1]), fmaxf(km4[2], km4[3])));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) kglob = fmaxf(kglob, __shfl_xor(kglob, off));
  }
  if constexpr (DESC) {
    wave_done = last_w < 0;
    if (lane == 0) wdone[0][wave] = wdone[1][wave] = wave_done ? 1 : 0;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  }

  // ---- the three parts of one key tile of this wave's queries ----
  f32x16 s[KB][QB];      // logits of the tile in flight
  bf16x8 pop[KS2][QB];   // its probabilities, P^T operand layout

  // On the diagonal-first (biased) walk, and with the distance bias on the
  // fused walk, the biases ride in the accumulator input of Q K^T with -m:
  // per element the distance bias (one fused multiply-add) and minus the
  // key's gate offset (one subtraction), formed before the products, so the
  // pass over the logits after them (soft, below) is left to the diagonal
  // tile's mask
  constexpr bool CB = DESC || (FUSED && ALIBI);
  f32x16 cb[CB ? KB : 1][CB ? QB : 1];
  auto bias_init = [&](int n, int t) __attribute__((always_inline)) {
    const int j0 = t * BN;
    const float* gt = reinterpret_cast<const float*>(smem + (n % NST) * STAGE + KTILE + VTILE);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      // the gate offsets of this lane's keys: 16 h2 + 8 hf + e of the block
      f32x4 gk[4] = {};
      if constexpr (FORGET) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          gk[u] = *reinterpret_cast<const f32x4*>(gt + 32 * kb + 16 * (u >> 1) + 8 * hf + 4 * (u & 1));
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int base = j0 + 8 * hf - (qw + 32 * qb + ln);  // key - query minus koff
        const float fbm = ALIBI ? fmaf(slope2, (float)base, cneg[qb][0]) : cneg[qb][0];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int koff = 32 * kb + 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3);
          float c = ALIBI ? fmaf(slope2, (float)koff, fbm) : fbm;
          if (FORGET) c -= gk[r >> 2][r & 3];
          cb[kb][qb][r] = c;
        }
      }
    }
  };
  auto qk = [&](int n) __attribute__((always_inline)) {
    const uint8_t* kt = smem + (n % NST) * STAGE;
    // S^T - m = K~ Q~^T + cneg
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int row = 32 * kb + ln;
      bf16x8 ka[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ka[ks] = *reinterpret_cast<const bf16x8*>(kt + row * KROW + (((2 * ks + hf) ^ swz<KROW>(row)) << 4));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        s[kb][qb] = mfma32(ka[0], qop[qb][0], CB ? cb[kb][qb] : cneg[qb]);
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) s[kb][qb] = mfma32(ka[ks], qop[qb][ks], s[kb][qb]);
      }
    }

  };

  // n: step (ring stage n % NST), t: key tile, first: the wave's first tile.
  // safe: the caller has established that no row of this tile can need a
  // rescale, so the maxima are not taken
  auto soft = [&](int n, int t, bool first, bool safe = false) __attribute__((always_inline)) {
    const int j0 = t * BN;
    // Element r of s[kb][qb] on this lane is key j0 + koff(kb, r) + 8 hf,
    // koff = 32 kb + 16 (r>>3) + 4 ((r>>2)&1) + (r&3); query qw + 32 qb + ln.
    const bool diag = (t == last_w);
    if (diag) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          // elements r = 8 h2 + e: keys koff + 8 hf, koff = 32 kb + 16 h2 + e (+4 for e >= 4)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const int base = j0 + 8 * hf - (qw + 32 * qb + ln);  // key - query minus koff
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int r = 8 * h2 + e;
              const int koff = 32 * kb + 16 * h2 + 4 * (e >> 2) + (e & 3);
              float x = s[kb][qb][r];
              if (diag && koff + base > 0) x = -INFINITY;
              s[kb][qb][r] = x;
            }
          }
        }
    }

    // Row maxima of the shifted logits (both half-waves) -- only when the
    // tile might need them: s_ij <= |q~_i| max_j |k~_j| (Cauchy-Schwarz) plus
    // the tile's largest bias (the mask only lowers scores), so while that
    // bound stays within TAU of the running maximum no rescale can be due.
    bool check = FUSED || first;
    if constexpr (DESC) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) check |= (tb[qb] > mrun[qb] + TAU);
    } else if constexpr (!FUSED) {
      if (!nb_safe) {
        const float km = kmax_bh[t];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) check |= (qn[qb] * km > mrun[qb] + TAU);
      }
    }
    if (!safe && __any(check)) {
    float mx[QB];
    bool need = first;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // a chain of three-input maxima (v_max3_f32), two new values per step
      float t = s[0][qb][0];
#pragma unroll
      for (int e = 1; e + 1 < 16 * KB; e += 2)
        t = fmaxf(fmaxf(t, s[e / 16][qb][e % 16]), s[(e + 1) / 16][qb][(e + 1) % 16]);
      t = fmaxf(t, s[KB - 1][qb][15]);
      t = halves_max(t);
      mx[qb] = t;
      need |= (t > TAU);
    }
    if (__any(need)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float delta = first ? mx[qb] : fmaxf(mx[qb], 0.f);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][qb][r] -= delta;
        if (!first) {
          const float alpha = __builtin_amdgcn_exp2f(-delta);
          lsum[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha;
        }
        mrun[qb] += delta;
#pragma unroll
        for (int r = 0; r < 16; ++r) cneg[qb][r] = FORGET ? gq[qb] - mrun[qb] : -mrun[qb];
      }
    }
    if constexpr (!DESC && !FUSED) {
      bool ok = true;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) ok &= (qn[qb] * kglob <= mrun[qb] + TAU);
      nb_safe = __all(ok);
    }
    }

    // P = 2^(s - m) in bf16, row sums, then O^T += V~^T P^T.
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
  };

  // The V^T operand A[m = d][k = keys 8 hf .. 8 hf + 7] of the P V product:
  // from the natural V rows, two transpose reads of four keys each.  Source
  // lane j = lane % 16 of group g = lane / 16 names keys 16 ks2 + 8 (g / 2) +
  // 4 u + j / 4 and d = 32 db + 16 (g % 2) + 4 (j % 4) .. + 3.
  const int trj = lane & 15, trg = (lane >> 4) & 1;
  auto pv = [&](int n) __attribute__((always_inline)) {
    const uint8_t* vtile = smem + (n % NST) * STAGE + KTILE;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int ks2 = 0; ks2 < KS2; ++ks2) {
        const int colb = 64 * db + 32 * trg + 8 * (trj & 3);  // byte offset in the row
        u32x2 t[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int row = 16 * ks2 + 8 * hf + 4 * u + (trj >> 2);
          t[u] = lds_read_tr16(vtile + row * KROW + (((colb >> 4) ^ swzv<KROW>(row)) << 4) +
                               (colb & 15));
        }
        const u32x4 w = {t[0][0], t[0][1], t[1][0], t[1][1]};
        const bf16x8 va = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = mfma32(va, pop[ks2][qb], oacc[db][qb]);
      }
    }
  };

  if constexpr (!FUSED) {
    // ---- key loop: NST-stage ring; tile n+NST-1 is loaded while n is computed ----
    constexpr int LOADS = KLD + VLD;  // direct loads per wave per tile
    auto sync_step = [&](int n) __attribute__((always_inline)) {
      // step n's tile has landed once at most the loads of the steps after it are pending
      if (n + NST - 2 <= last_tile) wait_loads<(NST - 2) * LOADS>();
      else wait_loads<0>();
      // Every wave's share of step n's tile is in place and every wave is
      // done with step n-1 (whose stage the next issue overwrites).  A bare
      // s_barrier: the wait above already covers this wave's loads, and a
      // fenced barrier would also wait for the loads of the tiles still in
      // flight.
      __builtin_amdgcn_s_barrier();
    };
    auto issue_ahead = [&](int n) __attribute__((always_inline)) {
      if (n + NST - 1 <= last_tile) issue(tile_at(n + NST - 1), smem + ((n + NST - 1) % NST) * STAGE);
    };
    int n0 = 0;
    if constexpr (SPLIT) {
      // The unbiased walk at d = 128 in three loops of one barrier per step
      // each (the waves of a workgroup may be in different loops at one
      // step): this first one until the key-norm bound holds for every later
      // tile (which stays so, since the running maximum never falls); the
      // next one over the tiles before the wave's diagonal, with no maxima
      // and so no branch between the products and the exponentials; the
      // diagonal tile and the steps after it in the main loop below.
      for (; n0 <= last_tile; ++n0) {
        sync_step(n0);
        issue_ahead(n0);
        if (n0 <= last_w) {
          qk(n0);
          soft(n0, n0, n0 == 0);
          pv(n0);
        }
        if (nb_safe && n0 + 1 < last_w) {
          ++n0;
          break;
        }
      }
      for (; n0 < last_w; ++n0) {
        sync_step(n0);
        issue_ahead(n0);
        qk(n0);
        soft(n0, n0, false, true);
        pv(n0);
      }
    }
    for (int n = n0; n <= last_tile; ++n) {
      const int t = tile_at(n);
      sync_step(n);
      if constexpr (DESC) {
        if (n > 0) {  // the flags of step n-1, the same for every wave
          bool all = true;
#pragma unroll
          for (int w = 0; w < NW; ++w) all &= wdone[(n - 1) & 1][w] != 0;
          if (all) break;
        }
      }
      issue_ahead(n);
      if constexpr (DESC) {
        if (t <= last_w && !wave_done) {
          // Bound the tile's logits per row: the key-norm bound plus the
          // tile's largest bias (distance bias at the tile end nearer the
          // query -- the far end for a negative slope -- and the gate bias
          // at its last key, where the non-increasing prefix is lowest).
          // With the wave-wide key-norm maximum and a non-negative slope the
          // same bound covers every tile not yet walked.
          const bool first = (t == last_w);
          const float km = kmax_bh[t];
          const float gl = FORGET ? reinterpret_cast<const float*>(
                                        smem + (n % NST) * STAGE + KTILE + VTILE)[BN - 1]
                                  : 0.f;
          bool dead = !first && !(ALIBI && slope2 < 0.f);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const int i = qw + 32 * qb + ln;
            float bb = 0.f;
            if (ALIBI)
              bb = fmaxf(slope2 * (float)(t * BN - i), slope2 * (float)(t * BN + BN - 1 - i));
            if (FORGET) {
              // the tile base difference, rounded once (the key tile's base
              // came into LDS with its gates)
              const double gkt = *reinterpret_cast<const double*>(smem + (n % NST) * STAGE + KTILE +
                                                                  VTILE + BN * 4);
              const float dt = (float)(gqb[qb] - gkt);
              bb += gq[qb] + dt - gl;
#pragma unroll
              for (int r = 0; r < 16; ++r) cneg[qb][r] = gq[qb] + dt - mrun[qb];
            }
            tb[qb] = fmaf(qn[qb], km, bb);
            dead &= (i >= L) || (fmaf(qn[qb], kglob, bb) < mrun[qb] - ZGAP);
          }
          if (__all(dead)) {
            wave_done = true;
          } else {
            bias_init(n, t);
            qk(n);
            soft(n, t, first);
            pv(n);
          }
        }
        if (wave_done && lane == 0) {
          wdone[n & 1][wave] = 1;
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the flag is in LDS before the next barrier
        }
      } else if (n <= last_w) {
        qk(n);
        soft(n, t, n == 0);
        pv(n);
      }
    }
    if constexpr (DESC) wait_loads<0>();  // no load into LDS outlives an early exit
  } else {
    // ---- key loop, fused rotation: tile n+1 is fetched into registers while
    // n is computed, then rotated into the other stage ----
    for (int n = 0; n <= last_tile; ++n) {
      if (n + 1 <= last_tile) fetch(n + 1);
      if (n <= last_w) {
        if constexpr (ALIBI) bias_init(n, n);
        qk(n);
        soft(n, n, n == 0);
        pv(n);
      }
      if (n + 1 <= last_tile) commit(smem + ((n + 1) & 1) * STAGE);
      __syncthreads();  // tile n+1 is in place; every wave is done with tile n
    }
  }

  // ---- epilogue: normalise, value-transport un-rotation, store bf16 ----
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int i = qw + 32 * qb + ln;
    const float ltot = halves_sum(lsum[qb]);
    if (i >= L) continue;
    const float inv = 1.f / ltot;
    // base-2 log-sum-exp of the row's scaled logits, for the backward pass
    if (lse != nullptr && hf == 0) lse[(size_t)bh * L + i] = mrun[qb] + __log2f(ltot);
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
          __sincosf(a.x, &s0, &c0);
          __sincosf(a.y, &s1, &c1);
          rotate_pair(x0, x1, c0, -s0);
          rotate_pair(x2, x3, c1, -s1);
        }
        u32x2 w = {pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
  }
}

// Logical tile order: longest tiles first; without a bias, heads grouped per
// XCD (blockIdx % 8) so that its L2 holds their K/V.  A biased walk stops
// early by an amount that differs from head to head (the slope, the gates),
// so there the tiles are dealt out across the XCDs, the last query tile of
// every head first: grouping would leave the XCD with the gentlest heads
// doing several times the average work, and the longest tiles of the last
// heads would start last.
// PAIR (unbiased, total_tiles a multiple of 16; which grids is decided at
// the launch below, and the paired walk is an instantiation of its own so
// that the unpaired one keeps its own register allocation): half as many
// workgroups, each taking the c-th longest and the c-th shortest
// tile of its XCD's share one after the other, so every workgroup has the
// same work and no CU waits for a second dispatch.
template <int D, int QPW, int NW, int NST, int MINB, bool FUSED, int BIAS, bool ROTV, bool PAIR>
__global__ __launch_bounds__(NW * 64, MINB) void attn_bf16_kernel(
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kr,
    const uint16_t* __restrict__ vt, const float* __restrict__ kmax,
    const float* __restrict__ theta, const float* __restrict__ alibi,
    const float* __restrict__ gate2, const double* __restrict__ gbase, uint16_t* __restrict__ o,
    float* __restrict__ lse, int L, int Lp, int vrows, int H, int Hphi, int nqt, int total_tiles,
    int rot_qk, float qscale, const float* __restrict__ hscale) {
  static_assert(!PAIR || BIAS == 0, "pairs are for unbiased walks");
  constexpr int STAGE = BN * D * 2 + D * BN * 2 + (((BIAS & 2) != 0) ? BN * 4 + 256 : 0);  // as in attn_tile
  // the tile ring and the waves' query angle rows (after the ring, or in its
  // space before it is loaded; as in attn_tile)
  constexpr int RING = NST * STAGE, TSTAGE = FUSED ? 0 : NW * QPW * D * 2;
  constexpr int LDSB = (!FUSED && RING + TSTAGE <= 163840 / MINB) ? RING + TSTAGE
                       : (RING > TSTAGE ? RING : TSTAGE);
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDSB];
  constexpr bool SPREAD = (BIAS != 0) && !FUSED;
  const int per = (total_tiles + 7) / 8;
  if constexpr (PAIR) {
    const int x = (int)(blockIdx.x % 8), c = (int)(blockIdx.x / 8);
    attn_tile<D, QPW, NW, NST, MINB, FUSED, BIAS, ROTV>(x * per + c, smem, qr, kr, vt, kmax, theta,
                                                        alibi, gate2, gbase, o, lse, L, Lp, vrows, H, Hphi, nqt,
                                                        total_tiles, rot_qk, qscale, hscale);
    __syncthreads();  // every wave is done with the LDS ring before it is refilled
    attn_tile<D, QPW, NW, NST, MINB, FUSED, BIAS, ROTV>(x * per + per - 1 - c, smem, qr, kr, vt,
                                                        kmax, theta, alibi, gate2, gbase, o, lse, L, Lp,
                                                        vrows, H, Hphi, nqt, total_tiles, rot_qk,
                                                        qscale, hscale);
    return;
  }
  const int logical = SPREAD ? (int)blockIdx.x : (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  attn_tile<D, QPW, NW, NST, MINB, FUSED, BIAS, ROTV>(logical, smem, qr, kr, vt, kmax, theta, alibi,
                                                      gate2, gbase, o, lse, L, Lp, vrows, H, Hphi, nqt,
                                                      total_tiles, rot_qk, qscale, hscale);
}

template <int D, int QPW, int NW, int NST, int MINB, bool FUSED>
hipError_t launch_bf16_cfg(const Geometry& g, const uint16_t* qr, const uint16_t* kr,
                           const uint16_t* vt, int vrows, const float* kmax, const float* theta,
                           const float* alibi, const float* gate2, const double* gbase, uint16_t* o,
                           float* lse, hipStream_t stream) {
  constexpr int BM = QPW * NW;
  const int nqt = (g.L + BM - 1) / BM;
  const int total = g.B * g.H * nqt;
  const bool rv = g.flags & ARP_ROTATE_V;
  const int bias = ((g.flags & ARP_ALIBI) ? 1 : 0) | ((g.flags & ARP_FORGET_GATE) ? 2 : 0);
  // Paired query tiles (a workgroup takes tile c of a run of its XCD and then
  // the tile as far from the end; every pair holds the same number of key
  // tiles): always for the 512-query shape; for 4 waves x 32 queries where
  // the pairs still fill every CU and a head's walks are at most 8192 keys
  // long (2 x 8 heads at 8192 tokens, d = 64: 182 -> 157 us; 8 x 8 at 2048:
  // 70 -> 56 us; at 16384 tokens the shorter unpaired walks keep a head's
  // K/V tiles shared in L2 better: 292 against 306 us).
  // The d = 128 8-wave shape pairs where its grid holds two or three
  // workgroups per CU (1 x 16 heads at 8192 tokens: 254 -> 239 us; 1 x 32:
  // 510 -> 493 us; at four and more, rope_8k_d128's 4 x 32 heads, it stays
  // unpaired: 2028 against 2030 us).
  // With the rotation fused into the staging the 4 x 32 shape pairs by the
  // same rule (8 x 8 heads at 2048 tokens 93.6 -> 82.1 us, 2 x 8 at 4096
  // 122.5 -> 95.7 us); the 512-query fused walk does not pair (2 x 8 heads
  // at 16384 tokens: 610 against 766 us paired).
  constexpr bool CAN_PAIR = (QPW == 64 && NW == 8 && !FUSED) || (QPW == 32 && NW == 4) ||
                           (QPW == 32 && NW == 8 && !FUSED);
  const bool pair_ok = (QPW == 64 && NW == 8) ||
                       (QPW == 32 && NW == 4 && g.L <= 8192 && total / 2 >= device_cus()) ||
                       (QPW == 32 && NW == 8 && total / 2 >= device_cus() && total / 2 < 4 * device_cus());
  const bool paired = CAN_PAIR && pair_ok && bias == 0 && total % 16 == 0;
  // spread (biased, pre-rotation): every head's groups of SG query
  // tiles, a whole number of rounds over the 8 XCDs
  constexpr int SG = spread_group<D>();
  const long groups = (long)g.B * g.H * ((nqt + SG - 1) / SG);
  const int grid = paired ? total / 2
                   : (bias != 0 && !FUSED) ? (int)(((groups + 7) / 8) * 8 * SG)
                                           : ((total + 7) / 8) * 8;
  const int rqk = (g.flags & ARP_ROTATE_QK) ? 1 : 0;
  const float qscale = g.scale * LOG2E;
#define ARP_BF16_LAUNCH(A, R, P)                                                               \
  hipLaunchKernelGGL((attn_bf16_kernel<D, QPW, NW, NST, MINB, FUSED, A, R, P>), dim3(grid),   \
                     dim3(NW * 64), 0, stream, qr, kr, vt, kmax, theta, alibi, gate2, gbase, o, \
                     lse,                                                                       \
                     g.L, g.Lp, vrows, g.H, g.Hphi, nqt, total, rqk, qscale, g.hscale)
#define ARP_BF16_LAUNCH_R(A, P) \
  do {                          \
    if (rv) ARP_BF16_LAUNCH(A, true, P); else ARP_BF16_LAUNCH(A, false, P); \
  } while (0)
  auto launch_unbiased = [&]() {
    if constexpr (CAN_PAIR) {
      if (paired) {
        ARP_BF16_LAUNCH_R(0, true);
        return;
      }
    }
    ARP_BF16_LAUNCH_R(0, false);
  };
  if constexpr (FUSED) {
    if (bias & 2) return hipErrorNotSupported;
    if (bias & 1) ARP_BF16_LAUNCH_R(1, false); else launch_unbiased();
  } else {
    switch (bias) {
      case 0: launch_unbiased(); break;
      case 1: ARP_BF16_LAUNCH_R(1, false); break;
      case 2: ARP_BF16_LAUNCH_R(2, false); break;
      default: ARP_BF16_LAUNCH_R(3, false); break;
    }
  }
#undef ARP_BF16_LAUNCH_R
#undef ARP_BF16_LAUNCH
  return hipGetLastError();
}

}  // namespace

// Compute units of the current device (256 on an MI355X), queried on every
// call (a host-side attribute lookup; the library keeps no mutable state).
hipError_t launch_attn_bf16_rotated(const Geometry& g, const uint16_t* q, const uint16_t* kr,
                                    const uint16_t* v, int vrows, const float* kmax,
                                    const float* theta, const float* alibi, const float* gate2,
                                    const double* gbase, uint16_t* o, float* lse,
                                    hipStream_t stream) {
  if (g.D == 64) {
    // Two shapes, every row computed the same way in both (bit-identical
    // results):
    //  * 512-query workgroups of 8 waves x 64 queries, one per CU: the most
    //    matrix-core work per LDS operand read; best on long, deep grids
    //    (2 x 8 heads at 16384 tokens: 0.51 ms against 0.60 ms);
    //  * 128-query workgroups of 4 waves x 32 queries, two per CU: finer
    //    grains, so a grid's causal tail and a biased walk's uneven early
    //    stops cost less (8 x 8 heads at 1024 tokens 28.5 -> 24.2 us, 1 x 8 at
    //    16384 408 -> 291 us, ALiBi on 1 x 16 at 32768 1.34 -> 1.02 ms).
    // The first is taken for an unbiased walk over at least 4096 tokens
    // whose 512-query grid fills every CU twice (4 x 16 heads at 8192: 553
    // against 491 us; 8 x 8 at 4096: 168 against 152 us; at 2048 tokens the
    // second is faster: 16 x 16 heads 184 against 197 us), the second
    // otherwise.
    const long wg512 = (long)g.B * g.H * ((g.L + 511) / 512);
    const bool biased = (g.flags & (ARP_ALIBI | ARP_FORGET_GATE)) != 0;
    if (!biased && g.L >= 4096 && wg512 >= 2L * device_cus())
      return launch_bf16_cfg<64, 64, 8, 2, 1, false>(g, q, kr, v, vrows, kmax, theta, alibi, gate2, gbase, o,
                                                     lse, stream);
    return launch_bf16_cfg<64, 32, 4, 2, 2, false>(g, q, kr, v, vrows, kmax, theta, alibi, gate2, gbase, o, lse,
                                                   stream);
  }
  // d = 128: 256-query workgroups of 8 waves x 32 queries for unbiased grids
  // of at least four per CU, or two per CU from 8192 tokens (4 x 32 heads at
  // 8192 tokens: 2.06 ms against 2.12 ms; 1 x 16 at 8192: 249 against 261
  // us), else 128-query workgroups of 4 waves x 32 queries, two per CU
  // (1 x 8 heads at 8192 tokens 213 -> 201 us, 2 x 8 at 2048 63 -> 51 us; 2 x
  // 16 at 4096, paired, 148 against 189 us for the larger workgroups).
  const long wg256 = (long)g.B * g.H * ((g.L + 255) / 256);
  const bool biased = (g.flags & (ARP_ALIBI | ARP_FORGET_GATE)) != 0;
  if (!biased && wg256 >= (g.L >= 8192 ? 2L : 4L) * device_cus())
    return launch_bf16_cfg<128, 32, 8, 2, 1, false>(g, q, kr, v, vrows, kmax, theta, alibi, gate2, gbase, o,
                                                    lse, stream);
  return launch_bf16_cfg<128, 32, 4, 2, 2, false>(g, q, kr, v, vrows, kmax, theta, alibi, gate2, gbase, o, lse,
                                                  stream);
}

hipError_t launch_attn_bf16_fused(const Geometry& g, const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, const float* theta, const float* alibi,
                                  uint16_t* o, hipStream_t stream) {
  if (g.D == 64) {
    // The 512-query shape on deep unbiased grids (the pre-rotation path's
    // rule) and with the distance bias (1 x 16 heads at 32768 tokens: 3.50
    // ms against 4.30 ms with 4 waves x 32 queries); otherwise 4 waves x 32
    // queries (8 x 8 heads at 1024 tokens 51.2 -> 37.8 us, 1 x 8 at 16384
    // tokens 527 -> 452 us).
    const long wg512 = (long)g.B * g.H * ((g.L + 511) / 512);
    const bool biased = (g.flags & ARP_ALIBI) != 0;
    if (biased || (g.L >= 4096 && wg512 >= 2L * device_cus()))
      return launch_bf16_cfg<64, 64, 8, 2, 1, true>(g, q, k, v, g.L, nullptr, theta, alibi, nullptr,
                                                    nullptr, o, nullptr, stream);
    return launch_bf16_cfg<64, 32, 4, 2, 2, true>(g, q, k, v, g.L, nullptr, theta, alibi, nullptr,
                                                  nullptr, o, nullptr, stream);
  }
  // d = 128: one shape (4 waves x 32 queries stage four 16-byte pieces per
  // thread and were slower on 8 x 8 heads at 1024 tokens: 62.3 against 51.1
  // us)
  return launch_bf16_cfg<128, 32, 8, 2, 1, true>(g, q, k, v, g.L, nullptr, theta, alibi, nullptr,
                                                 nullptr, o, nullptr, stream);
}

}  // namespace arp
