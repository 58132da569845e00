// Chunk prep: the state-independent half of the chunked gated delta rule,
// fully parallel over (chunk, value head). For a chunk of 64 rows, with
// gamma = cumsum(g) inside the chunk and rk, rq the inverse L2 norms of the
// k and q rows (folded into the kernel as in the Megatron-LM pull request
// "fold q/k L2-norm into the gated_delta_rule kernel", section What):
//
//   A[r,i] = beta_r exp(gamma_r - gamma_i) rk_r rk_i (k_r . k_i),   i < r
//   T      = (I + A)^-1                        (unit lower triangular)
//   P[r,i] = scale exp(gamma_r - gamma_i) rq_r rk_i (q_r . k_i),    i <= r
//   T' = T diag(beta),  aa = e^gamma rk,  cw = e^(gamma_C - gamma) rk,
//   zc = scale e^gamma rq
//
// which the chunk-state kernel consumes as
//   Vn = T' V - T' (aa (.) (K S0^T)),   O = zc (.) (Q S0^T) + P Vn,
//   S  = e^gamma_C S0 + K^T (cw (.) Vn).
// This is the WY/UT form of the delta rule (Yang et al., NeurIPS 2024) with
// the gating of Gated DeltaNet (ICLR 2025); only non-positive exponents are
// evaluated. T is computed in FP32: the four 16 x 16 diagonal blocks by
// forward substitution, then T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj, one
// block column per wave, on the FP32 MFMA with the column's blocks kept in
// registers. Results go to the caller's workspace in MFMA operand order
// (layout in gdn_internal.h).
//
// One workgroup per (chunk, NV value heads of one GQA group), four wavefronts
// per value head: the NV heads share the q/k tiles, which are read once (NV = 2
// when the group size is even). Packed sequences: a one-block kernel first
// turns cu_seqlens into chunk offsets.
#include <type_traits>

#include "gdn_internal.h"
#include "mfma_tiles.h"

namespace gdn {
namespace {

constexpr int BT = 64;
constexpr int kPrepThreads = 256;  // per value head

// cu_chunks[n] = sum over sequences m < n of ceil(len_m / 64).
__global__ __launch_bounds__(256) void chunk_index_kernel(const int32_t *__restrict__ cu, int64_t n,
                                                          int32_t *__restrict__ cuc) {
  __shared__ int32_t part[256];
  const int tid = threadIdx.x;
  const int64_t per = (n + 255) / 256;
  const int64_t b = tid * per, e = b + per < n ? b + per : n;
  int32_t sum = 0;
  for (int64_t i = b; i < e; ++i) sum += (cu[i + 1] - cu[i] + BT - 1) / BT;
  part[tid] = sum;
  __syncthreads();
  if (tid == 0) {
    int32_t acc = 0;
    for (int i = 0; i < 256; ++i) {
      const int32_t x = part[i];
      part[i] = acc;
      acc += x;
    }
  }
  __syncthreads();
  int32_t acc = part[tid];
  for (int64_t i = b; i < e; ++i) {
    cuc[i] = acc;
    acc += (cu[i + 1] - cu[i] + BT - 1) / BT;
  }
  if (b < e && e == n) cuc[n] = acc;
  if (n == 0 && tid == 0) cuc[0] = 0;
}

enum { P_GAM = 0, P_BT, P_EG, P_ECG, P_RK, P_RQ, P_N };

template <int DK, int NV>
struct PrepLds {
  static constexpr int RB = DK * 2;    // bytes per q/k row (16-bit elements)
  static constexpr int CPR = RB / 16;  // 16-byte chunks per row
  static constexpr int TILE = BT * RB;
  struct Mats {                        // lower 16 x 16 blocks, FP32, column-major
    float a[10][256];                  //   a[blk][col * 16 + row] = A block; the
                                       //   off-diagonal T blocks replace it
    float t[4][256];                   //   diagonal T blocks
  };
  struct Tiles {
    unsigned char k[TILE];
    unsigned char q[TILE];
  };
  union alignas(16) {
    Tiles x;                           // k and q rows, dead after the products
    Mats m[NV];                        // per value head
  } u;
  alignas(16) float fac[NV][P_N][BT];
  float eC[NV];
};

__device__ __forceinline__ int blk(int mi, int ni) { return mi * (mi + 1) / 2 + ni; }

template <typename T, int DK, int NV>
__global__ __launch_bounds__(kPrepThreads * NV) __attribute__((amdgpu_waves_per_eu(DK == 256 ? 4 : NV == 2 ? 8 : 6))) void chunk_prep_kernel(
    ChunkArgs p) {
  using MF = M2<T>;
  using f8 = typename MF::f8;
  using v4 = typename MF::v4;
  using SM = PrepLds<DK, NV>;
  constexpr int KT = DK / 32;
  constexpr int RB = SM::RB, CPR = SM::CPR;
  __shared__ SM sm;

  const int lane = threadIdx.x & 63, hv = threadIdx.x >> 8, wave = (threadIdx.x >> 6) & 3;
  const int g = lane >> 4, c = lane & 15;
  // The head groups of one chunk read the same g and beta cache lines (token
  // rows of all heads): consecutive linear block ids go to different XCDs,
  // so the ids are permuted to place the blocks of a chunk on one XCD and
  // its L2.
  int64_t lid = blockIdx.x + (int64_t)gridDim.x * blockIdx.y;
  const int64_t nwg = (int64_t)gridDim.x * gridDim.y;
  if (nwg % 8 == 0) lid = (lid % 8) * (nwg / 8) + lid / 8;
  const int64_t gc = lid / gridDim.y, hy = lid % gridDim.y;
  const int64_t h = hy * NV + hv;
  const int64_t hk = h / (p.Hv / p.Hqk);
  float(&fac)[P_N][BT] = sm.fac[hv];
  typename SM::Mats &mm = sm.u.m[hv];
  int64_t ch, bos, L, brow;
  if (p.cu_seqlens) {
    const int32_t *cuc = p.cu_chunks;
    if (gc >= cuc[p.n_seqs]) return;  // whole block: past the last chunk
    int64_t lo = 0, hi = p.n_seqs;    // cuc[lo] <= gc < cuc[hi]
    while (hi - lo > 1) {
      const int64_t mid = (lo + hi) >> 1;
      if (cuc[mid] <= gc) lo = mid; else hi = mid;
    }
    ch = gc - cuc[lo];
    bos = p.cu_seqlens[lo];
    L = p.cu_seqlens[lo + 1] - bos;
    brow = 0;
  } else {
    const int64_t nc = (p.T + BT - 1) / BT;
    brow = gc / nc;
    ch = gc % nc;
    bos = 0;
    L = p.T;
  }
  const int64_t t0 = bos + ch * BT;
  const int nr = (int)(L - ch * BT < BT ? L - ch * BT : BT);
  const T *qb = static_cast<const T *>(p.q) + brow * p.sq_b + hk * p.sq_h + t0 * p.sq_t;
  const T *kb = static_cast<const T *>(p.k) + brow * p.sk_b + hk * p.sk_h + t0 * p.sk_t;
  unsigned char *rec = p.ws_rec + (gc * p.Hv + h) * kRecBytes;

  // g and beta of value head hv' of the block, loaded by workgroup wave hv'
  // and issued first so that their latency overlaps the tile loads
  const int wid = threadIdx.x >> 6;
  float graw = 0.f, braw = 0.f;
  if (wid < NV) {
    const int64_t hs = hy * NV + wid;
    const float *gp = p.g + brow * p.sg_b + hs * p.sg_h + t0 * p.sg_t;
    const float *bp = p.beta + brow * p.sbt_b + hs * p.sbt_h + t0 * p.sbt_t;
    const int64_t li = lane < nr ? lane : nr - 1;
    graw = gp[li * p.sg_t];
    braw = bp[li * p.sbt_t];
  }

  // 1. k and q tiles, rows past the chunk repeat its last row (their beta
  //    and g are zero, which makes them inert). All loads are issued before
  //    the first LDS write.
  constexpr int NLD = BT * CPR / (kPrepThreads * NV);
  static_assert(NLD * kPrepThreads * NV == BT * CPR, "tile split");
  uint4 kr[NLD], qr[NLD];
#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int i = threadIdx.x + u * kPrepThreads * NV;
    const int r = i / CPR, jp = i % CPR;
    const int j = jp ^ kswz<DK>(r);
    const int rr = r < nr ? r : nr - 1;
    kr[u] = *reinterpret_cast<const uint4 *>(kb + (int64_t)rr * p.sk_t + 8 * j);
    qr[u] = *reinterpret_cast<const uint4 *>(qb + (int64_t)rr * p.sq_t + 8 * j);
  }
#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int i = threadIdx.x + u * kPrepThreads * NV;
    const int r = i / CPR, jp = i % CPR;
    *reinterpret_cast<uint4 *>(sm.u.x.k + r * RB + jp * 16) = kr[u];
    *reinterpret_cast<uint4 *>(sm.u.x.q + r * RB + jp * 16) = qr[u];
  }
  __syncthreads();

  // Fragments over dk: lane group g of k step pp holds dk 32 pp + 8 g .. + 7 of
  // row c (one 16-byte read); both operands of the products use this order.
  int fo[KT];
#pragma unroll
  for (int pp = 0; pp < KT; ++pp) fo[pp] = c * RB + (((4 * pp + g) ^ kswz<DK>(c)) << 4);

  // 2. The lower 16 x 16 tiles of K K^T and of P^T = K Q^T, which the NV
  //    value heads share, are computed once per workgroup in eight groups of
  //    tiles: Gram / q-form x {(0,0) (1,0) (1,1)}, {(2,0) (2,1) (2,2)},
  //    {(3,0) (3,1)}, {(3,2) (3,3)}; wave w takes groups w and w + 4 NV.
  //    1/|k| comes from the diagonal Gram tiles, 1/|q| from the q fragments.
  //    Waves 0 .. NV - 1 also scan gamma of their value head.
  // Gram tile (mi, ni): lane (g, c) holds k_{16 mi + 4 g + j} . k_{16 ni + c};
  // q-form tile: q_{16 mi + c} . k_{16 ni + 4 g + j}.
  constexpr int NW = 4 * NV;
  constexpr int NGW = (8 + NW - 1) / NW;  // groups per wave
  f32x4 acc[NGW][3];
  // tile list of group sub: sub 0: (0,0) (1,0) (1,1); sub 1: (2,0) (2,1) (2,2);
  // sub 2: (3,0) (3,1); sub 3: (3,2) (3,3)
  auto tile_mi = [](int sub, int t) { return sub == 0 ? (t == 0 ? 0 : 1) : sub == 1 ? 2 : 3; };
  auto tile_ni = [](int sub, int t) { return sub == 0 ? (t == 0 ? 0 : t - 1) : sub == 1 ? t : sub == 2 ? t : 2 + t; };
  auto products = [&](auto sub_t, auto qform_t, f32x4(&ac)[3]) {
    constexpr int SUB = decltype(sub_t)::value;
    constexpr bool QF = decltype(qform_t)::value;
    constexpr int NTL = SUB < 2 ? 3 : 2;
    constexpr int MLO = SUB == 0 ? 0 : SUB == 1 ? 2 : 3, MHI = SUB == 0 ? 1 : SUB == 1 ? 2 : 3;
#pragma unroll
    for (int t = 0; t < 3; ++t) ac[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float ssq[2] = {0.f, 0.f};
#pragma unroll 1  // unrolling hoists the fragment loads of later k steps (VGPRs)
    for (int pp = 0; pp < KT; ++pp) {
      f8 kf[4], qf[2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        bool used = false;
#pragma unroll
        for (int t = 0; t < NTL; ++t) used |= tile_ni(SUB, t) == mt || (!QF && tile_mi(SUB, t) == mt);
        if (used) kf[mt] = *reinterpret_cast<const f8 *>(sm.u.x.k + mt * 16 * RB + fo[pp]);
      }
      if constexpr (QF) {
#pragma unroll
        for (int m = MLO; m <= MHI; ++m) {
          qf[m - MLO] = *reinterpret_cast<const f8 *>(sm.u.x.q + m * 16 * RB + fo[pp]);
          ssq[m - MLO] = sumsq8<T>(qf[m - MLO], ssq[m - MLO]);
        }
      }
#pragma unroll
      for (int t = 0; t < NTL; ++t) {
        const int mi = tile_mi(SUB, t), ni = tile_ni(SUB, t);
        if constexpr (QF) ac[t] = MF::k32(kf[ni], qf[mi - MLO], ac[t]);
        else ac[t] = MF::k32(kf[mi], kf[ni], ac[t]);
      }
    }
    if constexpr (QF) {
      if constexpr (SUB != 3) {  // sub 3 shares row 3 with sub 2
#pragma unroll
        for (int m = MLO; m <= MHI; ++m) {
          float sq = ssq[m - MLO];
          sq += __shfl_xor(sq, 16, 64);
          sq += __shfl_xor(sq, 32, 64);
          const float rq = p.use_l2 ? rsqrtf(sq + p.l2_eps) : 1.f;
          if (g == 0)
#pragma unroll
            for (int v = 0; v < NV; ++v) sm.fac[v][P_RQ][16 * m + c] = rq;
        }
      }
    } else if ((c >> 2) == g) {
      // lane (g, c) with c / 4 == g holds |k_{16 mi + c}|^2 in a diagonal tile
#pragma unroll
      for (int t = 0; t < NTL; ++t) {
        const int mi = tile_mi(SUB, t), ni = tile_ni(SUB, t);
        if (mi != ni) continue;
        const int e = c & 3;
        const float sq = e == 0 ? ac[t][0] : e == 1 ? ac[t][1] : e == 2 ? ac[t][2] : ac[t][3];
        const float rk = p.use_l2 ? rsqrtf(sq + p.l2_eps) : 1.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) sm.fac[v][P_RK][16 * mi + c] = rk;
      }
    }
  };
  auto group = [&](int gid, auto fn) {
    switch (gid) {
      case 0: fn(std::integral_constant<int, 0>{}, std::false_type{}); break;
      case 1: fn(std::integral_constant<int, 1>{}, std::false_type{}); break;
      case 2: fn(std::integral_constant<int, 2>{}, std::false_type{}); break;
      case 3: fn(std::integral_constant<int, 3>{}, std::false_type{}); break;
      case 4: fn(std::integral_constant<int, 0>{}, std::true_type{}); break;
      case 5: fn(std::integral_constant<int, 1>{}, std::true_type{}); break;
      case 6: fn(std::integral_constant<int, 2>{}, std::true_type{}); break;
      case 7: fn(std::integral_constant<int, 3>{}, std::true_type{}); break;
      default: break;
    }
  };
  if (wid < NV) {
    float(&fv)[P_N][BT] = sm.fac[wid];
    const bool live = lane < nr;
    float gam = live ? graw : 0.f;
    const float bv = live ? braw : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(gam, off, 64);
      if (lane >= off) gam += o;
    }
    const float gC = __shfl(gam, 63, 64);
    fv[P_GAM][lane] = gam;
    fv[P_BT][lane] = bv;
    fv[P_EG][lane] = fast_exp(gam);
    fv[P_ECG][lane] = fast_exp(gC - gam);
    if (lane == 0) sm.eC[wid] = fast_exp(gC);
  }
#pragma unroll
  for (int u = 0; u < NGW; ++u)
    group(wid + u * NW, [&](auto sub_t, auto qform_t) { products(sub_t, qform_t, acc[u]); });
  __syncthreads();  // the q/k tiles are dead from here on (their space holds A, T)

  // 3. For every value head of the block: A blocks (Gram groups) and P
  //    fragments (q-form groups) of the tiles each wave holds; the row
  //    factors to the record (wave hv'). The row and column factors are read
  //    once as vectors; every exponential is evaluated (with its argument
  //    clamped to <= 0, exact where the mask keeps it since gamma is
  //    non-increasing) and masked by a select, so the epilogues have no
  //    branches.
  auto epilogue = [&](auto sub_t, auto qform_t, const f32x4(&ac)[3], int v) {
    constexpr int SUB = decltype(sub_t)::value;
    constexpr bool QF = decltype(qform_t)::value;
    constexpr int NTL = SUB < 2 ? 3 : 2;
    const float(&fv)[P_N][BT] = sm.fac[v];
    if constexpr (!QF) {
      // lane (g, c) of tile (mi, ni): rows r = 16 mi + 4 g + i, column 16 ni + c
#pragma unroll
      for (int t = 0; t < NTL; ++t) {
        const int mi = tile_mi(SUB, t), ni = tile_ni(SUB, t);
        const int col = 16 * ni + c;
        const float gcol = fv[P_GAM][col], kcol = fv[P_RK][col];
        const f32x4 gr = *reinterpret_cast<const f32x4 *>(&fv[P_GAM][16 * mi + 4 * g]);
        const f32x4 br = *reinterpret_cast<const f32x4 *>(&fv[P_BT][16 * mi + 4 * g]) *
                         *reinterpret_cast<const f32x4 *>(&fv[P_RK][16 * mi + 4 * g]);
        f32x4 av;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * mi + 4 * g + i;
          const float e = fast_exp(fminf(gr[i] - gcol, 0.f));
          const float x = br[i] * kcol * e * ac[t][i];
          av[i] = col < r ? x : 0.f;
        }
        *reinterpret_cast<f32x4 *>(&sm.u.m[v].a[blk(mi, ni)][c * 16 + 4 * g]) = av;  // column c, rows 4g..
      }
    } else {
      // P fragment f = (mt, q) = cat(tile (mt, 2 q), tile (mt, 2 q + 1)); lane
      // (g, c) of tile (mi, ni): query row r = 16 mi + c, key i = 16 ni + 4 g + j.
      unsigned char *rv = p.ws_rec + (gc * p.Hv + hy * NV + v) * kRecBytes;
      f32x4 pv[3];
#pragma unroll
      for (int t = 0; t < NTL; ++t) {
        const int mi = tile_mi(SUB, t), ni = tile_ni(SUB, t);
        const int r = 16 * mi + c;
        const float grow = fv[P_GAM][r], srq = p.scale * fv[P_RQ][r];
        const f32x4 gk = *reinterpret_cast<const f32x4 *>(&fv[P_GAM][16 * ni + 4 * g]);
        const f32x4 rkk = *reinterpret_cast<const f32x4 *>(&fv[P_RK][16 * ni + 4 * g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 16 * ni + 4 * g + j;
          const float e = fast_exp(fminf(grow - gk[j], 0.f));
          const float x = srq * rkk[j] * e * ac[t][j];
          pv[t][j] = i <= r ? x : 0.f;
        }
      }
      const v4 z4 = cvt4<T>(f32x4{0.f, 0.f, 0.f, 0.f});
      auto put = [&](int f, const v4 &lo, const v4 &hi) {
        *reinterpret_cast<f8 *>(rv + kRecP + f * 1024 + lane * 16) = cat8<T>(lo, hi);
      };
      if constexpr (SUB == 0) {
        put(0, cvt4<T>(pv[0]), z4);                   // f0 = (0,0) | 0
        put(1, cvt4<T>(pv[1]), cvt4<T>(pv[2]));       // f1 = (1,0) | (1,1)
      } else if constexpr (SUB == 1) {
        put(2, cvt4<T>(pv[0]), cvt4<T>(pv[1]));       // f2 = (2,0) | (2,1)
        put(4, cvt4<T>(pv[2]), z4);                   // f4 = (2,2) | 0
      } else if constexpr (SUB == 2) {
        put(3, cvt4<T>(pv[0]), cvt4<T>(pv[1]));       // f3 = (3,0) | (3,1)
      } else {
        put(5, cvt4<T>(pv[0]), cvt4<T>(pv[1]));       // f5 = (3,2) | (3,3)
      }
    }
  };
#pragma unroll
  for (int u = 0; u < NGW; ++u)
    group(wid + u * NW, [&](auto sub_t, auto qform_t) {
#pragma unroll
      for (int v = 0; v < NV; ++v) epilogue(sub_t, qform_t, acc[u], v);
    });
  if (wid < NV) {
    const float(&fv)[P_N][BT] = sm.fac[wid];
    float *rf = reinterpret_cast<float *>(p.ws_rec + (gc * p.Hv + hy * NV + wid) * kRecBytes + kRecF);
    const float eg = fv[P_EG][lane], rk = fv[P_RK][lane];
    rf[0 * BT + lane] = eg * rk;                          // aa (beta is in T')
    rf[1 * BT + lane] = fv[P_ECG][lane] * rk;             // cw
    rf[2 * BT + lane] = p.scale * eg * fv[P_RQ][lane];    // zc
    rf[3 * BT + lane] = fv[P_BT][lane];                   // beta
    if (lane == 0) rf[4 * BT] = sm.eC[wid];
  }
  __syncthreads();

  // 4. T = (I + A)^-1. Diagonal blocks: wave j, lane c < 16 solves column c
  //    of (I + A_jj) x = e_c by forward substitution in FP32.
  {
    const int j = wave;
    const float *ab = mm.a[blk(j, j)];
    if (lane < 16) {
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = r == lane ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < 15; ++i) {
        f32x4 col4[4];
#pragma unroll
        for (int v = (i + 1) >> 2; v < 4; ++v) col4[v] = *reinterpret_cast<const f32x4 *>(&ab[i * 16 + 4 * v]);
#pragma unroll
        for (int r = i + 1; r < 16; ++r) x[r] -= col4[r >> 2][r & 3] * x[i];
      }
      float *tb = mm.t[j];
#pragma unroll
      for (int v = 0; v < 4; ++v)
        *reinterpret_cast<f32x4 *>(&tb[lane * 16 + 4 * v]) = f32x4{x[4 * v], x[4 * v + 1], x[4 * v + 2], x[4 * v + 3]};
    }
  }
  __syncthreads();
  //    Off-diagonal blocks: wave j owns block column j and computes, for
  //    i = j + 1 .. 3, T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj on the FP32 MFMA
  //    (16x16x4). The k index of MFMA kk in lane group g is 4 g + kk, so a
  //    16 x 16 accumulator (lane (g, c) holds rows 4 g .. 4 g + 3 of column c)
  //    is directly the B operand of the next product: X and the T_kj of this
  //    column stay in registers. The A blocks and diagonal T blocks it needs
  //    are read into registers first; after a barrier the off-diagonal T
  //    blocks are written over the A blocks.
  {
    f32x4 tjj;           // B operand T_JJ[4 g + kk][c] (column-major, four consecutive floats)
    float aop[4][4][4];  // A_ik[c][4 g + kk] for i > k >= J
    float tio[4][4];     // T_ii[c][4 g + kk] for i > J
    auto load = [&](auto jt) {
      constexpr int J = decltype(jt)::value;
      tjj = *reinterpret_cast<const f32x4 *>(&mm.t[J][c * 16 + 4 * g]);
#pragma unroll
      for (int i = J + 1; i < 4; ++i) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) tio[i][kk] = mm.t[i][(4 * g + kk) * 16 + c];
#pragma unroll
        for (int k = J; k < i; ++k)
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) aop[i][k][kk] = mm.a[blk(i, k)][(4 * g + kk) * 16 + c];
      }
    };
    auto solve = [&](auto jt) {
      constexpr int J = decltype(jt)::value;
      f32x4 tk[4];  // T_kJ, k > J
#pragma unroll
      for (int i = J + 1; i < 4; ++i) {
        f32x4 xv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = J; k < i; ++k) {
          const f32x4 bk = k == J ? tjj : tk[k];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) xv = __builtin_amdgcn_mfma_f32_16x16x4f32(aop[i][k][kk], bk[kk], xv, 0, 0, 0);
        }
        f32x4 tv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) tv = __builtin_amdgcn_mfma_f32_16x16x4f32(tio[i][kk], xv[kk], tv, 0, 0, 0);
        tk[i] = -tv;
      }
#pragma unroll
      for (int i = J + 1; i < 4; ++i) *reinterpret_cast<f32x4 *>(&mm.a[blk(i, J)][c * 16 + 4 * g]) = tk[i];
    };
    using J0 = std::integral_constant<int, 0>;
    using J1 = std::integral_constant<int, 1>;
    using J2 = std::integral_constant<int, 2>;
    if (wave == 0) load(J0{}); else if (wave == 1) load(J1{}); else if (wave == 2) load(J2{});
    __syncthreads();  // every A operand is in registers: T may replace A
    if (wave == 0) solve(J0{}); else if (wave == 1) solve(J1{}); else if (wave == 2) solve(J2{});
  }
  __syncthreads();

  // 5. T' = T diag(beta) fragments to the record: wave w writes fragments w
  //    and w + 4.
  for (int f = wave; f < 6; f += 4) {
    const int mt = f < 4 ? f : f - 2, q = f < 4 ? 0 : 1;
    f32x4 lo, hi;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int nb = 2 * q + hh;  // block column
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (nb <= mt) {
        const float *tb = nb == mt ? mm.t[mt] : mm.a[blk(mt, nb)];
#pragma unroll
        for (int i = 0; i < 4; ++i)  // T[row c][col 4g + i] beta_col
          v[i] = tb[(4 * g + i) * 16 + c] * fac[P_BT][16 * nb + 4 * g + i];
      }
      if (hh == 0) lo = v; else hi = v;
    }
    *reinterpret_cast<f8 *>(rec + kRecT + f * 1024 + lane * 16) = cat8<T>(cvt4<T>(lo), cvt4<T>(hi));
  }
}

template <typename T, int DK>
hipError_t launch_prep(const ChunkArgs &a, hipStream_t s) {
  const bool pair = (a.Hv / a.Hqk) % 2 == 0;
  if (a.cu_seqlens) {
    hipLaunchKernelGGL(chunk_index_kernel, dim3(1), dim3(256), 0, s, a.cu_seqlens, a.n_seqs, a.cu_chunks);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (pair)
    hipLaunchKernelGGL((chunk_prep_kernel<T, DK, 2>), dim3((unsigned)a.chunk_bound, (unsigned)(a.Hv / 2)),
                       dim3(2 * kPrepThreads), 0, s, a);
  else
    hipLaunchKernelGGL((chunk_prep_kernel<T, DK, 1>), dim3((unsigned)a.chunk_bound, (unsigned)a.Hv),
                       dim3(kPrepThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_index(const int32_t *cu, int64_t n_seqs, int32_t *cuc, hipStream_t s) {
  hipLaunchKernelGGL(chunk_index_kernel, dim3(1), dim3(256), 0, s, cu, n_seqs, cuc);
  return hipGetLastError();
}

hipError_t launch_chunk_prep(const ChunkArgs &a, hipStream_t s) {
  if (a.act == kBF16)
    return a.dk == 64 ? launch_prep<bf16, 64>(a, s) : a.dk == 128 ? launch_prep<bf16, 128>(a, s) : launch_prep<bf16, 256>(a, s);
  if (a.act == kF16)
    return a.dk == 64 ? launch_prep<f16, 64>(a, s) : a.dk == 128 ? launch_prep<f16, 128>(a, s) : launch_prep<f16, 256>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace gdn
