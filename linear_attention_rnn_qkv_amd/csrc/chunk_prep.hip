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
    float a[10][256];                  //   a[blk][col * 16 + row] = A block
    float t[10][256];                  //   same for T
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
__global__ __launch_bounds__(kPrepThreads * NV) __attribute__((amdgpu_waves_per_eu(6))) void chunk_prep_kernel(
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
  const int64_t gc = blockIdx.x;
  const int64_t h = blockIdx.y * NV + hv;
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

  // g and beta of the chunk (wave 2 of each head), issued first so that their
  // latency overlaps the tile loads
  const float *gp = p.g + brow * p.sg_b + h * p.sg_h + t0 * p.sg_t;
  const float *bp = p.beta + brow * p.sbt_b + h * p.sbt_h + t0 * p.sbt_t;
  float graw = 0.f, braw = 0.f;
  if (wave == 2) {
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

  // 2. K K^T (wave 0), P^T = K Q^T (wave 1), gamma and decay factors (wave 2)
  f32x4 acc[10];
#pragma unroll
  for (int t = 0; t < 10; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (wave == 0) {
#pragma unroll 1  // unrolling hoists the fragment loads of later k steps (VGPRs)
    for (int pp = 0; pp < KT; ++pp) {
      f8 kf[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) kf[mt] = *reinterpret_cast<const f8 *>(sm.u.x.k + mt * 16 * RB + fo[pp]);
      int t = 0;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni <= mi; ++ni, ++t) acc[t] = MF::k32(kf[mi], kf[ni], acc[t]);
    }
    // 1/|k| from the diagonal: lane (g, c) with c / 4 == g holds |k_{16 mi + c}|^2
    if ((c >> 2) == g) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const f32x4 d = acc[blk(mi, mi)];
        const int e = c & 3;
        const float sq = e == 0 ? d[0] : e == 1 ? d[1] : e == 2 ? d[2] : d[3];
        fac[P_RK][16 * mi + c] = p.use_l2 ? rsqrtf(sq + p.l2_eps) : 1.f;
      }
    }
  } else if (wave == 1) {
    // lane (g, c) of tile (mi, ni): q_{16 mi + c} . k_{16 ni + 4 g + j}
    float ssqs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1  // unrolling hoists the fragment loads of later k steps (VGPRs)
    for (int pp = 0; pp < KT; ++pp) {
      f8 kf[4], qf[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        kf[mt] = *reinterpret_cast<const f8 *>(sm.u.x.k + mt * 16 * RB + fo[pp]);
        qf[mt] = *reinterpret_cast<const f8 *>(sm.u.x.q + mt * 16 * RB + fo[pp]);
        ssqs[mt] = sumsq8<T>(qf[mt], ssqs[mt]);
      }
      int t = 0;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni <= mi; ++ni, ++t) acc[t] = MF::k32(kf[ni], qf[mi], acc[t]);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      float ssq = ssqs[mt];
      ssq += __shfl_xor(ssq, 16, 64);
      ssq += __shfl_xor(ssq, 32, 64);
      if (g == 0) fac[P_RQ][16 * mt + c] = p.use_l2 ? rsqrtf(ssq + p.l2_eps) : 1.f;
    }
  } else if (wave == 2) {
    const bool live = lane < nr;
    float gam = live ? graw : 0.f;
    const float bv = live ? braw : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(gam, off, 64);
      if (lane >= off) gam += o;
    }
    const float gC = __shfl(gam, 63, 64);
    fac[P_GAM][lane] = gam;
    fac[P_BT][lane] = bv;
    fac[P_EG][lane] = fast_exp(gam);
    fac[P_ECG][lane] = fast_exp(gC - gam);
    if (lane == 0) sm.eC[hv] = fast_exp(gC);
  }
  __syncthreads();  // the q tile is dead from here on (its space holds A, T)

  // 3. A blocks (wave 0), P fragments (wave 1), row factors (wave 2). The
  //    row and column factors are read once as vectors; every exponential is
  //    evaluated (with its argument clamped to <= 0, exact where the mask keeps
  //    it since gamma is non-increasing) and masked by a select, so the
  //    epilogues have no branches.
  if (wave == 0) {
    // lane (g, c) of tile (mi, ni): rows r = 16 mi + 4 g + i, column 16 ni + c
    float gcol[4], kcol[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      gcol[m] = fac[P_GAM][16 * m + c];
      kcol[m] = fac[P_RK][16 * m + c];
    }
    int t = 0;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const f32x4 gr = *reinterpret_cast<const f32x4 *>(&fac[P_GAM][16 * mi + 4 * g]);
      const f32x4 br = *reinterpret_cast<const f32x4 *>(&fac[P_BT][16 * mi + 4 * g]) *
                       *reinterpret_cast<const f32x4 *>(&fac[P_RK][16 * mi + 4 * g]);
#pragma unroll
      for (int ni = 0; ni <= mi; ++ni, ++t) {
        const int col = 16 * ni + c;
        f32x4 av;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * mi + 4 * g + i;
          const float e = fast_exp(fminf(gr[i] - gcol[ni], 0.f));
          const float x = br[i] * kcol[ni] * e * acc[t][i];
          av[i] = col < r ? x : 0.f;
        }
        *reinterpret_cast<f32x4 *>(&mm.a[t][c * 16 + 4 * g]) = av;  // column c, rows 4g..
      }
    }
  } else if (wave == 1) {
    // P^T tile (mi, ni), lane (g, c): row r = 16 mi + c, key i = 16 ni + 4 g + j
    float grow[4], qrow[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      grow[m] = fac[P_GAM][16 * m + c];
      qrow[m] = p.scale * fac[P_RQ][16 * m + c];
    }
    auto ptile = [&](int mi, int ni) -> f32x4 {
      const int r = 16 * mi + c;
      const f32x4 a = acc[blk(mi, ni)];
      const f32x4 gk = *reinterpret_cast<const f32x4 *>(&fac[P_GAM][16 * ni + 4 * g]);
      const f32x4 rkk = *reinterpret_cast<const f32x4 *>(&fac[P_RK][16 * ni + 4 * g]);
      f32x4 pv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 16 * ni + 4 * g + j;
        const float e = fast_exp(fminf(grow[mi] - gk[j], 0.f));
        const float x = qrow[mi] * rkk[j] * e * a[j];
        pv[j] = i <= r ? x : 0.f;
      }
      return pv;
    };
    const v4 z4 = cvt4<T>(f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int f = 0; f < 6; ++f) {
      const int mt = f < 4 ? f : f - 2, q = f < 4 ? 0 : 1;
      const v4 lo = cvt4<T>(ptile(mt, 2 * q));
      const v4 hi = (2 * q + 1 <= mt) ? cvt4<T>(ptile(mt, 2 * q + 1)) : z4;
      *reinterpret_cast<f8 *>(rec + kRecP + f * 1024 + lane * 16) = cat8<T>(lo, hi);
    }
  } else if (wave == 2) {
    float *rf = reinterpret_cast<float *>(rec + kRecF);
    const float bt = fac[P_BT][lane], eg = fac[P_EG][lane], rk = fac[P_RK][lane];
    rf[0 * BT + lane] = eg * rk;                                 // aa (beta is in T')
    rf[1 * BT + lane] = fac[P_ECG][lane] * rk;                // cw
    rf[2 * BT + lane] = p.scale * eg * fac[P_RQ][lane];       // zc
    rf[3 * BT + lane] = bt;                                      // beta
    if (lane == 0) rf[4 * BT] = sm.eC[hv];
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
      float *tb = mm.t[blk(j, j)];
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
  //    column stay in registers, and only A blocks and the diagonal T blocks
  //    (phase 4) are read from LDS.
  {
    auto column = [&](auto jt) {
      constexpr int J = decltype(jt)::value;
      if constexpr (J < 3) {
        // B operand T_JJ[4 g + kk][c]: column-major, four consecutive floats
        const f32x4 tjj = *reinterpret_cast<const f32x4 *>(&mm.t[blk(J, J)][c * 16 + 4 * g]);
        f32x4 tk[4];  // T_kJ, k > J
#pragma unroll
        for (int i = J + 1; i < 4; ++i) {
          f32x4 xv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = J; k < i; ++k) {
            const float *ab = mm.a[blk(i, k)];
            const f32x4 bk = k == J ? tjj : tk[k];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
              xv = __builtin_amdgcn_mfma_f32_16x16x4f32(ab[(4 * g + kk) * 16 + c], bk[kk], xv, 0, 0, 0);
          }
          const float *ti = mm.t[blk(i, i)];
          f32x4 tv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            tv = __builtin_amdgcn_mfma_f32_16x16x4f32(ti[(4 * g + kk) * 16 + c], xv[kk], tv, 0, 0, 0);
          tk[i] = -tv;
        }
#pragma unroll
        for (int i = J + 1; i < 4; ++i) *reinterpret_cast<f32x4 *>(&mm.t[blk(i, J)][c * 16 + 4 * g]) = tk[i];
      }
    };
    switch (wave) {
      case 0: column(std::integral_constant<int, 0>{}); break;
      case 1: column(std::integral_constant<int, 1>{}); break;
      case 2: column(std::integral_constant<int, 2>{}); break;
      default: break;
    }
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
        const float *tb = mm.t[blk(mt, nb)];
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

hipError_t launch_chunk_prep(const ChunkArgs &a, hipStream_t s) {
  if (a.act == kBF16) return a.dk == 64 ? launch_prep<bf16, 64>(a, s) : launch_prep<bf16, 128>(a, s);
  if (a.act == kF16) return a.dk == 64 ? launch_prep<f16, 64>(a, s) : launch_prep<f16, 128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace gdn
