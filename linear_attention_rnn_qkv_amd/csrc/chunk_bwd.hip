// Backward of the chunked gated delta rule (first-order gradients of q, k, v,
// g, beta and the initial state), FP32 arithmetic throughout.
//
// The forward, per chunk of C = 64 tokens of one value head, with S0 the
// state entering the chunk (dv x dk), gamma the running sum of g inside the
// chunk, E_ts = exp(gamma_t - gamma_s) and unit q, k rows (the L2 fold):
//   A     = strictly lower part of diag(beta) (E o K K^T)
//   M     = (I + A)^-1
//   R     = V - diag(exp gamma) K S0^T
//   Delta = M diag(beta) R                 (the corrected values)
//   O     = scale (diag(exp gamma) Q S0^T + Pt Delta),  Pt = lower part of E o Q K^T
//   S_C   = exp(gamma_C) S0 + Delta^T diag(exp(gamma_C - gamma)) K
// (the gated delta rule of Gated DeltaNet, Yang, Kautz and Hatamizadeh, in
// the chunked form that the flash-linear-attention pull request's chunk mode
// and the Megatron-LM L2-fold pull request run; first-order autograd of the
// fused stages: Megatron Core "GDN Elementwise Fusion", Execution and
// numerical behavior).
//
// Kernels, in launch order:
//   bwd_prep_kernel    per (chunk, q/k head): unit q, k rows, then per value
//                      head gamma, M (forward substitution) and scale * Pt
//   bwd_states_kernel  per (sequence, value head, 16 value rows), serial
//                      over chunks: S0 of every chunk, R and Delta
//   bwd_dstate_kernel  per (sequence, value head, 16 value rows), serial
//                      over chunks in reverse: dS_C (gradient of the state
//                      leaving each chunk), dR' = M^T dDelta, dv and dS0
//   bwd_grad_kernel    per (chunk, q/k head), the value heads of the group
//                      in turn: dq, dk (through the L2 fold), dg, dbeta
// Products run in FP32 on the vector ALU from LDS tiles; the forward's MFMA
// records (BF16 fragments of M diag(beta), not M) are not reused. For BF16
// and FP16 activations at dk 64/128 the prep also writes matrix-core records
// and the state passes and the gradients run on the matrix cores
// (chunk_bwd_state_mma.hip, chunk_bwd_mma.hip); the two state passes are
// independent of each other and run side by side in one launch there.
#include <type_traits>

#include "chunk_bwd_common.h"
#include "device_common.h"
#include "gdn_internal.h"
#include "mfma_tiles.h"

namespace gdn {
namespace {

constexpr int BT = 64;
constexpr int kThreads = 256;
constexpr int MP = 65;  // row stride of [64][64] tiles

template <int RM, int CN>
__device__ __forceinline__ void zero(float (&acc)[RM][CN]) {
#pragma unroll
  for (int r = 0; r < RM; ++r)
#pragma unroll
    for (int c = 0; c < CN; ++c) acc[r][c] = 0.f;
}

template <typename T>
__device__ __forceinline__ void store_grad(void *base, int32_t dt, int64_t i, float x) {
  if (dt == kF32) static_cast<float *>(base)[i] = x;
  else static_cast<T *>(base)[i] = to<T>(x);
}

// Sequence n: batch row, first token, length, first chunk of the call.
__device__ __forceinline__ void seq_pos(const ChunkBwdArgs &p, int64_t n, int64_t &brow, int64_t &bos, int64_t &L,
                                        int64_t &gc0) {
  if (p.cu_seqlens) {
    brow = 0;
    bos = p.cu_seqlens[n];
    L = p.cu_seqlens[n + 1] - bos;
    gc0 = p.cu_chunks[n];
  } else {
    brow = n;
    bos = 0;
    L = p.T;
    gc0 = n * ((p.T + BT - 1) / BT);
  }
}

// ---------------------------------------------------------------------------
// Vector-read products for the serial kernels. Operands in LDS, FP32.
//   mm_kk: A(i, k) = A[k * lda + i] (k-major), B(k, j) = B[k * ldb + j]
//   mm_rk: A(i, k) = A[i * lda + k] (row-major; k0, k1 multiples of 4)
//   mm_rr: as mm_rk, and B(k, j) = B[j * ldb + k] (so the product is A B^T)
// acc[r][c] += sum_{k0 <= k < k1} A(r0 + r, k) B(k, c0 + c). Strides and
// r0, c0 keep every vector read aligned to its size.
// ---------------------------------------------------------------------------
typedef float fv4 __attribute__((ext_vector_type(4)));
typedef float fv2 __attribute__((ext_vector_type(2)));

template <int N>
__device__ __forceinline__ void ldv(const float *p, float (&o)[N]) {
  if constexpr (N == 4) {
    const fv4 v = *reinterpret_cast<const fv4 *>(p);
    o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
  } else if constexpr (N == 2) {
    const fv2 v = *reinterpret_cast<const fv2 *>(p);
    o[0] = v[0]; o[1] = v[1];
  } else if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const fv4 v = *reinterpret_cast<const fv4 *>(p + i);
      o[i] = v[0]; o[i + 1] = v[1]; o[i + 2] = v[2]; o[i + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) o[i] = p[i];
  }
}

template <int N>
__device__ __forceinline__ void stv(float *p, const float (&o)[N]) {
  if constexpr (N == 4) {
    *reinterpret_cast<fv4 *>(p) = fv4{o[0], o[1], o[2], o[3]};
  } else if constexpr (N == 2) {
    *reinterpret_cast<fv2 *>(p) = fv2{o[0], o[1]};
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) p[i] = o[i];
  }
}

template <int RM, int CN>
__device__ __forceinline__ void mm_kk(float (&acc)[RM][CN], const float *A, int lda, int r0, const float *B, int ldb,
                                      int c0, int k0, int k1) {
  // four contraction steps per block, all their reads issued before the FMAs
  int k = k0;
#pragma unroll 2
  for (; k + 4 <= k1; k += 4) {
    float a[4][RM], b[4][CN];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      ldv<RM>(A + (k + kk) * lda + r0, a[kk]);
      ldv<CN>(B + (k + kk) * ldb + c0, b[kk]);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int r = 0; r < RM; ++r)
#pragma unroll
        for (int c = 0; c < CN; ++c) acc[r][c] = fmaf(a[kk][r], b[kk][c], acc[r][c]);
  }
  for (; k < k1; ++k) {
    float a[RM], b[CN];
    ldv<RM>(A + k * lda + r0, a);
    ldv<CN>(B + k * ldb + c0, b);
#pragma unroll
    for (int r = 0; r < RM; ++r)
#pragma unroll
      for (int c = 0; c < CN; ++c) acc[r][c] = fmaf(a[r], b[c], acc[r][c]);
  }
}

template <int RM, int CN>
__device__ __forceinline__ void mm_rk(float (&acc)[RM][CN], const float *A, int lda, int r0, const float *B, int ldb,
                                      int c0, int k0, int k1) {
#pragma unroll 2
  for (int k = k0; k < k1; k += 4) {
    float a[RM][4], b[4][CN];
#pragma unroll
    for (int r = 0; r < RM; ++r) ldv<4>(A + (r0 + r) * lda + k, a[r]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) ldv<CN>(B + (k + kk) * ldb + c0, b[kk]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int r = 0; r < RM; ++r)
#pragma unroll
        for (int c = 0; c < CN; ++c) acc[r][c] = fmaf(a[r][kk], b[kk][c], acc[r][c]);
  }
}

template <int RM, int CN>
__device__ __forceinline__ void mm_rr(float (&acc)[RM][CN], const float *A, int lda, int r0, const float *B, int ldb,
                                      int c0, int k0, int k1) {
#pragma unroll 2
  for (int k = k0; k < k1; k += 4) {
    float a[RM][4], b[CN][4];
#pragma unroll
    for (int r = 0; r < RM; ++r) ldv<4>(A + (r0 + r) * lda + k, a[r]);
#pragma unroll
    for (int c = 0; c < CN; ++c) ldv<4>(B + (c0 + c) * ldb + k, b[c]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int r = 0; r < RM; ++r)
#pragma unroll
        for (int c = 0; c < CN; ++c) acc[r][c] = fmaf(a[r][kk], b[c][kk], acc[r][c]);
  }
}

// The serial kernels run kSer threads (kSerW waves, two per SIMD).
constexpr int kSer = 512, kSerW = kSer / 64;

// A 64 x 16 product split over the contraction: wave w's lanes hold 4 x 4
// tiles (rows 4 (lane >> 2), columns 4 (lane & 3)) of its partial sum; the
// kSerW partials meet in `red` and thread tid gets row tid >> 3, columns
// 2 (tid & 7) and + 1 of the total.
__device__ __forceinline__ void ksplit_sum(float *red, const float (&acc)[4][4], float (&out)[2]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tg = lane >> 2, ig = lane & 3;
#pragma unroll
  for (int r = 0; r < 4; ++r) stv<4>(red + w * 1024 + (4 * tg + r) * 16 + 4 * ig, acc[r]);
  __syncthreads();
  const int t = threadIdx.x >> 3, i2 = 2 * (threadIdx.x & 7);
  ldv<2>(red + t * 16 + i2, out);
#pragma unroll
  for (int ww = 1; ww < kSerW; ++ww) {
    float x[2];
    ldv<2>(red + ww * 1024 + t * 16 + i2, x);
    out[0] += x[0];
    out[1] += x[1];
  }
}

// Chunk factors shared by the serial kernels: exp(gamma), exp(gamma_C - gamma)
// (0 past the last row), beta (0 past the last row), exp(gamma_C).
struct Fac {
  float eg[BT], cw[BT], beta[BT], eC;
};

// (value-row slice start, value head, sequence) of a serial-kernel workgroup.
// Consecutive workgroup ids go to different XCDs; the ids are permuted so that
// the slices of a head, and the value heads of a GQA group, share one XCD
// and its L2, which then serves their common chunk operands (k, q, M, P).
__device__ __forceinline__ void serial_ids(const ChunkBwdArgs &p, int64_t &j0, int64_t &h, int64_t &n) {
  const int64_t ns = gridDim.x, nwg = (int64_t)gridDim.x * gridDim.y * gridDim.z;
  int64_t lid = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
  if (nwg % 8 == 0) lid = (lid % 8) * (nwg / 8) + lid / 8;
  j0 = (lid % ns) * 16;
  h = (lid / ns) % p.Hv;
  n = lid / (ns * p.Hv);
}

// Rows [0, 64) x cols [0, D) of a contiguous FP32 [64][D] array into LDS rows
// of stride ld (float4 copies).
template <int D>
__device__ __forceinline__ void copy_rows(float *dst, int ld, const float *src) {
  constexpr int Q = D / 4;
  for (int e = threadIdx.x; e < BT * Q; e += blockDim.x) {
    const int t = e / Q, j = 4 * (e % Q);
    *reinterpret_cast<fv4 *>(dst + t * ld + j) = *reinterpret_cast<const fv4 *>(src + t * D + j);
  }
}

// ---------------------------------------------------------------------------
// Prep: unit q, k rows per (chunk, q/k head); gamma, M and scale * Pt per
// value head of the group. MMA (BF16 or FP16 activations, dk 64/128, 16-byte
// rows, the matrix-core passes downstream): the raw q, k rows go to LDS as
// swizzled 16-bit tiles and K K^T, Q K^T run on the matrix cores (exact
// products of the 16-bit inputs, FP32 accumulation), scaled by the inverse
// norms afterwards; nothing reads unit rows then, so none are written.
// ---------------------------------------------------------------------------
template <int DK, bool MMA>
struct PrepX {  // FP32 unit rows
  static constexpr int KP = DK + 4;
  float q[BT * KP], k[BT * KP];
};
template <int DK>
struct PrepX<DK, true> {  // raw BF16 rows (swizzled), then K K^T and Q K^T in FP32
  union {
    struct {
      unsigned char q[BT * DK * 2], k[BT * DK * 2];
    } t;
    struct {
      float gg[BT * MP], qk[BT * MP];
    } r;
  };
};

template <typename T, int DK, bool MMA = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void bwd_prep_kernel(ChunkBwdArgs p) {
  constexpr int KP = DK + 4;
  // the q/k tiles are dead once K K^T and Q K^T are in registers; A and M
  // then reuse their LDS
  __shared__ alignas(16) union {
    PrepX<DK, MMA> x;
    struct {
      float a[BT * MP], m[BT * MP], p[BT * MP];
    } y;
  } lds;
  float *sA = lds.y.a, *sM = lds.y.m, *sP = lds.y.p;
  __shared__ float sgam[BT], sbeta[BT], srq[BT], srk[BT];
  const int tid = threadIdx.x, rg = tid >> 4, cg = tid & 15;
  const int64_t gc = blockIdx.x, hk = blockIdx.y;
  const ChunkPos cp = chunk_pos(p, gc);
  if (!cp.valid) return;
  const int nr = cp.nr;
  const int64_t G = p.Hv / p.Hqk;

  // q, k rows of the chunk (zero past the last token), four lanes per row
  float gg[4][4], qk[4][4];  // thread owns rows 4 rg .., columns 4 cg ..
  if constexpr (MMA) {
    using F8 = typename M2<T>::f8;
    constexpr int RB = DK * 2, SEG = DK / 4, NU = SEG / 8;  // 16-byte units per lane
    const int t = tid >> 2, part = tid & 3;
    const int64_t tt = cp.t0 + (t < nr ? t : nr - 1);
    uint4 qv[NU], kv[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      qv[u] = *reinterpret_cast<const uint4 *>(static_cast<const T *>(p.q) + cp.brow * p.sq_b + tt * p.sq_t +
                                               hk * p.sq_h + part * SEG + 8 * u);
      kv[u] = *reinterpret_cast<const uint4 *>(static_cast<const T *>(p.k) + cp.brow * p.sk_b + tt * p.sk_t +
                                               hk * p.sk_h + part * SEG + 8 * u);
    }
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if (t >= nr) qv[u] = kv[u] = uint4{0u, 0u, 0u, 0u};
      const F8 a = __builtin_bit_cast(F8, qv[u]), b = __builtin_bit_cast(F8, kv[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sq = fmaf(f(a[e]), f(a[e]), sq);
        sk = fmaf(f(b[e]), f(b[e]), sk);
      }
      const int un = part * NU + u, off = t * RB + ((un ^ kswz<DK>(t)) << 4);
      *reinterpret_cast<uint4 *>(lds.x.t.q + off) = qv[u];
      *reinterpret_cast<uint4 *>(lds.x.t.k + off) = kv[u];
    }
    sq = lane_sum<4>(sq);
    sk = lane_sum<4>(sk);
    const float rq = p.use_l2 ? 1.f / sqrtf(sq + p.l2_eps) : 1.f;
    const float rk = p.use_l2 ? 1.f / sqrtf(sk + p.l2_eps) : 1.f;
    if (part == 0) {
      p.rq[(gc * p.Hqk + hk) * BT + t] = rq;
      p.rk[(gc * p.Hqk + hk) * BT + t] = rk;
      srq[t] = rq;
      srk[t] = rk;
    }
    __syncthreads();
    // lower 16 x 16 tiles (w, n <= w) of K K^T and Q K^T, row tile w = wave
    const int lane = tid & 63, w = tid >> 6, g = lane >> 4, c = lane & 15;
    auto rowk = [&](const unsigned char *x, int tile, int pp) -> F8 {
      const int r = 16 * tile + c;
      return *reinterpret_cast<const F8 *>(x + r * RB + (((4 * pp + g) ^ kswz<DK>(r)) << 4));
    };
    f32x4 ag[4], aq[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) ag[n] = aq[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pp = 0; pp < DK / 32; ++pp) {
      const F8 kt = rowk(lds.x.t.k, w, pp), qt = rowk(lds.x.t.q, w, pp);
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        if (n > w) continue;
        const F8 ks = rowk(lds.x.t.k, n, pp);
        ag[n] = M2<T>::k32(kt, ks, ag[n]);
        aq[n] = M2<T>::k32(qt, ks, aq[n]);
      }
    }
    __syncthreads();  // the tiles are read: their LDS takes the FP32 products
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * g + i, col = 16 * n + c;
        lds.x.r.gg[r * MP + col] = n <= w ? ag[n][i] * srk[r] * srk[col] : 0.f;
        lds.x.r.qk[r * MP + col] = n <= w ? aq[n][i] * srq[r] * srk[col] : 0.f;
      }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        gg[r][cc] = lds.x.r.gg[(4 * rg + r) * MP + 4 * cg + cc];
        qk[r][cc] = lds.x.r.qk[(4 * rg + r) * MP + 4 * cg + cc];
      }
    __syncthreads();  // A, M and P reuse this LDS
  } else {
    float *sQ = lds.x.q, *sK = lds.x.k;
    const int t = tid >> 2, part = tid & 3;
    constexpr int SEG = DK / 4;  // columns part * SEG .. + SEG - 1
    float qv[SEG], kv[SEG];
#pragma unroll
    for (int q = 0; q < SEG; ++q) qv[q] = kv[q] = 0.f;
    if (t < nr) {
      const int64_t tt = cp.t0 + t;
      load_vec<T, SEG>(static_cast<const T *>(p.q) + cp.brow * p.sq_b + tt * p.sq_t + hk * p.sq_h + part * SEG,
                       (int)sizeof(T), qv);
      load_vec<T, SEG>(static_cast<const T *>(p.k) + cp.brow * p.sk_b + tt * p.sk_t + hk * p.sk_h + part * SEG,
                       (int)sizeof(T), kv);
    }
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int q = 0; q < SEG; ++q) {
      sq = fmaf(qv[q], qv[q], sq);
      sk = fmaf(kv[q], kv[q], sk);
    }
    sq = lane_sum<4>(sq);
    sk = lane_sum<4>(sk);
    const float rq = p.use_l2 ? 1.f / sqrtf(sq + p.l2_eps) : 1.f;
    const float rk = p.use_l2 ? 1.f / sqrtf(sk + p.l2_eps) : 1.f;
    const int64_t un = ((gc * p.Hqk + hk) * BT + t) * DK + part * SEG;  // unit rows (when written)
#pragma unroll
    for (int q = 0; q < SEG; q += 4) {
      float a[4] = {qv[q] * rq, qv[q + 1] * rq, qv[q + 2] * rq, qv[q + 3] * rq};
      float b[4] = {kv[q] * rk, kv[q + 1] * rk, kv[q + 2] * rk, kv[q + 3] * rk};
      stv<4>(sQ + t * KP + part * SEG + q, a);
      stv<4>(sK + t * KP + part * SEG + q, b);
      if (p.qn) {
        stv<4>(p.qn + un + q, a);
        stv<4>(p.kn + un + q, b);
      }
    }
    if (part == 0) {
      p.rq[(gc * p.Hqk + hk) * BT + t] = rq;
      p.rk[(gc * p.Hqk + hk) * BT + t] = rk;
      srq[t] = rq;
      srk[t] = rk;
    }
    __syncthreads();
    // G = K K^T and QK = Q K^T
    zero(gg);
    zero(qk);
    mm_rr(gg, sK, KP, 4 * rg, sK, KP, 4 * cg, 0, DK);
    mm_rr(qk, sQ, KP, 4 * rg, sK, KP, 4 * cg, 0, DK);
    __syncthreads();  // A, M and P reuse this LDS
  }

  for (int64_t vh = 0; vh < G; ++vh) {
    const int64_t h = hk * G + vh;
    if (tid < 64) {  // gamma: inclusive scan of g over the chunk's rows
      const int t = tid;
      float gv = 0.f, bv = 0.f;
      if (t < nr) {
        const int64_t tt = cp.t0 + t;
        gv = p.g[cp.brow * p.sg_b + tt * p.sg_t + h * p.sg_h];
        bv = p.beta[cp.brow * p.sbt_b + tt * p.sbt_t + h * p.sbt_h];
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(gv, off, 64);
        if (t >= off) gv += o;
      }
      sgam[t] = gv;  // rows past nr repeat the last row's gamma (g = 0 there)
      sbeta[t] = bv;
      p.gam[(gc * p.Hv + h) * BT + t] = gv;
    }
    __syncthreads();
    // A (strict lower, beta-weighted) to LDS; scale * Pt to the workspace
    {
      const int64_t pb = (gc * p.Hv + h) * BT * BT;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * rg + r;
        float pv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int s = 4 * cg + c;
          const float e = s <= t ? __expf(sgam[t] - sgam[s]) : 0.f;
          sA[t * MP + s] = s < t ? sbeta[t] * e * gg[r][c] : 0.f;
          pv[c] = p.scale * e * qk[r][c];
          sP[t * MP + s] = t < nr ? pv[c] : 0.f;
        }
        if (p.pp) stv<4>(p.pp + pb + t * BT + 4 * cg, pv);
      }
    }
    __syncthreads();
    // M = (I + A)^-1 in 16 x 16 blocks. Diagonal blocks: wave j, lane c < 16
    // solves column c of (I + A_jj) x = e_c by forward substitution; the
    // strict upper blocks are zero.
    {
      const int lane = tid & 63, j = tid >> 6;
      if (lane < 16) {
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = r == lane ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < 15; ++i)
#pragma unroll
          for (int r = i + 1; r < 16; ++r) x[r] = fmaf(-sA[(16 * j + r) * MP + 16 * j + i], x[i], x[r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) sM[(16 * j + r) * MP + 16 * j + lane] = x[r];
      }
      for (int e = tid; e < 6 * 256; e += kThreads) {  // blocks (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
        const int b = e >> 8, r = (e >> 4) & 15, cc = e & 15;
        const int bi = b < 3 ? 0 : (b < 5 ? 1 : 2), bj = b < 3 ? b + 1 : (b < 5 ? b - 1 : 3);
        sM[(16 * bi + r) * MP + 16 * bj + cc] = 0.f;
      }
    }
    __syncthreads();
    //   Off-diagonal blocks: wave J owns block column J and forms, for
    //   i = J + 1 .. 3, M_iJ = -M_ii sum_{k=J}^{i-1} A_ik M_kJ on the FP32
    //   matrix cores (16x16x4, k index 4 g + kk in lane group g), so that an
    //   accumulator (rows 4 g .. 4 g + 3 of column c) is directly the B
    //   operand of the next product.
    {
      const int lane = tid & 63, g = lane >> 4, c = lane & 15;
      auto column = [&](auto jt) {
        constexpr int J = decltype(jt)::value;
        f32x4 mk[4];  // M_kJ, k > J
#pragma unroll
        for (int i = J + 1; i < 4; ++i) {
          f32x4 xv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = J; k < i; ++k) {
            f32x4 bk;
            if (k == J) {
#pragma unroll
              for (int kk = 0; kk < 4; ++kk) bk[kk] = sM[(16 * J + 4 * g + kk) * MP + 16 * J + c];
            } else {
              bk = mk[k];
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
              xv = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 * i + c) * MP + 16 * k + 4 * g + kk], bk[kk], xv, 0, 0, 0);
          }
          f32x4 tv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            tv = __builtin_amdgcn_mfma_f32_16x16x4f32(sM[(16 * i + c) * MP + 16 * i + 4 * g + kk], xv[kk], tv, 0, 0, 0);
          mk[i] = -tv;
        }
#pragma unroll
        for (int i = J + 1; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) sM[(16 * i + 4 * g + r) * MP + 16 * J + c] = mk[i][r];
      };
      const int wv = tid >> 6;
      if (wv == 0) column(std::integral_constant<int, 0>{});
      else if (wv == 1) column(std::integral_constant<int, 1>{});
      else if (wv == 2) column(std::integral_constant<int, 2>{});
    }
    __syncthreads();
    if (p.mm) {
      float *mm_ = p.mm + (gc * p.Hv + h) * BT * BT;
      for (int e = tid; e < BT * BT; e += kThreads) mm_[e] = sM[(e >> 6) * MP + (e & 63)];
    }
    if (p.brec) {  // the matrix-core reverse pass's record (16-bit activations)
      unsigned char *br = p.brec + (gc * p.Hv + h) * kBrBytes;
      // 6 fragments x 3 matrices (M^T, P'^T, M) x 64 lanes; hi and lo
      // written together
      for (int it = tid; it < 3 * 6 * 64; it += kThreads) {
        const int lane = it & 63, fi = (it >> 6) % 6, mat = it / 384, g = lane >> 4, c = lane & 15;
        float x[8];
        if (mat < 2) {  // upper triangular: (0,0) (1,0) (0,1) (1,1) (2,1) (3,1), transposed reads
          const int mt = fi < 2 ? fi : fi - 2, q = fi < 2 ? 0 : 1;
          const float *src = mat == 0 ? sM : sP;
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = src[(32 * q + 16 * (e >> 2) + 4 * g + (e & 3)) * MP + 16 * mt + c];
        } else {  // M, lower triangular: (0,0) (1,0) (2,0) (3,0) (2,1) (3,1)
          const int mt = fi < 4 ? fi : fi - 2, q = fi < 4 ? 0 : 1;
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = sM[(16 * mt + c) * MP + 32 * q + 16 * (e >> 2) + 4 * g + (e & 3)];
        }
        // 16-bit parts in the activations' type (FP32 activations write no record)
        using R16 = typename std::conditional<std::is_same<T, f16>::value, f16, bf16>::type;
        R16 hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          hi[e] = to<R16>(x[e]);
          lo[e] = to<R16>(x[e] - f(hi[e]));
        }
        const int64_t oh = (mat == 0 ? kBrMtH : mat == 1 ? kBrPH : kBrMH) + fi * 1024 + lane * 16;
        const int64_t ol = (mat == 0 ? kBrMtL : mat == 1 ? kBrPL : kBrML) + fi * 1024 + lane * 16;
        __builtin_memcpy(br + oh, hi, 16);
        __builtin_memcpy(br + ol, lo, 16);
      }
      if (tid < BT) {
        const int t = tid;
        float *fr = reinterpret_cast<float *>(br + kBrF);
        const float gl = sgam[nr - 1], eg = __expf(sgam[t]);
        const float cw = t < nr ? __expf(gl - sgam[t]) : 0.f;
        fr[0 * BT + t] = eg;
        fr[1 * BT + t] = cw * srk[t];
        fr[2 * BT + t] = sbeta[t];
        fr[3 * BT + t] = t < nr ? p.scale * eg * srq[t] : 0.f;
        fr[4 * BT + t] = -eg * sbeta[t] * srk[t];
        fr[5 * BT + t] = t == 0 ? __expf(gl) : 0.f;
        fr[6 * BT + t] = eg * srk[t];
        fr[7 * BT + t] = 0.f;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Forward states: S0 of every chunk, R and Delta, for 16 value rows. The
// state slice is kept transposed in LDS (sST[j][i]).
// ---------------------------------------------------------------------------
template <typename T, int DK>
__global__ __launch_bounds__(kSer) void bwd_states_kernel(ChunkBwdArgs p) {
  // state update tiles: RI value rows by CJ dk columns per thread
  constexpr int KP = DK + 4, RI = DK >= 128 ? 4 : 2, CJ = DK / 32 / RI, NIG = 16 / RI;
  __shared__ alignas(16) float sK[BT * KP];    // unit k rows [t][j]
  __shared__ alignas(16) float sM[BT * 68];    // M [t][s]
  __shared__ alignas(16) float sST[DK * 16];   // S^T [j][i]
  __shared__ alignas(16) float sX[BT * 16];    // beta R [s][i]
  __shared__ alignas(16) float sV[BT * 16];    // v, then cw Delta [s][i]
  __shared__ alignas(16) float red[kSerW * 1024];
  __shared__ Fac F;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int64_t j0, h, n;
  serial_ids(p, j0, h, n);
  const int64_t hk = h / (p.Hv / p.Hqk);
  int64_t brow, bos, L, gc0;
  seq_pos(p, n, brow, bos, L, gc0);
  const int64_t nch = (L + BT - 1) / BT;
  const int et = tid >> 3, ei = 2 * (tid & 7);  // epilogue: row et, columns ei .. ei + 3
  const int ig = tid % NIG, jg = tid / NIG;     // state update: rows RI ig .., columns CJ jg ..

  for (int e = tid; e < 16 * DK; e += kSer) {
    const int i = e / DK, j = e % DK;
    sST[j * 16 + i] = p.init_state ? p.init_state[((n * p.Hv + h) * p.dv + j0 + i) * DK + j] : 0.f;
  }
  // The next chunk's operands are staged in registers while this one is
  // computed: unit k rows, M, the v slice and the factors.
  constexpr int NK = DK / 32;
  fv4 rk[NK], rm[2];
  float rv[2], rg = 0.f, rgl = 0.f, rb = 0.f;
  auto fetch = [&](int64_t c) {
    const int64_t gc = gc0 + c, t0 = bos + c * BT;
    const int nr = (int)(L - c * BT < BT ? L - c * BT : BT);
    const float *kn = p.kn + (gc * p.Hqk + hk) * BT * DK, *mm_ = p.mm + (gc * p.Hv + h) * BT * BT;
#pragma unroll
    for (int m = 0; m < NK; ++m) rk[m] = *reinterpret_cast<const fv4 *>(kn + 4 * (tid + kSer * m));
#pragma unroll
    for (int m = 0; m < 2; ++m) rm[m] = *reinterpret_cast<const fv4 *>(mm_ + 4 * (tid + kSer * m));
#pragma unroll
    for (int q = 0; q < 2; ++q) rv[q] = 0.f;
    if (et < nr) load_vec<T, 2>(static_cast<const T *>(p.v) + brow * p.sv_b + (t0 + et) * p.sv_t + h * p.sv_h + j0 + ei,
                                (int)sizeof(T), rv);
    if (tid < BT) {
      const float *gm = p.gam + (gc * p.Hv + h) * BT;
      rg = gm[tid];
      rgl = gm[nr - 1];
      rb = tid < nr ? p.beta[brow * p.sbt_b + (t0 + tid) * p.sbt_t + h * p.sbt_h] : 0.f;
    }
  };
  if (nch > 0) fetch(0);
  __syncthreads();
  for (int64_t c = 0; c < nch; ++c) {
    const int64_t gc = gc0 + c;
    const int nr = (int)(L - c * BT < BT ? L - c * BT : BT);
    float *s0 = p.s0 + ((gc * p.Hv + h) * p.dv + j0) * DK;
    for (int e = tid; e < 16 * DK; e += kSer) s0[e] = sST[(e % DK) * 16 + e / DK];
#pragma unroll
    for (int m = 0; m < NK; ++m) {
      const int e = 4 * (tid + kSer * m);
      *reinterpret_cast<fv4 *>(sK + (e / DK) * KP + e % DK) = rk[m];
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int e = 4 * (tid + kSer * m);
      *reinterpret_cast<fv4 *>(sM + (e >> 6) * 68 + (e & 63)) = rm[m];
    }
    stv<2>(sV + et * 16 + ei, rv);
    if (tid < BT) {
      F.eg[tid] = __expf(rg);
      F.cw[tid] = tid < nr ? __expf(rgl - rg) : 0.f;
      F.beta[tid] = rb;
      if (tid == 0) F.eC = __expf(rgl);
    }
    __syncthreads();
    if (c + 1 < nch) fetch(c + 1);
    // KS = K S0^T (contraction over dk, an eighth per wave); R = V - exp(gamma) KS
    {
      float acc[4][4];
      zero(acc);
      mm_rk(acc, sK, KP, 4 * (lane >> 2), sST, 16, 4 * (lane & 3), w * (DK / kSerW), (w + 1) * (DK / kSerW));
      float ks[2];
      ksplit_sum(red, acc, ks);
      float vv[2], R[2], X[2];
      ldv<2>(sV + et * 16 + ei, vv);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        R[q] = vv[q] - F.eg[et] * ks[q];
        X[q] = F.beta[et] * R[q];
      }
      stv<2>(p.rr + ((gc * p.Hv + h) * BT + et) * p.dv + j0 + ei, R);
      stv<2>(sX + et * 16 + ei, X);
    }
    __syncthreads();
    // Delta = M X (contraction over s, 8 per wave)
    {
      float acc[4][4];
      zero(acc);
      mm_rk(acc, sM, 68, 4 * (lane >> 2), sX, 16, 4 * (lane & 3), 8 * w, 8 * w + 8);
      float dl[2], cd[2];
      ksplit_sum(red, acc, dl);
#pragma unroll
      for (int q = 0; q < 2; ++q) cd[q] = F.cw[et] * dl[q];
      stv<2>(p.del + ((gc * p.Hv + h) * BT + et) * p.dv + j0 + ei, dl);
      stv<2>(sV + et * 16 + ei, cd);
    }
    __syncthreads();
    // S = exp(gamma_C) S + (cw Delta)^T K
    {
      float acc[RI][CJ];
#pragma unroll
      for (int r = 0; r < RI; ++r)
#pragma unroll
        for (int q = 0; q < CJ; ++q) acc[r][q] = F.eC * sST[(CJ * jg + q) * 16 + RI * ig + r];
      mm_kk(acc, sV, 16, RI * ig, sK, KP, CJ * jg, 0, BT);  // rows past nr are zero
#pragma unroll
      for (int r = 0; r < RI; ++r)
#pragma unroll
        for (int q = 0; q < CJ; ++q) sST[(CJ * jg + q) * 16 + RI * ig + r] = acc[r][q];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Reverse pass: dS carried from the last chunk to the first (kept transposed,
// sDT[j][i]).
// ---------------------------------------------------------------------------
template <typename T, int DK>
__global__ __launch_bounds__(kSer) void bwd_dstate_kernel(ChunkBwdArgs p) {
  // state update tiles: RI value rows by CJ dk columns per thread
  constexpr int KP = DK + 4, RI = DK >= 128 ? 4 : 2, CJ = DK / 32 / RI, NIG = 16 / RI;
  // dk 256: the unit q rows are read from the workspace (L2) in the state
  // update instead of being staged in LDS, which would not hold them
  constexpr bool QG = DK > 128;
  __shared__ alignas(16) float sK[BT * KP], sQs[QG ? 4 : BT * KP];  // unit rows [s][j]
  __shared__ alignas(16) float sP[BT * BT], sM[BT * BT];  // as stored: [s][t]
  __shared__ alignas(16) float sDT[DK * 16];              // dS^T [j][i]
  __shared__ alignas(16) float sO[BT * 16], sR[BT * 16];  // dO, then scale exp(gamma) dO; -exp(gamma) dv
  __shared__ alignas(16) float red[kSerW * 1024];             // partials; red[0 .. 1024) then holds dDelta
  __shared__ Fac F;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int64_t j0, h, n;
  serial_ids(p, j0, h, n);
  const int64_t hk = h / (p.Hv / p.Hqk);
  int64_t brow, bos, L, gc0;
  seq_pos(p, n, brow, bos, L, gc0);
  const int64_t nch = (L + BT - 1) / BT;
  const int et = tid >> 3, ei = 2 * (tid & 7);
  const int ig = tid % NIG, jg = tid / NIG;

  for (int e = tid; e < 16 * DK; e += kSer) {
    const int i = e / DK, j = e % DK;
    sDT[j * 16 + i] = p.d_final ? p.d_final[((n * p.Hv + h) * p.dv + j0 + i) * DK + j] : 0.f;
  }
  // The next chunk's operands are staged in registers while this one is
  // computed: unit k and q rows, M, scale * Pt, the dO slice and the factors.
  constexpr int NK = DK / 32, NQ = QG ? 1 : NK;
  fv4 rk[NK], rq[NQ], rm[2], rp[2];
  float ro[2], rg = 0.f, rgl = 0.f, rb = 0.f;
  auto fetch = [&](int64_t c) {
    const int64_t gc = gc0 + c, t0 = bos + c * BT;
    const int nr = (int)(L - c * BT < BT ? L - c * BT : BT);
    const float *kn = p.kn + (gc * p.Hqk + hk) * BT * DK, *qn = p.qn + (gc * p.Hqk + hk) * BT * DK;
    const float *mm_ = p.mm + (gc * p.Hv + h) * BT * BT, *pp = p.pp + (gc * p.Hv + h) * BT * BT;
#pragma unroll
    for (int m = 0; m < NK; ++m) rk[m] = *reinterpret_cast<const fv4 *>(kn + 4 * (tid + kSer * m));
    if constexpr (!QG) {
#pragma unroll
      for (int m = 0; m < NQ; ++m) rq[m] = *reinterpret_cast<const fv4 *>(qn + 4 * (tid + kSer * m));
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      rm[m] = *reinterpret_cast<const fv4 *>(mm_ + 4 * (tid + kSer * m));
      rp[m] = *reinterpret_cast<const fv4 *>(pp + 4 * (tid + kSer * m));
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) ro[q] = 0.f;
    if (et < nr)
      load_vec<T, 2>(static_cast<const T *>(p.d_o) + brow * p.sdo_b + (t0 + et) * p.sdo_t + h * p.sdo_h + j0 + ei,
                     (int)sizeof(T), ro);
    if (tid < BT) {
      const float *gm = p.gam + (gc * p.Hv + h) * BT;
      rg = gm[tid];
      rgl = gm[nr - 1];
      rb = tid < nr ? p.beta[brow * p.sbt_b + (t0 + tid) * p.sbt_t + h * p.sbt_h] : 0.f;
    }
  };
  if (nch > 0) fetch(nch - 1);
  __syncthreads();
  for (int64_t c = nch - 1; c >= 0; --c) {
    const int64_t gc = gc0 + c, t0 = bos + c * BT;
    const int nr = (int)(L - c * BT < BT ? L - c * BT : BT);
    float *ds = p.ds + ((gc * p.Hv + h) * p.dv + j0) * DK;
    for (int e = tid; e < 16 * DK; e += kSer) ds[e] = sDT[(e % DK) * 16 + e / DK];
#pragma unroll
    for (int m = 0; m < NK; ++m) {
      const int e = 4 * (tid + kSer * m);
      *reinterpret_cast<fv4 *>(sK + (e / DK) * KP + e % DK) = rk[m];
    }
    if constexpr (!QG) {
#pragma unroll
      for (int m = 0; m < NQ; ++m) {
        const int e = 4 * (tid + kSer * m);
        *reinterpret_cast<fv4 *>(sQs + (e / DK) * KP + e % DK) = rq[m];
      }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int e = 4 * (tid + kSer * m);
      *reinterpret_cast<fv4 *>(sM + e) = rm[m];
      *reinterpret_cast<fv4 *>(sP + e) = rp[m];
    }
    stv<2>(sO + et * 16 + ei, ro);
    if (tid < BT) {
      F.eg[tid] = __expf(rg);
      F.cw[tid] = tid < nr ? __expf(rgl - rg) : 0.f;
      F.beta[tid] = rb;
      if (tid == 0) F.eC = __expf(rgl);
    }
    __syncthreads();
    if (c > 0) fetch(c - 1);
    // dDelta = cw (K dS^T) + Pt'^T dO: both contractions split over the waves
    {
      float a1[4][4];
      zero(a1);
      const int r0 = 4 * (lane >> 2), c0 = 4 * (lane & 3);
      mm_rk(a1, sK, KP, r0, sDT, 16, c0, w * (DK / kSerW), (w + 1) * (DK / kSerW));
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) a1[r][q] *= F.cw[r0 + r];
      mm_kk(a1, sP, BT, r0, sO, 16, c0, 8 * w, 8 * w + 8);
      float dd[2];
      ksplit_sum(red, a1, dd);
      __syncthreads();  // every partial is read before red[0 ..) is overwritten
      stv<2>(red + et * 16 + ei, dd);
    }
    __syncthreads();
    // dR' = M^T dDelta; dv = beta dR'
    {
      float a1[4][4];
      zero(a1);
      mm_kk(a1, sM, BT, 4 * (lane >> 2), red, 16, 4 * (lane & 3), 8 * w, 8 * w + 8);
      __syncthreads();  // dDelta in red[0 ..) is read by every wave before the partials land
      float dr[2], dvv[2], er[2], oo[2];
      ksplit_sum(red, a1, dr);
      stv<2>(p.drp + ((gc * p.Hv + h) * BT + et) * p.dv + j0 + ei, dr);
      ldv<2>(sO + et * 16 + ei, oo);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        dvv[q] = F.beta[et] * dr[q];
        er[q] = -F.eg[et] * dvv[q];
        oo[q] *= p.scale * F.eg[et];
      }
      if (et < nr) {
        const int64_t o = brow * p.sdv_b + (t0 + et) * p.sdv_t + h * p.dv + j0 + ei;
#pragma unroll
        for (int q = 0; q < 2; ++q) store_grad<T>(p.dvv, p.grad_dtype, o + q, dvv[q]);
      }
      stv<2>(sR + et * 16 + ei, er);
      stv<2>(sO + et * 16 + ei, oo);
    }
    __syncthreads();
    // dS0 = exp(gamma_C) dS + (scale exp(gamma) dO)^T Q - (exp(gamma) dv)^T K
    {
      float a1[RI][CJ];
#pragma unroll
      for (int r = 0; r < RI; ++r)
#pragma unroll
        for (int q = 0; q < CJ; ++q) a1[r][q] = F.eC * sDT[(CJ * jg + q) * 16 + RI * ig + r];
      if constexpr (QG)
        mm_kk(a1, sO, 16, RI * ig, p.qn + (gc * p.Hqk + hk) * BT * DK, DK, CJ * jg, 0, BT);  // rows past nr are zero
      else
        mm_kk(a1, sO, 16, RI * ig, sQs, KP, CJ * jg, 0, BT);
      mm_kk(a1, sR, 16, RI * ig, sK, KP, CJ * jg, 0, BT);
#pragma unroll
      for (int r = 0; r < RI; ++r)
#pragma unroll
        for (int q = 0; q < CJ; ++q) sDT[(CJ * jg + q) * 16 + RI * ig + r] = a1[r][q];
    }
    __syncthreads();
  }
  if (p.d_init) {
    for (int e = tid; e < 16 * DK; e += kSer) {
      const int i = e / DK, j = e % DK;
      p.d_init[((n * p.Hv + h) * p.dv + j0 + i) * DK + j] = sDT[j * 16 + i];
    }
  }
}

// ---------------------------------------------------------------------------
// Gradients of q, k, g and beta per (chunk, q/k head). The value-column
// tiles are stored transposed ([i][t]) so that every product reads vectors.
// Thread tid owns rows 4 (tid >> 4) .. + 3 and, of the 64 chunk columns,
// 4 (tid & 15) .. + 3; of the dk columns, NJ (tid & 15) .. + NJ - 1.
// ---------------------------------------------------------------------------
template <int DK>
struct GradTiles {
  float o[16 * BT], d[16 * BT], rp[16 * BT], r[16 * BT];  // dO, Delta, dR', R as [i][t]
  float s0[16 * DK], ds[16 * DK];                          // S0, dS_C rows [i][j]
};

// Threads of the gradient kernel: 512 (two waves per SIMD; each thread holds
// 4 chunk rows by 2 chunk columns and by dk / 32 dk columns). For dk 256 the
// unit q, k rows are read from the workspace (L2) instead of LDS.
template <int DK>
constexpr int grad_threads() { return 512; }

template <typename T, int DK>
__global__ __launch_bounds__(grad_threads<DK>()) void bwd_grad_kernel(ChunkBwdArgs p) {
  constexpr int NT = grad_threads<DK>();
  constexpr bool QKG = DK > 128;
  constexpr int CG = NT / 16;        // column groups: threads per row group
  constexpr int CCN = BT / CG;       // chunk columns per thread (4 or 2)
  constexpr int NJ = DK / CG;        // dk columns per thread
  constexpr int TPR = 1024 / NT;     // tile elements per thread per [64][16] array
  constexpr int KP = DK + 4, ZP = 68;
  __shared__ alignas(16) float sQK[QKG ? 4 : 2 * BT * KP];
  __shared__ alignas(16) float sZ1[BT * ZP], sZ2[BT * ZP];  // dQK, dG
  __shared__ alignas(16) union {
    GradTiles<DK> t;
    float z[BT * ZP];  // a + p, for its column sums
  } u;
  __shared__ float sgam[BT], seg[BT], scw[BT], sbeta[BT];
  __shared__ float vrow[BT], vm[BT], vb[BT], red[NT / 64];
  const int tid = threadIdx.x, rg = tid / CG, cg = tid % CG;
  const int r0 = 4 * rg, c0 = CCN * cg, j0c = NJ * cg;
  const int64_t gc = blockIdx.x, hk = blockIdx.y;
  const ChunkPos cp = chunk_pos(p, gc);
  if (!cp.valid) return;
  const int nr = cp.nr;
  const int64_t G = p.Hv / p.Hqk, dvn = p.dv;

  const float *sQ, *sK;  // unit q, k rows, row stride QS
  int QS;
  if constexpr (QKG) {
    sQ = p.qn + (gc * p.Hqk + hk) * BT * DK;
    sK = p.kn + (gc * p.Hqk + hk) * BT * DK;
    QS = DK;
  } else {
    copy_rows<DK>(sQK + BT * KP, KP, p.kn + (gc * p.Hqk + hk) * BT * DK);
    copy_rows<DK>(sQK, KP, p.qn + (gc * p.Hqk + hk) * BT * DK);
    sQ = sQK;
    sK = sQK + BT * KP;
    QS = KP;
  }
  __syncthreads();
  float gg[4][CCN], qk[4][CCN];
  zero(gg);
  zero(qk);
  mm_rr(gg, sK, QS, r0, sK, QS, c0, 0, DK);
  mm_rr(qk, sQ, QS, r0, sK, QS, c0, 0, DK);
  float dq[4][NJ], dk[4][NJ];
  zero(dq);
  zero(dk);

  for (int64_t vh = 0; vh < G; ++vh) {
    const int64_t h = hk * G + vh;
    __syncthreads();  // the previous head's readers of the factors and tiles are done
    if (tid < BT) {
      const float *gm = p.gam + (gc * p.Hv + h) * BT;
      const float gl = gm[nr - 1], gt = gm[tid];
      sgam[tid] = gt;
      seg[tid] = __expf(gt);
      scw[tid] = tid < nr ? __expf(gl - gt) : 0.f;
      sbeta[tid] = tid < nr ? p.beta[cp.brow * p.sbt_b + (cp.t0 + tid) * p.sbt_t + h * p.sbt_h] : 0.f;
    }
    float c1[4][CCN], c2[4][CCN], k1[4][NJ], k2[4][NJ], k3[4][NJ];
    zero(c1);
    zero(c2);
    zero(k1);
    zero(k2);
    zero(k3);
    float db1 = 0.f, sdot = 0.f;
    const int64_t rowbase = (gc * p.Hv + h) * BT * dvn;
    const int64_t stbase = (gc * p.Hv + h) * dvn * DK;
    for (int64_t jv = 0; jv < dvn; jv += 16) {
      __syncthreads();
      {  // row t of the tiles, value columns i4 .. i4 + TPR - 1
        const int t = tid / (16 / TPR), i4 = TPR * (tid % (16 / TPR));
        float o4[TPR], d4[TPR], rp4[TPR], r4[TPR];
#pragma unroll
        for (int q = 0; q < TPR; ++q) o4[q] = 0.f;
        if (t < nr)
          load_vec<T, TPR>(static_cast<const T *>(p.d_o) + cp.brow * p.sdo_b + (cp.t0 + t) * p.sdo_t + h * p.sdo_h +
                               jv + i4,
                           (int)sizeof(T), o4);
        const int64_t wo = rowbase + t * dvn + jv + i4;
        ldv<TPR>(p.del + wo, d4);
        ldv<TPR>(p.drp + wo, rp4);
        ldv<TPR>(p.rr + wo, r4);
#pragma unroll
        for (int q = 0; q < TPR; ++q) {
          u.t.o[(i4 + q) * BT + t] = o4[q];
          u.t.d[(i4 + q) * BT + t] = d4[q];
          u.t.rp[(i4 + q) * BT + t] = rp4[q];
          u.t.r[(i4 + q) * BT + t] = r4[q];
        }
      }
      for (int e = 4 * tid; e < 16 * DK; e += 4 * NT) {
        float a[4], b[4];
        ldv<4>(p.s0 + stbase + jv * DK + e, a);
        ldv<4>(p.ds + stbase + jv * DK + e, b);
        stv<4>(u.t.s0 + e, a);
        stv<4>(u.t.ds + e, b);
#pragma unroll
        for (int q = 0; q < 4; ++q) sdot = fmaf(a[q], b[q], sdot);
      }
      __syncthreads();
      mm_kk(c1, u.t.o, BT, r0, u.t.d, BT, c0, 0, 16);
      mm_kk(c2, u.t.rp, BT, r0, u.t.d, BT, c0, 0, 16);
      mm_kk(k1, u.t.o, BT, r0, u.t.s0, DK, j0c, 0, 16);
      mm_kk(k2, u.t.d, BT, r0, u.t.ds, DK, j0c, 0, 16);
      mm_kk(k3, u.t.rp, BT, r0, u.t.s0, DK, j0c, 0, 16);
      if (tid < BT)
#pragma unroll
        for (int i = 0; i < 16; ++i) db1 = fmaf(u.t.rp[i * BT + tid], u.t.r[i * BT + tid], db1);
    }
    __syncthreads();  // tiles dead: the union now holds a + p
    float rowz[4], roww[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = r0 + r;
      rowz[r] = 0.f;
      roww[r] = 0.f;
#pragma unroll
      for (int c = 0; c < CCN; ++c) {
        const int s = c0 + c;
        const float e = s <= t ? __expf(sgam[t] - sgam[s]) : 0.f;
        const float dqk = s <= t ? p.scale * c1[r][c] * e : 0.f;  // dPt o E
        const float pz = dqk * qk[r][c];                           // dPt * Pt
        const float da = s < t ? -c2[r][c] : 0.f;                  // dA
        const float eg = e * gg[r][c];
        const float az = da * sbeta[t] * eg;                       // dA * A
        sZ1[t * ZP + s] = dqk;
        sZ2[t * ZP + s] = da * sbeta[t] * e;                       // dG
        u.z[t * ZP + s] = az + pz;
        rowz[r] += az + pz;
        roww[r] = fmaf(da, eg, roww[r]);
      }
    }
    float rdot[4], rm[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = r0 + r;
      float a = 0.f, b = 0.f, m = 0.f;
#pragma unroll
      for (int q = 0; q < NJ; ++q) {
        const int j = j0c + q;
        a = fmaf(sQ[t * QS + j], k1[r][q], a);
        b = fmaf(sK[t * QS + j], k3[r][q], b);
        m = fmaf(sK[t * QS + j], k2[r][q], m);
      }
      const float rd = p.scale * seg[t] * a - seg[t] * sbeta[t] * b - scw[t] * m;
      rdot[r] = group_sum<CG>(rd + rowz[r]);
      rm[r] = group_sum<CG>(scw[t] * m);
      roww[r] = group_sum<CG>(roww[r]);
    }
    if (cg == 0)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        vrow[r0 + r] = rdot[r];
        vm[r0 + r] = rm[r];
        vb[r0 + r] = roww[r];
      }
    {  // per-wave total of <dS, S0>
      const float a = group_sum<64>(sdot);
      if ((tid & 63) == 0) red[tid >> 6] = a;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = r0 + r;
#pragma unroll
      for (int q = 0; q < NJ; ++q) {
        dq[r][q] = fmaf(p.scale * seg[t], k1[r][q], dq[r][q]);
        dk[r][q] += scw[t] * k2[r][q] - seg[t] * sbeta[t] * k3[r][q];
      }
    }
    __syncthreads();
    mm_rk(dq, sZ1, ZP, r0, sK, QS, j0c, 0, BT);
    mm_rk(dk, sZ2, ZP, r0, sK, QS, j0c, 0, BT);
    mm_kk(dk, sZ2, ZP, r0, sK, QS, j0c, 0, BT);
    mm_kk(dk, sZ1, ZP, r0, sQ, QS, j0c, 0, BT);
    if (tid < BT) {  // wave 0: dgamma, its reverse running sum (dg), dbeta
      const int t = tid;
      float colz = 0.f;
      for (int s = 0; s < BT; ++s) colz += u.z[s * ZP + t];
      float tot = 0.f;
      for (int i = 0; i < NT / 64; ++i) tot += red[i];
      float sm = 0.f;
      for (int s = 0; s < BT; ++s) sm += vm[s];
      float dgam = vrow[t] - colz;
      if (t == nr - 1) dgam += __expf(sgam[t]) * tot + sm;
      if (t >= nr) dgam = 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_down(dgam, off, 64);
        if (t + off < 64) dgam += o;
      }
      if (t < nr) {
        const int64_t o = (cp.brow * p.T + cp.t0 + t) * p.Hv + h;
        p.dg[o] = dgam;
        p.dbeta[o] = db1 + vb[t];
      }
    }
  }
  // through the L2 fold: d(x / n) = (dx_hat - x_hat (x_hat . dx_hat)) / n
  {
    const float *rq = p.rq + (gc * p.Hqk + hk) * BT, *rk = p.rk + (gc * p.Hqk + hk) * BT;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = r0 + r;
      float a = 0.f, b = 0.f;
      if (p.use_l2) {
#pragma unroll
        for (int q = 0; q < NJ; ++q) {
          const int j = j0c + q;
          a = fmaf(sQ[t * QS + j], dq[r][q], a);
          b = fmaf(sK[t * QS + j], dk[r][q], b);
        }
        a = group_sum<CG>(a);
        b = group_sum<CG>(b);
      }
      if (t < nr) {
        const int64_t tt = cp.t0 + t, hq = hk * DK + j0c;
        const int64_t bq = cp.brow * p.sdq_b + tt * p.sdq_t + hq, bk = cp.brow * p.sdk_b + tt * p.sdk_t + hq;
#pragma unroll
        for (int q = 0; q < NJ; ++q) {
          const int j = j0c + q;
          store_grad<T>(p.dqq, p.grad_dtype, bq + q, (dq[r][q] - sQ[t * QS + j] * a) * rq[t]);
          store_grad<T>(p.dkk, p.grad_dtype, bk + q, (dk[r][q] - sK[t * QS + j] * b) * rk[t]);
        }
      }
    }
  }
}

template <typename T, int DK>
hipError_t launch_t(const ChunkBwdArgs &a0, hipStream_t s) {
  // The matrix-core state passes read the records the prep writes, and no
  // (I + A)^-1 or P in FP32; with the matrix-core gradient kernel as well,
  // nothing reads the unit q, k rows, and R is recomputed there instead of
  // stored. The prep and the state passes skip what is not read.
  ChunkBwdArgs a = a0;
  const bool ds_mma = chunk_bwd_state_mma_supported(a), grad_mma = chunk_bwd_grad_mma_supported(a);
  if (!ds_mma) a.brec = nullptr;
  if (ds_mma) a.mm = a.pp = nullptr;
  if (ds_mma && grad_mma) a.qn = a.kn = a.rr = nullptr;
  const int64_t N = a.n_seqs;
  // the matrix-core prep serves the all-matrix-core path (BF16 or FP16, dk
  // 64/128)
  if constexpr ((std::is_same<T, bf16>::value || std::is_same<T, f16>::value) && DK <= 128) {
    if (ds_mma && grad_mma)
      hipLaunchKernelGGL((bwd_prep_kernel<T, DK, true>), dim3((unsigned)a.chunk_bound, (unsigned)a.Hqk),
                         dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_prep_kernel<T, DK>), dim3((unsigned)a.chunk_bound, (unsigned)a.Hqk), dim3(kThreads),
                         0, s, a);
  } else {
    hipLaunchKernelGGL((bwd_prep_kernel<T, DK>), dim3((unsigned)a.chunk_bound, (unsigned)a.Hqk), dim3(kThreads), 0,
                       s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 sg((unsigned)(a.dv / 16), (unsigned)a.Hv, (unsigned)N);
  if (ds_mma) {
    e = launch_chunk_bwd_state_passes_mma(a, s);
  } else {
    hipLaunchKernelGGL((bwd_states_kernel<T, DK>), sg, dim3(kSer), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dstate_kernel<T, DK>), sg, dim3(kSer), 0, s, a);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  if (grad_mma) return launch_chunk_bwd_grad_mma(a, s);
  hipLaunchKernelGGL((bwd_grad_kernel<T, DK>), dim3((unsigned)a.chunk_bound, (unsigned)a.Hqk),
                     dim3(grad_threads<DK>()), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dk(const ChunkBwdArgs &a, hipStream_t s) {
  if (a.dk == 64) return launch_t<T, 64>(a, s);
  if (a.dk == 128) return launch_t<T, 128>(a, s);
  if (a.dk == 256) return launch_t<T, 256>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

bool chunk_bwd_supported(int64_t dk, int64_t dv) { return (dk == 64 || dk == 128 || dk == 256) && dv % 16 == 0; }

hipError_t launch_chunk_bwd(const ChunkBwdArgs &a, hipStream_t s) {
  if (a.cu_seqlens) {
    const hipError_t e = launch_chunk_index(a.cu_seqlens, a.n_seqs, a.cu_chunks, s);
    if (e != hipSuccess) return e;
  }
  if (a.act == kF32) return launch_dk<float>(a, s);
  if (a.act == kBF16) return launch_dk<bf16>(a, s);
  if (a.act == kF16) return launch_dk<f16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace gdn
