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
// and the Megatron-LM L2-fold pull request run; the pages state that the
// fused stages support first-order autograd, Megatron Core "GDN Elementwise
// Fusion", Execution and numerical behavior).
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
// Products run on the vector ALU from LDS tiles (a first version; the
// forward's MFMA layouts are not reused here).
#include "device_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int BT = 64;
constexpr int kThreads = 256;
constexpr int XP = 17;  // row stride of [64][16] tiles
constexpr int MP = 65;  // row stride of [64][64] tiles

// acc[r][c] += sum_k A(ty + 16 r, k) * B(k, tx + 16 c), with
// A(i, k) = A[i * ars + k * acs] and B(k, j) = B[k * brs + j * bcs].
template <int RM, int CN>
__device__ __forceinline__ void mm(float (&acc)[RM][CN], const float *A, int ars, int acs, const float *B, int brs,
                                   int bcs, int kn, int ty, int tx) {
  for (int kk = 0; kk < kn; ++kk) {
    float a[RM], b[CN];
#pragma unroll
    for (int r = 0; r < RM; ++r) a[r] = A[(ty + 16 * r) * ars + kk * acs];
#pragma unroll
    for (int c = 0; c < CN; ++c) b[c] = B[kk * brs + (tx + 16 * c) * bcs];
#pragma unroll
    for (int r = 0; r < RM; ++r)
#pragma unroll
      for (int c = 0; c < CN; ++c) acc[r][c] = fmaf(a[r], b[c], acc[r][c]);
  }
}

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

// Where chunk gc of the whole call lies: batch row, first token, rows.
struct ChunkPos {
  int64_t brow, t0;
  int nr;
  bool valid;
};

__device__ __forceinline__ ChunkPos chunk_pos(const ChunkBwdArgs &p, int64_t gc) {
  ChunkPos c;
  if (p.cu_seqlens) {
    const int32_t *cuc = p.cu_chunks;
    c.valid = gc < cuc[p.n_seqs];
    if (!c.valid) return c;
    int64_t lo = 0, hi = p.n_seqs;  // cuc[lo] <= gc < cuc[hi]
    while (hi - lo > 1) {
      const int64_t mid = (lo + hi) >> 1;
      if (cuc[mid] <= gc) lo = mid; else hi = mid;
    }
    const int64_t ch = gc - cuc[lo], bos = p.cu_seqlens[lo], L = p.cu_seqlens[lo + 1] - bos;
    c.brow = 0;
    c.t0 = bos + ch * BT;
    c.nr = (int)(L - ch * BT < BT ? L - ch * BT : BT);
  } else {
    const int64_t nc = (p.T + BT - 1) / BT;
    c.valid = gc < p.B * nc;
    if (!c.valid) return c;
    c.brow = gc / nc;
    const int64_t ch = gc % nc;
    c.t0 = ch * BT;
    c.nr = (int)(p.T - c.t0 < BT ? p.T - c.t0 : BT);
  }
  return c;
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
// Prep: unit q, k rows per (chunk, q/k head); gamma, M and scale * Pt per
// value head of the group.
// ---------------------------------------------------------------------------
template <typename T, int DK>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(ChunkBwdArgs p) {
  constexpr int KP = DK + 1;
  __shared__ float sQ[BT * KP], sK[BT * KP];
  __shared__ float sA[BT * MP], sM[BT * MP];
  __shared__ float sgam[BT], sbeta[BT];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t gc = blockIdx.x, hk = blockIdx.y;
  const ChunkPos cp = chunk_pos(p, gc);
  if (!cp.valid) return;
  const int nr = cp.nr;
  const int64_t G = p.Hv / p.Hqk;

  // q, k rows of the chunk (zero past the last token)
  for (int e = tid; e < BT * DK; e += kThreads) {
    const int t = e / DK, j = e % DK;
    float qv = 0.f, kv = 0.f;
    if (t < nr) {
      const int64_t tt = cp.t0 + t;
      qv = f(static_cast<const T *>(p.q)[cp.brow * p.sq_b + tt * p.sq_t + hk * p.sq_h + j]);
      kv = f(static_cast<const T *>(p.k)[cp.brow * p.sk_b + tt * p.sk_t + hk * p.sk_h + j]);
    }
    sQ[t * KP + j] = qv;
    sK[t * KP + j] = kv;
  }
  __syncthreads();
  // inverse norms: four lanes per row
  {
    const int t = tid >> 2, part = tid & 3;
    float sq = 0.f, sk = 0.f;
    for (int j = part; j < DK; j += 4) {
      sq = fmaf(sQ[t * KP + j], sQ[t * KP + j], sq);
      sk = fmaf(sK[t * KP + j], sK[t * KP + j], sk);
    }
    sq = group_sum<4>(sq);
    sk = group_sum<4>(sk);
    const float rq = p.use_l2 ? 1.f / sqrtf(sq + p.l2_eps) : 1.f;
    const float rk = p.use_l2 ? 1.f / sqrtf(sk + p.l2_eps) : 1.f;
    __syncthreads();
    for (int j = part; j < DK; j += 4) {
      sQ[t * KP + j] *= rq;
      sK[t * KP + j] *= rk;
    }
    if (part == 0) {
      p.rq[(gc * p.Hqk + hk) * BT + t] = rq;
      p.rk[(gc * p.Hqk + hk) * BT + t] = rk;
    }
  }
  __syncthreads();
  {
    float *qn = p.qn + (gc * p.Hqk + hk) * BT * DK, *kn = p.kn + (gc * p.Hqk + hk) * BT * DK;
    for (int e = tid; e < BT * DK; e += kThreads) {
      const int t = e / DK, j = e % DK;
      qn[e] = sQ[t * KP + j];
      kn[e] = sK[t * KP + j];
    }
  }
  // G = K K^T and QK = Q K^T; thread owns rows ty + 16 r, columns tx + 16 c
  float gg[4][4], qk[4][4];
  zero(gg);
  zero(qk);
  mm(gg, sK, KP, 1, sK, 1, KP, DK, ty, tx);
  mm(qk, sQ, KP, 1, sK, 1, KP, DK, ty, tx);

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
      float *pp = p.pp + (gc * p.Hv + h) * BT * BT;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int t = ty + 16 * r, s = tx + 16 * c;
          const float e = s <= t ? __expf(sgam[t] - sgam[s]) : 0.f;
          sA[t * MP + s] = s < t ? sbeta[t] * e * gg[r][c] : 0.f;
          pp[t * BT + s] = p.scale * e * qk[r][c];
        }
    }
    __syncthreads();
    // M = (I + A)^-1 by forward substitution, column c by four lanes; lane
    // `part` keeps rows 4 u + part of its column in registers.
    {
      const int c = tid >> 2, part = tid & 3;
      float mr[16];
#pragma unroll
      for (int t = 0; t < BT; ++t) {
        float sum = 0.f;
#pragma unroll
        for (int u = 0; u < (t + 3) / 4; ++u) {
          const int s = 4 * u + part;
          if (s < t) sum = fmaf(sA[t * MP + s], mr[u], sum);
        }
        sum = group_sum<4>(sum);
        const float mt = t == c ? 1.f : (t > c ? -sum : 0.f);
        if ((t & 3) == part) mr[t >> 2] = mt;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) sM[(4 * u + part) * MP + c] = mr[u];
    }
    __syncthreads();
    {
      float *mm_ = p.mm + (gc * p.Hv + h) * BT * BT;
      for (int e = tid; e < BT * BT; e += kThreads) mm_[e] = sM[(e >> 6) * MP + (e & 63)];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Forward states: S0 of every chunk, R and Delta, for 16 value rows.
// ---------------------------------------------------------------------------
template <typename T, int DK>
__global__ __launch_bounds__(kThreads) void bwd_states_kernel(ChunkBwdArgs p) {
  constexpr int KP = DK + 1, CN = DK / 16;
  __shared__ float sK[BT * KP], sM[BT * MP], sS[16 * KP];
  __shared__ float sX[BT * XP], sV[BT * XP];
  __shared__ float seg[BT], scw[BT], sbeta[BT];
  __shared__ float seC;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t j0 = (int64_t)blockIdx.x * 16, h = blockIdx.y, n = blockIdx.z;
  const int64_t hk = h / (p.Hv / p.Hqk);
  int64_t brow, bos, L, gc0;
  seq_pos(p, n, brow, bos, L, gc0);
  const int64_t nch = (L + BT - 1) / BT;

  for (int e = tid; e < 16 * DK; e += kThreads) {
    const int i = e / DK, j = e % DK;
    sS[i * KP + j] = p.init_state ? p.init_state[((n * p.Hv + h) * p.dv + j0 + i) * DK + j] : 0.f;
  }
  __syncthreads();
  for (int64_t c = 0; c < nch; ++c) {
    const int64_t gc = gc0 + c, t0 = bos + c * BT;
    const int nr = (int)(L - c * BT < BT ? L - c * BT : BT);
    float *s0 = p.s0 + ((gc * p.Hv + h) * p.dv + j0) * DK;
    for (int e = tid; e < 16 * DK; e += kThreads) s0[e] = sS[(e / DK) * KP + e % DK];
    const float *kn = p.kn + (gc * p.Hqk + hk) * BT * DK;
    for (int e = tid; e < BT * DK; e += kThreads) sK[(e / DK) * KP + e % DK] = kn[e];
    const float *mm_ = p.mm + (gc * p.Hv + h) * BT * BT;
    for (int e = tid; e < BT * BT; e += kThreads) sM[(e >> 6) * MP + (e & 63)] = mm_[e];
    if (tid < BT) {
      const float *gm = p.gam + (gc * p.Hv + h) * BT;
      const float gl = gm[nr - 1], gt = gm[tid];
      seg[tid] = __expf(gt);
      scw[tid] = tid < nr ? __expf(gl - gt) : 0.f;
      sbeta[tid] = tid < nr ? p.beta[brow * p.sbt_b + (t0 + tid) * p.sbt_t + h * p.sbt_h] : 0.f;
      if (tid == 0) seC = __expf(gl);
    }
    for (int e = tid; e < BT * 16; e += kThreads) {
      const int t = e >> 4, i = e & 15;
      sV[t * XP + i] = t < nr ? f(static_cast<const T *>(p.v)[brow * p.sv_b + (t0 + t) * p.sv_t + h * p.sv_h + j0 + i])
                              : 0.f;
    }
    __syncthreads();
    // KS = K S0^T; R = V - exp(gamma) KS; X = beta R
    {
      float ks[4][1];
      zero(ks);
      mm(ks, sK, KP, 1, sS, 1, KP, DK, ty, tx);
      float *rr = p.rr + (gc * p.Hv + h) * BT * p.dv + j0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = ty + 16 * r;
        const float R = sV[t * XP + tx] - seg[t] * ks[r][0];
        rr[t * p.dv + tx] = R;
        sX[t * XP + tx] = sbeta[t] * R;
      }
    }
    __syncthreads();
    // Delta = M X; cw Delta to sV for the state update
    {
      float dl[4][1];
      zero(dl);
      mm(dl, sM, MP, 1, sX, XP, 1, BT, ty, tx);
      float *del = p.del + (gc * p.Hv + h) * BT * p.dv + j0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = ty + 16 * r;
        del[t * p.dv + tx] = dl[r][0];
        sV[t * XP + tx] = scw[t] * dl[r][0];
      }
    }
    __syncthreads();
    // S = exp(gamma_C) S + (cw Delta)^T K; row i = ty, columns tx + 16 c
    {
      float sn[1][CN];
#pragma unroll
      for (int cc = 0; cc < CN; ++cc) sn[0][cc] = seC * sS[ty * KP + tx + 16 * cc];
      mm(sn, sV, 1, XP, sK, KP, 1, nr, ty, tx);
#pragma unroll
      for (int cc = 0; cc < CN; ++cc) sS[ty * KP + tx + 16 * cc] = sn[0][cc];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Reverse pass: dS carried from the last chunk to the first.
// ---------------------------------------------------------------------------
template <typename T, int DK>
__global__ __launch_bounds__(kThreads) void bwd_dstate_kernel(ChunkBwdArgs p) {
  constexpr int KP = DK + 1, CN = DK / 16;
  __shared__ float sK[BT * KP], sQ[BT * KP], sP[BT * MP], sM[BT * MP], sS[16 * KP];
  __shared__ float sO[BT * XP], sD[BT * XP], sR[BT * XP];
  __shared__ float seg[BT], scw[BT], sbeta[BT];
  __shared__ float seC;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t j0 = (int64_t)blockIdx.x * 16, h = blockIdx.y, n = blockIdx.z;
  const int64_t hk = h / (p.Hv / p.Hqk);
  int64_t brow, bos, L, gc0;
  seq_pos(p, n, brow, bos, L, gc0);
  const int64_t nch = (L + BT - 1) / BT;

  for (int e = tid; e < 16 * DK; e += kThreads) {
    const int i = e / DK, j = e % DK;
    sS[i * KP + j] = p.d_final ? p.d_final[((n * p.Hv + h) * p.dv + j0 + i) * DK + j] : 0.f;
  }
  __syncthreads();
  for (int64_t c = nch - 1; c >= 0; --c) {
    const int64_t gc = gc0 + c, t0 = bos + c * BT;
    const int nr = (int)(L - c * BT < BT ? L - c * BT : BT);
    float *ds = p.ds + ((gc * p.Hv + h) * p.dv + j0) * DK;
    for (int e = tid; e < 16 * DK; e += kThreads) ds[e] = sS[(e / DK) * KP + e % DK];
    const float *kn = p.kn + (gc * p.Hqk + hk) * BT * DK, *qn = p.qn + (gc * p.Hqk + hk) * BT * DK;
    for (int e = tid; e < BT * DK; e += kThreads) {
      sK[(e / DK) * KP + e % DK] = kn[e];
      sQ[(e / DK) * KP + e % DK] = qn[e];
    }
    const float *mm_ = p.mm + (gc * p.Hv + h) * BT * BT, *pp = p.pp + (gc * p.Hv + h) * BT * BT;
    for (int e = tid; e < BT * BT; e += kThreads) {
      sM[(e >> 6) * MP + (e & 63)] = mm_[e];
      sP[(e >> 6) * MP + (e & 63)] = pp[e];
    }
    if (tid < BT) {
      const float *gm = p.gam + (gc * p.Hv + h) * BT;
      const float gl = gm[nr - 1], gt = gm[tid];
      seg[tid] = __expf(gt);
      scw[tid] = tid < nr ? __expf(gl - gt) : 0.f;
      sbeta[tid] = tid < nr ? p.beta[brow * p.sbt_b + (t0 + tid) * p.sbt_t + h * p.sbt_h] : 0.f;
      if (tid == 0) seC = __expf(gl);
    }
    for (int e = tid; e < BT * 16; e += kThreads) {
      const int t = e >> 4, i = e & 15;
      sO[t * XP + i] =
          t < nr ? f(static_cast<const T *>(p.d_o)[brow * p.sdo_b + (t0 + t) * p.sdo_t + h * p.sdo_h + j0 + i]) : 0.f;
    }
    __syncthreads();
    // dDelta = Pt'^T dO + cw (K dS^T)   (scale is inside the stored Pt)
    {
      float a1[4][1], a2[4][1];
      zero(a1);
      zero(a2);
      mm(a1, sP, 1, MP, sO, XP, 1, nr, ty, tx);
      mm(a2, sK, KP, 1, sS, 1, KP, DK, ty, tx);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = ty + 16 * r;
        sD[t * XP + tx] = a1[r][0] + scw[t] * a2[r][0];
      }
    }
    __syncthreads();
    // dR' = M^T dDelta; dv = beta dR'; exp(gamma) dv and scale exp(gamma) dO
    // for the state update
    {
      float a1[4][1];
      zero(a1);
      mm(a1, sM, 1, MP, sD, XP, 1, BT, ty, tx);
      float *drp = p.drp + (gc * p.Hv + h) * BT * p.dv + j0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = ty + 16 * r;
        drp[t * p.dv + tx] = a1[r][0];
        const float dvv = sbeta[t] * a1[r][0];
        if (t < nr)
          store_grad<T>(p.dvv, p.grad_dtype, ((brow * p.T + t0 + t) * p.Hv + h) * p.dv + j0 + tx, dvv);
        sR[t * XP + tx] = seg[t] * dvv;
        sO[t * XP + tx] *= p.scale * seg[t];
      }
    }
    __syncthreads();
    // dS0 = exp(gamma_C) dS + (scale exp(gamma) dO)^T Q - (exp(gamma) dv)^T K
    {
      float a1[1][CN], a2[1][CN];
#pragma unroll
      for (int cc = 0; cc < CN; ++cc) {
        a1[0][cc] = seC * sS[ty * KP + tx + 16 * cc];
        a2[0][cc] = 0.f;
      }
      mm(a1, sO, 1, XP, sQ, KP, 1, nr, ty, tx);
      mm(a2, sR, 1, XP, sK, KP, 1, nr, ty, tx);
#pragma unroll
      for (int cc = 0; cc < CN; ++cc) sS[ty * KP + tx + 16 * cc] = a1[0][cc] - a2[0][cc];
    }
    __syncthreads();
  }
  if (p.d_init) {
    for (int e = tid; e < 16 * DK; e += kThreads) {
      const int i = e / DK, j = e % DK;
      p.d_init[((n * p.Hv + h) * p.dv + j0 + i) * DK + j] = sS[i * KP + j];
    }
  }
}

// ---------------------------------------------------------------------------
// Gradients of q, k, g and beta per (chunk, q/k head).
// ---------------------------------------------------------------------------
template <int DK>
struct GradTiles {
  static constexpr int KP = DK + 1;
  float o[BT * XP], d[BT * XP], rp[BT * XP], r[BT * XP];  // dO, Delta, dR', R
  float s0[16 * KP], ds[16 * KP];                          // S0, dS_C rows
};

template <typename T, int DK>
__global__ __launch_bounds__(kThreads) void bwd_grad_kernel(ChunkBwdArgs p) {
  constexpr int KP = DK + 1, CN = DK / 16;
  __shared__ float sQ[BT * KP], sK[BT * KP];
  __shared__ float sZ1[BT * MP], sZ2[BT * MP];  // dQK, dG
  __shared__ union {
    GradTiles<DK> t;
    float z[BT * MP];  // a + p, for its column sums
  } u;
  __shared__ float sgam[BT], seg[BT], scw[BT], sbeta[BT];
  __shared__ float vrow[BT], vm[BT], vb[BT], red[kThreads];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t gc = blockIdx.x, hk = blockIdx.y;
  const ChunkPos cp = chunk_pos(p, gc);
  if (!cp.valid) return;
  const int nr = cp.nr;
  const int64_t G = p.Hv / p.Hqk, dvn = p.dv;

  {
    const float *kn = p.kn + (gc * p.Hqk + hk) * BT * DK, *qn = p.qn + (gc * p.Hqk + hk) * BT * DK;
    for (int e = tid; e < BT * DK; e += kThreads) {
      sK[(e / DK) * KP + e % DK] = kn[e];
      sQ[(e / DK) * KP + e % DK] = qn[e];
    }
  }
  __syncthreads();
  float gg[4][4], qk[4][4];
  zero(gg);
  zero(qk);
  mm(gg, sK, KP, 1, sK, 1, KP, DK, ty, tx);
  mm(qk, sQ, KP, 1, sK, 1, KP, DK, ty, tx);
  float dq[4][CN], dk[4][CN];
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
    float c1[4][4], c2[4][4], k1[4][CN], k2[4][CN], k3[4][CN];
    zero(c1);
    zero(c2);
    zero(k1);
    zero(k2);
    zero(k3);
    float db1 = 0.f, sdot = 0.f;
    const int64_t rowbase = (gc * p.Hv + h) * BT * dvn;
    const int64_t stbase = (gc * p.Hv + h) * dvn * DK;
    for (int64_t j0 = 0; j0 < dvn; j0 += 16) {
      __syncthreads();
      for (int e = tid; e < BT * 16; e += kThreads) {
        const int t = e >> 4, i = e & 15;
        u.t.o[t * XP + i] = t < nr ? f(static_cast<const T *>(p.d_o)[cp.brow * p.sdo_b + (cp.t0 + t) * p.sdo_t +
                                                                      h * p.sdo_h + j0 + i])
                                   : 0.f;
        const int64_t w = rowbase + t * dvn + j0 + i;
        u.t.d[t * XP + i] = p.del[w];
        u.t.rp[t * XP + i] = p.drp[w];
        u.t.r[t * XP + i] = p.rr[w];
      }
      for (int e = tid; e < 16 * DK; e += kThreads) {
        const int i = e / DK, j = e % DK;
        const int64_t w = stbase + (j0 + i) * DK + j;
        const float a = p.s0[w], b = p.ds[w];
        u.t.s0[i * KP + j] = a;
        u.t.ds[i * KP + j] = b;
        sdot = fmaf(a, b, sdot);
      }
      __syncthreads();
      mm(c1, u.t.o, XP, 1, u.t.d, 1, XP, 16, ty, tx);
      mm(c2, u.t.rp, XP, 1, u.t.d, 1, XP, 16, ty, tx);
      mm(k1, u.t.o, XP, 1, u.t.s0, KP, 1, 16, ty, tx);
      mm(k2, u.t.d, XP, 1, u.t.ds, KP, 1, 16, ty, tx);
      mm(k3, u.t.rp, XP, 1, u.t.s0, KP, 1, 16, ty, tx);
      if (tid < BT)
#pragma unroll
        for (int i = 0; i < 16; ++i) db1 = fmaf(u.t.rp[tid * XP + i], u.t.r[tid * XP + i], db1);
    }
    __syncthreads();  // tiles dead: the union now holds a + p
    // Elementwise C x C terms. Thread owns rows t = ty + 16 r, columns
    // s = tx + 16 c.
    float rowz[4], roww[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = ty + 16 * r;
      rowz[r] = 0.f;
      roww[r] = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int s = tx + 16 * c;
        const float e = s <= t ? __expf(sgam[t] - sgam[s]) : 0.f;
        const float dpt = p.scale * c1[r][c] * (s <= t ? 1.f : 0.f);  // dPt
        const float dqk = dpt * e;
        const float pz = dqk * qk[r][c];                               // dPt * Pt
        const float da = s < t ? -c2[r][c] : 0.f;                      // dA
        const float eg = e * gg[r][c];
        const float dg = da * sbeta[t] * e;                            // dG
        const float az = da * sbeta[t] * eg;                           // dA * A
        sZ1[t * MP + s] = dqk;
        sZ2[t * MP + s] = dg;
        u.z[t * MP + s] = az + pz;
        rowz[r] += az + pz;
        roww[r] = fmaf(da, eg, roww[r]);
      }
    }
    // row dots of the C x dk terms with the unit q, k rows
    float rdot[4], rm[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = ty + 16 * r;
      float a = 0.f, b = 0.f, m = 0.f;
#pragma unroll
      for (int cc = 0; cc < CN; ++cc) {
        const int j = tx + 16 * cc;
        a = fmaf(sQ[t * KP + j], k1[r][cc], a);
        b = fmaf(sK[t * KP + j], k3[r][cc], b);
        m = fmaf(sK[t * KP + j], k2[r][cc], m);
      }
      const float rd = p.scale * seg[t] * a - seg[t] * sbeta[t] * b - scw[t] * m;
      rdot[r] = group_sum<16>(rd + rowz[r]);
      rm[r] = group_sum<16>(scw[t] * m);
      roww[r] = group_sum<16>(roww[r]);
    }
    if (tx == 0)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        vrow[ty + 16 * r] = rdot[r];
        vm[ty + 16 * r] = rm[r];
        vb[ty + 16 * r] = roww[r];
      }
    red[tid] = sdot;
    // the q/k gradients of this value head
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = ty + 16 * r;
#pragma unroll
      for (int cc = 0; cc < CN; ++cc) {
        dq[r][cc] = fmaf(p.scale * seg[t], k1[r][cc], dq[r][cc]);
        dk[r][cc] += scw[t] * k2[r][cc] - seg[t] * sbeta[t] * k3[r][cc];
      }
    }
    __syncthreads();
    mm(dq, sZ1, MP, 1, sK, KP, 1, BT, ty, tx);
    mm(dk, sZ2, MP, 1, sK, KP, 1, BT, ty, tx);
    mm(dk, sZ2, 1, MP, sK, KP, 1, BT, ty, tx);
    mm(dk, sZ1, 1, MP, sQ, KP, 1, BT, ty, tx);
    if (tid < BT) {  // wave 0: dgamma, its reverse running sum (dg), dbeta
      const int t = tid;
      float colz = 0.f;
      for (int s = 0; s < BT; ++s) colz += u.z[s * MP + t];
      float tot = 0.f;
      for (int i = 0; i < kThreads; ++i) tot += red[i];
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
  __syncthreads();
  // through the L2 fold: d(x / n) = (dx_hat - x_hat (x_hat . dx_hat)) / n
  {
    const float *rq = p.rq + (gc * p.Hqk + hk) * BT, *rk = p.rk + (gc * p.Hqk + hk) * BT;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = ty + 16 * r;
      float a = 0.f, b = 0.f;
      if (p.use_l2) {
#pragma unroll
        for (int cc = 0; cc < CN; ++cc) {
          const int j = tx + 16 * cc;
          a = fmaf(sQ[t * KP + j], dq[r][cc], a);
          b = fmaf(sK[t * KP + j], dk[r][cc], b);
        }
        a = group_sum<16>(a);
        b = group_sum<16>(b);
      }
      if (t < nr) {
        const int64_t base = ((cp.brow * p.T + cp.t0 + t) * p.Hqk + hk) * DK;
#pragma unroll
        for (int cc = 0; cc < CN; ++cc) {
          const int j = tx + 16 * cc;
          store_grad<T>(p.dqq, p.grad_dtype, base + j, (dq[r][cc] - sQ[t * KP + j] * a) * rq[t]);
          store_grad<T>(p.dkk, p.grad_dtype, base + j, (dk[r][cc] - sK[t * KP + j] * b) * rk[t]);
        }
      }
    }
  }
}

template <typename T, int DK>
hipError_t launch_t(const ChunkBwdArgs &a, hipStream_t s) {
  const int64_t N = a.n_seqs;
  hipLaunchKernelGGL((bwd_prep_kernel<T, DK>), dim3((unsigned)a.chunk_bound, (unsigned)a.Hqk), dim3(kThreads), 0, s,
                     a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 sg((unsigned)(a.dv / 16), (unsigned)a.Hv, (unsigned)N);
  hipLaunchKernelGGL((bwd_states_kernel<T, DK>), sg, dim3(kThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dstate_kernel<T, DK>), sg, dim3(kThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_grad_kernel<T, DK>), dim3((unsigned)a.chunk_bound, (unsigned)a.Hqk), dim3(kThreads), 0, s,
                     a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dk(const ChunkBwdArgs &a, hipStream_t s) {
  if (a.dk == 64) return launch_t<T, 64>(a, s);
  if (a.dk == 128) return launch_t<T, 128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

bool chunk_bwd_supported(int64_t dk, int64_t dv) { return (dk == 64 || dk == 128) && dv % 16 == 0; }

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
