// Chunked gated delta rule, forward, with q/k L2 normalisation folded in.
//
// The Megatron-LM pull request "fold q/k L2-norm into the gated_delta_rule
// kernel" (What, Why) moves the per-head q/k L2 normalisation (eps 1e-6) into
// the recurrence kernel; the flash-linear-attention pull request on the fused
// short conv runs that recurrence in chunk mode. The recurrence (Gated
// DeltaNet, Yang, Kautz and Hatamizadeh, ICLR 2025) is
//     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
//     o_t = scale * S_t q_t.
// Its chunked form (WY / UT transform of the delta rule, Yang et al., NeurIPS
// 2024, with gating): for a chunk of C = 64 rows entering with state S0,
//     gamma = cumsum(g)                      (inside the chunk)
//     A[r,i] = beta_r exp(gamma_r - gamma_i) k_r.k_i   (i < r)
//     T = (I + A)^-1                         (unit lower triangular, FP32)
//     R = diag(beta) (V - diag(exp(gamma)) K S0^T)
//     Vn = T R                               (the chunk's corrected values)
//     P[r,i] = exp(gamma_r - gamma_i) q_r.k_i          (i <= r)
//     O = scale (diag(exp(gamma)) Q S0^T + P Vn)
//     S = exp(gamma_C) S0 + Vn^T diag(exp(gamma_C - gamma)) K
// Only non-positive exponents appear (g <= 0), so nothing overflows.
//
// Mapping to gfx950. One workgroup (4 wavefronts) owns one (sequence, value
// head, 16-row slice of dv) and walks that sequence's chunks in order; the
// 16 x dk FP32 slice of S stays in MFMA accumulator registers for the whole
// sequence and is also kept as an act-dtype copy in LDS for use as an MFMA
// operand. All contractions (K K^T, Q K^T, K S^T, Q S^T, T R, P Vn and the
// state update) are v_mfma_f32_16x16x32 {bf16,f16} tiles on LDS-staged
// operands (v_mfma_f32_16x16x4_f32 for FP32 inputs); the triangular inverse
// is solved in FP32: 16 x 16 diagonal blocks by forward substitution (one
// lane per column), then the three off-diagonal levels. Value head h reads
// query/key head h / (Hv / Hqk) (GQA map, no copy). Padded rows of a partial
// chunk carry zero q, k, v, g and beta, which makes them inert.
#include "device_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int BT = 64;   // chunk length
constexpr int DVT = 16;  // dv rows per workgroup

template <typename T> struct Mfma;
template <> struct Mfma<bf16> {
  static constexpr int KS = 32, E = 8;
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<f16> {
  static constexpr int KS = 32, E = 8;
  typedef f16x8 frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  static constexpr int KS = 4, E = 1;
  typedef float frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Operand fragment of a row-major LDS matrix M (leading dimension ld):
// lane l supplies M[m0 + l%16][k0 + (l/16)*E + j], j < E. Used for the A
// operand (rows = output rows) and, with M = B^T, for the B operand
// (rows = output columns); both use the same k mapping, so the contraction is
// over matching k.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag frag_rows(const T *M, int ld, int m0, int k0,
                                                            int lane) {
  const T *p = M + (m0 + (lane & 15)) * ld + k0 + (lane >> 4) * Mfma<T>::E;
  return *reinterpret_cast<const typename Mfma<T>::frag *>(p);
}

// B operand read from a row-major LDS matrix M[k][n] without a transposed
// copy: lane l supplies M[k0 + (l/16)*E + j][n0 + l%16].
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag frag_cols(const T *M, int ld, int k0, int n0,
                                                            int lane) {
  typename Mfma<T>::frag fr;
  if constexpr (Mfma<T>::E == 1) {
    fr = M[(k0 + (lane >> 4)) * ld + n0 + (lane & 15)];
  } else {
#pragma unroll
    for (int j = 0; j < Mfma<T>::E; ++j)
      fr[j] = M[(k0 + (lane >> 4) * Mfma<T>::E + j) * ld + n0 + (lane & 15)];
  }
  return fr;
}

template <typename T, int DK>
struct Smem {
  static constexpr int PAD = 16 / (int)sizeof(T);
  static constexpr int LDK = DK + PAD;  // rows of length dk
  static constexpr int LDC = BT + PAD;  // rows of length BT
  static constexpr int LDF = BT + 1;    // FP32 64 x 64 scratch
  alignas(16) T q[BT * LDK];            // normalised q rows
  alignas(16) T k[BT * LDK];            // normalised k rows
  alignas(16) T s[DVT * LDK];           // state slice (act dtype copy)
  // T = (I + A)^-1 as an MFMA operand; for FP32 inputs the FP32 copy below
  // is used directly.
  static constexpr bool kTmIsTf = sizeof(T) == 4;
  alignas(16) T tm[kTmIsTf ? 4 : BT * LDC];
  alignas(16) T pm[BT * LDC];           // P
  alignas(16) T vt[DVT * LDC];          // V^T slice
  alignas(16) T rt[DVT * LDC];          // R^T
  alignas(16) T wt[DVT * LDC];          // Vn^T
  alignas(16) T wdt[DVT * LDC];         // (diag(exp(gamma_C - gamma)) Vn)^T
  float a[BT * LDF];                    // A (strictly lower)
  float tf[BT * LDF];                   // T in FP32
  float x[3 * 256];                     // off-diagonal products
  float gam[BT], beta[BT];
};

template <typename T, int DK>
__global__ __launch_bounds__(kThreads) void chunk_rule_kernel(ChunkArgs p) {
  using MF = Mfma<T>;
  using SM = Smem<T, DK>;
  constexpr int KS = MF::KS;
  constexpr int LDK = SM::LDK, LDC = SM::LDC, LDF = SM::LDF;
  __shared__ SM sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t j0 = (int64_t)blockIdx.x * DVT;
  const int64_t h = blockIdx.y;
  const int64_t n = blockIdx.z;
  const int64_t hk = h / (p.Hv / p.Hqk);

  int64_t bos, eos, brow;
  if (p.cu_seqlens) {
    bos = p.cu_seqlens[n];
    eos = p.cu_seqlens[n + 1];
    brow = 0;
  } else {
    bos = 0;
    eos = p.T;
    brow = n;
  }
  const T *qb = static_cast<const T *>(p.q) + brow * p.sq_b + hk * p.sq_h;
  const T *kb = static_cast<const T *>(p.k) + brow * p.sk_b + hk * p.sk_h;
  const T *vb = static_cast<const T *>(p.v) + brow * p.sv_b + h * p.sv_h + j0;
  const float *gb = p.g + brow * p.sg_b + h * p.sg_h;
  const float *bb = p.beta + brow * p.sbt_b + h * p.sbt_h;
  T *ob = static_cast<T *>(p.o) + brow * p.so_b + h * p.so_h + j0;

  // State slice S[j0 + row][col], rows 4*(lane/16)+i, cols 16*nt + lane%16,
  // N-tiles nt = wave + 4u.
  constexpr int NTW = DK / 64;  // state N-tiles per wave
  f32x4 S[NTW];
  const int64_t st_base = ((n * p.Hv + h) * p.dv + j0) * DK;
#pragma unroll
  for (int u = 0; u < NTW; ++u) {
    const int nt = wave + 4 * u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * (lane >> 4) + i, col = 16 * nt + (lane & 15);
      const float v0 = p.init_state ? p.init_state[st_base + (int64_t)row * DK + col] : 0.f;
      S[u][i] = v0;
      sm.s[row * LDK + col] = to<T>(v0);
    }
  }

  for (int64_t c0 = bos; c0 < eos; c0 += BT) {
    const int nr = (int)(eos - c0 < BT ? eos - c0 : BT);

    // ---- stage q, k (normalised), v^T, beta and gamma in LDS ----
    {
      constexpr int SEG = DK / 8;          // 8-element segments per row
      constexpr int RPP = kThreads / SEG;  // rows per pass
      const int s = tid % SEG;
#pragma unroll
      for (int r0 = 0; r0 < BT; r0 += RPP) {
        const int r = r0 + tid / SEG;
        float qv[8], kv[8];
        if (r < nr) {
          load_vec<T, 8>(qb + (c0 + r) * p.sq_t + s * 8, 16, qv);
          load_vec<T, 8>(kb + (c0 + r) * p.sk_t + s * 8, 16, kv);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) qv[i] = kv[i] = 0.f;
        }
        if (p.use_l2) {
          float sq = 0.f, sk = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            sq += qv[i] * qv[i];
            sk += kv[i] * kv[i];
          }
          sq = group_sum<SEG>(sq);
          sk = group_sum<SEG>(sk);
          const float rq = rsqrtf(sq + p.l2_eps), rk = rsqrtf(sk + p.l2_eps);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            qv[i] *= rq;
            kv[i] *= rk;
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          sm.q[r * LDK + s * 8 + i] = to<T>(qv[i]);
          sm.k[r * LDK + s * 8 + i] = to<T>(kv[i]);
        }
      }
      {
        const int r = tid >> 2, cc = (tid & 3) * 4;
        float vv[4];
        if (r < nr) {
          load_vec<T, 4>(vb + (c0 + r) * p.sv_t + cc, 4 * (int)sizeof(T), vv);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) vv[i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.vt[(cc + i) * LDC + r] = to<T>(vv[i]);
      }
      if (wave == 0) {
        float gv = lane < nr ? gb[(c0 + lane) * p.sg_t] : 0.f;
        const float bv = lane < nr ? bb[(c0 + lane) * p.sbt_t] : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float o = __shfl_up(gv, off, 64);
          if (lane >= off) gv += o;
        }
        sm.gam[lane] = gv;
        sm.beta[lane] = bv;
      }
    }
    __syncthreads();

    // ---- K K^T -> A (FP32), Q K^T -> P; 10 lower tiles each ----
    for (int task = wave; task < 20; task += 4) {
      const int tt = task % 10;
      const int mi = tt < 1 ? 0 : tt < 3 ? 1 : tt < 6 ? 2 : 3;
      const int ni = tt - mi * (mi + 1) / 2;
      const T *lhs = task < 10 ? sm.k : sm.q;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK / KS; ++ks)
        acc = MF::mma(frag_rows(lhs, LDK, 16 * mi, ks * KS, lane),
                      frag_rows(sm.k, LDK, 16 * ni, ks * KS, lane), acc);
      const int c = 16 * ni + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mi + 4 * (lane >> 4) + i;
        const float d = sm.gam[r] - sm.gam[c];
        if (task < 10) {
          sm.a[r * LDF + c] = c < r ? sm.beta[r] * fast_exp(fminf(d, 0.f)) * acc[i] : 0.f;
        } else {
          sm.pm[r * LDC + c] = to<T>(c <= r ? fast_exp(fminf(d, 0.f)) * acc[i] : 0.f);
        }
      }
    }
    // zero the upper tiles of P
    for (int e = tid; e < BT * BT; e += kThreads) {
      const int r = e / BT, c = e % BT;
      if ((c >> 4) > (r >> 4)) sm.pm[r * LDC + c] = to<T>(0.f);
    }
    __syncthreads();

    // ---- T = (I + A)^-1: diagonal 16 x 16 blocks, one lane per column ----
    if (wave == 0) {
      const int blk = lane >> 4, c = lane & 15, o = 16 * blk;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = r == c ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) s -= sm.a[(o + r) * LDF + o + i] * x[i];
        x[r] = s;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.tf[(o + r) * LDF + o + c] = x[r];
    }
    __syncthreads();
    // off-diagonal blocks, level d: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj, i = j + d
    for (int d = 1; d < 4; ++d) {
      const int nb = 4 - d;
      for (int e = tid; e < nb * 256; e += kThreads) {
        const int jb = e >> 8, rr = (e >> 4) & 15, cc = e & 15, ib = jb + d;
        float acc = 0.f;
        for (int kb = jb; kb < ib; ++kb)
#pragma unroll
          for (int m = 0; m < 16; ++m)
            acc += sm.a[(16 * ib + rr) * LDF + 16 * kb + m] * sm.tf[(16 * kb + m) * LDF + 16 * jb + cc];
        sm.x[e] = acc;
      }
      __syncthreads();
      for (int e = tid; e < nb * 256; e += kThreads) {
        const int jb = e >> 8, rr = (e >> 4) & 15, cc = e & 15, ib = jb + d;
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m)
          acc += sm.tf[(16 * ib + rr) * LDF + 16 * ib + m] * sm.x[(jb << 8) + m * 16 + cc];
        sm.tf[(16 * ib + rr) * LDF + 16 * jb + cc] = -acc;
      }
      __syncthreads();
    }
    for (int e = tid; e < BT * BT; e += kThreads) {
      const int r = e / BT, c = e % BT;
      const float tv = c <= r ? sm.tf[r * LDF + c] : 0.f;
      if constexpr (SM::kTmIsTf) sm.tf[r * LDF + c] = tv;
      else sm.tm[r * LDC + c] = to<T>(tv);
    }
    __syncthreads();
    const T *tmat;
    int ldt;
    if constexpr (SM::kTmIsTf) {
      tmat = reinterpret_cast<const T *>(sm.tf);
      ldt = LDF;
    } else {
      tmat = sm.tm;
      ldt = LDC;
    }

    // ---- state-dependent part; wave w owns chunk rows 16w .. 16w+15 ----
    const int w16 = 16 * wave;
    f32x4 Y = {0.f, 0.f, 0.f, 0.f}, Z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DK / KS; ++ks) {
      const auto bs = frag_rows(sm.s, LDK, 0, ks * KS, lane);
      Y = MF::mma(frag_rows(sm.k, LDK, w16, ks * KS, lane), bs, Y);
      Z = MF::mma(frag_rows(sm.q, LDK, w16, ks * KS, lane), bs, Z);
    }
    const int col = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = w16 + 4 * (lane >> 4) + i;
      const float eg = fast_exp(sm.gam[r]);
      const float R = sm.beta[r] * (f(sm.vt[col * LDC + r]) - eg * Y[i]);
      sm.rt[col * LDC + r] = to<T>(R);
      Z[i] *= eg;
    }
    __syncthreads();

    // Vn = T R (T is lower triangular: k < 16w + 16)
    constexpr int KST = KS;
    const int nks = (w16 + 16 + KST - 1) / KST;
    f32x4 W = {0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < nks; ++ks)
      W = MF::mma(frag_rows(tmat, ldt, w16, ks * KS, lane), frag_rows(sm.rt, LDC, 0, ks * KS, lane), W);
    const float gC = sm.gam[BT - 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = w16 + 4 * (lane >> 4) + i;
      sm.wt[col * LDC + r] = to<T>(W[i]);
      sm.wdt[col * LDC + r] = to<T>(fast_exp(gC - sm.gam[r]) * W[i]);
    }
    __syncthreads();

    // O = scale (diag(exp(gamma)) Q S^T + P Vn)
    f32x4 Oa = Z;
    for (int ks = 0; ks < nks; ++ks)
      Oa = MF::mma(frag_rows(sm.pm, LDC, w16, ks * KS, lane), frag_rows(sm.wt, LDC, 0, ks * KS, lane), Oa);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = w16 + 4 * (lane >> 4) + i;
      if (r < nr) ob[(c0 + r) * p.so_t + col] = to<T>(p.scale * Oa[i]);
    }

    // S = exp(gamma_C) S + Vn^T diag(exp(gamma_C - gamma)) K
    const float eC = fast_exp(gC);
#pragma unroll
    for (int u = 0; u < NTW; ++u) {
      const int nt = wave + 4 * u;
      f32x4 acc = S[u] * eC;
#pragma unroll
      for (int ks = 0; ks < BT / KS; ++ks)
        acc = MF::mma(frag_rows(sm.wdt, LDC, 0, ks * KS, lane), frag_cols(sm.k, LDK, ks * KS, 16 * nt, lane),
                      acc);
      S[u] = acc;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sm.s[(4 * (lane >> 4) + i) * LDK + 16 * nt + (lane & 15)] = to<T>(acc[i]);
    }
    __syncthreads();
  }

  if (p.final_state) {
#pragma unroll
    for (int u = 0; u < NTW; ++u) {
      const int nt = wave + 4 * u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * (lane >> 4) + i, c = 16 * nt + (lane & 15);
        p.final_state[st_base + (int64_t)row * DK + c] = S[u][i];
      }
    }
  }
}

template <typename T, int DK>
hipError_t launch_dk(const ChunkArgs &a, hipStream_t s) {
  dim3 grid((unsigned)(a.dv / DVT), (unsigned)a.Hv, (unsigned)a.n_seqs);
  hipLaunchKernelGGL((chunk_rule_kernel<T, DK>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const ChunkArgs &a, hipStream_t s) {
  switch (a.dk) {
    case 64: return launch_dk<T, 64>(a, s);
    case 128: return launch_dk<T, 128>(a, s);
    case 256:
      if constexpr (sizeof(T) == 2) return launch_dk<T, 256>(a, s);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool chunk_rule_supported(int64_t dk, int32_t act) {
  if (act == kF32) return dk == 64 || dk == 128;
  if (act == kBF16 || act == kF16) return dk == 64 || dk == 128 || dk == 256;
  return false;
}

hipError_t launch_chunk_rule(const ChunkArgs &a, hipStream_t s) {
  if (a.n_seqs == 0 || a.dv == 0) return hipSuccess;
  if (a.ws_rec && chunk_split_supported(a.dk, a.dv, a.act) && a.rows16 && a.o8) return launch_chunk_split(a, s);
  switch (a.act) {
    case kF32: return launch_t<float>(a, s);
    case kBF16: return launch_t<bf16>(a, s);
    case kF16: return launch_t<f16>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
