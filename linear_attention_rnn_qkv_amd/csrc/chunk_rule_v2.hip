// Chunked gated delta rule, software-pipelined across wavefronts (16-bit
// inputs, dk in {64, 128}).
//
// Same mathematics as the basic kernel in chunk_rule.hip (the gated delta rule
// of Gated DeltaNet in its chunked WY / UT form, q/k L2 normalisation folded
// in as in the Megatron-LM pull request "fold q/k L2-norm into the
// gated_delta_rule kernel"), scheduled differently. For a chunk of 64 rows
// entering with state S0 (dv x dk):
//   gamma = cumsum(g);  rk, rq = inverse L2 norms of the k and q rows
//   A[r,i] = beta_r exp(gamma_r - gamma_i) rk_r rk_i (k_r . k_i),   i < r
//   Vn = (I + A)^-1 R,   R = beta (.) V - (beta exp(gamma) rk) (.) (K S0^T)
//   O  = (scale exp(gamma) rq) (.) (Q S0^T) + P Vn,
//        P[r,i] = scale exp(gamma_r - gamma_i) rq_r rk_i (q_r . k_i), i <= r
//   S  = exp(gamma_C) S0 + (K^T) ((exp(gamma_C - gamma) rk) (.) Vn)
// q and k are used raw (exactly as stored); the norms enter as row factors.
//
// One workgroup = (sequence, value head, 16 rows of dv), four wavefronts with
// fixed roles, one barrier per step. At step s:
//   wave 0  state(s):   K S^T, R, the triangular solve by 16 x 16 blocks
//                       (diagonal inverses from wave 3, -A blocks from wave 1),
//                       the state update; S lives in MFMA accumulators.
//   wave 1  prep(s+2):  loads k, g, beta; norms, gamma and row factors; K K^T
//                       -> A (FP32 diagonal blocks, act-dtype -A blocks);
//                       stores the k rows for waves 0 and 2.
//   wave 2  prep(s+1):  loads q and the v slice; norms; Q K^T -> P.
//   wave 3  inv(s+1):   (I + A_bb)^-1 of the four diagonal blocks (FP32
//                       forward substitution, one lane per column);
//           out(s-1):   Q S^T and P Vn -> o.
// Every hand-off crosses at least one barrier; ring buffers in LDS are sized
// so that no slot is written while another wave reads it.
//
// Operand layouts. With v_mfma_f32_16x16x32, lane l = 16 g + c supplies 8 k
// values; an accumulator tile holds rows 4 g + i (i < 4) of column c. Two
// accumulator tiles (rows 16 t .. 16 t + 15, t = 2q, 2q + 1) therefore form
// one B operand whose k slots are {32q + 4g + i} then {32q + 16 + 4g + i}.
// Every matrix used against such an operand is stored in LDS with its k
// columns permuted to that order (pcol below), so one 16-byte read yields a
// matching A fragment. The state update contracts K over chunk rows; its A
// fragments come straight from the row-major k tile through two
// ds_read_b64_tr_b16 transposing reads.
#include "device_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int BT = 64;
constexpr int DVT = 16;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <typename T> struct M2;
template <> struct M2<bf16> {
  typedef bf16x8 f8;
  typedef bf16x4 v4;
  typedef s16x4 f4;  // K16 operand
  static __device__ __forceinline__ f32x4 k32(f8 a, f8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 k16(f4 a, f4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f4 as_f4(v4 x) { return __builtin_bit_cast(s16x4, x); }
};
template <> struct M2<f16> {
  typedef f16x8 f8;
  typedef f16x4 v4;
  typedef f16x4 f4;
  static __device__ __forceinline__ f32x4 k32(f8 a, f8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 k16(f4 a, f4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f4 as_f4(v4 x) { return x; }
};

// Storage column of logical column x inside rows whose k order is permuted
// per 32-block: logical 4a + i -> 8a + i, logical 16 + 4a + i -> 8a + 4 + i.
__device__ __forceinline__ int pcol(int x) {
  const int xi = x & 31;
  return (x & ~31) + ((xi & 15) >> 2) * 8 + ((xi >> 4) << 2) + (xi & 3);
}

enum { F_GAM = 0, F_BETA, F_RK, F_RQ, F_A, F_CW, F_BQ, F_MISC, F_N };

template <typename T, int DK>
struct Lds2 {
  static constexpr int LDK = DK + 8;  // k rows (dk columns, permuted)
  static constexpr int LDP = BT + 8;  // P rows (chunk columns, permuted)
  static constexpr int LDV = BT + 8;  // V^T rows
  alignas(16) T k[3][BT * LDK];
  alignas(16) T p[3][BT * LDP];
  alignas(16) T vt[2][DVT * LDV];
  alignas(16) T ao[3][6][256];        // -A_ij, i > j, row-major 16 x 16
  alignas(16) T tii[2][4][256];       // (I + A_bb)^-1, row-major 16 x 16
  alignas(16) T sfrag[2][64 * (DK / 4)];
  alignas(16) T wfrag[2][64 * 16];
  alignas(16) float ad[3][4][256];    // A_bb, FP32, row-major 16 x 16
  alignas(16) float fac[4][F_N][BT];  // per-row factors of a chunk
};

__device__ __forceinline__ int off_idx(int i, int j) { return i * (i - 1) / 2 + j; }

// Workgroup barrier for LDS hand-offs only. Waves exchange data through LDS
// alone, so each wave waits for its own LDS accesses (lgkmcnt 0) and then
// meets the others; outstanding global loads (prefetches for later steps) and
// stores (outputs) stay in flight across the barrier. The memory clobber keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Keeps the global loads issued above it (prefetches for the next step) from
// being scheduled below it, so they are in flight during this step's work.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

template <typename T>
__device__ __forceinline__ typename M2<T>::f8 cat8(typename M2<T>::v4 a, typename M2<T>::v4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <typename T>
__device__ __forceinline__ typename M2<T>::v4 cvt4(f32x4 x) {
  return __builtin_convertvector(x, typename M2<T>::v4);
}

// Rows [0, nr) of a chunk (row stride st, elements, nr >= 1) into fragments
// with the permuted k order: fr[mt][p] = row 16 mt + c, k slots 32p + 4g + i
// and 32p + 16 + 4g + i. Rows beyond nr repeat row nr - 1 (in bounds, no
// branches, no use of the data at issue time). Such padding rows are inert:
// their beta and g are zero, so their rows of A, R and Vn vanish, a padding
// column only meets valid rows above the diagonal (masked), and their
// outputs are not stored.
template <typename T, int KT>
__device__ __forceinline__ void load_rows(typename M2<T>::f8 (&fr)[4][KT], const T *base, int64_t st,
                                          int nr, int g, int c) {
  using f8 = typename M2<T>::f8;
  struct Pair {
    uint2 lo, hi;
  };
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int row = 16 * mt + c;
    const T *rp = base + (int64_t)(row < nr ? row : nr - 1) * st;
#pragma unroll
    for (int pp = 0; pp < KT; ++pp) {
      Pair v;
      v.lo = *reinterpret_cast<const uint2 *>(rp + 32 * pp + 4 * g);
      v.hi = *reinterpret_cast<const uint2 *>(rp + 32 * pp + 16 + 4 * g);
      fr[mt][pp] = __builtin_bit_cast(f8, v);
    }
  }
}

// Row sums of squares of fragments (row 16 mt + c), summed over the 4 groups.
template <typename T, int KT>
__device__ __forceinline__ void row_sumsq(const typename M2<T>::f8 (&fr)[4][KT], float (&ss)[4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    float s = 0.f;
#pragma unroll
    for (int pp = 0; pp < KT; ++pp)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = f(fr[mt][pp][j]);
        s += x * x;
      }
    s += __shfl_xor(s, 16, 64);
    s += __shfl_xor(s, 32, 64);
    ss[mt] = s;
  }
}

__device__ __forceinline__ float pick4(const float (&v)[4], int i) {
  return i == 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : v[3];
}

template <typename T, int DK>
__global__ __launch_bounds__(kThreads) void chunk_rule_v2_kernel(ChunkArgs p) {
  using MF = M2<T>;
  using f8 = typename MF::f8;
  using f4 = typename MF::f4;
  using v4 = typename MF::v4;
  using SM = Lds2<T, DK>;
  constexpr int KT = DK / 32;  // k-steps over dk
  constexpr int NT = DK / 16;  // 16-row tiles of dk
  constexpr int LDK = SM::LDK, LDP = SM::LDP, LDV = SM::LDV;
  constexpr int SF = DK / 4;   // state-fragment elements per lane
  typedef f8 Frags[4][KT];
  __shared__ SM sm;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  // Workgroups are dispatched round-robin over the 8 XCDs by linear id. Remap
  // so that the dv slices of one head (which read the same q/k tiles) run on
  // one XCD and share its L2.
  const int64_t ntile = gridDim.x, nwg = (int64_t)gridDim.x * gridDim.y * gridDim.z;
  int64_t lid = blockIdx.x + ntile * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
  if (nwg % 8 == 0) lid = (lid % 8) * (nwg / 8) + lid / 8;
  const int64_t j0 = (lid % ntile) * DVT;
  const int64_t h = (lid / ntile) % gridDim.y;
  const int64_t n = lid / (ntile * gridDim.y);
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
  const int64_t L = eos - bos;
  const int Nc = (int)((L + BT - 1) / BT);
  const T *qb = static_cast<const T *>(p.q) + brow * p.sq_b + hk * p.sq_h + bos * p.sq_t;
  const T *kb = static_cast<const T *>(p.k) + brow * p.sk_b + hk * p.sk_h + bos * p.sk_t;
  const T *vb = static_cast<const T *>(p.v) + brow * p.sv_b + h * p.sv_h + j0 + bos * p.sv_t;
  const float *gb = p.g + brow * p.sg_b + h * p.sg_h + bos * p.sg_t;
  const float *bb = p.beta + brow * p.sbt_b + h * p.sbt_h + bos * p.sbt_t;
  T *ob = static_cast<T *>(p.o) + brow * p.so_b + h * p.so_h + j0 + bos * p.so_t;
  const int64_t st_base = ((n * p.Hv + h) * p.dv + j0) * DK;
  auto rows_of = [&](int ch) -> int {
    const int64_t r = L - (int64_t)ch * BT;
    return (int)(r < BT ? r : BT);
  };
  // Steps s = -2 .. Nc; every wave runs them all (one barrier each). Roles
  // with prefetched operands alternate between two register buffers so that
  // the loads for the next step land directly where that step reads them.
  auto run_steps = [&](auto &&step) {
    int s = -2;
    for (; s + 1 <= Nc; s += 2) {
      step(s, 0);
      step(s + 1, 1);
    }
    if (s <= Nc) step(s, 0);
  };

  if (wave == 0) {
    // ---------------------------------------------------------------- state
    // S[mt][i] = S[dv row c][dk 16 mt + 4 g + i], FP32 accumulators.
    f32x4 S[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[mt][i] = p.init_state ? p.init_state[st_base + (int64_t)c * DK + 16 * mt + 4 * g + i] : 0.f;
    run_steps([&](int s, int) {
      lds_barrier();
      if (s < 0 || s >= Nc) return;
      const int k3 = s % 3, k2 = s & 1, k4 = s & 3;
      const T *kt = sm.k[k3];
      const float *fa = &sm.fac[k4][0][0];
      // operands that do not depend on S: read them all first
      Frags kf;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int pp = 0; pp < KT; ++pp)
          kf[mt][pp] = *reinterpret_cast<const f8 *>(&kt[(16 * mt + c) * LDK + 32 * pp + 8 * g]);
      v4 vv[4];
      f32x4 be[4], aa[4], cw[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int r0 = 16 * mt + 4 * g;
        vv[mt] = *reinterpret_cast<const v4 *>(&sm.vt[k2][c * LDV + r0]);
        be[mt] = *reinterpret_cast<const f32x4 *>(&fa[F_BETA * BT + r0]);
        aa[mt] = *reinterpret_cast<const f32x4 *>(&fa[F_A * BT + r0]);
        cw[mt] = *reinterpret_cast<const f32x4 *>(&fa[F_CW * BT + r0]);
      }
      const float eC = fa[F_MISC * BT];
      const T *ti = sm.tii[k2][0];
      const T *ao = sm.ao[k3][0];
      f4 tf[4], af[6];
#pragma unroll
      for (int b = 0; b < 4; ++b) tf[b] = *reinterpret_cast<const f4 *>(&ti[b * 256 + c * 16 + 4 * g]);
#pragma unroll
      for (int b = 0; b < 6; ++b) af[b] = *reinterpret_cast<const f4 *>(&ao[b * 256 + c * 16 + 4 * g]);
      // A fragments of K^T for the state update (transposing reads)
      f8 kt8[NT][2];
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        const int colst = pcol(16 * mt + 4 * (c & 3));
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const T *a1 = &kt[(32 * q + 4 * g + (c >> 2)) * LDK + colst];
          const T *a2 = &kt[(32 * q + 16 + 4 * g + (c >> 2)) * LDK + colst];
          const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<T *>(a1));
          const s16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<T *>(a2));
          kt8[mt][q] = cat8<T>(__builtin_bit_cast(v4, r1), __builtin_bit_cast(v4, r2));
        }
      }
      // state fragments (also handed to the output wave)
      f8 Sf[KT];
#pragma unroll
      for (int pp = 0; pp < KT; ++pp) Sf[pp] = cat8<T>(cvt4<T>(S[2 * pp]), cvt4<T>(S[2 * pp + 1]));
#pragma unroll
      for (int pp = 0; pp < KT; ++pp) *reinterpret_cast<f8 *>(&sm.sfrag[k2][lane * SF + 8 * pp]) = Sf[pp];
      // Y = K S^T (four independent accumulators)
      f32x4 Y[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) Y[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pp = 0; pp < KT; ++pp)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) Y[mt] = MF::k32(kf[mt][pp], Sf[pp], Y[mt]);
      f32x4 R[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) R[mt][i] = be[mt][i] * f(vv[mt][i]) - aa[mt][i] * Y[mt][i];
      // Vn = (I + A)^-1 R by 16-row blocks
      const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
      f32x4 W[4];
      W[0] = MF::k16(tf[0], MF::as_f4(cvt4<T>(R[0])), zero4);
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        f32x4 x = R[i];
#pragma unroll
        for (int j = 0; j < i; ++j) x = MF::k16(af[off_idx(i, j)], MF::as_f4(cvt4<T>(W[j])), x);
        W[i] = MF::k16(tf[i], MF::as_f4(cvt4<T>(x)), zero4);
      }
      f8 Bw[2], Wf[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        Wf[q] = cat8<T>(cvt4<T>(W[2 * q]), cvt4<T>(W[2 * q + 1]));
        Bw[q] = cat8<T>(cvt4<T>(cw[2 * q] * W[2 * q]), cvt4<T>(cw[2 * q + 1] * W[2 * q + 1]));
      }
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) S[mt] = S[mt] * eC;
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) S[mt] = MF::k32(kt8[mt][q], Bw[q], S[mt]);
#pragma unroll
      for (int q = 0; q < 2; ++q) *reinterpret_cast<f8 *>(&sm.wfrag[k2][lane * 16 + 8 * q]) = Wf[q];
    });
    if (p.final_state) {
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) p.final_state[st_base + (int64_t)c * DK + 16 * mt + 4 * g + i] = S[mt][i];
    }
  } else if (wave == 1) {
    // --------------------------------------------------------- prep(s + 2): k
    Frags kbuf[2];
    float gbuf[2], bbuf[2];
    auto load_k = [&](int ch, int slot) {
      const int nr = rows_of(ch);
      const int64_t t0 = (int64_t)ch * BT;
      load_rows<T, KT>(kbuf[slot], kb + t0 * p.sk_t, p.sk_t, nr, g, c);
      const int lr = lane < nr ? lane : nr - 1;
      gbuf[slot] = gb[(t0 + lr) * p.sg_t];  // rows >= nr are zeroed at use
      bbuf[slot] = bb[(t0 + lr) * p.sbt_t];
    };
    if (Nc > 0) load_k(0, 0);
    run_steps([&](int s, int par) {
      lds_barrier();
      const int ch = s + 2;
      if (ch >= Nc) return;
      if (ch + 1 < Nc) load_k(ch + 1, par ^ 1);
      issue_fence();
      Frags &cur = kbuf[par];
      const bool live = lane < rows_of(ch);
      const float bv = live ? bbuf[par] : 0.f;
      const int k3 = ch % 3, k4 = ch & 3;
      float ss[4], rk[4];
      row_sumsq<T, KT>(cur, ss);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) rk[mt] = p.use_l2 ? rsqrtf(ss[mt] + p.l2_eps) : 1.f;
      float gam = live ? gbuf[par] : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(gam, off, 64);
        if (lane >= off) gam += o;
      }
      const float gC = __shfl(gam, 63, 64);
      const float rko = pick4(rk, g);  // row `lane`
      // factors of the rows this lane's accumulators hold (16 mi + 4 g + i)
      // and of its columns (16 ni + c)
      float gR[4][4], bR[4][4], kR[4][4], gCol[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * mi + 4 * g + i;
          gR[mi][i] = __shfl(gam, r, 64);
          bR[mi][i] = __shfl(bv, r, 64);
          kR[mi][i] = __shfl(rk[mi], 4 * g + i, 64);
        }
        gCol[mi] = __shfl(gam, 16 * mi + c, 64);
      }
      f32x4 acc[10];
#pragma unroll
      for (int t = 0; t < 10; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pp = 0; pp < KT; ++pp) {
        int t = 0;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni <= mi; ++ni, ++t) acc[t] = MF::k32(cur[mi][pp], cur[ni][pp], acc[t]);
      }
      float *fa = &sm.fac[k4][0][0];
      fa[F_GAM * BT + lane] = gam;
      fa[F_BETA * BT + lane] = bv;
      fa[F_RK * BT + lane] = rko;
      fa[F_A * BT + lane] = bv * fast_exp(gam) * rko;
      fa[F_CW * BT + lane] = fast_exp(gC - gam) * rko;
      if (lane == 0) fa[F_MISC * BT] = fast_exp(gC);
      T *kt = sm.k[k3];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int pp = 0; pp < KT; ++pp)
          *reinterpret_cast<f8 *>(&kt[(16 * mt + c) * LDK + 32 * pp + 8 * g]) = cur[mt][pp];
      int t = 0;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni <= mi; ++ni, ++t) {
          const int col = 16 * ni + c;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * mi + 4 * g + i;
            const float av =
                col < r ? bR[mi][i] * fast_exp(fminf(gR[mi][i] - gCol[ni], 0.f)) * kR[mi][i] * rk[ni] * acc[t][i]
                        : 0.f;
            if (mi == ni) sm.ad[k3][mi][(4 * g + i) * 16 + c] = av;
            else sm.ao[k3][off_idx(mi, ni)][(4 * g + i) * 16 + c] = to<T>(-av);
          }
        }
    });
  } else if (wave == 2) {
    // ------------------------------------------------------ prep(s + 1): q, v
    Frags qbuf[2];
    uint2 vbuf[2][4];
    auto load_q = [&](int ch, int slot) {
      const int nr = rows_of(ch);
      const int64_t t0 = (int64_t)ch * BT;
      load_rows<T, KT>(qbuf[slot], qb + t0 * p.sq_t, p.sq_t, nr, g, c);
      const int lr = lane < nr ? lane : nr - 1;
      const T *vr = vb + (t0 + lr) * p.sv_t;
#pragma unroll
      for (int i = 0; i < 4; ++i) vbuf[slot][i] = *reinterpret_cast<const uint2 *>(vr + 4 * i);
    };
    run_steps([&](int s, int par) {
      lds_barrier();
      const int ch = s + 1;
      if (ch >= Nc) return;
      if (ch + 1 < Nc) load_q(ch + 1, par ^ 1);
      issue_fence();
      if (ch < 0) return;
      Frags &cur = qbuf[par];
      const int k3 = ch % 3, k2 = ch & 1, k4 = ch & 3;
      float *fa = &sm.fac[k4][0][0];
      const T *kt = sm.k[k3];
      // LDS operands first: k fragments, gamma and 1/|k| of rows and columns
      Frags kf;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int pp = 0; pp < KT; ++pp)
          kf[mt][pp] = *reinterpret_cast<const f8 *>(&kt[(16 * mt + c) * LDK + 32 * pp + 8 * g]);
      f32x4 gR[4];
      float gCol[4], kCol[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        gR[mi] = *reinterpret_cast<const f32x4 *>(&fa[F_GAM * BT + 16 * mi + 4 * g]);
        gCol[mi] = fa[F_GAM * BT + 16 * mi + c];
        kCol[mi] = fa[F_RK * BT + 16 * mi + c];
      }
      const float gOwn = fa[F_GAM * BT + lane];
      float ss[4], rq[4];
      row_sumsq<T, KT>(cur, ss);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) rq[mt] = p.use_l2 ? rsqrtf(ss[mt] + p.l2_eps) : 1.f;
      float qR[4][4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) qR[mi][i] = __shfl(rq[mi], 4 * g + i, 64);
      f32x4 acc[10];
#pragma unroll
      for (int t = 0; t < 10; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pp = 0; pp < KT; ++pp) {
        int t = 0;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni <= mi; ++ni, ++t) acc[t] = MF::k32(cur[mi][pp], kf[ni][pp], acc[t]);
      }
      // writes: v slice (transposed), factors, P
      {
        T vv[16];
        __builtin_memcpy(vv, vbuf[par], sizeof vv);
#pragma unroll
        for (int j = 0; j < 16; ++j) sm.vt[k2][j * LDV + lane] = vv[j];
      }
      const float rqo = pick4(rq, g);
      fa[F_RQ * BT + lane] = rqo;
      fa[F_BQ * BT + lane] = p.scale * fast_exp(gOwn) * rqo;
      T *pm = sm.p[k3];
      int t = 0;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni <= mi; ++ni, ++t) {
          const int col = 16 * ni + c;
          const int pc = pcol(col);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * mi + 4 * g + i;
            const float pv =
                col <= r ? p.scale * fast_exp(fminf(gR[mi][i] - gCol[ni], 0.f)) * qR[mi][i] * kCol[ni] * acc[t][i]
                         : 0.f;
            pm[r * LDP + pc] = to<T>(pv);
          }
        }
      // upper tiles read by the 32-wide k steps: (0, 1) and (2, 3)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pm[(4 * g + i) * LDP + pcol(16 + c)] = to<T>(0.f);
        pm[(32 + 4 * g + i) * LDP + pcol(48 + c)] = to<T>(0.f);
      }
    });
  } else {
    // -------------------------------------------- inv(s + 1), out(s - 1)
    Frags qbuf[2];
    run_steps([&](int s, int par) {
      lds_barrier();
      if (s >= 0 && s < Nc)
        load_rows<T, KT>(qbuf[par ^ 1], qb + (int64_t)s * BT * p.sq_t, p.sq_t, rows_of(s), g, c);
      issue_fence();
      const int ci = s + 1;
      if (ci >= 0 && ci < Nc) {
        // forward substitution, lane = (block g, column c); rows read as
        // float4 vectors, four rows at a time
        const float *ad = sm.ad[ci % 3][g];
        float x[16];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          f32x4 arow[4][4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int v = 0; v <= rb; ++v)
              arow[rr][v] = *reinterpret_cast<const f32x4 *>(&ad[(4 * rb + rr) * 16 + 4 * v]);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int r = 4 * rb + rr;
            float acc = r == c ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) acc -= arow[rr][i >> 2][i & 3] * x[i];
            x[r] = acc;
          }
        }
        T *ti = sm.tii[ci & 1][g];
#pragma unroll
        for (int r = 0; r < 16; ++r) ti[r * 16 + c] = to<T>(x[r]);
      }
      const int co = s - 1;
      if (co < 0 || co >= Nc) return;
      Frags &cur = qbuf[par];  // q rows of chunk co, loaded one step ago
      const int k3 = co % 3, k2 = co & 1, k4 = co & 3;
      const int nr = rows_of(co);
      const float *fa = &sm.fac[k4][0][0];
      const T *pm = sm.p[k3];
      f8 Sf[KT], Wf[2], pf[6];
      f32x4 bq[4];
#pragma unroll
      for (int pp = 0; pp < KT; ++pp) Sf[pp] = *reinterpret_cast<const f8 *>(&sm.sfrag[k2][lane * SF + 8 * pp]);
#pragma unroll
      for (int q = 0; q < 2; ++q) Wf[q] = *reinterpret_cast<const f8 *>(&sm.wfrag[k2][lane * 16 + 8 * q]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) bq[mt] = *reinterpret_cast<const f32x4 *>(&fa[F_BQ * BT + 16 * mt + 4 * g]);
      {
        int t = 0;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int q = 0; q <= mt / 2; ++q, ++t)
            pf[t] = *reinterpret_cast<const f8 *>(&pm[(16 * mt + c) * LDP + 32 * q + 8 * g]);
      }
      f32x4 z[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) z[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pp = 0; pp < KT; ++pp)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) z[mt] = MF::k32(cur[mt][pp], Sf[pp], z[mt]);
      T *orow = ob + (int64_t)co * BT * p.so_t;
      int t = 0;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 o = bq[mt] * z[mt];
#pragma unroll
        for (int q = 0; q <= mt / 2; ++q, ++t) o = MF::k32(pf[t], Wf[q], o);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * mt + 4 * g + i;
          if (r < nr) orow[(int64_t)r * p.so_t + c] = to<T>(o[i]);
        }
      }
    });
  }
}

template <typename T, int DK>
hipError_t launch_dk(const ChunkArgs &a, hipStream_t s) {
  dim3 grid((unsigned)(a.dv / DVT), (unsigned)a.Hv, (unsigned)a.n_seqs);
  hipLaunchKernelGGL((chunk_rule_v2_kernel<T, DK>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool chunk_rule_v2_supported(int64_t dk, int32_t act) {
  return (act == kBF16 || act == kF16) && (dk == 64 || dk == 128);
}

hipError_t launch_chunk_rule_v2(const ChunkArgs &a, hipStream_t s) {
  if (a.n_seqs == 0 || a.dv == 0) return hipSuccess;
  if (a.act == kBF16) return a.dk == 64 ? launch_dk<bf16, 64>(a, s) : launch_dk<bf16, 128>(a, s);
  if (a.act == kF16) return a.dk == 64 ? launch_dk<f16, 64>(a, s) : launch_dk<f16, 128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace gdn
