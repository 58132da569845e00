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
// fixed roles and one barrier per step. At step s:
//   wave 0  state(s):  K S^T, R, the triangular solve by 16 x 16 blocks, the
//                      state update; S lives in MFMA accumulators.
//   wave 1  prep(s+1): K K^T -> 1/|k| (its diagonal) and A; the four
//                      16 x 16 diagonal inverses (FP32, right-looking
//                      substitution, one lane per column); -A blocks.
//   wave 2  loads:     g, beta of chunk s+3 and their per-row factors (gamma
//                      scan, exponentials); then streams the k tile of chunk
//                      s+3 and the q, v tiles of chunk s+2 from HBM straight
//                      into LDS rings (global_load_lds, no registers). Copies
//                      issued at step s have retired before barrier s+2, which
//                      publishes them: a step of latency is hidden.
//   wave 3  out(s):    Q S^T and P^T = K Q^T for chunk s (P^T accumulators are
//                      exactly the A operands of P Vn); finishes o(s-1) with
//                      Vn(s-1) from wave 0.
// Ring sizes make sure no slot is overwritten while another wave reads it.
//
// Operand layouts. With v_mfma_f32_16x16x32, lane l = 16 g + c supplies 8 k
// values; an accumulator tile holds rows 4 g + i (i < 4) of column c. Two
// accumulator tiles (rows 16 t .. 16 t + 15, t = 2q, 2q + 1) therefore form
// one B operand whose k slots are {32q + 4g + i} then {32q + 16 + 4g + i},
// and every A operand used against it is read in that k order (two 8-byte
// LDS reads). q/k tiles are stored row-major with the 16-byte chunks of each
// row XOR-swizzled by the row index, which keeps these reads and the
// ds_read_b64_tr_b16 transposing reads (K^T fragments of the state update)
// free of bank conflicts.
#include "gdn_internal.h"
#include "mfma_tiles.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int BT = 64;
constexpr int DVT = 16;

enum { F_GAM = 0, F_BETA, F_EG, F_ECG, F_RK, F_MISC, F_N };

template <typename T, int DK>
struct Lds3 {
  static constexpr int RB = DK * 2;    // bytes per q/k row
  static constexpr int CPR = RB / 16;  // 16-byte chunks per row
  static constexpr int TILE = BT * RB;
  alignas(16) unsigned char k[4][TILE];  // k rows of chunk c in slot c % 4
  alignas(16) unsigned char q[3][TILE];  // q rows of chunk c in slot c % 3
  alignas(16) T v[3][BT * DVT];          // v slice, row-major [64][16]
  alignas(16) float adt[4][256];         // A_bb, FP32, column-major (wave 1 only)
  alignas(16) T ao[2][6][256];           // -A_ij (i > j), row-major 16 x 16
  alignas(16) T tii[2][4][256];          // (I + A_bb)^-1, row-major 16 x 16
  alignas(16) T sfrag[2][64 * (DK / 4)]; // state fragments per lane
  alignas(16) T wfrag[2][64 * 16];       // Vn fragments per lane
  alignas(16) float fac[4][F_N][BT];     // per-row factors of chunk c, slot c % 4
};

__device__ __forceinline__ int off_idx(int i, int j) { return i * (i - 1) / 2 + j; }

template <typename T, int DK>
__global__ __launch_bounds__(kThreads) void chunk_rule_v2_kernel(ChunkArgs p) {
  using MF = M2<T>;
  using f8 = typename MF::f8;
  using f4 = typename MF::f4;
  using v4 = typename MF::v4;
  using SM = Lds3<T, DK>;
  constexpr int KT = DK / 32;  // k-steps over dk
  constexpr int NT = DK / 16;  // 16-row tiles of dk
  constexpr int SF = DK / 4;   // state-fragment elements per lane
  constexpr int RB = SM::RB, CPR = SM::CPR;
  constexpr int NI = SM::TILE / 1024;  // 1 KB global_load_lds rounds per tile
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
  // Per-lane byte offsets inside a swizzled q/k tile (XOR of the 16-byte
  // chunk index with the row's low bits; rows 16 mt + c share c's bits):
  // fragment of row 16 mt + c, k-step pp, half h  ->  fo[pp][h] + mt * 16 RB.
  int fo[KT][2];
#pragma unroll
  for (int pp = 0; pp < KT; ++pp)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      fo[pp][hh] = c * RB + (((4 * pp + (g >> 1) + 2 * hh) ^ (c & (CPR - 1))) << 4) + 8 * (g & 1);
  // Steps s = -3 .. Nc, one barrier each, in every wave.
  if (wave == 0) {
    // ---------------------------------------------------------------- state
    // S[mt][i] = S[dv row c][dk 16 mt + 4 g + i], FP32 accumulators; Sf are
    // the act-dtype B fragments of S for the next K S^T.
    f32x4 S[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[mt][i] = p.init_state ? p.init_state[st_base + (int64_t)c * DK + 16 * mt + 4 * g + i] : 0.f;
    f8 Sf[KT];
#pragma unroll
    for (int pp = 0; pp < KT; ++pp) {
      Sf[pp] = cat8<T>(cvt4<T>(S[2 * pp]), cvt4<T>(S[2 * pp + 1]));
      *reinterpret_cast<f8 *>(&sm.sfrag[0][lane * SF + 8 * pp]) = Sf[pp];
    }
    // transposing-read offsets: row 32 q + 16 hh + 4 g + (c >> 2), columns
    // 16 mt + 4 (c & 3) .. + 3  ->  trb + trc[mt] + (32 q + 16 hh) RB
    const int yrow = (4 * g + (c >> 2)) & (CPR - 1);
    const int trb = (4 * g + (c >> 2)) * RB + 8 * (c & 1);
    int trc[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) trc[mt] = trb + (((2 * mt + ((c & 3) >> 1)) ^ yrow) << 4);
    for (int s = -3; s <= Nc; ++s) {
      lds_barrier();
      if (s < 0 || s >= Nc) continue;
      const unsigned char *kt = sm.k[s & 3];
      const int s2 = s & 1;
      const float *fa = &sm.fac[s & 3][0][0];
      // operands that do not depend on S: read them all first
      f8 kf[4][KT];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int pp = 0; pp < KT; ++pp)
          kf[mt][pp] = frag_at<T>(kt + mt * 16 * RB, fo[pp][0], fo[pp][1]);
      f32x4 be[4], aa[4], cw[4], vv[4];
      const T *vt = sm.v[s % 3];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int r0 = 16 * mt + 4 * g;
        be[mt] = *reinterpret_cast<const f32x4 *>(&fa[F_BETA * BT + r0]);
        const f32x4 eg = *reinterpret_cast<const f32x4 *>(&fa[F_EG * BT + r0]);
        const f32x4 ecg = *reinterpret_cast<const f32x4 *>(&fa[F_ECG * BT + r0]);
        const f32x4 rk = *reinterpret_cast<const f32x4 *>(&fa[F_RK * BT + r0]);
        aa[mt] = be[mt] * eg * rk;
        cw[mt] = ecg * rk;
#pragma unroll
        for (int i = 0; i < 4; ++i) vv[mt][i] = f(vt[(r0 + i) * DVT + c]);
      }
      const float eC = fa[F_MISC * BT];
      const T *ti = sm.tii[s2][0];
      const T *ao = sm.ao[s2][0];
      f4 tf[4], af[6];
#pragma unroll
      for (int b = 0; b < 4; ++b) tf[b] = *reinterpret_cast<const f4 *>(&ti[b * 256 + c * 16 + 4 * g]);
#pragma unroll
      for (int b = 0; b < 6; ++b) af[b] = *reinterpret_cast<const f4 *>(&ao[b * 256 + c * 16 + 4 * g]);
      // A fragments of K^T for the state update (transposing reads)
      f8 kt8[NT][2];
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const unsigned char *a1 = kt + trc[mt] + (32 * q) * RB;
          const unsigned char *a2 = kt + trc[mt] + (32 * q + 16) * RB;
          const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(a1));
          const s16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(a2));
          kt8[mt][q] = cat8<T>(__builtin_bit_cast(v4, r1), __builtin_bit_cast(v4, r2));
        }
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
      for (int mt = 0; mt < 4; ++mt) R[mt] = be[mt] * vv[mt] - aa[mt] * Y[mt];
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
      f8 Bw[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f8 wf = cat8<T>(cvt4<T>(W[2 * q]), cvt4<T>(W[2 * q + 1]));
        *reinterpret_cast<f8 *>(&sm.wfrag[s2][lane * 16 + 8 * q]) = wf;
        Bw[q] = cat8<T>(cvt4<T>(cw[2 * q] * W[2 * q]), cvt4<T>(cw[2 * q + 1] * W[2 * q + 1]));
      }
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) S[mt] = S[mt] * eC;
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) S[mt] = MF::k32(kt8[mt][q], Bw[q], S[mt]);
#pragma unroll
      for (int pp = 0; pp < KT; ++pp) {
        Sf[pp] = cat8<T>(cvt4<T>(S[2 * pp]), cvt4<T>(S[2 * pp + 1]));
        *reinterpret_cast<f8 *>(&sm.sfrag[s2 ^ 1][lane * SF + 8 * pp]) = Sf[pp];
      }
    }
    if (p.final_state) {
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) p.final_state[st_base + (int64_t)c * DK + 16 * mt + 4 * g + i] = S[mt][i];
    }
  } else if (wave == 1) {
    // ----------------------------------------------------------- prep(s + 1)
    for (int s = -3; s <= Nc; ++s) {
      lds_barrier();
      const int ch = s + 1;
      if (ch < 0 || ch >= Nc) continue;
      const int c2 = ch & 1;
      const unsigned char *kt = sm.k[ch & 3];
      float *fa = &sm.fac[ch & 3][0][0];
      f8 kf[4][KT];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int pp = 0; pp < KT; ++pp)
          kf[mt][pp] = frag_at<T>(kt + mt * 16 * RB, fo[pp][0], fo[pp][1]);
      // K K^T, lower tiles
      f32x4 acc[10];
#pragma unroll
      for (int t = 0; t < 10; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pp = 0; pp < KT; ++pp) {
        int t = 0;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni <= mi; ++ni, ++t) acc[t] = MF::k32(kf[mi][pp], kf[ni][pp], acc[t]);
      }
      // 1/|k| from the diagonal of K K^T: lane (g, c) with c >> 2 == g holds
      // |k_{16 mi + c}|^2 in element c & 3 of diagonal tile mi.
      if ((c >> 2) == g) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const f32x4 d = acc[mi * (mi + 1) / 2 + mi];
          const int e = c & 3;
          const float sq = e == 0 ? d[0] : e == 1 ? d[1] : e == 2 ? d[2] : d[3];
          fa[F_RK * BT + 16 * mi + c] = p.use_l2 ? rsqrtf(sq + p.l2_eps) : 1.f;
        }
      }
      lds_fence_wave();
      f32x4 gR[4], bR[4], kR[4];
      float gCol[4], kCol[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        gR[mi] = *reinterpret_cast<const f32x4 *>(&fa[F_GAM * BT + 16 * mi + 4 * g]);
        bR[mi] = *reinterpret_cast<const f32x4 *>(&fa[F_BETA * BT + 16 * mi + 4 * g]);
        kR[mi] = *reinterpret_cast<const f32x4 *>(&fa[F_RK * BT + 16 * mi + 4 * g]);
        gCol[mi] = fa[F_GAM * BT + 16 * mi + c];
        kCol[mi] = fa[F_RK * BT + 16 * mi + c];
      }
      T *ao = sm.ao[c2][0];
      int t = 0;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const f32x4 rowf = bR[mi] * kR[mi];
#pragma unroll
        for (int ni = 0; ni <= mi; ++ni, ++t) {
          const int col = 16 * ni + c;
          f32x4 av;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * mi + 4 * g + i;
            const float e = fast_exp(gR[mi][i] - gCol[ni]);
            av[i] = col < r ? rowf[i] * kCol[ni] * e * acc[t][i] : 0.f;
          }
          if (mi == ni) {
            *reinterpret_cast<f32x4 *>(&sm.adt[mi][c * 16 + 4 * g]) = av;  // column-major
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) ao[off_idx(mi, ni) * 256 + (4 * g + i) * 16 + c] = to<T>(-av[i]);
          }
        }
      }
      // (I + A_bb)^-1, lane = (block g, column c): right-looking substitution
      lds_fence_wave();
      {
        const float *adb = sm.adt[g];
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = r == c ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < 15; ++i) {
          f32x4 col4[4];
#pragma unroll
          for (int v = (i + 1) >> 2; v < 4; ++v) col4[v] = *reinterpret_cast<const f32x4 *>(&adb[i * 16 + 4 * v]);
#pragma unroll
          for (int r = i + 1; r < 16; ++r) x[r] -= col4[r >> 2][r & 3] * x[i];
        }
        T *ti = sm.tii[c2][g];
#pragma unroll
        for (int r = 0; r < 16; ++r) ti[r * 16 + c] = to<T>(x[r]);
      }
    }
  } else if (wave == 2) {
    // --------------------------------------------------- loads and factors
    for (int s = -3; s <= Nc; ++s) {
      lds_barrier();
      // factors of chunk s + 3 first: its g and beta come through ordinary
      // loads, whose wait also retires the tile copies issued one step ago
      const int cf = s + 3;
      if (cf < Nc) {
        const bool live = lane < rows_of(cf);
        const int64_t t = (int64_t)cf * BT + (live ? lane : 0);
        float gam = gb[t * p.sg_t];
        float bv = bb[t * p.sbt_t];
        gam = live ? gam : 0.f;
        bv = live ? bv : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float o = __shfl_up(gam, off, 64);
          if (lane >= off) gam += o;
        }
        const float gC = __shfl(gam, 63, 64);
        float *fa = &sm.fac[cf & 3][0][0];
        fa[F_GAM * BT + lane] = gam;
        fa[F_BETA * BT + lane] = bv;
        fa[F_EG * BT + lane] = fast_exp(gam);
        fa[F_ECG * BT + lane] = fast_exp(gC - gam);
        if (lane == 0) fa[F_MISC * BT] = fast_exp(gC);
      }
      // tile copies of the previous step must have landed before the next
      // barrier publishes them
      wait_vm<0>();
      const int ck = s + 3;  // k
      if (ck < Nc) {
        const int nr = rows_of(ck);
        const int64_t t0 = (int64_t)ck * BT;
        unsigned char *base = sm.k[ck & 3];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int b = 1024 * i + 16 * lane;
          const int r = b / RB, jp = (b % RB) >> 4;
          const int j = jp ^ (r & (CPR - 1));
          const int rr = r < nr ? r : nr - 1;
          g2l16(kb + (t0 + rr) * p.sk_t + 8 * j, base + 1024 * i);
        }
      }
      const int cq = s + 2;  // q, v
      if (cq >= 0 && cq < Nc) {
        const int nr = rows_of(cq);
        const int64_t t0 = (int64_t)cq * BT;
        const int sl = cq % 3;
        unsigned char *base = sm.q[sl];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int b = 1024 * i + 16 * lane;
          const int r = b / RB, jp = (b % RB) >> 4;
          const int j = jp ^ (r & (CPR - 1));
          const int rr = r < nr ? r : nr - 1;
          g2l16(qb + (t0 + rr) * p.sq_t + 8 * j, base + 1024 * i);
        }
        unsigned char *vbase = reinterpret_cast<unsigned char *>(sm.v[sl]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = 32 * i + (lane >> 1);
          const int rr = r < nr ? r : nr - 1;
          g2l16(vb + (t0 + rr) * p.sv_t + 8 * (lane & 1), vbase + 1024 * i);
        }
      }
    }
    wait_vm<0>();
  } else {
    // ------------------------------------------------- out(s), o(s - 1)
    f32x4 Zc[4];
    f8 Pf[6];
    for (int s = -3; s <= Nc; ++s) {
      lds_barrier();
      const int co = s - 1;
      if (co >= 0 && co < Nc) {
        const int nr = rows_of(co);
        f8 Wf[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) Wf[q] = *reinterpret_cast<const f8 *>(&sm.wfrag[co & 1][lane * 16 + 8 * q]);
        T *orow = ob + (int64_t)co * BT * p.so_t;
        int t = 0;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 o = Zc[mt];
#pragma unroll
          for (int q = 0; q <= mt / 2; ++q, ++t) o = MF::k32(Pf[t], Wf[q], o);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * mt + 4 * g + i;
            if (r < nr) orow[(int64_t)r * p.so_t + c] = to<T>(o[i]);
          }
        }
      }
      if (s < 0 || s >= Nc) continue;
      const unsigned char *qt = sm.q[s % 3];
      const unsigned char *kt = sm.k[s & 3];
      const float *fa = &sm.fac[s & 3][0][0];
      f8 qf[4][KT], kf[4][KT], Sf[KT];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int pp = 0; pp < KT; ++pp) {
          qf[mt][pp] = frag_at<T>(qt + mt * 16 * RB, fo[pp][0], fo[pp][1]);
          kf[mt][pp] = frag_at<T>(kt + mt * 16 * RB, fo[pp][0], fo[pp][1]);
        }
#pragma unroll
      for (int pp = 0; pp < KT; ++pp) Sf[pp] = *reinterpret_cast<const f8 *>(&sm.sfrag[s & 1][lane * SF + 8 * pp]);
      f32x4 gRow[4], egRow[4], kK[4];
      float gC4[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        gRow[m] = *reinterpret_cast<const f32x4 *>(&fa[F_GAM * BT + 16 * m + 4 * g]);
        egRow[m] = *reinterpret_cast<const f32x4 *>(&fa[F_EG * BT + 16 * m + 4 * g]);
        kK[m] = *reinterpret_cast<const f32x4 *>(&fa[F_RK * BT + 16 * m + 4 * g]);
        gC4[m] = fa[F_GAM * BT + 16 * m + c];
      }
      // 1/|q| of rows 16 mt + c
      float rq[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        float ssq = 0.f;
#pragma unroll
        for (int pp = 0; pp < KT; ++pp) ssq = sumsq8<T>(qf[mt][pp], ssq);
        ssq += __shfl_xor(ssq, 16, 64);
        ssq += __shfl_xor(ssq, 32, 64);
        rq[mt] = p.use_l2 ? rsqrtf(ssq + p.l2_eps) : 1.f;
      }
      // Z = Q S^T, scaled by scale exp(gamma_r) rq_r (rows 16 mt + 4 g + i)
      f32x4 z[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) z[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pp = 0; pp < KT; ++pp)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) z[mt] = MF::k32(qf[mt][pp], Sf[pp], z[mt]);
      // P^T tiles (ni <= mi): lane holds q_{16 mi + c} . k_{16 ni + 4 g + i}
      f32x4 pt[10];
#pragma unroll
      for (int t = 0; t < 10; ++t) pt[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pp = 0; pp < KT; ++pp) {
        int t = 0;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni <= mi; ++ni, ++t) pt[t] = MF::k32(kf[ni][pp], qf[mi][pp], pt[t]);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float rqr = __shfl(rq[mt], 4 * g + i, 64);
          Zc[mt][i] = p.scale * egRow[mt][i] * rqr * z[mt][i];
        }
      // P[r, i] = scale exp(gamma_r - gamma_i) rq_r rk_i (q_r . k_i), i <= r,
      // r = 16 mi + c, i = 16 ni + 4 g + j; packed as A fragments of P Vn.
      f32x4 pv[10];
      {
        int t = 0;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const float rowf = p.scale * rq[mi];
#pragma unroll
          for (int ni = 0; ni <= mi; ++ni, ++t) {
            const int r = 16 * mi + c;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int i = 16 * ni + 4 * g + j;
              const float e = fast_exp(gC4[mi] - gRow[ni][j]);
              pv[t][j] = i <= r ? rowf * kK[ni][j] * e * pt[t][j] : 0.f;
            }
          }
        }
      }
      auto tix = [](int mi, int ni) { return mi * (mi + 1) / 2 + ni; };
      const v4 z4 = cvt4<T>(f32x4{0.f, 0.f, 0.f, 0.f});
      {
        int t = 0;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int q = 0; q <= mt / 2; ++q, ++t) {
            const v4 lo = cvt4<T>(pv[tix(mt, 2 * q)]);
            const v4 hi = (2 * q + 1 <= mt) ? cvt4<T>(pv[tix(mt, 2 * q + 1)]) : z4;
            Pf[t] = cat8<T>(lo, hi);
          }
      }
    }
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
