// Chunk state: the state-dependent half of the chunked gated delta rule,
// serial over the chunks of a sequence. With the per-chunk record written by
// the chunk-prep kernel (T' = (I + A)^-1 diag(beta), P and row factors aa,
// cw, zc, e^{gamma_C}; see chunk_prep.hip), a chunk of 64 rows entering with
// state S0 (dv x dk, FP32) gives
//
//   X = K S0^T,   Vn = T' V - T' (aa (.) X)
//   O = zc (.) (Q S0^T) + P Vn          (computed transposed, O^T)
//   S = e^{gamma_C} S0 + K^T (cw (.) Vn)
//
// (the WY/UT form of the gated delta rule; q and k are used raw, their
// inverse norms are inside the factors).
//
// One workgroup = (sequence, value head, 16 rows of dv) with eight
// wavefronts and one barrier per step s:
//   wave 0  chain(s): U, X, Vn, the state update; S lives in MFMA
//           accumulators; Vn and the next S are handed over as fragments.
//   wave 1  out(s):   (Q S0^T)^T for chunk s and, with Vn(s - 1), finishes
//                     o(s - 1) transposed, so that each lane stores 4
//                     consecutive dv values of a row (8-byte stores).
//   waves 2-7 loads:  stream the k, q, v tiles and the record of chunk s + 2
//                     into three-slot LDS rings (global_load_lds); the copies
//                     of a step are complete before the barrier that ends the
//                     next step, so two steps of latency are hidden.
#include "gdn_internal.h"
#include "mfma_tiles.h"

namespace gdn {
namespace {

constexpr int kStateThreads = 512;
constexpr int BT = 64;
constexpr int DVT = 16;

template <typename T, int DK>
struct StateLds {
  static constexpr int RB = DK * 2;
  static constexpr int CPR = RB / 16;
  static constexpr int TILE = BT * RB;
  alignas(16) unsigned char k[3][TILE];      // k rows of chunk c in slot c % 3 (swizzled)
  alignas(16) unsigned char q[3][TILE];      // q rows
  alignas(16) T v[3][BT * DVT];              // v slice, row-major [64][16]
  alignas(16) unsigned char rec[3][kRecBytes];
  alignas(16) T sfrag[2][64 * (DK / 4)];     // state fragments per lane
  alignas(16) T wfrag[2][64 * 16];           // Vn fragments per lane
};

// The dk axis of the state tiles is permuted so that every MFMA operand
// fragment over dk is one contiguous 16-byte run: accumulator tile mt = 2 pp + h,
// row 4 g + i holds dk 32 pp + 8 g + 4 h + i. The state fragment of k step pp
// (tiles 2 pp and 2 pp + 1 side by side) then covers dk 32 pp + 8 g .. + 7 in
// lane group g, matching one 16-byte read of a k or q row.
__device__ __forceinline__ constexpr int dk_of(int mt, int r) {
  return 32 * (mt >> 1) + 8 * (r >> 2) + 4 * (mt & 1) + (r & 3);
}

// fragment index of (row tile mt, k pair q) in a record matrix
__device__ __forceinline__ constexpr int frag_id(int mt, int q) { return q == 0 ? mt : 2 + mt; }

template <int N> struct Slot { static constexpr int v = N; };

// Runs body(s, Slot<s mod 3>) for s = -2 .. last in order: the ring slot of
// chunk s is a compile-time constant in every call, so LDS addresses are
// loop-invariant.
template <typename F>
__device__ __forceinline__ void for_steps(int last, F &&body) {
  for (int base = -3; base <= last; base += 3) {
    if (base >= -2) body(base, Slot<0>{});
    if (base + 1 >= -2 && base + 1 <= last) body(base + 1, Slot<1>{});
    if (base + 2 <= last) body(base + 2, Slot<2>{});
  }
}

template <typename T, int DK>
__global__ __launch_bounds__(kStateThreads) void chunk_state_kernel(ChunkArgs p) {
  using MF = M2<T>;
  using f8 = typename MF::f8;
  using v4 = typename MF::v4;
  using SM = StateLds<T, DK>;
  constexpr int KT = DK / 32;
  constexpr int NT = DK / 16;
  constexpr int SF = DK / 4;
  constexpr int RB = SM::RB;
  constexpr int NI = SM::TILE / 1024;          // 1 KB copies per q/k tile
  constexpr int NR = (int)(kRecBytes / 1024);  // 1 KB copies per record
  static_assert(NI % 2 == 0 && NR % 2 == 0 && NI / 2 <= 31 && NR / 2 + 1 <= 31, "copy split");
  __shared__ SM sm;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  // The dv slices of one head (which read the same q/k tiles and records) are
  // placed on one XCD so that they share its L2.
  const int64_t ntile = gridDim.x, nwg = (int64_t)gridDim.x * gridDim.y * gridDim.z;
  int64_t lid = blockIdx.x + ntile * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
  if (nwg % 8 == 0) lid = (lid % 8) * (nwg / 8) + lid / 8;
  const int64_t j0 = (lid % ntile) * DVT;
  const int64_t h = (lid / ntile) % gridDim.y;
  const int64_t n = lid / (ntile * gridDim.y);
  const int64_t hk = h / (p.Hv / p.Hqk);
  int64_t bos, eos, brow, cbase;
  if (p.cu_seqlens) {
    bos = p.cu_seqlens[n];
    eos = p.cu_seqlens[n + 1];
    brow = 0;
    cbase = p.cu_chunks[n];
  } else {
    bos = 0;
    eos = p.T;
    brow = n;
    cbase = n * ((p.T + BT - 1) / BT);
  }
  const int64_t L = eos - bos;
  const int Nc = (int)((L + BT - 1) / BT);
  const T *qb = static_cast<const T *>(p.q) + brow * p.sq_b + hk * p.sq_h + bos * p.sq_t;
  const T *kb = static_cast<const T *>(p.k) + brow * p.sk_b + hk * p.sk_h + bos * p.sk_t;
  const T *vb = static_cast<const T *>(p.v) + brow * p.sv_b + h * p.sv_h + j0 + bos * p.sv_t;
  T *ob = static_cast<T *>(p.o) + brow * p.so_b + h * p.so_h + j0 + bos * p.so_t;
  const unsigned char *recb = p.ws_rec + (cbase * p.Hv + h) * kRecBytes;
  const int64_t rec_stride = p.Hv * kRecBytes;
  const int64_t st_base = ((n * p.Hv + h) * p.dv + j0) * DK;
  auto rows_of = [&](int ch) -> int {
    const int64_t r = L - (int64_t)ch * BT;
    return (int)(r < BT ? r : BT);
  };
  int fo[KT];  // row c of a 16-row tile, dk 32 pp + 8 g .. + 7
#pragma unroll
  for (int pp = 0; pp < KT; ++pp) fo[pp] = c * RB + (((4 * pp + g) ^ kswz<DK>(c)) << 4);

  // Steps s = -2 .. Nc, one barrier each, in every wave.
  if (wave == 0) {
    // ---------------------------------------------------------------- chain
    f32x4 S[NT];  // S[mt][i] = S[dv row c][dk dk_of(mt, 4 g + i)]
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[mt][i] = p.init_state ? p.init_state[st_base + (int64_t)c * DK + dk_of(mt, 4 * g + i)] : 0.f;
    f8 Sf[KT];
#pragma unroll
    for (int pp = 0; pp < KT; ++pp) {
      Sf[pp] = cat8<T>(cvt4<T>(S[2 * pp]), cvt4<T>(S[2 * pp + 1]));
      *reinterpret_cast<f8 *>(&sm.sfrag[0][lane * SF + 8 * pp]) = Sf[pp];
    }
    // transposing-read offsets (K^T fragments of the state update): lane
    // 16 g + c addresses row 4 g + c / 4 at dk dk_of(mt, 4 (c % 4)) .. + 3, so
    // that lane c of the group receives dk dk_of(mt, c) of rows 4 g .. 4 g + 3
    const int yrow = 4 * g + (c >> 2);
    int trc[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
      trc[mt] = yrow * RB + (((4 * (mt >> 1) + (c & 3)) ^ kswz<DK>(yrow)) << 4) + 8 * (mt & 1);
    // V fragments (B operand of T' V) by transposing reads of the [64][16]
    // v tile: lane 16 g + L reads the 4 values of row 4 g + L / 4 starting at
    // column 4 (L % 4); lane c then holds V[t0 .. t0 + 3][c].
    const int vtr = (4 * g + (c >> 2)) * (DVT * 2) + 8 * (c & 3);
    for_steps(Nc, [&](int s, auto SL) {
      lds_barrier();
      if (s < 0 || s >= Nc) return;
      constexpr int sl = decltype(SL)::v;
      const unsigned char *kt = sm.k[sl];
      const unsigned char *rec = sm.rec[sl];
      const float *fa = reinterpret_cast<const float *>(rec + kRecF);
      const T *vt = sm.v[sl];
      f8 Tf[6];
#pragma unroll
      for (int f = 0; f < 6; ++f) Tf[f] = *reinterpret_cast<const f8 *>(rec + kRecT + f * 1024 + lane * 16);
      f8 kf[4][KT];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int pp = 0; pp < KT; ++pp) kf[mt][pp] = *reinterpret_cast<const f8 *>(kt + mt * 16 * RB + fo[pp]);
      f32x4 aa[4], cw[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int r0 = 16 * mt + 4 * g;
        aa[mt] = *reinterpret_cast<const f32x4 *>(&fa[0 * BT + r0]);
        cw[mt] = *reinterpret_cast<const f32x4 *>(&fa[1 * BT + r0]);
      }
      const float eC = fa[4 * BT];
      // B operands of T' V: rows 32 q + 16 hh + 4 g + i, column c
      f8 Bv[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const unsigned char *vb8 = reinterpret_cast<const unsigned char *>(vt) + vtr + 32 * q * (DVT * 2);
        const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(vb8));
        const s16x4 r1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(vb8 + 16 * DVT * 2));
        Bv[q] = cat8<T>(__builtin_bit_cast(v4, r0), __builtin_bit_cast(v4, r1));
      }
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
      const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
      // X = K S0^T
      f32x4 X[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) X[mt] = zero4;
#pragma unroll
      for (int pp = 0; pp < KT; ++pp)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) X[mt] = MF::k32(kf[mt][pp], Sf[pp], X[mt]);
      // U = T' V, independent of S
      f32x4 U[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        U[mt] = MF::k32(Tf[frag_id(mt, 0)], Bv[0], zero4);
        if (mt >= 2) U[mt] = MF::k32(Tf[frag_id(mt, 1)], Bv[1], U[mt]);
      }
      // Vn = U - T' (aa (.) X)
      f8 Rf[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) Rf[q] = cat8<T>(cvt4<T>(aa[2 * q] * X[2 * q]), cvt4<T>(aa[2 * q + 1] * X[2 * q + 1]));
      f32x4 Vn[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 y = MF::k32(Tf[frag_id(mt, 0)], Rf[0], zero4);
        if (mt >= 2) y = MF::k32(Tf[frag_id(mt, 1)], Rf[1], y);
        Vn[mt] = U[mt] - y;
      }
      f8 Bw[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        *reinterpret_cast<f8 *>(&sm.wfrag[s & 1][lane * 16 + 8 * q]) =
            cat8<T>(cvt4<T>(Vn[2 * q]), cvt4<T>(Vn[2 * q + 1]));
        Bw[q] = cat8<T>(cvt4<T>(cw[2 * q] * Vn[2 * q]), cvt4<T>(cw[2 * q + 1] * Vn[2 * q + 1]));
      }
      // S = e^{gamma_C} S0 + K^T (cw (.) Vn)
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) S[mt] = S[mt] * eC;
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) S[mt] = MF::k32(kt8[mt][q], Bw[q], S[mt]);
#pragma unroll
      for (int pp = 0; pp < KT; ++pp) {
        Sf[pp] = cat8<T>(cvt4<T>(S[2 * pp]), cvt4<T>(S[2 * pp + 1]));
        *reinterpret_cast<f8 *>(&sm.sfrag[(s & 1) ^ 1][lane * SF + 8 * pp]) = Sf[pp];
      }
    });
    if (p.final_state) {
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) p.final_state[st_base + (int64_t)c * DK + dk_of(mt, 4 * g + i)] = S[mt][i];
    }
  } else if (wave == 1) {
    // ------------------------------------------------- out(s), o(s - 1)
    f32x4 Zc[4];
    f8 Pf[6];
    for_steps(Nc, [&](int s, auto SL) {
      lds_barrier();
      const int co = s - 1;
      if (co >= 0 && co < Nc) {
        const int nr = rows_of(co);
        f8 Wf[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) Wf[q] = *reinterpret_cast<const f8 *>(&sm.wfrag[co & 1][lane * 16 + 8 * q]);
        T *orow = ob + (int64_t)co * BT * p.so_t;
        // O^T = Zc^T + Vn^T P^T: lane (g, c) holds o[16 mt + c][4 g .. 4 g + 3]
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 o = MF::k32(Wf[0], Pf[frag_id(mt, 0)], Zc[mt]);
          if (mt >= 2) o = MF::k32(Wf[1], Pf[frag_id(mt, 1)], o);
          const int r = 16 * mt + c;
          if (r < nr) *reinterpret_cast<v4 *>(orow + (int64_t)r * p.so_t + 4 * g) = cvt4<T>(o);
        }
      }
      if (s < 0 || s >= Nc) return;
      constexpr int sl = decltype(SL)::v;
      const unsigned char *qt = sm.q[sl];
      const unsigned char *rec = sm.rec[sl];
      const float *fa = reinterpret_cast<const float *>(rec + kRecF);
      f8 qf[4][KT], Sf[KT];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int pp = 0; pp < KT; ++pp) qf[mt][pp] = *reinterpret_cast<const f8 *>(qt + mt * 16 * RB + fo[pp]);
#pragma unroll
      for (int pp = 0; pp < KT; ++pp) Sf[pp] = *reinterpret_cast<const f8 *>(&sm.sfrag[s & 1][lane * SF + 8 * pp]);
#pragma unroll
      for (int f = 0; f < 6; ++f) Pf[f] = *reinterpret_cast<const f8 *>(rec + kRecP + f * 1024 + lane * 16);
      f32x4 z[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) z[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // Z^T = S0 Q^T: lane (g, c) holds Z[16 mt + c][dv 4 g + i]
#pragma unroll
      for (int pp = 0; pp < KT; ++pp)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) z[mt] = MF::k32(Sf[pp], qf[mt][pp], z[mt]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) Zc[mt] = z[mt] * fa[2 * BT + 16 * mt + c];
    });
  } else {
    // ------------------------------------------------------------- loads
    // Six loader waves with at most 8 copies each per step: waves 2, 3 copy
    // the halves of the k tile, waves 4, 5 those of the q tile, waves 6, 7
    // the halves of the record and of the v slice. Spreading the copies over
    // many waves keeps more of them in flight per CU.
    const int role = wave - 2;
    if (role < 4) {
      constexpr int NH = NI / 2;
      const bool isk = role < 2;
      const int i0 = (role & 1) * NH;
      const int64_t st = isk ? p.sk_t : p.sq_t;
      const T *xb = isk ? kb : qb;
      // per-lane byte offsets of the copies inside a full chunk (rows of the
      // tile with the XOR swizzle): a block-uniform base plus these
      uint32_t xoff[NH];
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        const int b = 1024 * (i0 + i) + 16 * lane;
        const int r = b / RB, jp = (b % RB) >> 4;
        const int j = jp ^ kswz<DK>(r);
        xoff[i] = (uint32_t)(((int64_t)r * st + 8 * j) * (int64_t)sizeof(T));
      }
      for_steps(Nc, [&](int s, auto SL) {
        lds_barrier();
        constexpr int sl = (decltype(SL)::v + 2) % 3;  // slot of chunk s + 2
        const int cl = s + 2;
        const bool issue = cl < Nc;
        unsigned char *xt = (isk ? sm.k[sl] : sm.q[sl]) + 1024 * i0;
        if (issue) {
          const int nr = rows_of(cl);
          const int64_t t0 = (int64_t)cl * BT;
          if (nr == BT) {
            const unsigned char *xg = reinterpret_cast<const unsigned char *>(xb + t0 * st);
#pragma unroll
            for (int i = 0; i < NH; ++i) g2l16(xg + xoff[i], xt + 1024 * i);
          } else {
            // last, partial chunk: rows past its end repeat its last row
#pragma unroll
            for (int i = 0; i < NH; ++i) {
              const int b = 1024 * (i0 + i) + 16 * lane;
              const int r = b / RB, jp = (b % RB) >> 4;
              const int j = jp ^ kswz<DK>(r);
              const int rr = r < nr ? r : nr - 1;
              g2l16(xb + (t0 + rr) * st + 8 * j, xt + 1024 * i);
            }
          }
        }
        // The copies of the previous step must be complete before the next
        // barrier publishes them; this step's stay in flight.
        if (issue) wait_vm<NH>(); else wait_vm<0>();
      });
    } else {
      constexpr int NRH = NR / 2;
      const int half = role - 4;
      const uint32_t voff =
          (uint32_t)(((int64_t)(32 * half + (lane >> 1)) * p.sv_t + 8 * (lane & 1)) * (int64_t)sizeof(T));
      for_steps(Nc, [&](int s, auto SL) {
        lds_barrier();
        constexpr int sl = (decltype(SL)::v + 2) % 3;
        const int cl = s + 2;
        const bool issue = cl < Nc;
        if (issue) {
          const int nr = rows_of(cl);
          const int64_t t0 = (int64_t)cl * BT;
          const unsigned char *rg = recb + (int64_t)cl * rec_stride + 1024 * NRH * half;
#pragma unroll
          for (int i = 0; i < NRH; ++i) g2l16(rg + 1024 * i + 16 * lane, sm.rec[sl] + 1024 * (NRH * half + i));
          unsigned char *vt = reinterpret_cast<unsigned char *>(sm.v[sl]) + 1024 * half;
          if (nr == BT) {
            g2l16(reinterpret_cast<const unsigned char *>(vb + t0 * p.sv_t) + voff, vt);
          } else {
            const int r = 32 * half + (lane >> 1);
            const int rr = r < nr ? r : nr - 1;
            g2l16(vb + (t0 + rr) * p.sv_t + 8 * (lane & 1), vt);
          }
        }
        if (issue) wait_vm<NRH + 1>(); else wait_vm<0>();
      });
    }
  }
}

// ---------------------------------------------------------------------------
// Multi-slice variant, for launches with many (sequence, head) pairs (packed
// or batched sequences): one workgroup = (sequence, value head, NS * 16 rows
// of dv), NS = 4 or 8. The step of chunk_state_kernel is bound by the bytes a
// CU moves, and its k, q and record copies serve one 16-row slice; here one
// copy of them serves NS. Waves 0 .. NS - 1 each own a 16-row slice and run
// the whole step for it (chain and output: X and Z = S0 Q^T from the same
// state fragments, U, Vn, O, the state update), with no LDS hand-off; the
// four waves after them copy the k tile, the q tile, the record and the
// [64][16 NS] v tile of chunk s + 1 into two-slot rings during step s
// (complete before the barrier that starts step s + 1). LDS at dk 128: 108 KB
// (NS 4) or 124 KB (NS 8), one workgroup per CU.
// ---------------------------------------------------------------------------
template <typename T, int DK, int NS>
struct QuadLds {
  static constexpr int RB = DK * 2;
  static constexpr int TILE = BT * RB;
  static constexpr int VB = NS * DVT * 2;  // bytes per v row
  alignas(16) unsigned char k[2][TILE];
  alignas(16) unsigned char q[2][TILE];
  alignas(16) unsigned char v[2][BT * VB];
  alignas(16) unsigned char rec[2][kRecBytes];
};

// Runs body(s, Slot<s mod 2>) for s = -1 .. last - 1 in order.
template <typename F>
__device__ __forceinline__ void for_steps2(int last, F &&body) {
  for (int base = -2; base < last; base += 2) {
    if (base >= -1) body(base, Slot<0>{});
    if (base + 1 < last) body(base + 1, Slot<1>{});
  }
}

template <typename T, int DK, int NS>
__global__ __launch_bounds__((NS + 4) * 64) void chunk_state_quad_kernel(ChunkArgs p) {
  using MF = M2<T>;
  using f8 = typename MF::f8;
  using v4 = typename MF::v4;
  using SM = QuadLds<T, DK, NS>;
  constexpr int KT = DK / 32;
  constexpr int NT = DK / 16;
  constexpr int RB = SM::RB;
  constexpr int VB = SM::VB;
  constexpr int NI = SM::TILE / 1024;          // 1 KB copies per q/k tile
  constexpr int NR = (int)(kRecBytes / 1024);  // 1 KB copies per record
  constexpr int NV = BT * VB / 1024;           // 1 KB copies per v tile
  constexpr int LV = VB / 16;                   // lanes per v row in a copy
  static_assert(NI <= 16 && NR <= 16 && NV <= 16, "copies per loader wave");
  __shared__ SM sm;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t ntile = gridDim.x, nwg = (int64_t)gridDim.x * gridDim.y * gridDim.z;
  int64_t lid = blockIdx.x + ntile * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
  if (nwg % 8 == 0) lid = (lid % 8) * (nwg / 8) + lid / 8;
  const int64_t jg = (lid % ntile) * (NS * DVT);  // first value row of the workgroup
  const int64_t h = (lid / ntile) % gridDim.y;
  const int64_t n = lid / (ntile * gridDim.y);
  const int64_t hk = h / (p.Hv / p.Hqk);
  int64_t bos, eos, brow, cbase;
  if (p.cu_seqlens) {
    bos = p.cu_seqlens[n];
    eos = p.cu_seqlens[n + 1];
    brow = 0;
    cbase = p.cu_chunks[n];
  } else {
    bos = 0;
    eos = p.T;
    brow = n;
    cbase = n * ((p.T + BT - 1) / BT);
  }
  const int64_t L = eos - bos;
  const int Nc = (int)((L + BT - 1) / BT);
  auto rows_of = [&](int ch) -> int {
    const int64_t r = L - (int64_t)ch * BT;
    return (int)(r < BT ? r : BT);
  };

  if (wave < NS) {
    // ------------------------------------------- one 16-row slice, whole step
    const int64_t j0 = jg + DVT * wave;
    T *ob = static_cast<T *>(p.o) + brow * p.so_b + h * p.so_h + j0 + bos * p.so_t;
    const int64_t st_base = ((n * p.Hv + h) * p.dv + j0) * DK;
    int fo[KT];  // row c of a 16-row tile, dk 32 pp + 8 g .. + 7
#pragma unroll
    for (int pp = 0; pp < KT; ++pp) fo[pp] = c * RB + (((4 * pp + g) ^ kswz<DK>(c)) << 4);
    const int yrow = 4 * g + (c >> 2);
    int trc[NT];  // transposing reads of K^T fragments (as in chunk_state_kernel)
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
      trc[mt] = yrow * RB + (((4 * (mt >> 1) + (c & 3)) ^ kswz<DK>(yrow)) << 4) + 8 * (mt & 1);
    // V fragments by transposing reads of this slice's 16 columns of the
    // [64][64] v tile
    const int vtr = (4 * g + (c >> 2)) * VB + 2 * DVT * wave + 8 * (c & 3);
    f32x4 S[NT];  // S[mt][i] = S[dv row c][dk dk_of(mt, 4 g + i)]
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[mt][i] = p.init_state ? p.init_state[st_base + (int64_t)c * DK + dk_of(mt, 4 * g + i)] : 0.f;
    f8 Sf[KT];
#pragma unroll
    for (int pp = 0; pp < KT; ++pp) Sf[pp] = cat8<T>(cvt4<T>(S[2 * pp]), cvt4<T>(S[2 * pp + 1]));
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    for_steps2(Nc, [&](int s, auto SL) {
      lds_barrier();
      if (s < 0) return;
      constexpr int sl = decltype(SL)::v;
      const unsigned char *kt = sm.k[sl], *qt = sm.q[sl], *rec = sm.rec[sl], *vt = sm.v[sl];
      const float *fa = reinterpret_cast<const float *>(rec + kRecF);
      // X = K S0^T
      f32x4 X[4];
      {
        f8 kf[4][KT];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int pp = 0; pp < KT; ++pp) kf[mt][pp] = *reinterpret_cast<const f8 *>(kt + mt * 16 * RB + fo[pp]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) X[mt] = zero4;
#pragma unroll
        for (int pp = 0; pp < KT; ++pp)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) X[mt] = MF::k32(kf[mt][pp], Sf[pp], X[mt]);
      }
      __builtin_amdgcn_sched_barrier(0);
      // Z^T = S0 Q^T (lane (g, c) holds Z[16 mt + c][dv 4 g + i]), scaled by zc
      f32x4 Zc[4];
      {
        f8 qf[4][KT];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int pp = 0; pp < KT; ++pp) qf[mt][pp] = *reinterpret_cast<const f8 *>(qt + mt * 16 * RB + fo[pp]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) Zc[mt] = zero4;
#pragma unroll
        for (int pp = 0; pp < KT; ++pp)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) Zc[mt] = MF::k32(Sf[pp], qf[mt][pp], Zc[mt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) Zc[mt] = Zc[mt] * fa[2 * BT + 16 * mt + c];
      }
      __builtin_amdgcn_sched_barrier(0);
      // U = T' V, Vn = U - T' (aa (.) X)
      f32x4 Vn[4];
      {
        f8 Tf[6];
#pragma unroll
        for (int f = 0; f < 6; ++f) Tf[f] = *reinterpret_cast<const f8 *>(rec + kRecT + f * 1024 + lane * 16);
        f8 Bv[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const unsigned char *vb8 = vt + vtr + 32 * q * VB;
          const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(vb8));
          const s16x4 r1 =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(vb8 + 16 * VB));
          Bv[q] = cat8<T>(__builtin_bit_cast(v4, r0), __builtin_bit_cast(v4, r1));
        }
        f8 Rf[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f32x4 a0 = *reinterpret_cast<const f32x4 *>(&fa[0 * BT + 32 * q + 4 * g]);
          const f32x4 a1 = *reinterpret_cast<const f32x4 *>(&fa[0 * BT + 32 * q + 16 + 4 * g]);
          Rf[q] = cat8<T>(cvt4<T>(a0 * X[2 * q]), cvt4<T>(a1 * X[2 * q + 1]));
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 u = MF::k32(Tf[frag_id(mt, 0)], Bv[0], zero4);
          f32x4 y = MF::k32(Tf[frag_id(mt, 0)], Rf[0], zero4);
          if (mt >= 2) {
            u = MF::k32(Tf[frag_id(mt, 1)], Bv[1], u);
            y = MF::k32(Tf[frag_id(mt, 1)], Rf[1], y);
          }
          Vn[mt] = u - y;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // o = zc (.) (Q S0^T) + P Vn, transposed: O^T = Zc^T + Vn^T P^T
      {
        f8 Wf[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) Wf[q] = cat8<T>(cvt4<T>(Vn[2 * q]), cvt4<T>(Vn[2 * q + 1]));
        const int nr = rows_of(s);
        T *orow = ob + (int64_t)s * BT * p.so_t;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 o = MF::k32(Wf[0], *reinterpret_cast<const f8 *>(rec + kRecP + frag_id(mt, 0) * 1024 + lane * 16), Zc[mt]);
          if (mt >= 2)
            o = MF::k32(Wf[1], *reinterpret_cast<const f8 *>(rec + kRecP + frag_id(mt, 1) * 1024 + lane * 16), o);
          const int r = 16 * mt + c;
          if (r < nr) *reinterpret_cast<v4 *>(orow + (int64_t)r * p.so_t + 4 * g) = cvt4<T>(o);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // S = e^{gamma_C} S0 + K^T (cw (.) Vn)
      {
        f8 Bw[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f32x4 c0 = *reinterpret_cast<const f32x4 *>(&fa[1 * BT + 32 * q + 4 * g]);
          const f32x4 c1 = *reinterpret_cast<const f32x4 *>(&fa[1 * BT + 32 * q + 16 + 4 * g]);
          Bw[q] = cat8<T>(cvt4<T>(c0 * Vn[2 * q]), cvt4<T>(c1 * Vn[2 * q + 1]));
        }
        const float eC = fa[4 * BT];
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
          f32x4 a = S[mt] * eC;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const unsigned char *a1 = kt + trc[mt] + (32 * q) * RB;
            const unsigned char *a2 = kt + trc[mt] + (32 * q + 16) * RB;
            const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(a1));
            const s16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(a2));
            a = MF::k32(cat8<T>(__builtin_bit_cast(v4, r1), __builtin_bit_cast(v4, r2)), Bw[q], a);
          }
          S[mt] = a;
        }
#pragma unroll
        for (int pp = 0; pp < KT; ++pp) Sf[pp] = cat8<T>(cvt4<T>(S[2 * pp]), cvt4<T>(S[2 * pp + 1]));
      }
    });
    if (p.final_state) {
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) p.final_state[st_base + (int64_t)c * DK + dk_of(mt, 4 * g + i)] = S[mt][i];
    }
  } else {
    // ------------------------------------------------------------- loads
    // wave NS: the k tile; NS + 1: the q tile; NS + 2: the record; NS + 3:
    // the v tile; for chunk s + 1, complete before the next barrier
    const int role = wave - NS;
    const bool isx = role < 2;
    const int64_t st = role == 0 ? p.sk_t : p.sq_t;
    const T *xb = (role == 0 ? static_cast<const T *>(p.k) + brow * p.sk_b + hk * p.sk_h + bos * p.sk_t
                             : static_cast<const T *>(p.q) + brow * p.sq_b + hk * p.sq_h + bos * p.sq_t);
    const T *vb = static_cast<const T *>(p.v) + brow * p.sv_b + h * p.sv_h + jg + bos * p.sv_t;
    const unsigned char *recb = p.ws_rec + (cbase * p.Hv + h) * kRecBytes;
    const int64_t rec_stride = p.Hv * kRecBytes;
    for_steps2(Nc, [&](int s, auto SL) {
      lds_barrier();
      constexpr int sl = (decltype(SL)::v + 1) % 2;  // slot of chunk s + 1
      const int cl = s + 1;
      if (cl < Nc) {
        const int nr = rows_of(cl);
        const int64_t t0 = (int64_t)cl * BT;
        if (isx) {
          unsigned char *xt = role == 0 ? sm.k[sl] : sm.q[sl];
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            const int b = 1024 * i + 16 * lane;
            const int r = b / RB, jp = (b % RB) >> 4;
            const int j = jp ^ kswz<DK>(r);
            const int rr = r < nr ? r : nr - 1;  // rows past the chunk's end repeat its last row
            g2l16(xb + (t0 + rr) * st + 8 * j, xt + 1024 * i);
          }
        } else if (role == 2) {
          const unsigned char *rg = recb + (int64_t)cl * rec_stride;
#pragma unroll
          for (int i = 0; i < NR; ++i) g2l16(rg + 1024 * i + 16 * lane, sm.rec[sl] + 1024 * i);
        } else {
          // copy i: rows (64 / LV) i + lane / LV, 16 bytes at column 8 (lane % LV)
#pragma unroll
          for (int i = 0; i < NV; ++i) {
            const int r = (64 / LV) * i + lane / LV;
            const int rr = r < nr ? r : nr - 1;
            g2l16(vb + (t0 + rr) * p.sv_t + 8 * (lane % LV), sm.v[sl] + 1024 * i);
          }
        }
      }
      wait_vm<0>();
    });
  }
}

template <typename T, int DK, int NS>
hipError_t launch_quad(const ChunkArgs &a, hipStream_t s) {
  dim3 grid((unsigned)(a.dv / (NS * DVT)), (unsigned)a.Hv, (unsigned)a.n_seqs);
  hipLaunchKernelGGL((chunk_state_quad_kernel<T, DK, NS>), grid, dim3((NS + 4) * 64), 0, s, a);
  return hipGetLastError();
}

// A multi-slice kernel when its launch has at least this many workgroups
// (half the CUs): below that, the NS times as many one-slice workgroups run
// more chunks at once than it saves per chunk.
constexpr int64_t kQuadMinWorkgroups = 128;

template <typename T, int DK>
hipError_t launch_multi(const ChunkArgs &a, hipStream_t s, bool &done) {
  done = true;
  const int64_t pairs = a.n_seqs * a.Hv;
  if (a.dv % (8 * DVT) == 0 && pairs * (a.dv / (8 * DVT)) >= kQuadMinWorkgroups) return launch_quad<T, DK, 8>(a, s);
  if (a.dv % (4 * DVT) == 0 && pairs * (a.dv / (4 * DVT)) >= kQuadMinWorkgroups) return launch_quad<T, DK, 4>(a, s);
  done = false;
  return hipSuccess;
}

template <typename T, int DK>
hipError_t launch_dk(const ChunkArgs &a, hipStream_t s) {
  dim3 grid((unsigned)(a.dv / DVT), (unsigned)a.Hv, (unsigned)a.n_seqs);
  hipLaunchKernelGGL((chunk_state_kernel<T, DK>), grid, dim3(kStateThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_prep(const ChunkArgs &a, hipStream_t s);
hipError_t launch_chunk_state_wide(const ChunkArgs &a, hipStream_t s);

// dv is covered in slices of 16 rows (dk <= 128) or 32 rows (dk 256).
bool chunk_split_supported(int64_t dk, int64_t dv, int32_t act) {
  if (act != kBF16 && act != kF16) return false;
  if (dk == 64 || dk == 128) return dv % 16 == 0;
  return dk == 256 && dv % 32 == 0;
}

hipError_t launch_chunk_split(const ChunkArgs &a, hipStream_t s) {
  if (a.n_seqs == 0 || a.dv == 0) return hipSuccess;
  if (!a.ws_rec || (a.cu_seqlens && !a.cu_chunks)) return hipErrorInvalidValue;
  hipError_t e = launch_chunk_prep(a, s);
  if (e != hipSuccess) return e;
  if (a.dk == 256) return launch_chunk_state_wide(a, s);
  {
    bool done = false;
    if (a.act == kBF16) e = a.dk == 64 ? launch_multi<bf16, 64>(a, s, done) : launch_multi<bf16, 128>(a, s, done);
    else if (a.act == kF16) e = a.dk == 64 ? launch_multi<f16, 64>(a, s, done) : launch_multi<f16, 128>(a, s, done);
    if (done) return e;
  }
  if (a.act == kBF16) return a.dk == 64 ? launch_dk<bf16, 64>(a, s) : launch_dk<bf16, 128>(a, s);
  if (a.act == kF16) return a.dk == 64 ? launch_dk<f16, 64>(a, s) : launch_dk<f16, 128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace gdn
