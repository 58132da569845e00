// The two serial state passes of the chunk-rule backward on the 16-bit
// matrix cores, for BF16 or FP16 activations with dk 64 or 128, run by one
// launch (bwd_state_passes_kernel at the end of this file): its first
// workgroups run the forward-state pass, the rest the reverse pass, each in
// a one-slice or a multi-slice form.
//
// Reverse pass: per (sequence, value head, 16 value
// rows), serial over the chunks from the last to the first, the gradient dS
// of the state leaving each chunk is carried in FP32 MFMA accumulators and
// each chunk gives (unit q, k rows q^, k^; the algebra is written out at the
// top of chunk_bwd.hip)
//
//   dDelta = cw (.) K^ dS^T + P'^T dO                 (P' = scale Pt)
//   dR'    = M^T dDelta,   dv = beta (.) dR'
//   dS0    = e^{gamma_C} dS + Q^T (fq (.) dO) + K^T (fk (.) dR')
//
// with fq = scale e^gamma rq and fk = -e^gamma beta rk on the raw 16-bit q, k
// rows. dS_C (for the gradient kernel) and dR' are written in FP32, dv in the
// gradient dtype.
//
// Precision. K, Q and dO are exact 16-bit operands (on the instruction of
// their own type); dS, dDelta, dR', the scaled rows and the record's M^T,
// P'^T are split as x = hi + lo in that type, and products of two split
// operands take ah bh + ah bl + al bh, so that each term carries a relative
// error near 2^-16 (BF16) or 2^-22 (FP16, for values inside its range).
//
// One workgroup = (sequence, value head, 16 rows of dv), eight wavefronts,
// two barriers per step (B0 at its start, B1 in its middle):
//   wave 0     the chain: before B1 U = K dS^T, after it dDelta, dR' and the
//              K^T part of the update; dS in accumulators;
//   wave 1     the products that do not depend on dS: before B1
//              G = P'^T dO (read by the chain after B1), after it the q term
//              Q^T (fq (.) dO) (added to dS by the chain at the next step);
//              and the stores of the previous step's dR' and dv from a
//              two-slot LDS stage, so that the chain issues only dS_C's;
//   waves 2-7  copies (global_load_lds) of the k and q tiles, the dO slice
//              and the record of the next chunk into a two-slot LDS ring.
#include <atomic>

#include "chunk_bwd_common.h"
#include "gdn_internal.h"
#include "mfma_tiles.h"

namespace gdn {
namespace {

// LDS of the state passes: one dynamic allocation of the launch's size, read
// by whichever pass a workgroup runs (each body views it as its own layout)
extern __shared__ __attribute__((aligned(16))) unsigned char g_pass_lds[];

constexpr int kThr = 512;
constexpr int BT = 64;
constexpr int DVT = 16;

// T is the activations' 16-bit type (bf16 or f16): the products run on the
// matrix-core instruction of that type and split operands use its hi / lo.
template <typename T>
__device__ __forceinline__ f32x4 mma(typename M2<T>::f8 a, typename M2<T>::f8 b, f32x4 c) {
  return M2<T>::k32(a, b, c);
}

// dk permutation of the state tiles (as in the forward state kernel):
// accumulator tile mt = 2 pp + h, row 4 g + i holds dk 32 pp + 8 g + 4 h + i.
__device__ __forceinline__ constexpr int dk_of(int mt, int r) {
  return 32 * (mt >> 1) + 8 * (r >> 2) + 4 * (mt & 1) + (r & 3);
}

// fragment of (row tile mt, k pair q) of an upper-triangular record matrix
__device__ __forceinline__ constexpr int up_frag(int mt, int q) { return q == 0 ? mt : 2 + mt; }

template <typename T>
__device__ __forceinline__ void split2x4(f32x4 a, f32x4 b, typename M2<T>::f8 &hi, typename M2<T>::f8 &lo) {
  using v4 = typename M2<T>::v4;
  const v4 ah = __builtin_convertvector(a, v4), bh = __builtin_convertvector(b, v4);
  const v4 al = __builtin_convertvector(a - __builtin_convertvector(ah, f32x4), v4);
  const v4 bl = __builtin_convertvector(b - __builtin_convertvector(bh, f32x4), v4);
  hi = cat8<T>(ah, bh);
  lo = cat8<T>(al, bl);
}
template <typename T>
__device__ __forceinline__ void split8(const float (&x)[8], typename M2<T>::f8 &hi, typename M2<T>::f8 &lo) {
  split2x4<T>(f32x4{x[0], x[1], x[2], x[3]}, f32x4{x[4], x[5], x[6], x[7]}, hi, lo);
}

// the reverse pass copies bytes [kBrF, kBrBytes) of each record: offsets
// within its copy
constexpr int64_t kDsRec = kBrBytes - kBrF;
constexpr int64_t kDsF = 0, kDsMtH = kBrMtH - kBrF, kDsMtL = kBrMtL - kBrF, kDsPH = kBrPH - kBrF,
                  kDsPL = kBrPL - kBrF;

template <typename T, int DK>
struct DsLds {
  static constexpr int RB = DK * 2;
  static constexpr int TILE = BT * RB;
  alignas(16) unsigned char k[2][TILE];   // raw k rows of the step's chunk (swizzled)
  alignas(16) unsigned char q[2][TILE];   // raw q rows
  alignas(16) T o[2][BT * DVT];           // dO slice [64][16]
  alignas(16) unsigned char rec[2][kDsRec];
  alignas(16) float gg[4 * 64 * 4];        // G = P'^T dO, accumulator layout [mt][lane][4]
  alignas(16) float hq[DK / 16 * 64 * 4];  // q term of the state update, [mt][lane][4]
  alignas(16) float stage[2][4 * 64 * 4 + 64];  // dR' [mt][lane][4], then beta
};

template <int N> struct Slot { static constexpr int v = N; };

// Runs body(s, Slot<s mod 2>) for s = -1 .. last in order.
template <typename F>
__device__ __forceinline__ void for_steps2(int last, F &&body) {
  for (int base = -2; base <= last; base += 2) {
    if (base >= -1) body(base, Slot<0>{});
    if (base + 1 <= last) body(base + 1, Slot<1>{});
  }
}

template <typename T, int DK>
__device__ __forceinline__ void dstate_pass(const ChunkBwdArgs &p, int64_t bid) {
  using SM = DsLds<T, DK>;
  SM &sm = *reinterpret_cast<SM *>(g_pass_lds);
  using f8 = typename M2<T>::f8;
  using v4 = typename M2<T>::v4;
  constexpr int KT = DK / 32, NT = DK / 16, RB = SM::RB;
  constexpr int NI = SM::TILE / 1024;           // 1 KB copies per q/k tile
  constexpr int NR = (int)(kDsRec / 1024);      // 1 KB copies per record
  static_assert(NI % 2 == 0 && NR % 2 == 0 && NI / 2 <= 31 && NR / 2 + 1 <= 31, "copy split");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  // slices of one head (which read the same tiles and records) on one XCD
  const int64_t ntile = p.dv / DVT, nwg = ntile * p.Hv * p.n_seqs;
  int64_t lid = bid;
  if (nwg % 8 == 0) lid = (lid % 8) * (nwg / 8) + lid / 8;
  const int64_t j0 = (lid % ntile) * DVT;
  const int64_t h = (lid / ntile) % p.Hv;
  const int64_t n = lid / (ntile * p.Hv);
  const int64_t hk = h / (p.Hv / p.Hqk);
  int64_t brow, bos, L, gc0;
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
  const int Nc = (int)((L + BT - 1) / BT);
  // step s works on chunk Nc - 1 - s
  auto rows_of = [&](int ch) -> int {
    const int64_t r = L - (int64_t)ch * BT;
    return (int)(r < BT ? r : BT);
  };
  const int64_t st_base = ((n * p.Hv + h) * p.dv + j0) * DK;

  // fragment offsets shared by the compute waves
  int fo[KT];  // row c of a 16-row tile, dk 32 pp + 8 g .. + 7
#pragma unroll
  for (int pp = 0; pp < KT; ++pp) fo[pp] = c * RB + (((4 * pp + g) ^ kswz<DK>(c)) << 4);
  // transposing-read offsets (K^T, Q^T fragments; see the forward state kernel)
  const int yrow = 4 * g + (c >> 2);
  int trc[NT];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt)
    trc[mt] = yrow * RB + (((4 * (mt >> 1) + (c & 3)) ^ kswz<DK>(yrow)) << 4) + 8 * (mt & 1);
  const int otr = (4 * g + (c >> 2)) * (DVT * 2) + 8 * (c & 3);
  // dO fragments of slot sl (B operand, k slots in tile-pair order), exact
  auto dO_frags = [&](int sl, f8 (&Bo)[2]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const unsigned char *ob = reinterpret_cast<const unsigned char *>(sm.o[sl]) + otr + 32 * q * (DVT * 2);
      const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(ob));
      const s16x4 r1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(ob + 16 * DVT * 2));
      Bo[q] = cat8<T>(__builtin_bit_cast(v4, r0), __builtin_bit_cast(v4, r1));
    }
  };
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // Steps s = -1 .. Nc - 1, two barriers each (B0 at the start, B1 in the
  // middle) in every wave, then one more after the last step.
  if (wave == 0) {
    // ---------------------------------------------------------------- chain
    f32x4 dS[NT];  // dS[mt][i] = dS[dv row c][dk dk_of(mt, 4 g + i)]
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dS[mt][i] = p.d_final ? p.d_final[st_base + (int64_t)c * DK + dk_of(mt, 4 * g + i)] : 0.f;

    for_steps2(Nc - 1, [&](int s, auto SL) {
      lds_barrier();  // B0
      constexpr int sl = decltype(SL)::v;
      const int ch = Nc - 1 - s;
      const int64_t gc = gc0 + ch;
      const unsigned char *kt = sm.k[sl], *rec = sm.rec[sl];
      const float *fa = reinterpret_cast<const float *>(rec + kDsF);
      f32x4 U[4];
      f8 mth[6], mtl[6], kTr[NT][2];
      if (s >= 0) {
        // U = K dS^T (raw k rows), with the q term of the previous step
        // added first; every LDS fragment is read before the VALU work that
        // precedes its products
        f8 kfr[4][KT];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int pp = 0; pp < KT; ++pp) kfr[mt][pp] = *reinterpret_cast<const f8 *>(kt + mt * 16 * RB + fo[pp]);
        if (s > 0) {
#pragma unroll
          for (int mt = 0; mt < NT; ++mt) dS[mt] += *reinterpret_cast<const f32x4 *>(&sm.hq[(mt * 64 + lane) * 4]);
        }
        f8 Sh[KT], Sl[KT];
#pragma unroll
        for (int pp = 0; pp < KT; ++pp) split2x4<T>(dS[2 * pp], dS[2 * pp + 1], Sh[pp], Sl[pp]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 u = zero4;
#pragma unroll
          for (int pp = 0; pp < KT; ++pp) {
            u = mma<T>(kfr[mt][pp], Sh[pp], u);
            u = mma<T>(kfr[mt][pp], Sl[pp], u);
          }
          U[mt] = u;
        }
        // the M^T and K^T fragments of the second half
#pragma unroll
        for (int f = 0; f < 6; ++f) {
          mth[f] = *reinterpret_cast<const f8 *>(rec + kDsMtH + f * 1024 + lane * 16);
          mtl[f] = *reinterpret_cast<const f8 *>(rec + kDsMtL + f * 1024 + lane * 16);
        }
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const unsigned char *ka1 = kt + trc[mt] + (32 * q) * RB, *ka2 = kt + trc[mt] + (32 * q + 16) * RB;
            const s16x4 k1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(ka1));
            const s16x4 k2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(ka2));
            kTr[mt][q] = cat8<T>(__builtin_bit_cast(v4, k1), __builtin_bit_cast(v4, k2));
          }
        // dS_C to the workspace (as [dv][dk]), issued after the products so
        // that the stores do not wait behind the step's copies
        float *dsw = p.ds + ((gc * p.Hv + h) * p.dv + j0 + c) * DK;
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) *reinterpret_cast<f32x4 *>(dsw + dk_of(mt, 4 * g)) = dS[mt];
      }
      lds_barrier();  // B1: G of this chunk is in LDS
      if (s < 0) return;
      // dDelta = cw rk (.) U + P'^T dO
      f32x4 dD[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 cr = *reinterpret_cast<const f32x4 *>(&fa[1 * BT + 16 * mt + 4 * g]);
        dD[mt] = U[mt] * cr + *reinterpret_cast<const f32x4 *>(&sm.gg[(mt * 64 + lane) * 4]);
      }
      // dR' = M^T dDelta
      f32x4 dR[4];
      {
        f8 Dh[2], Dl[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) split2x4<T>(dD[2 * q], dD[2 * q + 1], Dh[q], Dl[q]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 r = zero4;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            if (q == 0 && mt >= 2) continue;
            const int f = up_frag(mt, q);
            r = mma<T>(mth[f], Dh[q], r);
            r = mma<T>(mth[f], Dl[q], r);
            r = mma<T>(mtl[f], Dh[q], r);
          }
          dR[mt] = r;
        }
      }
      // dR' and beta to the stage; wave 1 stores them (and dv) next step
      {
        float *stg = sm.stage[sl];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) *reinterpret_cast<f32x4 *>(&stg[(mt * 64 + lane) * 4]) = dR[mt];
        stg[4 * 64 * 4 + lane] = fa[2 * BT + lane];
      }
      // dS0 = e^{gamma_C} dS + K^T (fk (.) dR') (+ the q term, next step)
      f8 Fkh[2], Fkl[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f32x4 fk0 = *reinterpret_cast<const f32x4 *>(&fa[4 * BT + 32 * q + 4 * g]);
        const f32x4 fk1 = *reinterpret_cast<const f32x4 *>(&fa[4 * BT + 32 * q + 16 + 4 * g]);
        split2x4<T>(fk0 * dR[2 * q], fk1 * dR[2 * q + 1], Fkh[q], Fkl[q]);
      }
      const float eC = fa[5 * BT];
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        f32x4 a = dS[mt] * eC;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          a = mma<T>(kTr[mt][q], Fkh[q], a);
          a = mma<T>(kTr[mt][q], Fkl[q], a);
        }
        dS[mt] = a;
      }
    });
    lds_barrier();  // the last q term is in LDS
    if (Nc > 0) {
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) dS[mt] += *reinterpret_cast<const f32x4 *>(&sm.hq[(mt * 64 + lane) * 4]);
    }
    if (p.d_init) {
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
        *reinterpret_cast<f32x4 *>(p.d_init + st_base + (int64_t)c * DK + dk_of(mt, 4 * g)) = dS[mt];
    }
  } else if (wave == 1) {
    // --------------------------------------- G = P'^T dO, q term, stores
    // stage of step s2 (chunk Nc - 1 - s2) to dR' (FP32) and dv = beta dR'
    auto store_stage = [&](int s2, const float *stg) {
      const int ch = Nc - 1 - s2;
      const int64_t gc = gc0 + ch, t0 = bos + (int64_t)ch * BT;
      const int nr = rows_of(ch);
      const int t = lane, mt = t >> 4, gg = (t >> 2) & 3, i = t & 3;
      float x[16];
#pragma unroll
      for (int cc = 0; cc < 16; ++cc) x[cc] = stg[(mt * 64 + 16 * gg + cc) * 4 + i];
      float *dr = p.drp + ((gc * p.Hv + h) * BT + t) * p.dv + j0;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        *reinterpret_cast<f32x4 *>(dr + 4 * v) = f32x4{x[4 * v], x[4 * v + 1], x[4 * v + 2], x[4 * v + 3]};
      if (t < nr) {
        const float bt = stg[4 * 64 * 4 + t];
        const int64_t o = brow * p.sdv_b + (t0 + t) * p.sdv_t + h * p.dv + j0;
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) x[cc] *= bt;
        if (p.grad_dtype == kF32) {
          float *dv = static_cast<float *>(p.dvv) + o;
#pragma unroll
          for (int v = 0; v < 4; ++v)
            *reinterpret_cast<f32x4 *>(dv + 4 * v) = f32x4{x[4 * v], x[4 * v + 1], x[4 * v + 2], x[4 * v + 3]};
        } else {
          T *dv = static_cast<T *>(p.dvv) + o;
#pragma unroll
          for (int v = 0; v < 4; ++v)
            *reinterpret_cast<v4 *>(dv + 4 * v) =
                __builtin_convertvector(f32x4{x[4 * v], x[4 * v + 1], x[4 * v + 2], x[4 * v + 3]}, v4);
        }
      }
    };
    for_steps2(Nc - 1, [&](int s, auto SL) {
      lds_barrier();  // B0
      constexpr int sl = decltype(SL)::v;
      const unsigned char *qt = sm.q[sl], *rec = sm.rec[sl];
      const float *fa = reinterpret_cast<const float *>(rec + kDsF);
      f8 Bo[2];
      if (s >= 0) {
        dO_frags(sl, Bo);
        // G = P'^T dO in the accumulator layout of dDelta
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 a = zero4;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            if (q == 0 && mt >= 2) continue;
            const int f = up_frag(mt, q);
            const f8 ph = *reinterpret_cast<const f8 *>(rec + kDsPH + f * 1024 + lane * 16);
            const f8 pl = *reinterpret_cast<const f8 *>(rec + kDsPL + f * 1024 + lane * 16);
            a = mma<T>(ph, Bo[q], a);
            a = mma<T>(pl, Bo[q], a);
          }
          *reinterpret_cast<f32x4 *>(&sm.gg[(mt * 64 + lane) * 4]) = a;
        }
      }
      lds_barrier();  // B1
      if (s < 0) return;
      // q term Q^T (fq (.) dO), added to dS by the chain at the next step
      f8 Fqh[2], Fql[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f32x4 fq0 = *reinterpret_cast<const f32x4 *>(&fa[3 * BT + 32 * q + 4 * g]);
        const f32x4 fq1 = *reinterpret_cast<const f32x4 *>(&fa[3 * BT + 32 * q + 16 + 4 * g]);
        float xq[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xq[e] = fq0[e] * f(Bo[q][e]);
          xq[4 + e] = fq1[e] * f(Bo[q][4 + e]);
        }
        split8<T>(xq, Fqh[q], Fql[q]);
      }
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        f32x4 a = zero4;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const unsigned char *qa1 = qt + trc[mt] + (32 * q) * RB, *qa2 = qt + trc[mt] + (32 * q + 16) * RB;
          const s16x4 q1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(qa1));
          const s16x4 q2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(qa2));
          const f8 qT = cat8<T>(__builtin_bit_cast(v4, q1), __builtin_bit_cast(v4, q2));
          a = mma<T>(qT, Fqh[q], a);
          a = mma<T>(qT, Fql[q], a);
        }
        *reinterpret_cast<f32x4 *>(&sm.hq[(mt * 64 + lane) * 4]) = a;
      }
      // the previous step's dR' and dv (its stage slot is rewritten only
      // after the next middle barrier)
      if (s >= 1) store_stage(s - 1, sm.stage[(sl + 1) % 2]);
    });
    lds_barrier();
    if (Nc > 0) store_stage(Nc - 1, sm.stage[(Nc - 1) % 2]);
  } else {
    // ------------------------------------------------------------- loads
    // Waves 2, 3 copy the halves of the k tile, waves 4, 5 those of the q
    // tile, waves 6, 7 the halves of the record and of the dO slice, for the
    // chunk of step s + 1; they are complete before the barrier ending step s.
    const int role = wave - 2;
    if (role < 4) {
      constexpr int NH = NI / 2;
      const bool isk = role < 2;
      const int i0 = (role & 1) * NH;
      const int64_t st = isk ? p.sk_t : p.sq_t;
      const T *xb = static_cast<const T *>(isk ? p.k : p.q) + brow * (isk ? p.sk_b : p.sq_b) +
                       hk * (isk ? p.sk_h : p.sq_h) + bos * st;
      uint32_t xoff[NH];
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        const int b = 1024 * (i0 + i) + 16 * lane;
        const int r = b / RB, jp = (b % RB) >> 4;
        const int j = jp ^ kswz<DK>(r);
        xoff[i] = (uint32_t)(((int64_t)r * st + 8 * j) * 2);
      }
      for_steps2(Nc - 1, [&](int s, auto SL) {
        lds_barrier();
        constexpr int sl = (decltype(SL)::v + 1) % 2;  // slot of step s + 1
        if (s + 1 < Nc) {
          const int ch = Nc - 2 - s;
          const int nr = rows_of(ch);
          const int64_t t0 = (int64_t)ch * BT;
          unsigned char *xt = (isk ? sm.k[sl] : sm.q[sl]) + 1024 * i0;
          if (nr == BT) {
            const unsigned char *xg = reinterpret_cast<const unsigned char *>(xb + t0 * st);
#pragma unroll
            for (int i = 0; i < NH; ++i) g2l16(xg + xoff[i], xt + 1024 * i);
          } else {
            // partial chunk: rows past its end repeat its last row
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
        lds_barrier();  // B1
        wait_vm<0>();
      });
      lds_barrier();
    } else {
      constexpr int NRH = NR / 2;
      const int half = role - 4;
      const T *ob = static_cast<const T *>(p.d_o) + brow * p.sdo_b + h * p.sdo_h + j0 + bos * p.sdo_t;
      for_steps2(Nc - 1, [&](int s, auto SL) {
        lds_barrier();
        constexpr int sl = (decltype(SL)::v + 1) % 2;
        if (s + 1 < Nc) {
          const int ch = Nc - 2 - s;
          const int nr = rows_of(ch);
          const int64_t t0 = (int64_t)ch * BT;
          const unsigned char *rg = p.brec + ((gc0 + ch) * p.Hv + h) * kBrBytes + kBrF + 1024 * NRH * half;
#pragma unroll
          for (int i = 0; i < NRH; ++i) g2l16(rg + 1024 * i + 16 * lane, sm.rec[sl] + 1024 * (NRH * half + i));
          // dO rows past the chunk's end repeat its last row (their factors are 0)
          const int r = 32 * half + (lane >> 1);
          const int rr = r < nr ? r : nr - 1;
          g2l16(ob + (t0 + rr) * p.sdo_t + 8 * (lane & 1),
                reinterpret_cast<unsigned char *>(sm.o[sl]) + 1024 * half);
        }
        lds_barrier();  // B1
        wait_vm<0>();
      });
      lds_barrier();
    }
  }
}

// ---------------------------------------------------------------------------
// Forward-state pass: per (sequence, value head, 16 value rows), serial over
// the chunks in order, the state S (16 x dk) is carried in FP32 MFMA
// accumulators and each chunk gives (raw 16-bit k rows, factors from the
// record)
//
//   U = K S^T,   R = V - (e^gamma rk) (.) U,   Delta = M (beta (.) R)
//   S <- e^{gamma_C} S + K^T ((cw rk) (.) Delta)
//
// writing S0 (the state entering the chunk), R and Delta in FP32 for the
// gradient kernel. Split operands as in the reverse pass. Wavefronts: 0 the
// chain; 1 stores the previous step's R and Delta from a two-slot LDS stage;
// 2-7 copy the k tile, the v slice and the record's [0, kBrMtH) part of the
// chunk two steps ahead into a three-slot ring (one barrier per step).
// ---------------------------------------------------------------------------
template <typename T, int DK>
struct StLds {
  static constexpr int RB = DK * 2;
  static constexpr int TILE = BT * RB;
  alignas(16) unsigned char k[3][TILE];
  alignas(16) T v[3][BT * DVT];
  alignas(16) unsigned char rec[3][kBrMtH];
  alignas(16) float stage[2][2 * 4 * 64 * 4];  // R, then Delta, [mt][lane][4]
};

// Runs body(s, Slot<s mod 3>) for s = -2 .. last in order.
template <typename F>
__device__ __forceinline__ void for_steps3(int last, F &&body) {
  for (int base = -3; base <= last; base += 3) {
    if (base >= -2) body(base, Slot<0>{});
    if (base + 1 >= -2 && base + 1 <= last) body(base + 1, Slot<1>{});
    if (base + 2 <= last) body(base + 2, Slot<2>{});
  }
}

template <typename T, int DK>
__device__ __forceinline__ void states_pass(const ChunkBwdArgs &p, int64_t bid) {
  using SM = StLds<T, DK>;
  SM &sm = *reinterpret_cast<SM *>(g_pass_lds);
  using f8 = typename M2<T>::f8;
  using v4 = typename M2<T>::v4;
  constexpr int KT = DK / 32, NT = DK / 16, RB = SM::RB;
  constexpr int NI = SM::TILE / 1024;        // 1 KB copies per k tile
  constexpr int NR = (int)(kBrMtH / 1024);   // 1 KB copies per record part
  static_assert(NI % 4 == 0 && NR % 2 == 0, "copy split");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t ntile = p.dv / DVT, nwg = ntile * p.Hv * p.n_seqs;
  int64_t lid = bid;
  if (nwg % 8 == 0) lid = (lid % 8) * (nwg / 8) + lid / 8;
  const int64_t j0 = (lid % ntile) * DVT;
  const int64_t h = (lid / ntile) % p.Hv;
  const int64_t n = lid / (ntile * p.Hv);
  const int64_t hk = h / (p.Hv / p.Hqk);
  int64_t brow, bos, L, gc0;
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
  const int Nc = (int)((L + BT - 1) / BT);
  auto rows_of = [&](int ch) -> int {
    const int64_t r = L - (int64_t)ch * BT;
    return (int)(r < BT ? r : BT);
  };
  const int64_t st_base = ((n * p.Hv + h) * p.dv + j0) * DK;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  if (wave == 0) {
    // ---------------------------------------------------------------- chain
    int fo[KT];
#pragma unroll
    for (int pp = 0; pp < KT; ++pp) fo[pp] = c * RB + (((4 * pp + g) ^ kswz<DK>(c)) << 4);
    const int yrow = 4 * g + (c >> 2);
    int trc[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
      trc[mt] = yrow * RB + (((4 * (mt >> 1) + (c & 3)) ^ kswz<DK>(yrow)) << 4) + 8 * (mt & 1);
    const int vtr = (4 * g + (c >> 2)) * (DVT * 2) + 8 * (c & 3);
    f32x4 S[NT];  // S[mt][i] = S[dv row c][dk dk_of(mt, 4 g + i)]
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[mt][i] = p.init_state ? p.init_state[st_base + (int64_t)c * DK + dk_of(mt, 4 * g + i)] : 0.f;
    for_steps3(Nc, [&](int s, auto SL) {
      lds_barrier();
      if (s < 0 || s >= Nc) return;
      constexpr int sl = decltype(SL)::v;
      const int64_t gc = gc0 + s;
      const unsigned char *kt = sm.k[sl], *rec = sm.rec[sl];
      const float *fa = reinterpret_cast<const float *>(rec + kBrF);
      // U = K S^T. Every LDS fragment of a product is read before the
      // VALU work that precedes it, so that the reads overlap that work
      // instead of feeding the products one at a time.
      f32x4 U[4];
      {
        f8 kfr[4][KT];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int pp = 0; pp < KT; ++pp) kfr[mt][pp] = *reinterpret_cast<const f8 *>(kt + mt * 16 * RB + fo[pp]);
        f8 Sh[KT], Sl[KT];
#pragma unroll
        for (int pp = 0; pp < KT; ++pp) split2x4<T>(S[2 * pp], S[2 * pp + 1], Sh[pp], Sl[pp]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 u = zero4;
#pragma unroll
          for (int pp = 0; pp < KT; ++pp) {
            u = mma<T>(kfr[mt][pp], Sh[pp], u);
            u = mma<T>(kfr[mt][pp], Sl[pp], u);
          }
          U[mt] = u;
        }
      }
      // the M fragments and the K^T fragments of the update
      f8 mfh[6], mfl[6], kTr[NT][2];
#pragma unroll
      for (int fi = 0; fi < 6; ++fi) {
        mfh[fi] = *reinterpret_cast<const f8 *>(rec + kBrMH + fi * 1024 + lane * 16);
        mfl[fi] = *reinterpret_cast<const f8 *>(rec + kBrML + fi * 1024 + lane * 16);
      }
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const unsigned char *ka1 = kt + trc[mt] + (32 * q) * RB, *ka2 = kt + trc[mt] + (32 * q + 16) * RB;
          const s16x4 k1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(ka1));
          const s16x4 k2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(ka2));
          kTr[mt][q] = cat8<T>(__builtin_bit_cast(v4, k1), __builtin_bit_cast(v4, k2));
        }
      {  // S0 to the workspace ([dv][dk]), after the products (the stores do
         // not wait behind the step's copies)
        float *sw = p.s0 + ((gc * p.Hv + h) * p.dv + j0 + c) * DK;
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) *reinterpret_cast<f32x4 *>(sw + dk_of(mt, 4 * g)) = S[mt];
      }
      // R = V - e^gamma rk (.) U; X = beta (.) R
      f8 Bv[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const unsigned char *vb = reinterpret_cast<const unsigned char *>(sm.v[sl]) + vtr + 32 * q * (DVT * 2);
        const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(vb));
        const s16x4 r1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(vb + 16 * DVT * 2));
        Bv[q] = cat8<T>(__builtin_bit_cast(v4, r0), __builtin_bit_cast(v4, r1));
      }
      float *stg = sm.stage[s & 1];
      f32x4 X[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 er = *reinterpret_cast<const f32x4 *>(&fa[6 * BT + 16 * mt + 4 * g]);
        const f32x4 bt = *reinterpret_cast<const f32x4 *>(&fa[2 * BT + 16 * mt + 4 * g]);
        f32x4 vv;
#pragma unroll
        for (int i = 0; i < 4; ++i) vv[i] = f(Bv[mt >> 1][4 * (mt & 1) + i]);
        const f32x4 r = vv - er * U[mt];
        *reinterpret_cast<f32x4 *>(&stg[(mt * 64 + lane) * 4]) = r;
        X[mt] = bt * r;
      }
      // Delta = M X
      f32x4 Dl4[4];
      {
        f8 Xh[2], Xl[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) split2x4<T>(X[2 * q], X[2 * q + 1], Xh[q], Xl[q]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 d = zero4;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            if (q == 1 && mt < 2) continue;
            const int fi = q == 0 ? mt : 2 + mt;
            d = mma<T>(mfh[fi], Xh[q], d);
            d = mma<T>(mfh[fi], Xl[q], d);
            d = mma<T>(mfl[fi], Xh[q], d);
          }
          Dl4[mt] = d;
          *reinterpret_cast<f32x4 *>(&stg[((4 + mt) * 64 + lane) * 4]) = d;
        }
      }
      // S = e^{gamma_C} S + K^T (cw rk (.) Delta)
      f8 Bwh[2], Bwl[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f32x4 c0 = *reinterpret_cast<const f32x4 *>(&fa[1 * BT + 32 * q + 4 * g]);
        const f32x4 c1 = *reinterpret_cast<const f32x4 *>(&fa[1 * BT + 32 * q + 16 + 4 * g]);
        split2x4<T>(c0 * Dl4[2 * q], c1 * Dl4[2 * q + 1], Bwh[q], Bwl[q]);
      }
      const float eC = fa[5 * BT];
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        f32x4 a = S[mt] * eC;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          a = mma<T>(kTr[mt][q], Bwh[q], a);
          a = mma<T>(kTr[mt][q], Bwl[q], a);
        }
        S[mt] = a;
      }
    });
  } else if (wave == 1) {
    // ------------------------------------ R and Delta of the previous step
    for_steps3(Nc, [&](int s, auto) {
      lds_barrier();
      const int ch = s - 1;
      if (ch < 0 || ch >= Nc) return;
      const float *stg = sm.stage[ch & 1];
      const int64_t gc = gc0 + ch;
      const int t = lane, mt = t >> 4, gg = (t >> 2) & 3, i = t & 3;
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        if (a == 0 && p.rr == nullptr) continue;  // R not kept (the gradient kernel recomputes it)
        float x[16];
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) x[cc] = stg[((4 * a + mt) * 64 + 16 * gg + cc) * 4 + i];
        float *dst = (a == 0 ? p.rr : p.del) + ((gc * p.Hv + h) * BT + t) * p.dv + j0;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          *reinterpret_cast<f32x4 *>(dst + 4 * v) = f32x4{x[4 * v], x[4 * v + 1], x[4 * v + 2], x[4 * v + 3]};
      }
    });
  } else {
    // ------------------------------------------------------------- loads
    // waves 2-5: quarters of the k tile; waves 6, 7: halves of the record
    // part and of the v slice; for the chunk of step s + 2
    const int role = wave - 2;
    if (role < 4) {
      constexpr int NQ = NI / 4;
      const int i0 = role * NQ;
      const T *xb = static_cast<const T *>(p.k) + brow * p.sk_b + hk * p.sk_h + bos * p.sk_t;
      uint32_t xoff[NQ];
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const int b = 1024 * (i0 + i) + 16 * lane;
        const int r = b / RB, jp = (b % RB) >> 4;
        const int j = jp ^ kswz<DK>(r);
        xoff[i] = (uint32_t)(((int64_t)r * p.sk_t + 8 * j) * 2);
      }
      for_steps3(Nc, [&](int s, auto SL) {
        lds_barrier();
        constexpr int sl = (decltype(SL)::v + 2) % 3;
        const int cl = s + 2;
        const bool issue = cl < Nc;
        if (issue) {
          const int nr = rows_of(cl);
          const int64_t t0 = (int64_t)cl * BT;
          unsigned char *xt = sm.k[sl] + 1024 * i0;
          if (nr == BT) {
            const unsigned char *xg = reinterpret_cast<const unsigned char *>(xb + t0 * p.sk_t);
#pragma unroll
            for (int i = 0; i < NQ; ++i) g2l16(xg + xoff[i], xt + 1024 * i);
          } else {
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
              const int b = 1024 * (i0 + i) + 16 * lane;
              const int r = b / RB, jp = (b % RB) >> 4;
              const int j = jp ^ kswz<DK>(r);
              const int rr = r < nr ? r : nr - 1;
              g2l16(xb + (t0 + rr) * p.sk_t + 8 * j, xt + 1024 * i);
            }
          }
        }
        // the previous step's copies are complete before the next barrier
        if (issue) wait_vm<NQ>(); else wait_vm<0>();
      });
    } else {
      constexpr int NRH = NR / 2;
      const int half = role - 4;
      const T *vb = static_cast<const T *>(p.v) + brow * p.sv_b + h * p.sv_h + j0 + bos * p.sv_t;
      for_steps3(Nc, [&](int s, auto SL) {
        lds_barrier();
        constexpr int sl = (decltype(SL)::v + 2) % 3;
        const int cl = s + 2;
        const bool issue = cl < Nc;
        if (issue) {
          const int nr = rows_of(cl);
          const int64_t t0 = (int64_t)cl * BT;
          const unsigned char *rg = p.brec + ((gc0 + cl) * p.Hv + h) * kBrBytes + 1024 * NRH * half;
#pragma unroll
          for (int i = 0; i < NRH; ++i) g2l16(rg + 1024 * i + 16 * lane, sm.rec[sl] + 1024 * (NRH * half + i));
          // v rows past the chunk's end repeat its last row (beta is 0 there)
          const int r = 32 * half + (lane >> 1);
          const int rr = r < nr ? r : nr - 1;
          g2l16(vb + (t0 + rr) * p.sv_t + 8 * (lane & 1), reinterpret_cast<unsigned char *>(sm.v[sl]) + 1024 * half);
        }
        if (issue) wait_vm<NRH + 1>(); else wait_vm<0>();
      });
    }
  }
}

// ---------------------------------------------------------------------------
// Multi-slice forward-state pass, for launches with many (sequence, head)
// pairs: one workgroup = (sequence, value head, NS * 16 value rows). One
// copy of the k tile and of the record's [0, kBrMtH) part serves NS chains;
// waves 0 .. NS - 1 each carry one 16-row slice through the chain of
// the one-slice pass, states_pass (the same products in the same order), and store its
// S0, R and Delta themselves; the four waves after them copy the halves of
// the k tile, the record part and the [64][16 NS] v tile of the next chunk
// into two-slot rings (one barrier per step; a chain step is longer than the
// copies' latency, so one step of look-ahead suffices, and the rings stay
// small enough for LDS offsets without extra address registers). NS is 2
// or 4; waves past NS + 4 (the launch's workgroups are sized for the reverse
// pass) only take part in the barriers.
// ---------------------------------------------------------------------------
template <typename T, int DK, int NS>
struct StMLds {
  static constexpr int RB = DK * 2;
  static constexpr int TILE = BT * RB;
  static constexpr int VB = NS * DVT * 2;  // bytes per v row
  alignas(16) unsigned char k[2][TILE];
  alignas(16) unsigned char v[2][BT * VB];
  alignas(16) unsigned char rec[2][kBrMtH];
};

template <typename T, int DK, int NS>
__device__ __forceinline__ void states_multi_pass(const ChunkBwdArgs &p, int64_t bid) {
  using SM = StMLds<T, DK, NS>;
  SM &sm = *reinterpret_cast<SM *>(g_pass_lds);
  using f8 = typename M2<T>::f8;
  using v4 = typename M2<T>::v4;
  constexpr int KT = DK / 32, NT = DK / 16, RB = SM::RB, VB = SM::VB;
  constexpr int NI = SM::TILE / 1024;        // 1 KB copies per k tile
  constexpr int NR = (int)(kBrMtH / 1024);   // 1 KB copies per record part
  constexpr int NV = BT * VB / 1024;         // 1 KB copies per v tile
  constexpr int LV = VB / 16;                // lanes per v row in a copy
  static_assert(NI % 2 == 0 && NI / 2 <= 16 && NR <= 16 && NV <= 16, "copies per loader wave");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t ntile = p.dv / (NS * DVT), nwg = ntile * p.Hv * p.n_seqs;
  int64_t lid = bid;
  if (nwg % 8 == 0) lid = (lid % 8) * (nwg / 8) + lid / 8;
  const int64_t jg = (lid % ntile) * (NS * DVT);
  const int64_t h = (lid / ntile) % p.Hv;
  const int64_t n = lid / (ntile * p.Hv);
  const int64_t hk = h / (p.Hv / p.Hqk);
  int64_t brow, bos, L, gc0;
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
  const int Nc = (int)((L + BT - 1) / BT);
  auto rows_of = [&](int ch) -> int {
    const int64_t r = L - (int64_t)ch * BT;
    return (int)(r < BT ? r : BT);
  };
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  if (wave >= NS + 4) {
    // waves beyond this pass's own (the launch's block also serves the
    // reverse pass): they only take part in the barriers
    for_steps2(Nc - 1, [&](int, auto) { lds_barrier(); });
    return;
  }
  if (wave < NS) {
    // ------------------------------------------------ the chain of one slice
    const int64_t j0 = jg + DVT * wave;
    const int64_t st_base = ((n * p.Hv + h) * p.dv + j0) * DK;
    int fo[KT];
#pragma unroll
    for (int pp = 0; pp < KT; ++pp) fo[pp] = c * RB + (((4 * pp + g) ^ kswz<DK>(c)) << 4);
    const int yrow = 4 * g + (c >> 2);
    int trc[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
      trc[mt] = yrow * RB + (((4 * (mt >> 1) + (c & 3)) ^ kswz<DK>(yrow)) << 4) + 8 * (mt & 1);
    const int vtr = (4 * g + (c >> 2)) * VB + 2 * DVT * wave + 8 * (c & 3);
    f32x4 S[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[mt][i] = p.init_state ? p.init_state[st_base + (int64_t)c * DK + dk_of(mt, 4 * g + i)] : 0.f;
    if (Nc > 0) {  // S0 of the first chunk
      float *sw = p.s0 + ((gc0 * p.Hv + h) * p.dv + j0 + c) * DK;
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) *reinterpret_cast<f32x4 *>(sw + dk_of(mt, 4 * g)) = S[mt];
    }
    for_steps2(Nc - 1, [&](int s, auto SL) {
      lds_barrier();
      if (s < 0) return;
      constexpr int sl = decltype(SL)::v;
      const int64_t gc = gc0 + s;
      const unsigned char *kt = sm.k[sl], *rec = sm.rec[sl];
      const float *fa = reinterpret_cast<const float *>(rec + kBrF);
      // U = K S^T
      f32x4 U[4];
      {
        f8 kfr[4][KT];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int pp = 0; pp < KT; ++pp) kfr[mt][pp] = *reinterpret_cast<const f8 *>(kt + mt * 16 * RB + fo[pp]);
        f8 Sh[KT], Sl[KT];
#pragma unroll
        for (int pp = 0; pp < KT; ++pp) split2x4<T>(S[2 * pp], S[2 * pp + 1], Sh[pp], Sl[pp]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 u = zero4;
#pragma unroll
          for (int pp = 0; pp < KT; ++pp) {
            u = mma<T>(kfr[mt][pp], Sh[pp], u);
            u = mma<T>(kfr[mt][pp], Sl[pp], u);
          }
          U[mt] = u;
        }
      }
      f8 mfh[6], mfl[6], kTr[NT][2];
#pragma unroll
      for (int fi = 0; fi < 6; ++fi) {
        mfh[fi] = *reinterpret_cast<const f8 *>(rec + kBrMH + fi * 1024 + lane * 16);
        mfl[fi] = *reinterpret_cast<const f8 *>(rec + kBrML + fi * 1024 + lane * 16);
      }
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const unsigned char *ka1 = kt + trc[mt] + (32 * q) * RB, *ka2 = kt + trc[mt] + (32 * q + 16) * RB;
          const s16x4 k1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(ka1));
          const s16x4 k2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(ka2));
          kTr[mt][q] = cat8<T>(__builtin_bit_cast(v4, k1), __builtin_bit_cast(v4, k2));
        }
      // R = V - e^gamma rk (.) U; X = beta (.) R
      f8 Bv[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const unsigned char *vb = sm.v[sl] + vtr + 32 * q * VB;
        const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(vb));
        const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(vb + 16 * VB));
        Bv[q] = cat8<T>(__builtin_bit_cast(v4, r0), __builtin_bit_cast(v4, r1));
      }
      // R and Delta rows of this slice: lane (g, c) holds rows 16 mt + 4 g + i
      // of column c; each store writes 64 contiguous bytes per row. The row
      // offsets (16 mt + i) dv are uniform, the lane's 4 g dv part is in its
      // base pointer (no per-row addresses held across steps).
      const int64_t dvs = p.dv;
      float *rrow = p.rr + ((gc * p.Hv + h) * BT + 4 * g) * dvs + j0 + c;
      float *drow = p.del + ((gc * p.Hv + h) * BT + 4 * g) * dvs + j0 + c;
      f32x4 X[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 er = *reinterpret_cast<const f32x4 *>(&fa[6 * BT + 16 * mt + 4 * g]);
        const f32x4 bt = *reinterpret_cast<const f32x4 *>(&fa[2 * BT + 16 * mt + 4 * g]);
        f32x4 vv;
#pragma unroll
        for (int i = 0; i < 4; ++i) vv[i] = f(Bv[mt >> 1][4 * (mt & 1) + i]);
        const f32x4 r = vv - er * U[mt];
        if (p.rr != nullptr) {  // R kept only for the FP32 gradient kernel
#pragma unroll
          for (int i = 0; i < 4; ++i) rrow[(16 * mt + i) * dvs] = r[i];
        }
        X[mt] = bt * r;
      }
      // Delta = M X
      f32x4 Dl4[4];
      {
        f8 Xh[2], Xl[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) split2x4<T>(X[2 * q], X[2 * q + 1], Xh[q], Xl[q]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 d = zero4;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            if (q == 1 && mt < 2) continue;
            const int fi = q == 0 ? mt : 2 + mt;
            d = mma<T>(mfh[fi], Xh[q], d);
            d = mma<T>(mfh[fi], Xl[q], d);
            d = mma<T>(mfl[fi], Xh[q], d);
          }
          Dl4[mt] = d;
#pragma unroll
          for (int i = 0; i < 4; ++i) drow[(16 * mt + i) * dvs] = d[i];
        }
      }
      // S = e^{gamma_C} S + K^T (cw rk (.) Delta)
      f8 Bwh[2], Bwl[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f32x4 c0 = *reinterpret_cast<const f32x4 *>(&fa[1 * BT + 32 * q + 4 * g]);
        const f32x4 c1 = *reinterpret_cast<const f32x4 *>(&fa[1 * BT + 32 * q + 16 + 4 * g]);
        split2x4<T>(c0 * Dl4[2 * q], c1 * Dl4[2 * q + 1], Bwh[q], Bwl[q]);
      }
      const float eC = fa[5 * BT];
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        f32x4 a = S[mt] * eC;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          a = mma<T>(kTr[mt][q], Bwh[q], a);
          a = mma<T>(kTr[mt][q], Bwl[q], a);
        }
        S[mt] = a;
      }
      // the state just formed is S0 of the next chunk: stored at the end of
      // the step, after the step's copies have drained from the CU's memory
      // queue
      if (s + 1 < Nc) {
        float *sw = p.s0 + (((gc + 1) * p.Hv + h) * p.dv + j0 + c) * DK;
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) *reinterpret_cast<f32x4 *>(sw + dk_of(mt, 4 * g)) = S[mt];
      }
    });
  } else {
    // ------------------------------------------------------------- loads
    // waves NS, NS + 1: halves of the k tile; NS + 2: the record part;
    // NS + 3: the v tile; for the chunk of step s + 1, complete before the
    // next barrier
    const int role = wave - NS;
    const T *xb = static_cast<const T *>(p.k) + brow * p.sk_b + hk * p.sk_h + bos * p.sk_t;
    const T *vb = static_cast<const T *>(p.v) + brow * p.sv_b + h * p.sv_h + jg + bos * p.sv_t;
    for_steps2(Nc - 1, [&](int s, auto SL) {
      lds_barrier();
      constexpr int sl = (decltype(SL)::v + 1) % 2;
      const int cl = s + 1;
      const bool issue = cl < Nc;
      if (issue) {
        const int nr = rows_of(cl);
        const int64_t t0 = (int64_t)cl * BT;
        if (role < 2) {
          constexpr int NH = NI / 2;
#pragma unroll
          for (int i = 0; i < NH; ++i) {
            const int b = 1024 * (role * NH + i) + 16 * lane;
            const int r = b / RB, jp = (b % RB) >> 4;
            const int j = jp ^ kswz<DK>(r);
            const int rr = r < nr ? r : nr - 1;
            g2l16(xb + (t0 + rr) * p.sk_t + 8 * j, sm.k[sl] + 1024 * (role * NH + i));
          }
        } else if (role == 2) {
          const unsigned char *rg = p.brec + ((gc0 + cl) * p.Hv + h) * kBrBytes;
#pragma unroll
          for (int i = 0; i < NR; ++i) g2l16(rg + 1024 * i + 16 * lane, sm.rec[sl] + 1024 * i);
        } else {
          // v rows past the chunk's end repeat its last row (beta is 0 there)
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

// ---------------------------------------------------------------------------
// Multi-slice reverse pass, for launches with many (sequence, head) pairs and
// for running beside the forward-state pass: one workgroup = (sequence, value
// head, NS * 16 value rows). One copy of the k and q tiles and of the
// record's reverse part serves NS slices. Waves 0 .. NS - 1 carry the chain
// of the one-slice pass, dstate_pass, for one slice each (the same products in the same
// order), waves NS .. 2 NS - 1 are their helpers (G = P'^T dO, the q term,
// the dR' and dv stores); the last four waves copy the k tile, the q tile and
// the halves of the record part and of the [64][16 NS] dO tile of the next
// chunk into two-slot rings. Two barriers per step as in the one-slice
// kernel. The dR' hand-off has one slot per slice: a helper reads the
// previous step's stage before the middle barrier, after which its chain
// writes the next one.
// ---------------------------------------------------------------------------
template <typename T, int DK, int NS>
struct DsMLds {
  static constexpr int RB = DK * 2;
  static constexpr int TILE = BT * RB;
  static constexpr int VB = NS * DVT * 2;  // bytes per dO row
  alignas(16) unsigned char k[2][TILE];
  alignas(16) unsigned char q[2][TILE];
  alignas(16) unsigned char o[2][BT * VB];
  alignas(16) unsigned char rec[2][kDsRec];
  alignas(16) float gg[NS][4 * 64 * 4];        // G of each slice, [mt][lane][4]
  alignas(16) float hq[NS][DK / 16 * 64 * 4];  // q term of each slice, [mt][lane][4]
  alignas(16) float stage[NS][4 * 64 * 4 + 64];  // dR' [mt][lane][4], then beta
};

template <typename T, int DK, int NS>
__device__ __forceinline__ void dstate_multi_pass(const ChunkBwdArgs &p, int64_t bid) {
  using SM = DsMLds<T, DK, NS>;
  SM &sm = *reinterpret_cast<SM *>(g_pass_lds);
  using f8 = typename M2<T>::f8;
  using v4 = typename M2<T>::v4;
  constexpr int KT = DK / 32, NT = DK / 16, RB = SM::RB, VB = SM::VB;
  constexpr int NI = SM::TILE / 1024;       // 1 KB copies per q/k tile
  constexpr int NR = (int)(kDsRec / 1024);  // 1 KB copies per record part
  constexpr int NO = BT * VB / 1024;        // 1 KB copies per dO tile
  constexpr int LV = VB / 16;               // lanes per dO row in a copy
  static_assert(NI <= 31 && NR % 2 == 0 && NO % 2 == 0 && NR / 2 + NO / 2 <= 31, "copies per loader wave");
  static_assert(sizeof(SM) <= 160 * 1024, "LDS");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t ntile = p.dv / (NS * DVT), nwg = ntile * p.Hv * p.n_seqs;
  int64_t lid = bid;
  if (nwg % 8 == 0) lid = (lid % 8) * (nwg / 8) + lid / 8;
  const int64_t jg = (lid % ntile) * (NS * DVT);
  const int64_t h = (lid / ntile) % p.Hv;
  const int64_t n = lid / (ntile * p.Hv);
  const int64_t hk = h / (p.Hv / p.Hqk);
  int64_t brow, bos, L, gc0;
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
  const int Nc = (int)((L + BT - 1) / BT);
  // step s works on chunk Nc - 1 - s
  auto rows_of = [&](int ch) -> int {
    const int64_t r = L - (int64_t)ch * BT;
    return (int)(r < BT ? r : BT);
  };
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  if (wave < 2 * NS) {
    const int sw = wave < NS ? wave : wave - NS;  // the slice of this wave
    const int64_t j0 = jg + DVT * sw;
    const int64_t st_base = ((n * p.Hv + h) * p.dv + j0) * DK;
    float *const gq = sm.gg[sw];
    float *const hq = sm.hq[sw];
    float *const stg = sm.stage[sw];
    const int yrow = 4 * g + (c >> 2);
    int trc[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
      trc[mt] = yrow * RB + (((4 * (mt >> 1) + (c & 3)) ^ kswz<DK>(yrow)) << 4) + 8 * (mt & 1);
    if (wave < NS) {
      // -------------------------------------------------------------- chain
      int fo[KT];
#pragma unroll
      for (int pp = 0; pp < KT; ++pp) fo[pp] = c * RB + (((4 * pp + g) ^ kswz<DK>(c)) << 4);
      f32x4 dS[NT];  // dS[mt][i] = dS[dv row c][dk dk_of(mt, 4 g + i)]
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dS[mt][i] = p.d_final ? p.d_final[st_base + (int64_t)c * DK + dk_of(mt, 4 * g + i)] : 0.f;

      for_steps2(Nc - 1, [&](int s, auto SL) {
        lds_barrier();  // B0
        constexpr int sl = decltype(SL)::v;
        const int ch = Nc - 1 - s;
        const int64_t gc = gc0 + ch;
        const unsigned char *kt = sm.k[sl], *rec = sm.rec[sl];
        const float *fa = reinterpret_cast<const float *>(rec + kDsF);
        f32x4 U[4];
        f8 mth[6], mtl[6], kTr[NT][2];
        if (s >= 0) {
          // U = K dS^T, with the q term of the previous step added first
          f8 kfr[4][KT];
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int pp = 0; pp < KT; ++pp) kfr[mt][pp] = *reinterpret_cast<const f8 *>(kt + mt * 16 * RB + fo[pp]);
          if (s > 0) {
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) dS[mt] += *reinterpret_cast<const f32x4 *>(&hq[(mt * 64 + lane) * 4]);
          }
          f8 Sh[KT], Sl[KT];
#pragma unroll
          for (int pp = 0; pp < KT; ++pp) split2x4<T>(dS[2 * pp], dS[2 * pp + 1], Sh[pp], Sl[pp]);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            f32x4 u = zero4;
#pragma unroll
            for (int pp = 0; pp < KT; ++pp) {
              u = mma<T>(kfr[mt][pp], Sh[pp], u);
              u = mma<T>(kfr[mt][pp], Sl[pp], u);
            }
            U[mt] = u;
          }
#pragma unroll
          for (int f = 0; f < 6; ++f) {
            mth[f] = *reinterpret_cast<const f8 *>(rec + kDsMtH + f * 1024 + lane * 16);
            mtl[f] = *reinterpret_cast<const f8 *>(rec + kDsMtL + f * 1024 + lane * 16);
          }
#pragma unroll
          for (int mt = 0; mt < NT; ++mt)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const unsigned char *ka1 = kt + trc[mt] + (32 * q) * RB, *ka2 = kt + trc[mt] + (32 * q + 16) * RB;
              const s16x4 k1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(ka1));
              const s16x4 k2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(ka2));
              kTr[mt][q] = cat8<T>(__builtin_bit_cast(v4, k1), __builtin_bit_cast(v4, k2));
            }
        }
        lds_barrier();  // B1: G of this chunk is in LDS, the stage has been read
        if (s < 0) return;
        {  // dS_C to the workspace (as [dv][dk]); issued after the middle
           // barrier, when the step's copies no longer fill the CU's memory
           // queue that the stores would wait behind
          float *dsw = p.ds + ((gc * p.Hv + h) * p.dv + j0 + c) * DK;
#pragma unroll
          for (int mt = 0; mt < NT; ++mt) *reinterpret_cast<f32x4 *>(dsw + dk_of(mt, 4 * g)) = dS[mt];
        }
        f32x4 dD[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const f32x4 cr = *reinterpret_cast<const f32x4 *>(&fa[1 * BT + 16 * mt + 4 * g]);
          dD[mt] = U[mt] * cr + *reinterpret_cast<const f32x4 *>(&gq[(mt * 64 + lane) * 4]);
        }
        f32x4 dR[4];
        {
          f8 Dh[2], Dl[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) split2x4<T>(dD[2 * q], dD[2 * q + 1], Dh[q], Dl[q]);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            f32x4 r = zero4;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              if (q == 0 && mt >= 2) continue;
              const int f = up_frag(mt, q);
              r = mma<T>(mth[f], Dh[q], r);
              r = mma<T>(mth[f], Dl[q], r);
              r = mma<T>(mtl[f], Dh[q], r);
            }
            dR[mt] = r;
          }
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) *reinterpret_cast<f32x4 *>(&stg[(mt * 64 + lane) * 4]) = dR[mt];
        stg[4 * 64 * 4 + lane] = fa[2 * BT + lane];
        f8 Fkh[2], Fkl[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f32x4 fk0 = *reinterpret_cast<const f32x4 *>(&fa[4 * BT + 32 * q + 4 * g]);
          const f32x4 fk1 = *reinterpret_cast<const f32x4 *>(&fa[4 * BT + 32 * q + 16 + 4 * g]);
          split2x4<T>(fk0 * dR[2 * q], fk1 * dR[2 * q + 1], Fkh[q], Fkl[q]);
        }
        const float eC = fa[5 * BT];
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
          f32x4 a = dS[mt] * eC;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            a = mma<T>(kTr[mt][q], Fkh[q], a);
            a = mma<T>(kTr[mt][q], Fkl[q], a);
          }
          dS[mt] = a;
        }
      });
      lds_barrier();  // the last q term is in LDS
      if (Nc > 0) {
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) dS[mt] += *reinterpret_cast<const f32x4 *>(&hq[(mt * 64 + lane) * 4]);
      }
      if (p.d_init) {
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
          *reinterpret_cast<f32x4 *>(p.d_init + st_base + (int64_t)c * DK + dk_of(mt, 4 * g)) = dS[mt];
      }
    } else {
      // ---------------------------------------------------------- helper
      // the stage (dR' of the previous step in accumulator layout, then
      // beta) as lane t's row t: x[cc] = dR'[t][j0 + cc]
      auto load_stage = [&](float (&x)[16], float &bt) {
        const int t = lane, mt = t >> 4, gr = (t >> 2) & 3, i = t & 3;
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) x[cc] = stg[(mt * 64 + 16 * gr + cc) * 4 + i];
        bt = stg[4 * 64 * 4 + t];
      };
      // dR' (FP32) and dv = beta dR' of step s2 (chunk Nc - 1 - s2)
      auto store_rows = [&](int s2, float (&x)[16], float bt) {
        const int ch = Nc - 1 - s2;
        const int64_t gc = gc0 + ch, t0 = bos + (int64_t)ch * BT;
        const int nr = rows_of(ch);
        const int t = lane;
        float *dr = p.drp + ((gc * p.Hv + h) * BT + t) * p.dv + j0;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          *reinterpret_cast<f32x4 *>(dr + 4 * v) = f32x4{x[4 * v], x[4 * v + 1], x[4 * v + 2], x[4 * v + 3]};
        if (t < nr) {
          const int64_t o = brow * p.sdv_b + (t0 + t) * p.sdv_t + h * p.dv + j0;
#pragma unroll
          for (int cc = 0; cc < 16; ++cc) x[cc] *= bt;
          if (p.grad_dtype == kF32) {
            float *dv = static_cast<float *>(p.dvv) + o;
#pragma unroll
            for (int v = 0; v < 4; ++v)
              *reinterpret_cast<f32x4 *>(dv + 4 * v) = f32x4{x[4 * v], x[4 * v + 1], x[4 * v + 2], x[4 * v + 3]};
          } else {
            T *dv = static_cast<T *>(p.dvv) + o;
#pragma unroll
            for (int v = 0; v < 4; ++v)
              *reinterpret_cast<v4 *>(dv + 4 * v) =
                  __builtin_convertvector(f32x4{x[4 * v], x[4 * v + 1], x[4 * v + 2], x[4 * v + 3]}, v4);
          }
        }
      };
      const int otr = (4 * g + (c >> 2)) * VB + 2 * DVT * sw + 8 * (c & 3);
      for_steps2(Nc - 1, [&](int s, auto SL) {
        lds_barrier();  // B0
        constexpr int sl = decltype(SL)::v;
        const unsigned char *qt = sm.q[sl], *rec = sm.rec[sl];
        const float *fa = reinterpret_cast<const float *>(rec + kDsF);
        f8 Bo[2];
        float x[16], bt = 0.f;
        if (s >= 1) load_stage(x, bt);
        if (s >= 0) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const unsigned char *ob = sm.o[sl] + otr + 32 * q * VB;
            const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(ob));
            const s16x4 r1 =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(ob + 16 * VB));
            Bo[q] = cat8<T>(__builtin_bit_cast(v4, r0), __builtin_bit_cast(v4, r1));
          }
          // G = P'^T dO in the accumulator layout of dDelta
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            f32x4 a = zero4;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              if (q == 0 && mt >= 2) continue;
              const int f = up_frag(mt, q);
              const f8 ph = *reinterpret_cast<const f8 *>(rec + kDsPH + f * 1024 + lane * 16);
              const f8 pl = *reinterpret_cast<const f8 *>(rec + kDsPL + f * 1024 + lane * 16);
              a = mma<T>(ph, Bo[q], a);
              a = mma<T>(pl, Bo[q], a);
            }
            *reinterpret_cast<f32x4 *>(&gq[(mt * 64 + lane) * 4]) = a;
          }
        }
        lds_barrier();  // B1
        if (s < 0) return;
        // q term Q^T (fq (.) dO), added to dS by the chain at the next step
        f8 Fqh[2], Fql[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f32x4 fq0 = *reinterpret_cast<const f32x4 *>(&fa[3 * BT + 32 * q + 4 * g]);
          const f32x4 fq1 = *reinterpret_cast<const f32x4 *>(&fa[3 * BT + 32 * q + 16 + 4 * g]);
          float xq[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xq[e] = fq0[e] * f(Bo[q][e]);
            xq[4 + e] = fq1[e] * f(Bo[q][4 + e]);
          }
          split8<T>(xq, Fqh[q], Fql[q]);
        }
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
          f32x4 a = zero4;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const unsigned char *qa1 = qt + trc[mt] + (32 * q) * RB, *qa2 = qt + trc[mt] + (32 * q + 16) * RB;
            const s16x4 q1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(qa1));
            const s16x4 q2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(qa2));
            const f8 qT = cat8<T>(__builtin_bit_cast(v4, q1), __builtin_bit_cast(v4, q2));
            a = mma<T>(qT, Fqh[q], a);
            a = mma<T>(qT, Fql[q], a);
          }
          *reinterpret_cast<f32x4 *>(&hq[(mt * 64 + lane) * 4]) = a;
        }
        if (s >= 1) store_rows(s - 1, x, bt);
      });
      lds_barrier();  // the last stage is in LDS
      if (Nc > 0) {
        float x[16], bt;
        load_stage(x, bt);
        store_rows(Nc - 1, x, bt);
      }
    }
  } else {
    // ------------------------------------------------------------- loads
    // role 0 the k tile, 1 the q tile, 2 and 3 the halves of the record part
    // and of the dO tile, for the chunk of step s + 1; complete before the
    // barrier that ends step s
    const int role = wave - 2 * NS;
    if (role < 2) {
      const bool isk = role == 0;
      const int64_t st = isk ? p.sk_t : p.sq_t;
      const T *xb = static_cast<const T *>(isk ? p.k : p.q) + brow * (isk ? p.sk_b : p.sq_b) +
                    hk * (isk ? p.sk_h : p.sq_h) + bos * st;
      uint32_t xoff[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int b = 1024 * i + 16 * lane;
        const int r = b / RB, jp = (b % RB) >> 4;
        const int j = jp ^ kswz<DK>(r);
        xoff[i] = (uint32_t)(((int64_t)r * st + 8 * j) * 2);
      }
      for_steps2(Nc - 1, [&](int s, auto SL) {
        lds_barrier();
        constexpr int sl = (decltype(SL)::v + 1) % 2;  // slot of step s + 1
        if (s + 1 < Nc) {
          const int ch = Nc - 2 - s;
          const int nr = rows_of(ch);
          const int64_t t0 = (int64_t)ch * BT;
          unsigned char *xt = isk ? sm.k[sl] : sm.q[sl];
          if (nr == BT) {
            const unsigned char *xg = reinterpret_cast<const unsigned char *>(xb + t0 * st);
#pragma unroll
            for (int i = 0; i < NI; ++i) g2l16(xg + xoff[i], xt + 1024 * i);
          } else {
            // partial chunk: rows past its end repeat its last row
#pragma unroll
            for (int i = 0; i < NI; ++i) {
              const int b = 1024 * i + 16 * lane;
              const int r = b / RB, jp = (b % RB) >> 4;
              const int j = jp ^ kswz<DK>(r);
              const int rr = r < nr ? r : nr - 1;
              g2l16(xb + (t0 + rr) * st + 8 * j, xt + 1024 * i);
            }
          }
        }
        lds_barrier();  // B1
        wait_vm<0>();
      });
      lds_barrier();
    } else {
      constexpr int NRH = NR / 2, NOH = NO / 2;
      const int half = role - 2;
      const T *ob = static_cast<const T *>(p.d_o) + brow * p.sdo_b + h * p.sdo_h + jg + bos * p.sdo_t;
      for_steps2(Nc - 1, [&](int s, auto SL) {
        lds_barrier();
        constexpr int sl = (decltype(SL)::v + 1) % 2;
        if (s + 1 < Nc) {
          const int ch = Nc - 2 - s;
          const int nr = rows_of(ch);
          const int64_t t0 = (int64_t)ch * BT;
          const unsigned char *rg = p.brec + ((gc0 + ch) * p.Hv + h) * kBrBytes + kBrF + 1024 * NRH * half;
#pragma unroll
          for (int i = 0; i < NRH; ++i) g2l16(rg + 1024 * i + 16 * lane, sm.rec[sl] + 1024 * (NRH * half + i));
          // dO rows past the chunk's end repeat its last row (their factors are 0)
#pragma unroll
          for (int i = 0; i < NOH; ++i) {
            const int ci = NOH * half + i;
            const int r = (64 / LV) * ci + lane / LV;
            const int rr = r < nr ? r : nr - 1;
            g2l16(ob + (t0 + rr) * p.sdo_t + 8 * (lane % LV), sm.o[sl] + 1024 * ci);
          }
        }
        lds_barrier();  // B1
        wait_vm<0>();
      });
      lds_barrier();
    }
  }
}

// A multi-slice form when its pass has at least this many workgroups (half
// the CUs), else the one-slice form.
constexpr int64_t kMultiMinWorkgroups = 128;

// One launch runs both passes: blocks [0, nst) the forward-state pass, the
// rest the reverse pass. The two read only the inputs and the records and
// write disjoint workspace arrays, so they run side by side; with few
// (sequence, head) pairs each takes half of the CUs. NSS / NSR: slices per
// workgroup of each pass (1 = the one-slice kernel's body).
template <int NS> constexpr int states_waves() { return NS == 1 ? kThr / 64 : NS + 4; }
template <int NS> constexpr int reverse_waves() { return NS == 1 ? kThr / 64 : 2 * NS + 4; }
template <int NSS, int NSR> constexpr int pair_waves() {
  return states_waves<NSS>() > reverse_waves<NSR>() ? states_waves<NSS>() : reverse_waves<NSR>();
}
template <typename T, int DK, int NS> struct StatesLds { using type = StMLds<T, DK, NS>; };
template <typename T, int DK> struct StatesLds<T, DK, 1> { using type = StLds<T, DK>; };
template <typename T, int DK, int NS> struct ReverseLds { using type = DsMLds<T, DK, NS>; };
template <typename T, int DK> struct ReverseLds<T, DK, 1> { using type = DsLds<T, DK>; };

template <typename T, int DK, int NSS, int NSR>
__global__ __launch_bounds__((pair_waves<NSS, NSR>() * 64)) void bwd_state_passes_kernel(ChunkBwdArgs p, int64_t nst) {
  // only the forward-state pass may have spare waves (its barrier-only waves)
  static_assert(reverse_waves<NSR>() == pair_waves<NSS, NSR>(), "reverse pass sets the block size");
  static_assert(NSS > 1 || states_waves<NSS>() == pair_waves<NSS, NSR>(), "one-slice state pass: no spare waves");
  // blocks [0, nst) run the forward-state pass, the rest the reverse pass;
  // nst is a multiple of 8 whenever Hv is, so each pass's workgroup index
  // keeps its block's XCD (index mod 8 = block mod 8)
  const int64_t b = blockIdx.x;
  const bool states = b < nst;
  const int64_t idx = states ? b : b - nst;
  if (states) {
    if constexpr (NSS == 1) states_pass<T, DK>(p, idx);
    else states_multi_pass<T, DK, NSS>(p, idx);
  } else {
    if constexpr (NSR == 1) dstate_pass<T, DK>(p, idx);
    else dstate_multi_pass<T, DK, NSR>(p, idx);
  }
}

// A kernel whose dynamic LDS exceeds 64 KB states its size as a function
// attribute (no allocation), once per kernel instance and device.
constexpr int kMaxDevices = 64;
template <typename K>
hipError_t lds_limit(K kernel, size_t bytes) {
  static std::atomic<bool> set[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (set[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)bytes);
  if (e == hipSuccess) set[dev].store(true, std::memory_order_release);
  return e;
}

template <typename T, int DK, int NSS, int NSR>
hipError_t launch_pair(const ChunkBwdArgs &a, hipStream_t s) {
  const int64_t pairs = a.n_seqs * a.Hv;
  const int64_t nst = pairs * (a.dv / (NSS * DVT)), nrv = pairs * (a.dv / (NSR * DVT));
  constexpr size_t bs = sizeof(typename StatesLds<T, DK, NSS>::type), br = sizeof(typename ReverseLds<T, DK, NSR>::type);
  constexpr size_t bytes = bs > br ? bs : br;
  const hipError_t e = lds_limit(bwd_state_passes_kernel<T, DK, NSS, NSR>, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_state_passes_kernel<T, DK, NSS, NSR>), dim3((unsigned)(nst + nrv)),
                     dim3(pair_waves<NSS, NSR>() * 64), bytes, s, a, nst);
  return hipGetLastError();
}

}  // namespace

// BF16 or FP16 activations, dk 64 or 128, dv a multiple of 16; q, k, v and
// d_o rows 16-byte aligned (LDS DMA copies), dv rows aligned to 4 elements.
bool chunk_bwd_state_mma_supported(const ChunkBwdArgs &a) {
  if ((a.act != kBF16 && a.act != kF16) || !(a.dk == 64 || a.dk == 128) || a.dv % 16 != 0) return false;
  const uint64_t vva = (uint64_t)(uintptr_t)a.v | (uint64_t)(a.sv_b * 2) | (uint64_t)(a.sv_t * 2) | (uint64_t)(a.sv_h * 2);
  if (align_of_host(vva) < 16) return false;
  const uint64_t qa = (uint64_t)(uintptr_t)a.q | (uint64_t)(a.sq_b * 2) | (uint64_t)(a.sq_t * 2) | (uint64_t)(a.sq_h * 2);
  const uint64_t ka = (uint64_t)(uintptr_t)a.k | (uint64_t)(a.sk_b * 2) | (uint64_t)(a.sk_t * 2) | (uint64_t)(a.sk_h * 2);
  const uint64_t oa =
      (uint64_t)(uintptr_t)a.d_o | (uint64_t)(a.sdo_b * 2) | (uint64_t)(a.sdo_t * 2) | (uint64_t)(a.sdo_h * 2);
  const int64_t es = a.grad_dtype == kF32 ? 4 : 2;
  const uint64_t va = (uint64_t)(uintptr_t)a.dvv | (uint64_t)(a.sdv_b * es) | (uint64_t)(a.sdv_t * es);
  return align_of_host(qa) >= 16 && align_of_host(ka) >= 16 && align_of_host(oa) >= 16 &&
         align_of_host(va) >= (int)(4 * es > 16 ? 16 : 4 * es);
}

namespace {
// Slices per workgroup: a multi-slice form when its launch has at least
// kMultiMinWorkgroups workgroups (with W(n) = pairs * dv / (16 n)): the
// forward-state pass takes 4 or 2, the reverse pass 2. Every pair runs in
// eight-wave workgroups, which leave each wave 256 VGPRs; twelve-wave pairs
// (eight state chains or four reverse chains at dk 64) would leave 170.
template <typename T, int DK>
hipError_t launch_passes(const ChunkBwdArgs &a, hipStream_t s) {
  const int64_t pairs = a.n_seqs * a.Hv;
  auto fits = [&](int ns) { return a.dv % (ns * DVT) == 0 && pairs * (a.dv / (ns * DVT)) >= kMultiMinWorkgroups; };
  if (fits(4)) return launch_pair<T, DK, 4, 2>(a, s);
  if (fits(2)) return launch_pair<T, DK, 2, 2>(a, s);
  return launch_pair<T, DK, 1, 1>(a, s);
}
}  // namespace

hipError_t launch_chunk_bwd_state_passes_mma(const ChunkBwdArgs &a, hipStream_t s) {
  if (a.act == kF16) return a.dk == 64 ? launch_passes<f16, 64>(a, s) : launch_passes<f16, 128>(a, s);
  return a.dk == 64 ? launch_passes<bf16, 64>(a, s) : launch_passes<bf16, 128>(a, s);
}

}  // namespace gdn
