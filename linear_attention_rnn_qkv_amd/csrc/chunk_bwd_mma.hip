// Gradient kernel of the chunk-rule backward on the 16-bit matrix cores
// (v_mfma_f32_16x16x32_bf16 or _f16, FP32 accumulation): dq, dk (through the
// L2 fold), dg and dbeta per (chunk, q/k head), the value heads of the GQA
// group in turn, for BF16 or FP16 activations with dk 64 or 128 and dv a
// multiple of 32. It computes what the FP32 gradient kernel of chunk_bwd.hip
// computes, from the same workspace arrays (gamma, inverse norms, Delta,
// M^T dDelta and the states S0, dS_C) and v in place of the corrected values
// R = V - e^gamma rk (.) (K S0^T), which dbeta needs only through the row sums
// sum_i dR' R = sum_i dR' V - e^gamma rk (k . (S0^T dR'^T)), and the row dot
// k . k3 on the right is formed for dk anyway; the forward and backward algebra is
// written out at the top of chunk_bwd.hip (gated delta rule of Gated
// DeltaNet in the chunked form of the flash-linear-attention and Megatron-LM
// pull requests; first-order autograd as in Megatron Core "GDN Elementwise
// Fusion", Execution and numerical behavior).
//
// Precision. q, k and d_o are 16-bit inputs and enter the products exactly
// (on the instruction of their own type). Every FP32 operand x (workspace
// arrays, and the 64 x 64 matrices built from them) is split into
// x = hi + lo, hi = T(x), lo = T(x - hi), and a product of two such operands
// is taken as ah bh + ah bl + al bh: each term then carries a relative error
// of about 2^-16 (BF16) or 2^-22 (FP16, for values inside its range) instead
// of a single 16-bit rounding.
//
// Products per value head (i runs over dv in slabs of 32, the MFMA depth):
//   c1 = dO Delta^T, c2 = dR' Delta^T                     (64 x 64, [t][s])
//   k1^T = S0^T dO^T, k2^T = dS^T Delta^T, k3^T = S0^T dR'^T   (dk x 64, [j][t])
// then, with Z1 = scale (E o c1) (s <= t) and Z2 = -beta (E o c2) (s < t),
//   dq^T += K^T (Z1 diag(rk))^T
//   dk^T += K^T ((Z2 + Z2^T) diag(rk))^T + Q^T (diag(rq) Z1)^T
// where K, Q are the raw BF16 rows and rq, rk the inverse norms, so that the
// unit rows never have to be rounded. The dk x 64 outputs are kept transposed
// so that each lane ends with 4 consecutive dk values of one row (8- or
// 16-byte stores).
//
// Work split: 8 wavefronts; wave w owns row tile tt = w % 4 of the chunk and
// half jh = w / 4 of the dk tiles (and of the s tiles of c1, c2).
#include "chunk_bwd_common.h"
#include "gdn_internal.h"
#include "mfma_tiles.h"

namespace gdn {
namespace {

constexpr int BT = 64;
constexpr int kThr = 512;
constexpr int SP = 40;  // row stride (16-bit elements) of the [64][32] slab tiles: 80-byte rows
constexpr int WP = 72;  // row stride of the [64][64] 16-bit operand matrices: 144-byte rows
constexpr int ZP = 65;  // row stride of the FP32 [64][64] matrices

// T is the activations' 16-bit type (bf16 or f16); the products run on the
// matrix-core instruction of that type and split operands use its hi / lo.
template <typename T>
__device__ __forceinline__ f32x4 mma(typename M2<T>::f8 a, typename M2<T>::f8 b, f32x4 c) {
  return M2<T>::k32(a, b, c);
}

// dk permutation of the dk x 64 tiles: row 4 g + i of tile mt is dk
// 32 (mt / 2) + 8 g + 4 (mt % 2) + i, so that 4 consecutive rows of a lane are
// 4 consecutive dk values and the transposing reads below deliver them.
__device__ __forceinline__ constexpr int dk_of(int mt, int r) {
  return 32 * (mt >> 1) + 8 * (r >> 2) + 4 * (mt & 1) + (r & 3);
}

template <typename V>
__device__ __forceinline__ void split4(f32x4 x, V &hi, V &lo) {
  hi = __builtin_convertvector(x, V);
  lo = __builtin_convertvector(x - __builtin_convertvector(hi, f32x4), V);
}

// threadIdx.x through an empty asm statement: LDS addresses derived from it
// inside the value-head loop are computed there, at their use, instead of
// being kept live from the kernel's start (at 256 VGPRs the compiler spills
// such addresses and every reload waits for all loads in flight)
__device__ __forceinline__ int fresh_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

template <typename T, int DK>
struct GradLds {
  static constexpr int RB = DK * 2;  // bytes per row of a dk-wide BF16 tile
  // raw q, k rows of the chunk (zero past the last token), 16-byte units
  // XOR-swizzled by row (kswz)
  alignas(16) unsigned char tq[BT * RB];
  alignas(16) unsigned char tk[BT * RB];
  union {
    struct {  // one slab of 32 value columns
      alignas(16) T o[BT * SP];                  // d_o [t][i]
      alignas(16) T dh[BT * SP], dl[BT * SP];    // Delta hi, lo
      alignas(16) T rh[BT * SP], rl[BT * SP];    // M^T dDelta hi, lo
      alignas(16) unsigned char s0h[32 * RB], s0l[32 * RB];  // S0 [i][j], swizzled like q, k
      alignas(16) unsigned char dsh[32 * RB], dsl[32 * RB];  // dS_C [i][j]
    } s;
    struct {  // per value head, after the slabs
      float z1[BT * ZP], z2[BT * ZP];
    } e;
  } u;
  alignas(16) T w[6][BT * WP];  // hi, lo of Z1 diag(rk), (Z2 + Z2^T) diag(rk), (diag(rq) Z1)^T
  float gam[BT], eg[BT], cw[BT], beta[BT], rq[BT], rk[BT];
  float rowz[2][BT], roww[2][BT], pa[2][BT], pb[2][BT], pm[2][BT];
  float colz[4][BT];  // column sums of z over the rows of each row tile
  float db[BT];
  alignas(16) float dgam[BT];
  float sdot[kThr / 64];
};

template <typename T, int DK>
__global__ __launch_bounds__(kThr) void bwd_grad_mma_kernel(ChunkBwdArgs p) {
  using SM = GradLds<T, DK>;
  using f8 = typename M2<T>::f8;
  using v4 = typename M2<T>::v4;
  constexpr int RB = SM::RB;
  constexpr int NJW = DK / 32;  // dk tiles per wave
  constexpr int KS = DK / 32;   // MFMA steps over dk
  constexpr int S4 = 32 * DK / 4 / kThr;  // float4 of S0 (and of dS) per thread per slab
  static_assert(S4 >= 1 && S4 * 4 * kThr == 32 * DK, "slab split");
  __shared__ SM sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int tt = wave & 3, jh = wave >> 2;
  const int64_t gc = blockIdx.x, hk = blockIdx.y;
  const ChunkPos cp = chunk_pos(p, gc);
  if (!cp.valid) return;
  const int nr = cp.nr;
  const int64_t G = p.Hv / p.Hqk, dvn = p.dv;
  const int nslab = (int)(dvn / 32);

  // staging of a slab: thread tid holds row tid / 8, value columns
  // 4 (tid % 8) .. + 3 of d_o, Delta, dR', v, and S4 float4 of S0, dS.
  // Slab `it` of the flattened (value head, slab) order is fetched into
  // registers while slab it - 1 is multiplied (the first slab of a value
  // head during the previous head's tail). Loads are never under a
  // branch (rows past the chunk's end read its last row and are zeroed when
  // stored), so that they stay in flight.
  const int st_t = tid >> 3, st_c = 4 * (tid & 7);
  const int st_tc = st_t < nr ? st_t : nr - 1;
  uint2 so;
  uint2 sv;
  f32x4 sd4, sr4, s04[S4], sds4[S4];
  auto fetch = [&](int it) {
    const int64_t h = hk * G + it / nslab, i0 = 32 * (int64_t)(it % nslab);
    so = *reinterpret_cast<const uint2 *>(static_cast<const T *>(p.d_o) + cp.brow * p.sdo_b +
                                          (cp.t0 + st_tc) * p.sdo_t + h * p.sdo_h + i0 + st_c);
    const int64_t wo = ((gc * p.Hv + h) * BT + st_t) * dvn + i0 + st_c;
    sd4 = *reinterpret_cast<const f32x4 *>(p.del + wo);
    sr4 = *reinterpret_cast<const f32x4 *>(p.drp + wo);
    sv = *reinterpret_cast<const uint2 *>(static_cast<const T *>(p.v) + cp.brow * p.sv_b +
                                         (cp.t0 + st_tc) * p.sv_t + h * p.sv_h + i0 + st_c);
#pragma unroll
    for (int m = 0; m < S4; ++m) {
      const int64_t e = ((gc * p.Hv + h) * dvn + i0) * DK + 4 * (tid + kThr * m);
      s04[m] = *reinterpret_cast<const f32x4 *>(p.s0 + e);
      sds4[m] = *reinterpret_cast<const f32x4 *>(p.ds + e);
    }
  };

  // raw q, k tiles (loads, then the first slab's fetch, then the stores)
  {
    constexpr int UPR = DK / 8, NQK = BT * UPR / kThr;
    static_assert(NQK * kThr == BT * UPR, "q/k tile split");
    uint4 qv[NQK], kv[NQK];
#pragma unroll
    for (int m = 0; m < NQK; ++m) {
      const int e = tid + kThr * m, r = e / UPR, un = e % UPR;
      const int64_t t = cp.t0 + (r < nr ? r : nr - 1);
      qv[m] = *reinterpret_cast<const uint4 *>(static_cast<const T *>(p.q) + cp.brow * p.sq_b + t * p.sq_t +
                                               hk * p.sq_h + 8 * un);
      kv[m] = *reinterpret_cast<const uint4 *>(static_cast<const T *>(p.k) + cp.brow * p.sk_b + t * p.sk_t +
                                               hk * p.sk_h + 8 * un);
    }
    fetch(0);
#pragma unroll
    for (int m = 0; m < NQK; ++m) {
      const int e = tid + kThr * m, r = e / UPR, un = e % UPR;
      if (r >= nr) qv[m] = kv[m] = uint4{0u, 0u, 0u, 0u};
      const int off = r * RB + ((un ^ kswz<DK>(r)) << 4);
      *reinterpret_cast<uint4 *>(sm.tq + off) = qv[m];
      *reinterpret_cast<uint4 *>(sm.tk + off) = kv[m];
    }
    if (tid < BT) {
      sm.rq[tid] = p.rq[(gc * p.Hqk + hk) * BT + tid];
      sm.rk[tid] = p.rk[(gc * p.Hqk + hk) * BT + tid];
    }
  }
  __syncthreads();

  // row fragment (A or B operand) of row 16 tile + c of a swizzled dk-wide
  // tile, MFMA step pp: dk 32 pp + 8 g .. + 7
  auto rowk = [&](const unsigned char *x, int tile, int pp) -> f8 {
    const int r = 16 * tile + c;
    return *reinterpret_cast<const f8 *>(x + r * RB + (((4 * pp + g) ^ kswz<DK>(r)) << 4));
  };
  // transposed fragment of a swizzled dk-wide tile: lane (g, c) receives
  // column dk_of(mt, c) of rows r0 + 8 g .. r0 + 8 g + 7 (two transposing
  // reads of 4 rows each)
  auto trk = [&](const unsigned char *x, int mt, int r0) -> f8 {
    const int ra = r0 + 8 * g + (c >> 2), rb = ra + 4, un = 4 * (mt >> 1) + (c & 3);
    const unsigned char *pa = x + ra * RB + ((un ^ kswz<DK>(ra)) << 4) + 8 * (mt & 1);
    const unsigned char *pb = x + rb * RB + ((un ^ kswz<DK>(rb)) << 4) + 8 * (mt & 1);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(pa));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(pb));
    return cat8<T>(__builtin_bit_cast(v4, a), __builtin_bit_cast(v4, b));
  };
  // row fragment of a [64][SP] slab tile: row 16 tile + c, columns 8 g .. + 7
  auto rows = [&](const T *x, int tile) -> f8 {
    return *reinterpret_cast<const f8 *>(x + (16 * tile + c) * SP + 8 * g);
  };

  f32x4 dq[NJW], dk[NJW];  // dq^T, dk^T tiles (jh NJW + m, tt)
#pragma unroll
  for (int m = 0; m < NJW; ++m) dq[m] = dk[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t vh = 0; vh < G; ++vh) {
    const int64_t h = hk * G + vh;
    if (tid < BT) {
      const float *gm = p.gam + (gc * p.Hv + h) * BT;
      const float gl = gm[nr - 1], gt = gm[tid];
      sm.gam[tid] = gt;
      sm.eg[tid] = __expf(gt);
      sm.cw[tid] = tid < nr ? __expf(gl - gt) : 0.f;
      sm.beta[tid] = tid < nr ? p.beta[cp.brow * p.sbt_b + (cp.t0 + tid) * p.sbt_t + h * p.sbt_h] : 0.f;
    }
    f32x4 c1[2], c2[2], k1[NJW], k2[NJW], k3[NJW];
#pragma unroll
    for (int a = 0; a < 2; ++a) c1[a] = c2[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NJW; ++m) k1[m] = k2[m] = k3[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dbp = 0.f, sdp = 0.f;  // this thread's part of sum_i dR' V (row st_t) and of <S0, dS>

    for (int sl = 0; sl < nslab; ++sl) {
      __syncthreads();  // the previous slab (or value head) is done with the union
      {
        v4 hi, lo;
        *reinterpret_cast<uint2 *>(&sm.u.s.o[st_t * SP + st_c]) = st_t < nr ? so : uint2{0u, 0u};
        split4(sd4, hi, lo);
        *reinterpret_cast<v4 *>(&sm.u.s.dh[st_t * SP + st_c]) = hi;
        *reinterpret_cast<v4 *>(&sm.u.s.dl[st_t * SP + st_c]) = lo;
        split4(sr4, hi, lo);
        *reinterpret_cast<v4 *>(&sm.u.s.rh[st_t * SP + st_c]) = hi;
        *reinterpret_cast<v4 *>(&sm.u.s.rl[st_t * SP + st_c]) = lo;
        const v4 vv = __builtin_bit_cast(v4, sv);
#pragma unroll
        for (int q = 0; q < 4; ++q) dbp = fmaf(sr4[q], f(vv[q]), dbp);
#pragma unroll
        for (int m = 0; m < S4; ++m) {
          const int e = 4 * (tid + kThr * m), i = e / DK, j = e % DK;
          const int off = i * RB + (((j >> 3) ^ kswz<DK>(i)) << 4) + 2 * (j & 7);
          split4(s04[m], hi, lo);
          *reinterpret_cast<v4 *>(sm.u.s.s0h + off) = hi;
          *reinterpret_cast<v4 *>(sm.u.s.s0l + off) = lo;
          split4(sds4[m], hi, lo);
          *reinterpret_cast<v4 *>(sm.u.s.dsh + off) = hi;
          *reinterpret_cast<v4 *>(sm.u.s.dsl + off) = lo;
#pragma unroll
          for (int q = 0; q < 4; ++q) sdp = fmaf(s04[m][q], sds4[m][q], sdp);
        }
      }
      __syncthreads();
      if (sl + 1 < nslab) fetch((int)vh * nslab + sl + 1);
      const f8 fo = rows(sm.u.s.o, tt);
      const f8 fdh = rows(sm.u.s.dh, tt), fdl = rows(sm.u.s.dl, tt);
      const f8 frh = rows(sm.u.s.rh, tt), frl = rows(sm.u.s.rl, tt);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int st = 2 * jh + a;
        const f8 sdh = rows(sm.u.s.dh, st), sdl = rows(sm.u.s.dl, st);
        c1[a] = mma<T>(fo, sdh, c1[a]);
        c1[a] = mma<T>(fo, sdl, c1[a]);
        c2[a] = mma<T>(frh, sdh, c2[a]);
        c2[a] = mma<T>(frh, sdl, c2[a]);
        c2[a] = mma<T>(frl, sdh, c2[a]);
      }
#pragma unroll
      for (int m = 0; m < NJW; ++m) {
        const int mt = jh * NJW + m;
        const f8 ash = trk(sm.u.s.s0h, mt, 0), asl = trk(sm.u.s.s0l, mt, 0);
        const f8 adh = trk(sm.u.s.dsh, mt, 0), adl = trk(sm.u.s.dsl, mt, 0);
        k1[m] = mma<T>(ash, fo, k1[m]);
        k1[m] = mma<T>(asl, fo, k1[m]);
        k2[m] = mma<T>(adh, fdh, k2[m]);
        k2[m] = mma<T>(adh, fdl, k2[m]);
        k2[m] = mma<T>(adl, fdh, k2[m]);
        k3[m] = mma<T>(ash, frh, k3[m]);
        k3[m] = mma<T>(ash, frl, k3[m]);
        k3[m] = mma<T>(asl, frh, k3[m]);
        // keep the scheduler from hoisting the next tile's fragment reads
        // (register pressure)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();  // the slab tiles are dead: the union now holds Z1, Z2, z
    // the next value head's first slab: its loads overlap this head's tail
    // (which holds no spilled values whose reloads would wait for them)
    if (vh + 1 < G) fetch((int)(vh + 1) * nslab);

    // gg = K^ K^T and qk = Q^ K^T on tiles (tt, 2 jh + a): lane holds rows
    // t = 16 tt + 4 g + i, column s = 16 (2 jh + a) + c
    f32x4 gg[2], qk[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) gg[a] = qk[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pp = 0; pp < KS; ++pp) {
      const f8 kt = rowk(sm.tk, tt, pp), qt = rowk(sm.tq, tt, pp);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const f8 ks = rowk(sm.tk, 2 * jh + a, pp);
        gg[a] = mma<T>(kt, ks, gg[a]);
        qk[a] = mma<T>(qt, ks, qk[a]);
      }
    }
    {
      // (addresses from fresh_tid: computed here, not held across the loop)
      const int ft = fresh_tid(), fw = ft >> 6, t0 = 16 * (fw & 3) + 4 * ((ft >> 4) & 3);
      const int s0 = 32 * (fw >> 2) + (ft & 15);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + i, s = s0 + 16 * a;
          gg[a][i] *= sm.rk[t] * sm.rk[s];
          qk[a][i] *= sm.rq[t] * sm.rk[s];
        }
    }

    // elementwise on the c tiles; row sums of z and of dA o E o gg, column
    // sums of z
    {
      float rz[4] = {0.f, 0.f, 0.f, 0.f}, rw[4] = {0.f, 0.f, 0.f, 0.f}, cz[2] = {0.f, 0.f};
      // the lane's row and column factors, read once (the stores below would
      // otherwise order every factor read behind them)
      const int ft = fresh_tid(), fw = ft >> 6, frow = 16 * (fw & 3) + 4 * ((ft & 63) >> 4);
      const int fcol = 32 * (fw >> 2) + (ft & 15);
      const f32x4 gtv = *reinterpret_cast<const f32x4 *>(&sm.gam[frow]);
      const f32x4 btv = *reinterpret_cast<const f32x4 *>(&sm.beta[frow]);
      const float gsv[2] = {sm.gam[fcol], sm.gam[fcol + 16]};
      float z1v[2][4], z2v[2][4];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * tt + 4 * g + i, s = 16 * (2 * jh + a) + c;
          const float e = s <= t ? __expf(gtv[i] - gsv[a]) : 0.f;
          const float z1 = s <= t ? p.scale * c1[a][i] * e : 0.f;  // dPt o E
          const float da = s < t ? -c2[a][i] : 0.f;                // dA
          const float ge = e * gg[a][i];
          const float zz = da * btv[i] * ge + z1 * qk[a][i];       // dA * A + dPt * Pt
          z1v[a][i] = z1;
          z2v[a][i] = da * btv[i] * e;                             // dG
          rz[i] += zz;
          cz[a] += zz;
          rw[i] = fmaf(da, ge, rw[i]);
        }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * tt + 4 * g + i, s = 16 * (2 * jh + a) + c;
          sm.u.e.z1[t * ZP + s] = z1v[a][i];
          sm.u.e.z2[t * ZP + s] = z2v[a][i];
        }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rz[i] = lane_sum<16>(rz[i]);
        rw[i] = lane_sum<16>(rw[i]);
      }
      if (c == 0) {
        const int ft = fresh_tid(), fw = ft >> 6, r0 = 16 * (fw & 3) + 4 * ((ft & 63) >> 4);
        float *zr = &sm.rowz[fw >> 2][r0], *wr = &sm.roww[fw >> 2][r0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          zr[i] = rz[i];
          wr[i] = rw[i];
        }
      }
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        cz[a] += __shfl_xor(cz[a], 16, 64);
        cz[a] += __shfl_xor(cz[a], 32, 64);
        if (g == 0) {
          const int ft = fresh_tid(), fw = ft >> 6;
          sm.colz[fw & 3][16 * (2 * (fw >> 2) + a) + (ft & 15)] = cz[a];
        }
      }
    }
    // row dots q_t . k1_t, k_t . k3_t, k_t . k2_t (raw rows) over this wave's
    // dk half; dq, dk gain their direct terms
    {
      const int t = 16 * tt + c;
      const float fq = p.scale * sm.eg[t], fk = sm.cw[t], fb = sm.eg[t] * sm.beta[t];
      float a = 0.f, b = 0.f, mm = 0.f;
#pragma unroll
      for (int m = 0; m < NJW; ++m) {
        const int mt = jh * NJW + m, un = 4 * (mt >> 1) + g;
        const int off = t * RB + ((un ^ kswz<DK>(t)) << 4) + 8 * (mt & 1);
        const v4 qv = *reinterpret_cast<const v4 *>(sm.tq + off), kv = *reinterpret_cast<const v4 *>(sm.tk + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a = fmaf(f(qv[i]), k1[m][i], a);
          b = fmaf(f(kv[i]), k3[m][i], b);
          mm = fmaf(f(kv[i]), k2[m][i], mm);
        }
      }
#pragma unroll
      for (int off = 16; off < 64; off <<= 1) {
        a += __shfl_xor(a, off, 64);
        b += __shfl_xor(b, off, 64);
        mm += __shfl_xor(mm, off, 64);
      }
      if (g == 0) {
        const int ft = fresh_tid(), fw = ft >> 6, ftt = 16 * (fw & 3) + (ft & 15);
        sm.pa[fw >> 2][ftt] = a;
        sm.pb[fw >> 2][ftt] = b;
        sm.pm[fw >> 2][ftt] = mm;
      }
#pragma unroll
      for (int m = 0; m < NJW; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dq[m][i] = fmaf(fq, k1[m][i], dq[m][i]);
          dk[m][i] += fk * k2[m][i] - fb * k3[m][i];
        }
    }
    {
      dbp = lane_sum<8>(dbp);
      if ((tid & 7) == 0) sm.db[fresh_tid() >> 3] = dbp;
      sdp = lane_sum<64>(sdp);
      if (lane == 0) sm.sdot[fresh_tid() >> 6] = sdp;
    }
    __syncthreads();

    // operand matrices of the products over s, split hi / lo: thread holds
    // row t = tid / 8, columns s0 .. s0 + 7
    {
      const int t = tid >> 3, s0 = 8 * (tid & 7);
      float w1[8], w2[8], w3[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int s = s0 + e;
        w1[e] = sm.u.e.z1[t * ZP + s] * sm.rk[s];
        w2[e] = (sm.u.e.z2[t * ZP + s] + sm.u.e.z2[s * ZP + t]) * sm.rk[s];
        w3[e] = sm.u.e.z1[s * ZP + t] * sm.rq[s];
      }
      auto put = [&](int k, const float (&x)[8]) {
        v4 h0, l0, h1, l1;
        split4(f32x4{x[0], x[1], x[2], x[3]}, h0, l0);
        split4(f32x4{x[4], x[5], x[6], x[7]}, h1, l1);
        *reinterpret_cast<f8 *>(&sm.w[2 * k][t * WP + s0]) = cat8<T>(h0, h1);
        *reinterpret_cast<f8 *>(&sm.w[2 * k + 1][t * WP + s0]) = cat8<T>(l0, l1);
      };
      put(0, w1);
      put(1, w2);
      put(2, w3);
    }
    // wave 0: dgamma, its reverse running sum (dg), dbeta
    if (tid < BT) {
      const int t = tid;
      const float colz = sm.colz[0][t] + sm.colz[1][t] + sm.colz[2][t] + sm.colz[3][t];
      float svm = sm.cw[t] * sm.rk[t] * (sm.pm[0][t] + sm.pm[1][t]);
      svm = lane_sum<64>(svm);
      float tot = 0.f;
#pragma unroll
      for (int i = 0; i < kThr / 64; ++i) tot += sm.sdot[i];
      const float at = sm.rq[t] * (sm.pa[0][t] + sm.pa[1][t]);
      const float bt = sm.rk[t] * (sm.pb[0][t] + sm.pb[1][t]);
      const float mt = sm.rk[t] * (sm.pm[0][t] + sm.pm[1][t]);
      const float rd = p.scale * sm.eg[t] * at - sm.eg[t] * sm.beta[t] * bt - sm.cw[t] * mt;
      float dgam = rd + sm.rowz[0][t] + sm.rowz[1][t] - colz;
      if (t == nr - 1) dgam += __expf(sm.gam[t]) * tot + svm;
      if (t >= nr) dgam = 0.f;
      // reverse running sum through LDS (broadcast reads; no cross-lane
      // permutes, whose index registers spill)
      sm.dgam[t] = dgam;
      lds_fence_wave();
      dgam = 0.f;
#pragma unroll
      for (int u = 0; u < BT; u += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(&sm.dgam[u]);
#pragma unroll
        for (int e = 0; e < 4; ++e) dgam += u + e >= t ? x[e] : 0.f;
      }
      if (t < nr) {
        const int64_t o = (cp.brow * p.T + cp.t0 + t) * p.Hv + h;
        p.dg[o] = dgam;
        p.dbeta[o] = (sm.db[t] - sm.eg[t] * bt) + sm.roww[0][t] + sm.roww[1][t];
      }
    }
    __syncthreads();
    // dq^T += K^T W1^T, dk^T += K^T W2^T + Q^T W3^T (contraction over s)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      f8 bw[6];
#pragma unroll
      for (int k = 0; k < 6; ++k) bw[k] = *reinterpret_cast<const f8 *>(&sm.w[k][(16 * tt + c) * WP + 32 * q + 8 * g]);
#pragma unroll
      for (int m = 0; m < NJW; ++m) {
        const int mt = jh * NJW + m;
        const f8 kT = trk(sm.tk, mt, 32 * q), qT = trk(sm.tq, mt, 32 * q);
        dq[m] = mma<T>(kT, bw[0], dq[m]);
        dq[m] = mma<T>(kT, bw[1], dq[m]);
        dk[m] = mma<T>(kT, bw[2], dk[m]);
        dk[m] = mma<T>(kT, bw[3], dk[m]);
        dk[m] = mma<T>(qT, bw[4], dk[m]);
        dk[m] = mma<T>(qT, bw[5], dk[m]);
      }
    }
  }

  // through the L2 fold: d(x / n) = (dx_hat - x_hat (x_hat . dx_hat)) / n
  __syncthreads();  // the last head's readers of pa, pb are done
  {
    const int t = 16 * tt + c;
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int m = 0; m < NJW; ++m) {
      const int mt = jh * NJW + m, un = 4 * (mt >> 1) + g;
      const int off = t * RB + ((un ^ kswz<DK>(t)) << 4) + 8 * (mt & 1);
      const v4 qv = *reinterpret_cast<const v4 *>(sm.tq + off), kv = *reinterpret_cast<const v4 *>(sm.tk + off);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a = fmaf(f(qv[i]), dq[m][i], a);
        b = fmaf(f(kv[i]), dk[m][i], b);
      }
    }
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
      a += __shfl_xor(a, off, 64);
      b += __shfl_xor(b, off, 64);
    }
    if (g == 0) {
      sm.pa[jh][t] = a;
      sm.pb[jh][t] = b;
    }
  }
  __syncthreads();
  {
    const int t = 16 * tt + c;
    const float rq = sm.rq[t], rk = sm.rk[t];
    const float aq = p.use_l2 ? rq * rq * (sm.pa[0][t] + sm.pa[1][t]) : 0.f;
    const float ak = p.use_l2 ? rk * rk * (sm.pb[0][t] + sm.pb[1][t]) : 0.f;
    if (t < nr) {
      const int64_t tg = cp.t0 + t;
#pragma unroll
      for (int m = 0; m < NJW; ++m) {
        const int mt = jh * NJW + m, un = 4 * (mt >> 1) + g;
        const int off = t * RB + ((un ^ kswz<DK>(t)) << 4) + 8 * (mt & 1);
        const v4 qv = *reinterpret_cast<const v4 *>(sm.tq + off), kv = *reinterpret_cast<const v4 *>(sm.tk + off);
        f32x4 oq, ok;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          oq[i] = (dq[m][i] - f(qv[i]) * aq) * rq;
          ok[i] = (dk[m][i] - f(kv[i]) * ak) * rk;
        }
        const int64_t j = hk * DK + dk_of(mt, 4 * g);
        const int64_t bq = cp.brow * p.sdq_b + tg * p.sdq_t + j, bk = cp.brow * p.sdk_b + tg * p.sdk_t + j;
        if (p.grad_dtype == kF32) {
          *reinterpret_cast<f32x4 *>(static_cast<float *>(p.dqq) + bq) = oq;
          *reinterpret_cast<f32x4 *>(static_cast<float *>(p.dkk) + bk) = ok;
        } else {
          *reinterpret_cast<v4 *>(static_cast<T *>(p.dqq) + bq) = __builtin_convertvector(oq, v4);
          *reinterpret_cast<v4 *>(static_cast<T *>(p.dkk) + bk) = __builtin_convertvector(ok, v4);
        }
      }
    }
  }
}

template <typename T, int DK>
hipError_t launch_grad(const ChunkBwdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((bwd_grad_mma_kernel<T, DK>), dim3((unsigned)a.chunk_bound, (unsigned)a.Hqk), dim3(kThr), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// BF16 or FP16 activations, dk 64 or 128, dv a multiple of 32; q, k rows
// 16-byte aligned, d_o rows 8-byte aligned, dq and dk rows aligned to 4
// elements.
bool chunk_bwd_grad_mma_supported(const ChunkBwdArgs &a) {
  if ((a.act != kBF16 && a.act != kF16) || !(a.dk == 64 || a.dk == 128) || a.dv % 32 != 0) return false;
  const uint64_t qa = (uint64_t)(uintptr_t)a.q | (uint64_t)(a.sq_b * 2) | (uint64_t)(a.sq_t * 2) | (uint64_t)(a.sq_h * 2);
  const uint64_t ka = (uint64_t)(uintptr_t)a.k | (uint64_t)(a.sk_b * 2) | (uint64_t)(a.sk_t * 2) | (uint64_t)(a.sk_h * 2);
  const uint64_t oa =
      (uint64_t)(uintptr_t)a.d_o | (uint64_t)(a.sdo_b * 2) | (uint64_t)(a.sdo_t * 2) | (uint64_t)(a.sdo_h * 2);
  const int64_t es = a.grad_dtype == kF32 ? 4 : 2;
  const uint64_t ga = (uint64_t)(uintptr_t)a.dqq | (uint64_t)(uintptr_t)a.dkk | (uint64_t)(a.sdq_b * es) |
                      (uint64_t)(a.sdq_t * es) | (uint64_t)(a.sdk_b * es) | (uint64_t)(a.sdk_t * es);
  const uint64_t va = (uint64_t)(uintptr_t)a.v | (uint64_t)(a.sv_b * 2) | (uint64_t)(a.sv_t * 2) | (uint64_t)(a.sv_h * 2);
  return align_of_host(qa) >= 16 && align_of_host(ka) >= 16 && align_of_host(oa) >= 8 && align_of_host(va) >= 8 &&
         align_of_host(ga) >= (int)(4 * es > 16 ? 16 : 4 * es);
}

hipError_t launch_chunk_bwd_grad_mma(const ChunkBwdArgs &a, hipStream_t s) {
  if (a.act == kF16) return a.dk == 64 ? launch_grad<f16, 64>(a, s) : launch_grad<f16, 128>(a, s);
  return a.dk == 64 ? launch_grad<bf16, 64>(a, s) : launch_grad<bf16, 128>(a, s);
}

}  // namespace gdn
