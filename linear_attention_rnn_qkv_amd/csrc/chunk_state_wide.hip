// Chunk state for wide heads (dk = 256): the state-dependent half of the
// chunked gated delta rule, serial over the chunks of a sequence, with the
// per-chunk record of the chunk-prep kernel (T' = (I + A)^-1 diag(beta), P
// and the row factors aa, cw, zc, e^{gamma_C}). A chunk of 64 rows entering
// with state S0 (dv x dk, FP32) gives
//
//   X = K S0^T,   Vn = T' V - T' (aa (.) X)
//   O = zc (.) (Q S0^T) + P Vn          (computed transposed, O^T)
//   S = e^{gamma_C} S0 + K^T (cw (.) Vn)
//
// (the WY/UT form of the gated delta rule; q and k are used raw, their
// inverse norms are inside the factors).
//
// At dk = 256 a q or k tile of a chunk is 32 KB, so the three-slot LDS rings
// of the dk <= 128 kernel do not fit. Here one workgroup = (sequence, value
// head, 32 rows of dv) with four wavefronts and one barrier per chunk:
//   waves 0, 1  the whole step of chunk s for 16 rows of dv each: X and
//               (Q S0^T)^T share the state fragments, then T' V, Vn, O^T
//               (stored) and the state update; S lives in MFMA
//               accumulators. Each wave loads its own V fragments for the
//               next chunk straight into registers.
//   waves 2, 3  copy the k tile, the q tile and the record of chunk s + 1
//               into the other slot of two-slot LDS rings (global_load_lds);
//               the copies are complete before the barrier that starts
//               step s + 1.
// Two compute waves per workgroup halve the workgroup count for the same
// LDS, so that a whole launch of the common shapes is resident at once (the
// rings take almost all of a CU's 160 KB).
// The operand layouts, the dk permutation of the state tiles and the XOR
// swizzle of the q/k tiles are those of the dk <= 128 kernel.
#include "gdn_internal.h"
#include "mfma_tiles.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int BT = 64;
constexpr int DVT = 32;  // dv rows per workgroup, 16 per compute wave
// bytes of the record the step reads: T', P and the factor rows aa, cw, zc,
// beta, then e^{gamma_C} (one 16-byte unit)
constexpr int kRecUse = (int)kRecF + 4 * BT * 4 + 16;

template <typename T, int DK>
struct WideLds {
  static constexpr int RB = DK * 2;
  static constexpr int TILE = BT * RB;
  alignas(16) unsigned char k[2][TILE];   // k rows of chunk c in slot c % 2 (swizzled)
  alignas(16) unsigned char q[2][TILE];   // q rows
  alignas(16) unsigned char rec[2][kRecUse];
};

// dk permutation of the state accumulator tiles: tile mt = 2 pp + h, row
// 4 g + i holds dk 32 pp + 8 g + 4 h + i, so that the state fragment of k step
// pp covers dk 32 pp + 8 g .. + 7 in lane group g (one 16-byte q/k read).
__device__ __forceinline__ constexpr int dk_of(int mt, int r) {
  return 32 * (mt >> 1) + 8 * (r >> 2) + 4 * (mt & 1) + (r & 3);
}

// fragment index of (row tile mt, k pair q) in a record matrix
__device__ __forceinline__ constexpr int frag_id(int mt, int q) { return q == 0 ? mt : 2 + mt; }

template <typename T, int DK>
// One workgroup per CU (the LDS rings), one wave per SIMD: the compute waves
// may use the whole register file.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void chunk_state_wide_kernel(
    ChunkArgs p) {
  using MF = M2<T>;
  using f8 = typename MF::f8;
  using v4 = typename MF::v4;
  using SM = WideLds<T, DK>;
  constexpr int KT = DK / 32;
  constexpr int NT = DK / 16;
  constexpr int RB = SM::RB;
  constexpr int NI = SM::TILE / 1024;  // 1 KB copies per q/k tile
  constexpr int NRC = kRecUse / 1024;  // whole 1 KB copies of the record
  static_assert(NI + NRC + 1 <= 48, "copies per lane and step");
  __shared__ SM sm;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  // the dv slices of one head (same q/k tiles and records) on one XCD
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

  if (wave < 2) {
    // ------------------------------------------------------------ the step
    const int64_t jw = 16 * wave;  // this wave's dv rows j0 + jw .. + 15
    int fo[KT];  // row c of a 16-row tile, dk 32 pp + 8 g .. + 7
#pragma unroll
    for (int pp = 0; pp < KT; ++pp) fo[pp] = c * RB + (((4 * pp + g) ^ kswz<DK>(c)) << 4);
    f32x4 S[NT];  // S[mt][i] = S[dv row c][dk dk_of(mt, 4 g + i)]
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[mt][i] = p.init_state ? p.init_state[st_base + (jw + c) * DK + dk_of(mt, 4 * g + i)] : 0.f;
    f8 Sf[KT];
#pragma unroll
    for (int pp = 0; pp < KT; ++pp) Sf[pp] = cat8<T>(cvt4<T>(S[2 * pp]), cvt4<T>(S[2 * pp + 1]));
    // transposing reads of K^T fragments for the state update: lane 16 g + c
    // addresses row 4 g + c / 4 at dk dk_of(mt, 4 (c % 4)) .. + 3
    const int yrow = 4 * g + (c >> 2);
    // V fragments (B operand of T' V): lane (g, c) holds V[32 q + 16 hh + 4 g + i]
    // [dv jw + c] in element 4 hh + i of fragment q; loaded from global one
    // chunk ahead (rows past the end repeat the last row)
    const T *vw = vb + jw + c;
    auto load_v = [&](int cl, f8(&bv)[2]) {
      const int nr = rows_of(cl);
      const T *vc = vw + (int64_t)cl * BT * p.sv_t;
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 32 * q + 16 * (e >> 2) + 4 * g + (e & 3);
          bv[q][e] = vc[(int64_t)(r < nr ? r : nr - 1) * p.sv_t];
        }
    };
    f8 Bn[2];
    if (Nc > 0) load_v(0, Bn);
    for (int s = 0; s < Nc; ++s) {
      lds_barrier();
      const f8 Bv[2] = {Bn[0], Bn[1]};
      if (s + 1 < Nc) load_v(s + 1, Bn);
      const int sl = s & 1;
      const unsigned char *kt = sm.k[sl];
      const unsigned char *qt = sm.q[sl];
      const unsigned char *rec = sm.rec[sl];
      const float *fa = reinterpret_cast<const float *>(rec + kRecF);
      const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
      // X = K S0^T and Z^T = S0 Q^T (lane (g, c) of z[mt]: Z[16 mt + c][dv 4 g + i])
      f32x4 X[4], z[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) X[mt] = z[mt] = zero4;
      // every fragment read of the step is issued before its products (LDS
      // latency, not the MFMA issue rate, bounds this wave's step)
      f8 kfa[KT][4], qfa[KT][4];
#pragma unroll
      for (int pp = 0; pp < KT; ++pp)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          kfa[pp][mt] = *reinterpret_cast<const f8 *>(kt + mt * 16 * RB + fo[pp]);
          qfa[pp][mt] = *reinterpret_cast<const f8 *>(qt + mt * 16 * RB + fo[pp]);
        }
#pragma unroll
      for (int pp = 0; pp < KT; ++pp) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          X[mt] = MF::k32(kfa[pp][mt], Sf[pp], X[mt]);
          z[mt] = MF::k32(Sf[pp], qfa[pp][mt], z[mt]);
        }
      }
      f8 Tf[6], Pf[6];
#pragma unroll
      for (int f = 0; f < 6; ++f) {
        Tf[f] = *reinterpret_cast<const f8 *>(rec + kRecT + f * 1024 + lane * 16);
        Pf[f] = *reinterpret_cast<const f8 *>(rec + kRecP + f * 1024 + lane * 16);
      }
      f32x4 aa[4], cw[4], Zc[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int r0 = 16 * mt + 4 * g;
        aa[mt] = *reinterpret_cast<const f32x4 *>(&fa[0 * BT + r0]);
        cw[mt] = *reinterpret_cast<const f32x4 *>(&fa[1 * BT + r0]);
        Zc[mt] = z[mt] * fa[2 * BT + 16 * mt + c];
      }
      const float eC = fa[4 * BT];
      // Vn = T' V - T' (aa (.) X)
      f8 Rf[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) Rf[q] = cat8<T>(cvt4<T>(aa[2 * q] * X[2 * q]), cvt4<T>(aa[2 * q + 1] * X[2 * q + 1]));
      f32x4 Vn[4];
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
      f8 Wf[2], Bw[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        Wf[q] = cat8<T>(cvt4<T>(Vn[2 * q]), cvt4<T>(Vn[2 * q + 1]));
        Bw[q] = cat8<T>(cvt4<T>(cw[2 * q] * Vn[2 * q]), cvt4<T>(cw[2 * q + 1] * Vn[2 * q + 1]));
      }
      // O^T = Zc^T + Vn^T P^T: lane (g, c) holds o[16 mt + c][4 g .. 4 g + 3]
      {
        const int nr = rows_of(s);
        T *orow = ob + jw + (int64_t)s * BT * p.so_t;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 o = MF::k32(Wf[0], Pf[frag_id(mt, 0)], Zc[mt]);
          if (mt >= 2) o = MF::k32(Wf[1], Pf[frag_id(mt, 1)], o);
          const int r = 16 * mt + c;
          if (r < nr) *reinterpret_cast<v4 *>(orow + (int64_t)r * p.so_t + 4 * g) = cvt4<T>(o);
        }
      }
      // S = e^{gamma_C} S0 + K^T (cw (.) Vn)
      f8 kt8[NT][2];
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        const int tro = yrow * RB + (((4 * (mt >> 1) + (c & 3)) ^ kswz<DK>(yrow)) << 4) + 8 * (mt & 1);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const unsigned char *a1 = kt + tro + (32 * q) * RB;
          const unsigned char *a2 = kt + tro + (32 * q + 16) * RB;
          const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(a1));
          const s16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)const_cast<unsigned char *>(a2));
          kt8[mt][q] = cat8<T>(__builtin_bit_cast(v4, r1), __builtin_bit_cast(v4, r2));
        }
      }
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        f32x4 acc = S[mt] * eC;
#pragma unroll
        for (int q = 0; q < 2; ++q) acc = MF::k32(kt8[mt][q], Bw[q], acc);
        S[mt] = acc;
      }
#pragma unroll
      for (int pp = 0; pp < KT; ++pp) Sf[pp] = cat8<T>(cvt4<T>(S[2 * pp]), cvt4<T>(S[2 * pp + 1]));
    }
    if (p.final_state) {
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) p.final_state[st_base + (jw + c) * DK + dk_of(mt, 4 * g + i)] = S[mt][i];
    }
  } else {
    // ------------------------------------------------------------ copies
    // wave 2: the k tile and the first half of the record; wave 3: the q
    // tile, the rest of the record and its last 16 bytes; of chunk cl into
    // slot cl % 2.
    const int role = wave - 2;
    constexpr int NR0 = (NRC + 1) / 2;
    auto issue = [&](int cl) {
      const int sl = cl & 1;
      const int nr = rows_of(cl);
      const int64_t t0 = (int64_t)cl * BT;
      const bool isk = role == 0;
      const int64_t st = isk ? p.sk_t : p.sq_t;
      const T *xb = (isk ? kb : qb) + t0 * st;
      unsigned char *xt = isk ? sm.k[sl] : sm.q[sl];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int b = 1024 * i + 16 * lane;
        const int r = b / RB, jp = (b % RB) >> 4;
        const int j = jp ^ kswz<DK>(r);
        const int rr = r < nr ? r : nr - 1;  // rows past the end repeat the last row
        g2l16(xb + (int64_t)rr * st + 8 * j, xt + 1024 * i);
      }
      const unsigned char *rg = recb + (int64_t)cl * rec_stride;
      const int i0 = isk ? 0 : NR0, i1 = isk ? NR0 : NRC;
      for (int i = i0; i < i1; ++i) g2l16(rg + 1024 * i + 16 * lane, sm.rec[sl] + 1024 * i);
      if (!isk && lane == 0) g2l16(rg + 1024 * NRC, sm.rec[sl] + 1024 * NRC);
    };
    if (Nc > 0) issue(0);
    wait_vm<0>();
    for (int s = 0; s < Nc; ++s) {
      lds_barrier();
      if (s + 1 < Nc) issue(s + 1);
      wait_vm<0>();
    }
  }
}

template <typename T, int DK>
hipError_t launch_dk(const ChunkArgs &a, hipStream_t s) {
  dim3 grid((unsigned)(a.dv / DVT), (unsigned)a.Hv, (unsigned)a.n_seqs);
  hipLaunchKernelGGL((chunk_state_wide_kernel<T, DK>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_state_wide(const ChunkArgs &a, hipStream_t s) {
  if (a.act == kBF16) return launch_dk<bf16, 256>(a, s);
  if (a.act == kF16) return launch_dk<f16, 256>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace gdn
