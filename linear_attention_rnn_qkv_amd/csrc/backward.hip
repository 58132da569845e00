// Backward (first-order gradients) of the gated norm and of the prologue.
//
// The Megatron Core page "GDN Elementwise Fusion" (Execution and numerical
// behavior) gives the fused stages first-order autograd; the pages do not
// print the formulas, which are the derivatives of the forward definitions
// (the activation-dtype roundings of the forward are treated as the
// identity; all arithmetic is FP32):
//
// gated norm, per row of dv: r = (mean(o^2) + eps)^-1/2, n = o r, y = n w,
//   out = y silu(gate):
//     dy = dout silu(gate),  d_gate = dout y silu'(gate),
//     dn = dy w,  d_o = r (dn - n mean(dn n)),  d_w = sum over rows of dy n
// conv + SiLU, per channel c of one sequence: y_t = b + sum_j w_j x_{t-3+j},
//   z_t = silu(y_t):
//     e_t = dz_t silu'(y_t),  dx_t = sum_j w_j e_{t+3-j} (inside the sequence),
//     dw_j = sum_t e_t x_{t-3+j},  db = sum_t e_t
// beta = sigmoid(b), g = -exp(A_log) softplus(a + dt_bias):
//     d_b = d_beta beta (1 - beta),  d_a = -d_g exp(A_log) sigmoid(a + dt_bias),
//     d_dt_bias = sum d_a,  d_A_log = sum d_g g
// with silu'(x) = s (1 + x (1 - s)), s = sigmoid(x).
//
// Parameter gradients are sums over tokens: each block writes its partial
// sums to a caller workspace and a second kernel adds them in a fixed order,
// so results do not depend on scheduling.
#include <type_traits>

#include "device_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

__device__ __forceinline__ float sigm(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float dsilu(float x) {
  const float s = sigm(x);
  return s * (1.0f + x * (1.0f - s));
}

// out[i] = sum_p part[p * n + i] in a fixed order, in two levels: block
// (x, g) sums the parts of group g for 64 outputs (four interleaved
// subgroups, then their sum in order) into mid[g][i]; then the groups are
// added in order.
constexpr int kRedGroups = 32;

__global__ __launch_bounds__(256) void sum_partials_a(const float *__restrict__ part, int64_t nparts, int64_t n,
                                                      float *__restrict__ mid) {
  __shared__ float red[4][64];
  const int sub = threadIdx.x >> 6, o = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 64 + o, g = blockIdx.y;
  const int64_t lo = nparts * g / gridDim.y, hi = nparts * (g + 1) / gridDim.y;
  float acc = 0.f;
  if (i < n)
    for (int64_t q = lo + sub; q < hi; q += 4) acc += part[q * n + i];
  red[sub][o] = acc;
  __syncthreads();
  if (sub == 0 && i < n) mid[g * n + i] = ((red[0][o] + red[1][o]) + red[2][o]) + red[3][o];
}

__global__ __launch_bounds__(256) void sum_partials_b(const float *__restrict__ mid, int64_t ng, int64_t n,
                                                      float *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float acc = 0.f;
  for (int64_t g = 0; g < ng; ++g) acc += mid[g * n + i];
  out[i] = acc;
}

// mid: scratch of kRedGroups * n floats
hipError_t sum_partials(const float *part, int64_t nparts, int64_t n, float *mid, float *out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t ng = nparts < kRedGroups ? (nparts > 0 ? nparts : 1) : kRedGroups;
  hipLaunchKernelGGL(sum_partials_a, dim3((unsigned)((n + 63) / 64), (unsigned)ng), dim3(256), 0, s, part, nparts, n,
                     mid);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sum_partials_b, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, mid, ng, n, out);
  return hipGetLastError();
}

// ----------------------------------------------------------------- norm bwd
constexpr int kNormThreads = 256;

template <typename T, typename TG, typename TW, int DV>
__global__ __launch_bounds__(kNormThreads) void gated_norm_bwd_kernel(NormBwdArgs p) {
  constexpr int E = 8;
  constexpr int LPR = DV / E;                      // lanes per row
  constexpr int RPW = 64 / LPR;                    // rows per wave
  constexpr int RPB = (kNormThreads / 64) * RPW;   // rows per block and pass
  __shared__ float red[RPB][DV];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = (lane % LPR) * E, rg = wave * RPW + lane / LPR;
  const int64_t nrows = p.B * p.T * p.H;

  float w[E], dw[E];
  load_vec<TW, E>(static_cast<const TW *>(p.w) + c0, 16, w);
#pragma unroll
  for (int i = 0; i < E; ++i) dw[i] = 0.f;

  // two rows per lane and pass, all six loads issued before any arithmetic
  for (int64_t row0 = (int64_t)blockIdx.x * 2 * RPB; row0 < nrows; row0 += (int64_t)gridDim.x * 2 * RPB) {
    float O[2][E], G[2][E], D[2][E];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t row = row0 + u * RPB + rg;
      if (row < nrows) {
        int64_t b, t, h;
        split_row(p.rd, p.T, p.H, row, b, t, h);
        load_vec_nt<T, E>(static_cast<const T *>(p.o) + b * p.so_b + t * p.so_t + h * p.so_h + c0, p.o_align, O[u]);
        load_vec_nt<TG, E>(static_cast<const TG *>(p.gate) + b * p.sg_b + t * p.sg_t + h * p.sg_h + c0, p.gate_align,
                           G[u]);
        load_vec_nt<T, E>(static_cast<const T *>(p.dout) + b * p.sd_b + t * p.sd_t + h * p.sd_h + c0, p.dout_align,
                          D[u]);
      } else {
#pragma unroll
        for (int i = 0; i < E; ++i) O[u][i] = G[u][i] = D[u][i] = 0.f;
      }
    }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t row = row0 + u * RPB + rg;
    const bool live = row < nrows;
    const float(&o)[E] = O[u];
    const float(&gt)[E] = G[u];
    const float(&du)[E] = D[u];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) ss += o[i] * o[i];
    ss = group_sum<LPR>(ss);
    const float r = rsqrtf(ss * (1.0f / DV) + p.eps);
    float n[E], dn[E], dgate[E], dot = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      n[i] = o[i] * r;
      const float sg = gt[i] * sigm(gt[i]);
      const float dy = du[i] * sg;
      dgate[i] = du[i] * n[i] * w[i] * dsilu(gt[i]);
      dn[i] = dy * w[i];
      dw[i] += dy * n[i];
      dot += dn[i] * n[i];
    }
    dot = group_sum<LPR>(dot) * (1.0f / DV);
    float d_o[E];
#pragma unroll
    for (int i = 0; i < E; ++i) d_o[i] = r * (dn[i] - n[i] * dot);
    if (live) {
      store_vec_nt<T, E>(static_cast<T *>(p.d_o) + row * DV + c0, d_o);
      store_vec_nt<TG, E>(static_cast<TG *>(p.d_gate) + row * DV + c0, dgate);
    }
  }
  }
  // block partial of d_w: rows groups of the block summed in a fixed order
#pragma unroll
  for (int i = 0; i < E; ++i) red[rg][c0 + i] = dw[i];
  __syncthreads();
  for (int c = threadIdx.x; c < DV; c += kNormThreads) {
    float acc = 0.f;
    for (int q = 0; q < RPB; ++q) acc += red[q][c];
    p.part[(int64_t)blockIdx.x * DV + c] = acc;
  }
}

template <typename T, typename TG, typename TW, int DV>
hipError_t norm_bwd_dv(const NormBwdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((gated_norm_bwd_kernel<T, TG, TW, DV>), dim3((unsigned)a.nblocks), dim3(kNormThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return sum_partials(a.part, a.nblocks, DV, a.mid, a.d_w, s);
}

template <typename T, typename TG, typename TW>
hipError_t norm_bwd_w(const NormBwdArgs &a, hipStream_t s) {
  switch (a.dv) {
    case 64: return norm_bwd_dv<T, TG, TW, 64>(a, s);
    case 128: return norm_bwd_dv<T, TG, TW, 128>(a, s);
    case 256: return norm_bwd_dv<T, TG, TW, 256>(a, s);
    case 512: return norm_bwd_dv<T, TG, TW, 512>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, typename TG>
hipError_t norm_bwd_g(const NormBwdArgs &a, hipStream_t s) {
  switch (a.w_dtype) {
    case kF32: return norm_bwd_w<T, TG, float>(a, s);
    case kBF16: return norm_bwd_w<T, TG, bf16>(a, s);
    case kF16: return norm_bwd_w<T, TG, f16>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t norm_bwd_t(const NormBwdArgs &a, hipStream_t s) {
  if (a.gate_dtype == kF32) return norm_bwd_g<T, float>(a, s);
  if (a.gate_dtype == a.act) return norm_bwd_g<T, T>(a, s);
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------- prologue bwd
constexpr int kConvThreads = 256;

template <typename T>
__device__ __forceinline__ float ldf(const void *p, int32_t dt, int64_t i) {
  if (dt == kF32) return static_cast<const float *>(p)[i];
  return f(static_cast<const T *>(p)[i]);
}

// Sequence bounds of a token, advanced monotonically (packed sequences from
// cu_seqlens, else rows of T tokens).
struct SeqTrack {
  const int32_t *cu;
  int64_t n_seqs, T;
  int64_t seq, s0, s1;
  __device__ void init(int64_t u) {
    if (cu) {
      int64_t lo = 0, hi = n_seqs;  // cu[lo] <= u < cu[hi]
      while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (cu[mid] <= u) lo = mid; else hi = mid;
      }
      seq = lo;
      s0 = cu[lo];
      s1 = cu[lo + 1];
    } else {
      seq = u / T;
      s0 = seq * T;
      s1 = s0 + T;
    }
  }
  __device__ void advance(int64_t u) {  // u >= the last token seen, u < total
    while (u >= s1 && (!cu || seq + 1 < n_seqs)) {
      ++seq;
      s0 = s1;
      s1 = cu ? cu[seq + 1] : s0 + T;
    }
  }
};

// The tile's partial sums of d_conv_w and d_conv_b for channels c .. c + VEC - 1.
template <int VEC>
__device__ __forceinline__ void write_conv_parts(const PrologueBwdArgs &p, int64_t tile, int64_t c,
                                                 const float (&dw)[4][VEC], const float (&db)[VEC]) {
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    float *pw = p.part_w + (tile * p.C + c + v) * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) pw[j] = dw[j][v];
    p.part_b[tile * p.C + c + v] = db[v];
  }
}

// Tiles whose window (3 tokens before, 3 after) lies inside one sequence and
// inside the call: four 16-bit channels per thread, token rows at x(u) =
// xrow + u st, dz(u) = dzrow + u C, dx(u) = dxrow + u ldx. No boundary
// conditions; x and dz are fetched 4 tokens at a time, a batch ahead of use,
// with fixed-width non-temporal loads (unconditional: indices past the last
// needed token repeat it). Three waves per SIMD fit (a deeper batch needs
// more registers than that allows and was not faster).
template <typename T, typename TD>
__device__ __forceinline__ void conv_bwd_interior(const T *xrow, int64_t st, const TD *dzrow, int64_t C, T *dxrow,
                                                  int64_t ldx, const float (&w)[4][4], const float (&bias)[4],
                                                  int64_t t0, int64_t t1, float (&dw)[4][4], float (&db)[4]) {
  typedef unsigned int u2 __attribute__((ext_vector_type(2)));
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  using DR = typename std::conditional<sizeof(TD) == 2, u2, u4>::type;
  constexpr int NB = 4;  // tokens per batch
  const int64_t last = t1 + 2;  // last token whose x and dz are needed
  auto ldxr = [&](int64_t u) -> u2 {
    u = u < last ? u : last;
    return __builtin_nontemporal_load(reinterpret_cast<const u2 *>(xrow + u * st));
  };
  auto ldzr = [&](int64_t u) -> DR {
    u = u < last ? u : last;
    return __builtin_nontemporal_load(reinterpret_cast<const DR *>(dzrow + u * C));
  };
  auto cvx = [](u2 r, float(&o)[4]) {
    T t[4];
    __builtin_memcpy(t, &r, 8);
#pragma unroll
    for (int v = 0; v < 4; ++v) o[v] = f(t[v]);
  };
  auto cvz = [](DR r, float(&o)[4]) {
    TD t[4];
    __builtin_memcpy(t, &r, sizeof(DR));
#pragma unroll
    for (int v = 0; v < 4; ++v) o[v] = f(t[v]);
  };
  // e = dz silu'(b + sum_j w_j x_{u-3+j}) from x rows xa .. xa + 3
  auto e_at = [&](const float(&x0)[4], const float(&x1)[4], const float(&x2)[4], const float(&x3)[4],
                  const float(&dz)[4], float(&e)[4]) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float y = fmaf(w[0][v], x0[v], fmaf(w[1][v], x1[v], fmaf(w[2][v], x2[v], fmaf(w[3][v], x3[v], bias[v]))));
      e[v] = dz[v] * dsilu(y);
    }
  };
  float xw[7][4], ew[3][4];  // x_{t-3} .. x_{t+3}; e_t .. e_{t+2}
#pragma unroll
  for (int k = 0; k < 7; ++k) cvx(ldxr(t0 - 3 + k), xw[k]);
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    float dz[4];
    cvz(ldzr(t0 + k), dz);
    e_at(xw[k], xw[k + 1], xw[k + 2], xw[k + 3], dz, ew[k]);
  }
  // batch for tokens tb .. tb + NB - 1: x_{t+4} and dz_{t+3}
  auto fetch = [&](int64_t tb, u2(&xb)[NB], DR(&zb)[NB]) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      xb[k] = ldxr(tb + 4 + k);
      zb[k] = ldzr(tb + 3 + k);
    }
  };
  auto run = [&](int64_t tb, const u2(&xb)[NB], const DR(&zb)[NB]) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      float dz[4], e3[4], dx[4];
      cvz(zb[k], dz);
      e_at(xw[3], xw[4], xw[5], xw[6], dz, e3);  // e_{t+3}
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        dx[v] = fmaf(w[0][v], e3[v], fmaf(w[1][v], ew[2][v], fmaf(w[2][v], ew[1][v], w[3][v] * ew[0][v])));
        db[v] += ew[0][v];
#pragma unroll
        for (int j = 0; j < 4; ++j) dw[j][v] = fmaf(ew[0][v], xw[j][v], dw[j][v]);
      }
      store_vec<T, 4>(dxrow + (tb + k) * ldx, dx);
#pragma unroll
      for (int q = 0; q < 6; ++q)
#pragma unroll
        for (int v = 0; v < 4; ++v) xw[q][v] = xw[q + 1][v];
      cvx(xb[k], xw[6]);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        ew[0][v] = ew[1][v];
        ew[1][v] = ew[2][v];
        ew[2][v] = e3[v];
      }
    }
  };
  u2 xa[NB], xb[NB];
  DR za[NB], zb[NB];
  fetch(t0, xa, za);
  for (int64_t tb = t0; tb < t1; tb += 2 * NB) {  // t1 - t0 is a multiple of 2 NB
    fetch(tb + NB, xb, zb);
    run(tb, xa, za);
    fetch(tb + 2 * NB, xa, za);
    run(tb + NB, xb, zb);
  }
}

// One thread per VEC adjacent channels walks the tokens of one tile in order
// with rolling windows: xw[k] = x_{t-3+k} (k < 8) and ew[k] = e_{t+k} (k < 4),
// where e_u = dz_u silu'(y_u). The tile reads 3 tokens of x before it and 4
// ahead; x and dz are fetched NB tokens at a time (vector accesses of VEC
// elements).
template <typename T, int VEC, bool FLAT>
__global__ __launch_bounds__(kConvThreads) __attribute__((amdgpu_waves_per_eu(3))) void conv_bwd_kernel(PrologueBwdArgs p) {
  constexpr int NB = 4;
  const int64_t c = ((int64_t)blockIdx.x * kConvThreads + threadIdx.x) * VEC;
  const int64_t tile = blockIdx.y;
  if (c >= p.C) return;
  const int64_t nq = p.Hqk * p.dk;
  const T *xs;
  int64_t sb, st, cc, ldx;
  T *dxs;
  if (c < nq) {
    xs = static_cast<const T *>(p.xq); sb = p.sxq_b; st = p.sxq_t; cc = c; dxs = static_cast<T *>(p.dxq); ldx = nq;
  } else if (c < 2 * nq) {
    xs = static_cast<const T *>(p.xk); sb = p.sxk_b; st = p.sxk_t; cc = c - nq; dxs = static_cast<T *>(p.dxk); ldx = nq;
  } else {
    xs = static_cast<const T *>(p.xv); sb = p.sxv_b; st = p.sxv_t; cc = c - 2 * nq; dxs = static_cast<T *>(p.dxv);
    ldx = p.Hv * p.dv;
  }
  float w[4][VEC], bias[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j][v] = ldf<T>(p.conv_w, p.w_dtype, 4 * (c + v) + j);
    bias[v] = p.conv_b ? ldf<T>(p.conv_b, p.b_dtype, c + v) : 0.f;
  }

  const int64_t ntok = p.B * p.T;
  const int64_t t0 = tile * p.tile_tokens;
  const int64_t t1 = t0 + p.tile_tokens < ntok ? t0 + p.tile_tokens : ntok;
  // FLAT: the x rows of consecutive batch entries follow each other
  // (batch stride T times the token stride), so no division is needed
  auto xat = [&](int64_t u, float(&out)[VEC]) {  // raw x at flattened token u, 0 outside [0, ntok)
    if (u < 0 || u >= ntok) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) out[v] = 0.f;
      return;
    }
    int64_t row;
    if constexpr (FLAT) row = u * st;
    else row = (u / p.T) * sb + (u % p.T) * st;
    load_vec<T, VEC>(xs + row + cc, p.x_align, out);
  };
  auto dzat = [&](int64_t u, float(&out)[VEC]) {
    if (u >= ntok) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) out[v] = 0.f;
      return;
    }
    if (p.dqkv_dtype == kF32) load_vec<float, VEC>(static_cast<const float *>(p.dqkv) + u * p.C + c, p.dq_align, out);
    else load_vec<T, VEC>(static_cast<const T *>(p.dqkv) + u * p.C + c, p.dq_align, out);
  };
  SeqTrack tt{p.cu_seqlens, p.n_seqs, p.T, 0, 0, 0};  // sequence of t
  SeqTrack tu{p.cu_seqlens, p.n_seqs, p.T, 0, 0, 0};  // sequence of the lookahead token
  tt.init(t0);
  tu.init(t0);
  float dw[4][VEC], db[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    db[v] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) dw[j][v] = 0.f;
  }
  if constexpr (VEC == 4 && sizeof(T) == 2) {
    // the tile's window [t0 - 3, t1 + 2] inside one sequence (one batch row)
    if (t1 - t0 == p.tile_tokens && p.tile_tokens % 16 == 0 && t0 >= 3 && t1 + 2 < ntok && tt.s0 <= t0 - 3 &&
        t1 + 2 < tt.s1) {
      const int64_t brow = FLAT ? 0 : t0 / p.T;
      const T *xrow = xs + cc + (FLAT ? 0 : brow * sb - brow * p.T * st);
      if (p.dqkv_dtype == kF32)
        conv_bwd_interior<T, float>(xrow, st, static_cast<const float *>(p.dqkv) + c, p.C, dxs + cc, ldx, w, bias, t0,
                                    t1, dw, db);
      else
        conv_bwd_interior<T, T>(xrow, st, static_cast<const T *>(p.dqkv) + c, p.C, dxs + cc, ldx, w, bias, t0, t1, dw,
                                db);
      write_conv_parts<VEC>(p, tile, c, dw, db);
      return;
    }
  }
  // e_u from x_{u-3} .. x_u (xw rows k0 .. k0 + 3), inside u's sequence
  float xw[8][VEC], ew[4][VEC];
  auto e_of = [&](int64_t u, int k0, const float(&dz)[VEC], float(&e)[VEC]) {
    if (u >= ntok) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) e[v] = 0.f;
      return;
    }
    tu.advance(u);
    const int64_t s0 = tu.s0;
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      float y = bias[v] + w[3][v] * xw[k0 + 3][v];
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (u - 3 + j >= s0) y += w[j][v] * xw[k0 + j][v];
      e[v] = dz[v] * dsilu(y);
    }
  };
#pragma unroll
  for (int k = 0; k < 8; ++k) xat(t0 - 3 + k, xw[k]);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float dz[VEC];
    dzat(t0 + k, dz);
    e_of(t0 + k, k, dz, ew[k]);
  }
  for (int64_t tb = t0; tb < t1; tb += NB) {
    // x_{t+5} and dz_{t+4} for the NB tokens t of this group, fetched together
    float xn[NB][VEC], dzn[NB][VEC];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      xat(tb + 5 + k, xn[k]);
      dzat(tb + 4 + k, dzn[k]);
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int64_t t = tb + k;
      if (t >= t1) break;
      tt.advance(t);
      // dx_t = sum_j w_j e_{t+3-j} over tokens of t's sequence
      float dx[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (t + 3 - j < tt.s1) acc += w[j][v] * ew[3 - j][v];
        dx[v] = acc;
        db[v] += ew[0][v];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (t - 3 + j >= tt.s0) dw[j][v] += ew[0][v] * xw[j][v];
      }
      store_vec<T, VEC>(dxs + t * ldx + cc, dx);
      // advance the windows to t + 1: e_{t+4} uses x_{t+1} .. x_{t+4}
      float e4[VEC];
      e_of(t + 4, 4, dzn[k], e4);
#pragma unroll
      for (int q = 0; q < 7; ++q)
#pragma unroll
        for (int v = 0; v < VEC; ++v) xw[q][v] = xw[q + 1][v];
#pragma unroll
      for (int v = 0; v < VEC; ++v) xw[7][v] = xn[k][v];
#pragma unroll
      for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int v = 0; v < VEC; ++v) ew[q][v] = ew[q + 1][v];
#pragma unroll
      for (int v = 0; v < VEC; ++v) ew[3][v] = e4[v];
    }
  }
  write_conv_parts<VEC>(p, tile, c, dw, db);
}

// One block per tile of head_tile tokens (head_tile * Hv <= 4096): d_a and
// d_b of every (token, head) element in order of memory, and per head the
// tile's sums of d_a and d_g g (contributions staged in LDS, then added in
// token order).
template <typename T>
__global__ __launch_bounds__(256) void beta_g_bwd_kernel(PrologueBwdArgs p) {
  __shared__ float ca[4096], cg[4096];
  const int64_t Hv = p.Hv;
  const int64_t ntok = p.B * p.T;
  const int64_t t0 = (int64_t)blockIdx.x * p.head_tile;
  const int64_t t1 = t0 + p.head_tile < ntok ? t0 + p.head_tile : ntok;
  const int64_t ne = (t1 - t0) * Hv;
  const bool fa = p.sa_b == p.T * p.sa_t, fb = p.sb_b == p.T * p.sb_t;
  for (int64_t k = threadIdx.x; k < ne; k += 256) {
    const int64_t t = t0 + k / Hv, h = k % Hv;
    const int64_t ra = fa ? t * p.sa_t : (t / p.T) * p.sa_b + (t % p.T) * p.sa_t;
    const int64_t rb = fb ? t * p.sb_t : (t / p.T) * p.sb_b + (t % p.T) * p.sb_t;
    const float av = f(static_cast<const T *>(p.a)[ra + h]);
    const float bv = f(static_cast<const T *>(p.b)[rb + h]);
    const int64_t e = t * Hv + h;
    const float dg = p.d_g[e], dbeta = p.d_beta[e];
    const float ea = __expf(p.A_log[h]);
    const float xa = av + p.dt_bias[h];
    const float sp = xa > 20.f ? xa : log1pf(__expf(xa));
    const float spd = xa > 20.f ? 1.f : sigm(xa);
    const float beta = sigm(bv);
    const float da = -dg * ea * spd;
    static_cast<T *>(p.d_b)[e] = to<T>(dbeta * beta * (1.f - beta));
    static_cast<T *>(p.d_a)[e] = to<T>(da);
    ca[k] = da;
    cg[k] = dg * (-ea * sp);
  }
  __syncthreads();
  for (int64_t h = threadIdx.x; h < Hv; h += 256) {
    float sa = 0.f, sg = 0.f;
    for (int64_t t = 0; t < t1 - t0; ++t) {
      sa += ca[t * Hv + h];
      sg += cg[t * Hv + h];
    }
    p.part_dt[blockIdx.x * Hv + h] = sa;
    p.part_al[blockIdx.x * Hv + h] = sg;
  }
}

template <typename T>
hipError_t prologue_bwd_t(const PrologueBwdArgs &a, hipStream_t s) {
  const dim3 g4((unsigned)((a.C / 4 + kConvThreads - 1) / kConvThreads), (unsigned)a.ntiles);
  const dim3 g1((unsigned)((a.C + kConvThreads - 1) / kConvThreads), (unsigned)a.ntiles);
  if (a.vec4 && a.x_flat) hipLaunchKernelGGL((conv_bwd_kernel<T, 4, true>), g4, dim3(kConvThreads), 0, s, a);
  else if (a.vec4) hipLaunchKernelGGL((conv_bwd_kernel<T, 4, false>), g4, dim3(kConvThreads), 0, s, a);
  else if (a.x_flat) hipLaunchKernelGGL((conv_bwd_kernel<T, 1, true>), g1, dim3(kConvThreads), 0, s, a);
  else hipLaunchKernelGGL((conv_bwd_kernel<T, 1, false>), g1, dim3(kConvThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((beta_g_bwd_kernel<T>), dim3((unsigned)a.nhtiles), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = sum_partials(a.part_w, a.ntiles, a.C * 4, a.mid, a.d_conv_w, s);
  if (e == hipSuccess && a.d_conv_b) e = sum_partials(a.part_b, a.ntiles, a.C, a.mid, a.d_conv_b, s);
  if (e == hipSuccess) e = sum_partials(a.part_dt, a.nhtiles, a.Hv, a.mid, a.d_dt_bias, s);
  if (e == hipSuccess) e = sum_partials(a.part_al, a.nhtiles, a.Hv, a.mid, a.d_A_log, s);
  return e;
}

}  // namespace

hipError_t launch_gated_norm_bwd(const NormBwdArgs &a, hipStream_t s) {
  if (a.B * a.T * a.H == 0) return hipSuccess;
  switch (a.act) {
    case kF32: return norm_bwd_t<float>(a, s);
    case kBF16: return norm_bwd_t<bf16>(a, s);
    case kF16: return norm_bwd_t<f16>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prologue_bwd(const PrologueBwdArgs &a, hipStream_t s) {
  if (a.B * a.T == 0) return hipSuccess;
  switch (a.act) {
    case kF32: return prologue_bwd_t<float>(a, s);
    case kBF16: return prologue_bwd_t<bf16>(a, s);
    case kF16: return prologue_bwd_t<f16>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
