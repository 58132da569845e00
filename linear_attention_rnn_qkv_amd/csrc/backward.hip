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
#include "device_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + __expf(-x)); }
__device__ __forceinline__ float dsilu(float x) {
  const float s = sigm(x);
  return s * (1.0f + x * (1.0f - s));
}

// out[i] = sum_p part[p * n + i], p in order.
__global__ __launch_bounds__(256) void sum_partials_kernel(const float *__restrict__ part, int64_t nparts, int64_t n,
                                                           float *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float acc = 0.f;
  for (int64_t p = 0; p < nparts; ++p) acc += part[p * n + i];
  out[i] = acc;
}

hipError_t sum_partials(const float *part, int64_t nparts, int64_t n, float *out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(sum_partials_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, nparts, n, out);
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

  for (int64_t row0 = (int64_t)blockIdx.x * RPB; row0 < nrows; row0 += (int64_t)gridDim.x * RPB) {
    const int64_t row = row0 + rg;
    const bool live = row < nrows;
    float o[E], gt[E], du[E];
    if (live) {
      const int64_t h = row % p.H, bt = row / p.H, t = bt % p.T, b = bt / p.T;
      load_vec<T, E>(static_cast<const T *>(p.o) + b * p.so_b + t * p.so_t + h * p.so_h + c0, p.o_align, o);
      load_vec<TG, E>(static_cast<const TG *>(p.gate) + b * p.sg_b + t * p.sg_t + h * p.sg_h + c0, p.gate_align,
                      gt);
      load_vec<T, E>(static_cast<const T *>(p.dout) + b * p.sd_b + t * p.sd_t + h * p.sd_h + c0, p.dout_align, du);
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) o[i] = gt[i] = du[i] = 0.f;
    }
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
      store_vec<T, E>(static_cast<T *>(p.d_o) + row * DV + c0, d_o);
      store_vec<TG, E>(static_cast<TG *>(p.d_gate) + row * DV + c0, dgate);
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
  return sum_partials(a.part, a.nblocks, DV, a.d_w, s);
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

// One thread per channel walks the tokens of one tile in order with rolling
// windows: xw[k] = x_{t-3+k} (k < 8) and ew[k] = e_{t+k} (k < 4), where
// e_u = dz_u silu'(y_u). The tile reads 3 tokens of x before it and 4 ahead;
// x and dz are fetched 8 tokens at a time.
template <typename T>
__global__ __launch_bounds__(kConvThreads) void conv_bwd_kernel(PrologueBwdArgs p) {
  const int64_t c = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
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
  float w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = ldf<T>(p.conv_w, p.w_dtype, 4 * c + j);
  const float bias = p.conv_b ? ldf<T>(p.conv_b, p.b_dtype, c) : 0.f;

  const int64_t ntok = p.B * p.T;
  const int64_t t0 = tile * p.tile_tokens;
  const int64_t t1 = t0 + p.tile_tokens < ntok ? t0 + p.tile_tokens : ntok;
  auto xat = [&](int64_t u) -> float {  // raw x at flattened token u, 0 outside [0, ntok)
    if (u < 0 || u >= ntok) return 0.f;
    return f(xs[(u / p.T) * sb + (u % p.T) * st + cc]);
  };
  auto dzat = [&](int64_t u) -> float { return u < ntok ? ldf<T>(p.dqkv, p.dqkv_dtype, u * p.C + c) : 0.f; };
  SeqTrack tt{p.cu_seqlens, p.n_seqs, p.T, 0, 0, 0};  // sequence of t
  SeqTrack tu{p.cu_seqlens, p.n_seqs, p.T, 0, 0, 0};  // sequence of the lookahead token
  tt.init(t0);
  tu.init(t0);
  // e_u from x_{u-3} .. x_u (window values xa..xd), inside u's sequence
  auto e_of = [&](int64_t u, float xa, float xb, float xc, float xd, float dz) -> float {
    if (u >= ntok) return 0.f;
    tu.advance(u);
    const int64_t s0 = tu.s0;
    const float y = bias + (u - 3 >= s0 ? w[0] * xa : 0.f) + (u - 2 >= s0 ? w[1] * xb : 0.f) +
                    (u - 1 >= s0 ? w[2] * xc : 0.f) + w[3] * xd;
    return dz * dsilu(y);
  };
  float xw[8], ew[4];
#pragma unroll
  for (int k = 0; k < 8; ++k) xw[k] = xat(t0 - 3 + k);
#pragma unroll
  for (int k = 0; k < 4; ++k) ew[k] = e_of(t0 + k, xw[k], xw[k + 1], xw[k + 2], xw[k + 3], dzat(t0 + k));
  float dw[4] = {0.f, 0.f, 0.f, 0.f}, db = 0.f;
  for (int64_t tb = t0; tb < t1; tb += 8) {
    // x_{t+5} and dz_{t+4} for the 8 tokens t of this group, fetched together
    float xn[8], dzn[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      xn[k] = xat(tb + 5 + k);
      dzn[k] = dzat(tb + 4 + k);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t t = tb + k;
      if (t >= t1) break;
      tt.advance(t);
      // dx_t = sum_j w_j e_{t+3-j} over tokens of t's sequence
      float dx = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (t + 3 - j < tt.s1) dx += w[j] * ew[3 - j];
      dxs[t * ldx + cc] = to<T>(dx);
      db += ew[0];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (t - 3 + j >= tt.s0) dw[j] += ew[0] * xw[j];
      // advance the windows to t + 1: e_{t+4} uses x_{t+1} .. x_{t+4}
      const float e4 = e_of(t + 4, xw[4], xw[5], xw[6], xw[7], dzn[k]);
#pragma unroll
      for (int q = 0; q < 7; ++q) xw[q] = xw[q + 1];
      xw[7] = xn[k];
#pragma unroll
      for (int q = 0; q < 3; ++q) ew[q] = ew[q + 1];
      ew[3] = e4;
    }
  }
  float *part = p.part_conv + (tile * p.C + c) * 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) part[j] = dw[j];
  part[4] = db;
}

// One block per (tile, value head): d_a, d_b per token and the tile's sums of
// d_a and d_g g.
template <typename T>
__global__ __launch_bounds__(256) void beta_g_bwd_kernel(PrologueBwdArgs p) {
  __shared__ float red[2][4];
  const int64_t tile = blockIdx.x, h = blockIdx.y;
  const int64_t ntok = p.B * p.T;
  const int64_t t0 = tile * p.tile_tokens;
  const int64_t t1 = t0 + p.tile_tokens < ntok ? t0 + p.tile_tokens : ntok;
  const float ea = __expf(p.A_log[h]), dtb = p.dt_bias[h];
  float sa = 0.f, sg = 0.f;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += 256) {
    const int64_t b = t / p.T, tt = t % p.T;
    const float bv = f(static_cast<const T *>(p.b)[b * p.sb_b + tt * p.sb_t + h]);
    const float av = f(static_cast<const T *>(p.a)[b * p.sa_b + tt * p.sa_t + h]);
    const float dg = p.d_g[t * p.Hv + h], dbeta = p.d_beta[t * p.Hv + h];
    const float beta = sigm(bv);
    const float xa = av + dtb;
    const float sp = xa > 20.f ? xa : log1pf(__expf(xa));
    const float spd = xa > 20.f ? 1.f : sigm(xa);
    const float da = -dg * ea * spd;
    static_cast<T *>(p.d_b)[t * p.Hv + h] = to<T>(dbeta * beta * (1.f - beta));
    static_cast<T *>(p.d_a)[t * p.Hv + h] = to<T>(da);
    sa += da;
    sg += dg * (-ea * sp);
  }
  sa = group_sum<64>(sa);
  sg = group_sum<64>(sg);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[0][wave] = sa;
    red[1][wave] = sg;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float* part = p.part_head + (tile * p.Hv + h) * 2;
    part[0] = red[0][0] + red[0][1] + red[0][2] + red[0][3];  // d_dt_bias
    part[1] = red[1][0] + red[1][1] + red[1][2] + red[1][3];  // d_A_log
  }
}

// [ntiles][Hv][2] -> d_dt_bias, d_A_log; [ntiles][C][5] -> d_w [C][4], d_b [C]
__global__ __launch_bounds__(256) void prologue_sums_kernel(PrologueBwdArgs p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nconv = p.C * 5;
  if (i < nconv) {
    float acc = 0.f;
    for (int64_t q = 0; q < p.ntiles; ++q) acc += p.part_conv[q * nconv + i];
    const int64_t c = i / 5, j = i % 5;
    if (j < 4) p.d_conv_w[c * 4 + j] = acc;
    else if (p.d_conv_b) p.d_conv_b[c] = acc;
  } else if (i < nconv + 2 * p.Hv) {
    const int64_t k = i - nconv, h = k / 2, j = k % 2;
    float acc = 0.f;
    for (int64_t q = 0; q < p.ntiles; ++q) acc += p.part_head[(q * p.Hv + h) * 2 + j];
    if (j == 0) p.d_dt_bias[h] = acc;
    else p.d_A_log[h] = acc;
  }
}

template <typename T>
hipError_t prologue_bwd_t(const PrologueBwdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((conv_bwd_kernel<T>), dim3((unsigned)((a.C + kConvThreads - 1) / kConvThreads), (unsigned)a.ntiles),
                     dim3(kConvThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((beta_g_bwd_kernel<T>), dim3((unsigned)a.ntiles, (unsigned)a.Hv), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = a.C * 5 + 2 * a.Hv;
  hipLaunchKernelGGL(prologue_sums_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
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
