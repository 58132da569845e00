// Pre-recurrence prologue: one depthwise causal conv1d (4 taps) + SiLU over
// the concatenated q|k|v channels, and beta / log-decay preparation.
//
// flash-linear-attention pull request fusing GatedDeltaNet's q/k/v short
// convolutions (Summary, Why): the three depthwise convolutions share kernel
// size and activation and mix no channels, so one convolution over the
// channel-concatenated projections with concatenated weights (and bias) is
// the same computation at one launch. Here the concatenation costs no copy:
// the kernel reads the three (possibly strided) projection views in place and
// writes one [B, T, C] buffer whose channel ranges are q, k and v.
// Megatron Core "GDN Elementwise Fusion" (option table) lists the same
// prologue operations plus beta and decay preparation; the formulas used for
// those are beta = sigmoid(b) and g = -exp(A_log) * softplus(a + dt_bias)
// (Gated DeltaNet's parameterisation; the pages do not print them).
//
// Layout and schedule (HBM-bound): a thread owns VEC consecutive channels and
// walks a tile of 128 tokens (16 when the launch would have few blocks) in
// batches of 8, double-buffered so that the
// next batch's loads (raw packed vectors) are in flight during the arithmetic
// of the current one. It convolves over a window that keeps the three previous
// inputs in registers, so each input element is read once (plus a 3-token halo
// per tile) and each output is written once, with VEC-wide coalesced accesses.
// History is zero before every sequence start: batch rows are sequences; with
// cu_seqlens the thread finds the boundaries inside its tile from the offsets.
// The blocks of a token tile also compute beta and g of its tokens, each an
// equal share of the (token, head) pairs.
#include <limits.h>

#include "device_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;   // tokens per load batch

template <typename TW>
__device__ __forceinline__ float ld_param(const void *p, int64_t i) {
  return f(static_cast<const TW *>(p)[i]);
}

__device__ __forceinline__ float ld_any(const void *p, int32_t dt, int64_t i) {
  if (dt == kF32) return ld_param<float>(p, i);
  if (dt == kBF16) return ld_param<bf16>(p, i);
  return ld_param<f16>(p, i);
}

constexpr float kLog2e = 1.4426950408889634f;

// silu(y) from y2 = y * log2(e): y * sigmoid(y) = y2 / (log2(e) * (1 + 2^-y2)).
// (Convolving with weights pre-scaled by log2(e) saves the scaling of the
// exponent's argument.) For y2 -> -inf the reciprocal is 0 and the result -0.
__device__ __forceinline__ float silu_log2(float y2) {
  return y2 * __builtin_amdgcn_rcpf(__builtin_fmaf(kLog2e, __builtin_amdgcn_exp2f(-y2), kLog2e));
}

// beta and g of the tile's (token, head) pairs [lo, hi) in token-major order
template <typename T>
__device__ void beta_g_tile(const PrologueArgs &p, int64_t b, int64_t t0, int64_t lo, int64_t hi) {
  const T *pa = static_cast<const T *>(p.a);
  const T *pb = static_cast<const T *>(p.b);
  for (int64_t i = lo + threadIdx.x; i < hi; i += blockDim.x) {
    const int64_t t = t0 + i / p.Hv, h = i % p.Hv;
    const float bb = f(pb[b * p.sb_b + t * p.sb_t + h * p.sb_h]);
    const float aa = f(pa[b * p.sa_b + t * p.sa_t + h * p.sa_h]);
    const float x = aa + p.dt_bias[h];
    const float sp = x > 20.f ? x : log1pf(expf(x));
    const int64_t o = (b * p.T + t) * p.Hv + h;
    p.beta[o] = 1.0f / (1.0f + expf(-bb));
    p.g[o] = -expf(p.A_log[h]) * sp;
  }
}

template <typename T, int VEC, int TILE>
__global__ __launch_bounds__(kThreads) void prologue_kernel(PrologueArgs p) {
  // Consecutive blocks cover consecutive token tiles of one channel block.
  const int cb = (int)blockIdx.y;
  const int64_t b = blockIdx.z;
  const int64_t t0 = (int64_t)blockIdx.x * TILE;
  const int64_t t1 = t0 + TILE < p.T ? t0 + TILE : p.T;
  const int64_t c0 = ((int64_t)cb * blockDim.x + threadIdx.x) * VEC;
  const bool active = c0 < p.C;
  const int64_t nq = p.Hqk * p.dk;

  // Source view for this thread's channels (lanes past C read the last
  // channels and store nothing, so every lane issues the same loads).
  const int64_t cl = active ? c0 : p.C - VEC;
  const T *src;
  int64_t st;
  if (cl < nq) {
    src = static_cast<const T *>(p.xq) + b * p.sxq_b + cl;
    st = p.sxq_t;
  } else if (cl < 2 * nq) {
    src = static_cast<const T *>(p.xk) + b * p.sxk_b + (cl - nq);
    st = p.sxk_t;
  } else {
    src = static_cast<const T *>(p.xv) + b * p.sxv_b + (cl - 2 * nq);
    st = p.sxv_t;
  }
  constexpr int AL = VEC * (int)sizeof(T);

  // The thread's taps are 4*VEC consecutive weights: vector loads.
  float w[VEC][4], bias[VEC];
  {
    float wf[4 * VEC];
    if (!active) {
#pragma unroll
      for (int i = 0; i < 4 * VEC; ++i) wf[i] = 0.f;
    } else if (p.w_dtype == kF32) {
      load_vec<float, 4 * VEC>(static_cast<const float *>(p.conv_w) + c0 * 4, align_of(16 * VEC) < p.w_align
                               ? align_of(16 * VEC) : p.w_align, wf);
    } else {
      load_vec<T, 4 * VEC>(static_cast<const T *>(p.conv_w) + c0 * 4,
                           align_of(8 * VEC) < p.w_align ? align_of(8 * VEC) : p.w_align, wf);
    }
    // taps and bias pre-scaled by log2(e): the convolution yields y * log2(e)
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) w[i][j] = wf[4 * i + j] * kLog2e;
      bias[i] = (active && p.conv_b) ? ld_any(p.conv_b, p.b_dtype, c0 + i) * kLog2e : 0.f;
    }
  }

  // Sequence containing t0, and the next boundary after it.
  int64_t bos = 0, next = LLONG_MAX, idx = 0;
  const int32_t *cu = p.cu_seqlens;
  if (cu) {
    // the last lo with cu[lo] <= t0 (cu[0] = 0 <= t0): 64 strided samples
    // per round, one memory round trip each, the interval narrowed by the
    // count of samples <= t0 (cu is nondecreasing)
    int64_t lo = 0, end = p.n_seqs + 1;  // candidates lo .. end - 1
    const int lane = threadIdx.x & 63;
    while (end - lo > 1) {
      const int64_t step = (end - lo + 63) / 64;
      const int64_t at = lo + lane * step;
      const bool le = at < end && cu[at] <= t0;
      const int cnt = __popcll(__ballot(le));  // >= 1: cu[lo] <= t0
      lo += (int64_t)(cnt - 1) * step;
      end = lo + step < end ? lo + step : end;
    }
    bos = cu[lo];
    idx = lo + 1;
    next = idx <= p.n_seqs ? cu[idx] : LLONG_MAX;
  }

  // Inputs at t0-1, t0-2, t0-3 (zero before the sequence start). The loads
  // are unconditional (clamped rows) so they overlap the first batch's.
  float h1[VEC], h2[VEC], h3[VEC];
  {
    const int64_t r1 = t0 - 1 >= 0 ? t0 - 1 : 0, r2 = t0 - 2 >= 0 ? t0 - 2 : 0, r3 = t0 - 3 >= 0 ? t0 - 3 : 0;
    load_vec<T, VEC>(src + r1 * st, AL, h1);
    load_vec<T, VEC>(src + r2 * st, AL, h2);
    load_vec<T, VEC>(src + r3 * st, AL, h3);
    const bool v1 = t0 - 1 >= bos, v2 = t0 - 2 >= bos, v3 = t0 - 3 >= bos;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      h1[i] = v1 ? h1[i] : 0.f;
      h2[i] = v2 ? h2[i] : 0.f;
      h3[i] = v3 ? h3[i] : 0.f;
    }
  }

  const bool l2 = p.caller_l2norm && c0 < 2 * nq;
  const int group = (int)(p.dk / VEC);  // lanes per q/k head
  T *dst = static_cast<T *>(p.qkv) + b * p.T * p.C + c0;

  // Batches of kUnroll tokens. Loads are unconditional (rows past the tile
  // end read the tile's last row, results unused) so the compiler can count
  // the outstanding loads exactly.
  auto load_batch = [&](int64_t tb, T (&raw)[kUnroll][VEC]) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t t = tb + u < t1 ? tb + u : t1 - 1;
      load_raw_nt<T, VEC>(src + t * st, AL, raw[u]);
    }
  };
  auto emit = [&](int64_t t, float (&z)[VEC]) {
    if (p.caller_l2norm) {  // block-uniform: every lane joins the shuffles
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) ss += z[i] * z[i];
      for (int off = group >> 1; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
      if (l2) {
        const float r = rsqrtf(ss + p.l2_eps);
#pragma unroll
        for (int i = 0; i < VEC; ++i) z[i] *= r;
      }
    }
    if (active && t < t1) store_vec_nt<T, VEC>(dst + t * p.C, z);
  };
  auto compute_batch = [&](int64_t tb, const T (&raw)[kUnroll][VEC]) {
    if (next >= tb + kUnroll) {
      // No sequence starts inside the batch: a rolling 4-input window per
      // channel over the fully unrolled batch (registers are renamed, not
      // moved).
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float z[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float x = f(raw[u][i]);
          z[i] = silu_log2(bias[i] + w[i][0] * h3[i] + w[i][1] * h2[i] + w[i][2] * h1[i] + w[i][3] * x);
          h3[i] = h2[i];
          h2[i] = h1[i];
          h1[i] = x;
        }
        emit(tb + u, z);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t t = tb + u;
      if (t >= t1) break;
      if (t == next) {  // a new sequence starts: drop the history
#pragma unroll
        for (int i = 0; i < VEC; ++i) h1[i] = h2[i] = h3[i] = 0.f;
        while (idx <= p.n_seqs && cu[idx] <= t) ++idx;
        next = idx <= p.n_seqs ? cu[idx] : LLONG_MAX;
      }
      float z[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const float x = f(raw[u][i]);
        z[i] = silu_log2(bias[i] + w[i][0] * h3[i] + w[i][1] * h2[i] + w[i][2] * h1[i] + w[i][3] * x);
      }
      emit(t, z);
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        h3[i] = h2[i];
        h2[i] = h1[i];
        h1[i] = f(raw[u][i]);
      }
    }
  };
  T ra[kUnroll][VEC], rb[kUnroll][VEC];
  if (t1 - t0 == TILE) {
    // Full tile: double-buffered with a fixed trip count, the loads of batch
    // i + 1 in flight during the arithmetic of batch i.
    constexpr int kPairs = TILE / (2 * kUnroll);
    load_batch(t0, ra);
    int64_t tb = t0;
    for (int i = 0; i < kPairs - 1; ++i, tb += 2 * kUnroll) {
      load_batch(tb + kUnroll, rb);
      compute_batch(tb, ra);
      load_batch(tb + 2 * kUnroll, ra);
      compute_batch(tb + kUnroll, rb);
    }
    load_batch(tb + kUnroll, rb);
    compute_batch(tb, ra);
    compute_batch(tb + kUnroll, rb);
  } else {
    for (int64_t tb = t0; tb < t1; tb += kUnroll) {
      load_batch(tb, ra);
      compute_batch(tb, ra);
    }
  }
  // beta and g of the tile's tokens, split evenly over its channel blocks
  {
    const int64_t n = (t1 - t0) * p.Hv, ncb = gridDim.y;
    beta_g_tile<T>(p, b, t0, n * cb / ncb, n * (cb + 1) / ncb);
  }
}

// Token tile: the largest of 128, 64, 32, 16 tokens that still gives the
// launch one block per CU, else 16 (each block walks its tile's tokens in
// order; a short launch would leave most of the chip idle). Smaller tiles
// re-read a 3-row halo per tile. Measured at 8192 tokens of 16 + 16 + 32
// heads (256 blocks of 128 tokens): more, smaller blocks (64- or 32-token
// tiles, or 128- and 64-thread blocks) were 2-27% slower.
constexpr int64_t kMinBlocks = 256;

template <typename T, int VEC, int TILE>
hipError_t launch_tile(const PrologueArgs &a, int64_t cblocks, int threads, hipStream_t s) {
  const int64_t tblocks = (a.T + TILE - 1) / TILE;
  dim3 grid((unsigned)tblocks, (unsigned)cblocks, (unsigned)a.B);
  hipLaunchKernelGGL((prologue_kernel<T, VEC, TILE>), grid, dim3(threads), 0, s, a);
  return hipGetLastError();
}

template <typename T, int VEC>
hipError_t launch_vec(const PrologueArgs &a, hipStream_t s) {
  const int threads = kThreads;
  const int64_t cblocks = (a.C + (int64_t)threads * VEC - 1) / ((int64_t)threads * VEC);
  auto blocks = [&](int64_t tile) { return ((a.T + tile - 1) / tile) * cblocks * a.B; };
  if (blocks(128) >= kMinBlocks) return launch_tile<T, VEC, 128>(a, cblocks, threads, s);
  if (blocks(64) >= kMinBlocks) return launch_tile<T, VEC, 64>(a, cblocks, threads, s);
  if (blocks(32) >= kMinBlocks) return launch_tile<T, VEC, 32>(a, cblocks, threads, s);
  return launch_tile<T, VEC, 16>(a, cblocks, threads, s);
}

template <typename T>
hipError_t launch_t(const PrologueArgs &a, hipStream_t s) {
  switch (a.vec) {
    case 1: return launch_vec<T, 1>(a, s);
    case 2: return launch_vec<T, 2>(a, s);
    case 4: return launch_vec<T, 4>(a, s);
    case 8:
      if constexpr (sizeof(T) == 2) return launch_vec<T, 8>(a, s);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs &a, hipStream_t s) {
  if (a.B * a.T == 0) return hipSuccess;
  switch (a.act) {
    case kF32: return launch_t<float>(a, s);
    case kBF16: return launch_t<bf16>(a, s);
    case kF16: return launch_t<f16>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
