// Output RMSNorm in the activation dtype, then the FP32 SiLU-gate multiply.
//
// Megatron Core developer guide "GDN Elementwise Fusion": the post-recurrence
// fusion (option table) applies the output RMSNorm and SiLU gating; its
// requirements (Post-GDR requirements) are a BF16/FP16 recurrence output, a
// gate of the same shape in the activation dtype or FP32 that may be a strided
// view with separate batch and sequence strides, read without a copy, a
// contiguous weight of length head_dim and contiguous outputs; the RMSNorm
// result is materialised in the activation dtype before the FP32 gate
// multiply (Execution and numerical behavior). FP32 recurrence outputs are
// accepted as well.
//
// Per (token, head) row of dv elements:
//   r = 1/sqrt(mean(o^2) + eps);  y = round_act(o*r*w);
//   out = round_act(y * silu(gate))          (all arithmetic in FP32)
//
// Memory-bound: each row is read once (o, gate) and written once (out). A row
// is handled by dv/8 lanes holding 8 elements each; the sum of squares is a
// butterfly reduction inside that lane group. Each lane handles two rows so
// that four independent 16-byte loads are in flight per lane; o, gate and out
// are streamed with non-temporal accesses (each byte is touched once).
#include "device_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerLane = 2;

template <typename T, typename TG, typename TW, int DV>
__global__ __launch_bounds__(kThreads) void gated_norm_kernel(NormArgs p) {
  constexpr int E = 8;
  constexpr int LPR = DV / E;                  // lanes per row
  constexpr int RPW = 64 / LPR;                // row groups per wave
  constexpr int RPB = (kThreads / 64) * RPW;   // row groups per block
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = (lane % LPR) * E;
  const int64_t nrows = p.B * p.T * p.H;

  float w[E];
  load_vec<TW, E>(static_cast<const TW *>(p.w) + c0, 16, w);

  float ov[kRowsPerLane][E], gv[kRowsPerLane][E];
  int64_t rows[kRowsPerLane];
#pragma unroll
  for (int u = 0; u < kRowsPerLane; ++u) {
    const int64_t row = ((int64_t)blockIdx.x * kRowsPerLane + u) * RPB + wave * RPW + lane / LPR;
    rows[u] = row;
    if (row < nrows) {
      int64_t b, t, h;
      split_row(p.rd, p.T, p.H, row, b, t, h);
      load_vec_nt<T, E>(static_cast<const T *>(p.o) + b * p.so_b + t * p.so_t + h * p.so_h + c0,
                     p.o_align, ov[u]);
      load_vec_nt<TG, E>(static_cast<const TG *>(p.gate) + b * p.sg_b + t * p.sg_t + h * p.sg_h + c0,
                      p.gate_align, gv[u]);
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) ov[u][i] = gv[u][i] = 0.f;
    }
  }
#pragma unroll
  for (int u = 0; u < kRowsPerLane; ++u) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) ss += ov[u][i] * ov[u][i];
    ss = group_sum<LPR>(ss);
    const float r = rsqrtf(ss * (1.0f / DV) + p.eps);
    float res[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float y = round_through<T>(ov[u][i] * r * w[i]);
      res[i] = y * silu(gv[u][i]);
    }
    if (rows[u] < nrows) store_vec_nt<T, E>(static_cast<T *>(p.out) + rows[u] * DV + c0, res);
  }
}

template <typename T, typename TG, typename TW, int DV>
hipError_t launch_dv(const NormArgs &a, hipStream_t s) {
  constexpr int RPB = (kThreads / 64) * (64 / (DV / 8));
  const int64_t nrows = a.B * a.T * a.H;
  const int64_t per_block = (int64_t)RPB * kRowsPerLane;
  const int64_t blocks = (nrows + per_block - 1) / per_block;
  hipLaunchKernelGGL((gated_norm_kernel<T, TG, TW, DV>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     s, a);
  return hipGetLastError();
}

template <typename T, typename TG, typename TW>
hipError_t launch_w(const NormArgs &a, hipStream_t s) {
  switch (a.dv) {
    case 64: return launch_dv<T, TG, TW, 64>(a, s);
    case 128: return launch_dv<T, TG, TW, 128>(a, s);
    case 256: return launch_dv<T, TG, TW, 256>(a, s);
    case 512: return launch_dv<T, TG, TW, 512>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, typename TG>
hipError_t launch_g(const NormArgs &a, hipStream_t s) {
  switch (a.w_dtype) {
    case kF32: return launch_w<T, TG, float>(a, s);
    case kBF16: return launch_w<T, TG, bf16>(a, s);
    case kF16: return launch_w<T, TG, f16>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_t(const NormArgs &a, hipStream_t s) {
  if (a.gate_dtype == kF32) return launch_g<T, float>(a, s);
  if (a.gate_dtype == a.act) return launch_g<T, T>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gated_norm(const NormArgs &a, hipStream_t s) {
  if (a.B * a.T * a.H == 0) return hipSuccess;
  switch (a.act) {
    case kF32: return launch_t<float>(a, s);
    case kBF16: return launch_t<bf16>(a, s);
    case kF16: return launch_t<f16>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
