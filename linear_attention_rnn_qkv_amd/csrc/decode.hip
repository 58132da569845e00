// One recurrent decode step of the layer core: a new token for each of N
// sequences, each carrying a conv cache (its last three inputs per channel)
// and an FP32 state per value head. Per sequence and value head:
//
//   conv:   y = bias + w0 c0 + w1 c1 + w2 c2 + w3 x, z = round_act(silu(y)),
//           cache <- (c1, c2, x)       (the conv of the prologue, last token)
//   gates:  beta = sigmoid(b), g = -exp(A_log) softplus(a + dt_bias)
//   rule:   q^ = q / |q|, k^ = k / |k| (in-kernel L2 fold), then
//           S <- e^g S;  u = v - S k^;  S <- S + beta u k^T;  o = scale S q^
//           (the gated delta rule of Gated DeltaNet, one token)
//   norm:   y = round_act(round_act(o) r w), out = round_act(y silu(gate))
//           (the gated RMSNorm of the Megatron Core "GDN Elementwise Fusion"
//           page, section Execution and numerical behavior)
//
// The same materialisation points as the prefill layer core: conv outputs,
// o, the RMSNorm result and the output in the activation dtype; g, beta and
// the state in FP32. Decode is bound by the state's HBM traffic (read and
// written once, 2 * dv * dk * 4 bytes per head and token); everything else is
// a few KB per sequence.
//
// One workgroup per (sequence, query/key head): it convolves the q and k
// channels of the head once and the v channels of its G value heads, then
// updates the G states. A state row (dk floats) is handled by dk / 8 lanes,
// 8 floats each (two 16-byte non-temporal loads and stores); the two dot
// products per row are lane-group reductions.
#include "device_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxVCh = 8192;  // G * dv (dynamic LDS: one FP32 row of this length)
constexpr int kMaxG = 64;

template <typename T>
__device__ __forceinline__ float ld_as(const void *p, int32_t dt, int64_t i) {
  if (dt == kF32) return static_cast<const float *>(p)[i];
  return f(static_cast<const T *>(p)[i]);
}

template <typename T, int DK>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs p) {
  constexpr int LR = DK / 8;             // lanes per state row
  constexpr int RP = kThreads / LR;      // rows per pass
  __shared__ float qv[DK], kv[DK];
  __shared__ float gdec[kMaxG], bet[kMaxG];
  __shared__ float nrm[2];
  // v of the G value heads; row i's o overwrites its v (the lanes that read
  // v[i] belong to the wave that writes o[i], and one wave's LDS accesses
  // complete in order)
  extern __shared__ float dyn[];
  float *vv = dyn, *ov = dyn;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t hk = blockIdx.x, n = blockIdx.y;
  const int64_t G = p.Hv / p.Hqk, nq = p.Hqk * DK;
  const int64_t nvc = G * p.dv;

  // 1. conv + SiLU of the head's q, k channels and its value heads' v
  //    channels; the cache shifts by one token
  const T *xq = static_cast<const T *>(p.xq) + n * p.sxq + hk * DK;
  const T *xk = static_cast<const T *>(p.xk) + n * p.sxk + hk * DK;
  const T *xv = static_cast<const T *>(p.xv) + n * p.sxv + hk * nvc;
  T *cs = static_cast<T *>(p.conv_state) + n * p.scs_n;
  for (int64_t i = tid; i < 2 * DK + nvc; i += kThreads) {
    int64_t ch;
    float x;
    if (i < DK) {
      ch = hk * DK + i;
      x = f(xq[i]);
    } else if (i < 2 * DK) {
      ch = nq + hk * DK + (i - DK);
      x = f(xk[i - DK]);
    } else {
      ch = 2 * nq + hk * nvc + (i - 2 * DK);
      x = f(xv[i - 2 * DK]);
    }
    const float c0 = f(cs[ch]), c1 = f(cs[p.scs_t + ch]), c2 = f(cs[2 * p.scs_t + ch]);
    float y = p.conv_b ? ld_as<T>(p.conv_b, p.b_dtype, ch) : 0.f;
    y += ld_as<T>(p.conv_w, p.w_dtype, 4 * ch) * c0 + ld_as<T>(p.conv_w, p.w_dtype, 4 * ch + 1) * c1 +
         ld_as<T>(p.conv_w, p.w_dtype, 4 * ch + 2) * c2 + ld_as<T>(p.conv_w, p.w_dtype, 4 * ch + 3) * x;
    const float z = round_through<T>(silu(y));
    if (i < DK) qv[i] = z;
    else if (i < 2 * DK) kv[i - DK] = z;
    else vv[i - 2 * DK] = z;
    cs[ch] = to<T>(c1);
    cs[p.scs_t + ch] = to<T>(c2);
    cs[2 * p.scs_t + ch] = to<T>(x);
  }
  // beta and g of the G value heads
  for (int64_t j = tid; j < G; j += kThreads) {
    const int64_t h = hk * G + j;
    const float bb = f(static_cast<const T *>(p.b)[n * p.sb + h]);
    const float xa = f(static_cast<const T *>(p.a)[n * p.sa + h]) + p.dt_bias[h];
    const float sp = xa > 20.f ? xa : log1pf(expf(xa));
    bet[j] = 1.0f / (1.0f + expf(-bb));
    gdec[j] = -expf(p.A_log[h]) * sp;
  }
  __syncthreads();

  // 2. inverse L2 norms of q (wave 0) and k (wave 1)
  if (wave < 2) {
    const float *src = wave == 0 ? qv : kv;
    float ss = 0.f;
    for (int i = lane; i < DK; i += 64) ss += src[i] * src[i];
    ss = group_sum<64>(ss);
    if (lane == 0) nrm[wave] = p.use_l2 ? rsqrtf(ss + p.l2_eps) : 1.f;
  }
  __syncthreads();

  // 3. state update, one value head at a time; lane group of row i holds dk
  //    columns 8 cb .. 8 cb + 7
  const int cb = tid % LR;
  float kh[8], qh[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    kh[e] = kv[8 * cb + e] * nrm[1];
    qh[e] = qv[8 * cb + e] * nrm[0];
  }
  for (int64_t j = 0; j < G; ++j) {
    const int64_t h = hk * G + j;
    const float decay = fast_exp(gdec[j]), bj = bet[j];
    float *sbase = p.state + ((n * p.Hv + h) * p.dv) * DK + 8 * cb;
    const int64_t np = p.dv / RP;  // passes of RP rows
    // batches of four passes: their rows are loaded before any is updated
    for (int64_t p0 = 0; p0 < np; p0 += 4) {
      float s[4][8];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (p0 + b < np) load_vec_nt<float, 8>(sbase + ((p0 + b) * RP + tid / LR) * DK, 16, s[b]);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (p0 + b >= np) break;
        const int64_t i = (p0 + b) * RP + tid / LR;
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s[b][e] *= decay;
          d += s[b][e] * kh[e];
        }
        d = group_sum<LR>(d);
        const float u = bj * (vv[j * p.dv + i] - d);
        float o = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s[b][e] += u * kh[e];
          o += s[b][e] * qh[e];
        }
        o = group_sum<LR>(o);
        store_vec_nt<float, 8>(sbase + i * DK, s[b]);
        if (cb == 0) ov[j * p.dv + i] = p.scale * o;
      }
    }
  }
  __syncthreads();

  // 4. gated RMSNorm of each value head's row (one wave per head)
  for (int64_t j = wave; j < G; j += kThreads / 64) {
    const int64_t h = hk * G + j;
    float ss = 0.f;
    for (int64_t i = lane; i < p.dv; i += 64) {
      const float o = round_through<T>(ov[j * p.dv + i]);
      ov[j * p.dv + i] = o;
      ss += o * o;
    }
    ss = group_sum<64>(ss);
    const float r = rsqrtf(ss / (float)p.dv + p.rms_eps);
    const int64_t gb = n * p.sgate_n + h * p.sgate_h;
    T *out = static_cast<T *>(p.out) + (n * p.Hv + h) * p.dv;
    for (int64_t i = lane; i < p.dv; i += 64) {
      const float y = round_through<T>(ov[j * p.dv + i] * r * ld_as<T>(p.norm_w, p.nw_dtype, i));
      const float gt = ld_as<T>(p.gate, p.gate_dtype, gb + i);
      out[i] = to<T>(y * silu(gt));
    }
  }
}

template <typename T>
hipError_t launch_t(const DecodeArgs &a, hipStream_t s) {
  dim3 grid((unsigned)a.Hqk, (unsigned)a.N);
  const size_t lds = (size_t)(a.Hv / a.Hqk) * a.dv * sizeof(float);
  switch (a.dk) {
    case 64: hipLaunchKernelGGL((decode_kernel<T, 64>), grid, dim3(kThreads), lds, s, a); break;
    case 128: hipLaunchKernelGGL((decode_kernel<T, 128>), grid, dim3(kThreads), lds, s, a); break;
    case 256: hipLaunchKernelGGL((decode_kernel<T, 256>), grid, dim3(kThreads), lds, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool decode_supported(int64_t dk, int64_t G, int64_t dv) {
  return (dk == 64 || dk == 128 || dk == 256) && G <= kMaxG && G * dv <= kMaxVCh && dv >= 64 && dv <= 512;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  if (a.act == kF32) return launch_t<float>(a, s);
  if (a.act == kBF16) return launch_t<bf16>(a, s);
  if (a.act == kF16) return launch_t<f16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace gdn
