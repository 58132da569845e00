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
// One workgroup of 1024 threads per (sequence, query/key head): it convolves
// the q and k channels of the head once and the v channels of its G value
// heads, then updates the G states, which are adjacent in memory (one block
// of G * dv rows of dk floats). A row is handled by dk / 4 lanes, 4 floats
// each (one 16-byte non-temporal load and store); the two dot products per
// row are lane-group reductions. Wide, short-lived workgroups matter here: on
// this part a read-modify-write stream of many independent workgroups runs
// faster the less work each workgroup holds (measured: 256 rows per 256-thread
// workgroup reach 5.1 TB/s, the same rows per 1024-thread workgroup 5.8 TB/s),
// and the row block of one (sequence, head group) cannot be split across
// workgroups without a race on the shared q/k conv cache.
#include "device_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 1024;
constexpr int kCols = 4;       // state columns per lane (one 16-byte access)
constexpr int kBatch = 4;      // state rows in flight per lane
constexpr int kWavesPerEU = 8;
constexpr int kMaxVCh = 8192;  // G * dv (dynamic LDS: one FP32 row of this length)
constexpr int kMaxG = 64;

template <typename T>
__device__ __forceinline__ float ld_as(const void *p, int32_t dt, int64_t i) {
  if (dt == kF32) return static_cast<const float *>(p)[i];
  return f(static_cast<const T *>(p)[i]);
}

template <typename T, int DK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU))) void decode_kernel(
    DecodeArgs p) {
  constexpr int LR = DK / kCols;     // lanes per state row
  constexpr int RP = kThreads / LR;  // rows per pass
  __shared__ __align__(16) float qv[DK], kv[DK];
  __shared__ float gexp[kMaxG], bet[kMaxG];
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
  const int cb = tid % LR, rw = tid / LR;  // column block and row within a pass
  const int64_t np = p.dv / RP;           // passes of RP rows per value head

  // The G value heads of query/key head hk are adjacent in the state, so the
  // workgroup's rows form one contiguous block of G * dv rows, walked in
  // passes of RP rows (a pass never straddles two heads: RP divides dv).
  const int nt = (int)(G * np);
  const int lnp = __builtin_ctz((unsigned)np);
  float *sbase = p.state + ((n * p.Hv + hk * G) * p.dv + rw) * DK + kCols * cb;

  // The rows of the first batch are requested before anything else: their
  // latency overlaps the conv below.
  float s[kBatch][kCols];
#pragma unroll
  for (int b = 0; b < kBatch; ++b)
    if (b < nt) load_vec_nt<float, kCols>(sbase + (int64_t)b * RP * DK, 16, s[b]);

  // 1. conv + SiLU of the head's q, k channels and its value heads' v
  //    channels; the cache shifts by one token
  // Offsets below are 32-bit from uniform base pointers (C < 2^31).
  T *cs0 = static_cast<T *>(p.conv_state) + n * p.scs_n;
  T *cs1 = cs0 + p.scs_t, *cs2 = cs1 + p.scs_t;
  const bool w32 = p.w_dtype == kF32, b32 = p.b_dtype == kF32;
  auto conv = [&](int ch, float x) {
    const float c0 = f(cs0[ch]), c1 = f(cs1[ch]), c2 = f(cs2[ch]);
    float w[4];
    if (w32) load_vec<float, 4>(static_cast<const float *>(p.conv_w) + 4 * ch, p.w_align, w);
    else load_vec<T, 4>(static_cast<const T *>(p.conv_w) + 4 * ch, p.w_align, w);
    float y = 0.f;
    if (p.conv_b) y = b32 ? static_cast<const float *>(p.conv_b)[ch] : f(static_cast<const T *>(p.conv_b)[ch]);
    y += w[0] * c0 + w[1] * c1 + w[2] * c2 + w[3] * x;
    cs0[ch] = to<T>(c1);
    cs1[ch] = to<T>(c2);
    cs2[ch] = to<T>(x);
    return round_through<T>(silu(y));
  };
  {
    const T *xq = static_cast<const T *>(p.xq) + n * p.sxq + hk * DK;
    const T *xk = static_cast<const T *>(p.xk) + n * p.sxk + hk * DK;
    const T *xv = static_cast<const T *>(p.xv) + n * p.sxv + hk * nvc;
    const int q0 = (int)(hk * DK), k0 = (int)(nq + hk * DK), v0 = (int)(2 * nq + hk * nvc);
    for (int i = tid; i < DK; i += kThreads) qv[i] = conv(q0 + i, f(xq[i]));
    for (int i = tid; i < DK; i += kThreads) kv[i] = conv(k0 + i, f(xk[i]));
    for (int i = tid; i < (int)nvc; i += kThreads) vv[i] = conv(v0 + i, f(xv[i]));
  }
  // beta and g of the G value heads
  for (int64_t j = tid; j < G; j += kThreads) {
    const int64_t h = hk * G + j;
    const float bb = f(static_cast<const T *>(p.b)[n * p.sb + h]);
    const float xa = f(static_cast<const T *>(p.a)[n * p.sa + h]) + p.dt_bias[h];
    const float sp = xa > 20.f ? xa : log1pf(expf(xa));
    bet[j] = 1.0f / (1.0f + expf(-bb));
    gexp[j] = fast_exp(-expf(p.A_log[h]) * sp);  // the decay e^g
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

  // 3. state update; the lane group of a row holds its columns
  //    kCols * cb .. kCols * cb + kCols - 1
  float kh[kCols], qh[kCols];
#pragma unroll
  for (int e = 0; e < kCols; ++e) {
    kh[e] = kv[kCols * cb + e] * nrm[1];
    qh[e] = qv[kCols * cb + e] * nrm[0];
  }
  // batches of kBatch passes: their rows are loaded before any is updated
  for (int t0 = 0; t0 < nt; t0 += kBatch) {
    if (t0 > 0) {
#pragma unroll
      for (int b = 0; b < kBatch; ++b)
        if (t0 + b < nt) load_vec_nt<float, kCols>(sbase + (int64_t)(t0 + b) * RP * DK, 16, s[b]);
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (t0 + b >= nt) break;
      const int t = t0 + b, j = t >> lnp;  // value head j of the group
      const int r = t * RP + rw;           // row of the block: j * dv + (row in head j)
      const float decay = gexp[j], bj = bet[j];
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < kCols; ++e) {
        s[b][e] *= decay;
        d += s[b][e] * kh[e];
      }
      d = group_sum<LR>(d);
      const float u = bj * (vv[r] - d);
      float o = 0.f;
#pragma unroll
      for (int e = 0; e < kCols; ++e) {
        s[b][e] += u * kh[e];
        o += s[b][e] * qh[e];
      }
      o = group_sum<LR>(o);
      store_vec_nt<float, kCols>(sbase + (int64_t)t * RP * DK, s[b]);
      if (cb == 0) ov[r] = p.scale * o;
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
