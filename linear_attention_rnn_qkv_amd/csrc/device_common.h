// Device helpers shared by the gfx950 kernels: element types, alignment-aware
// vector loads/stores, fast transcendentals and 64-wide wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

// float <-> element; the conversion to 16-bit types rounds to nearest even.
template <typename T> __device__ __forceinline__ float f(T x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T to(float x) { return static_cast<T>(x); }

// Load N consecutive elements starting at p into floats. `align` is the
// number of bytes p is known to be aligned to (a power of two, >= sizeof(T));
// the widest access that alignment allows is used, up to 16 bytes.
template <typename T, int N>
__device__ __forceinline__ void load_vec(const T *__restrict__ p, int align, float (&out)[N]) {
  constexpr int BYTES = N * (int)sizeof(T);
  T tmp[N];
  const char *src = reinterpret_cast<const char *>(p);
  char *dst = reinterpret_cast<char *>(tmp);
  if (BYTES % 16 == 0 && align >= 16) {
#pragma unroll
    for (int c = 0; c < BYTES / 16; ++c) {
      uint4 u = *reinterpret_cast<const uint4 *>(src + 16 * c);
      __builtin_memcpy(dst + 16 * c, &u, 16);
    }
  } else if (BYTES % 8 == 0 && align >= 8) {
#pragma unroll
    for (int c = 0; c < BYTES / 8; ++c) {
      uint2 u = *reinterpret_cast<const uint2 *>(src + 8 * c);
      __builtin_memcpy(dst + 8 * c, &u, 8);
    }
  } else if (BYTES % 4 == 0 && align >= 4) {
#pragma unroll
    for (int c = 0; c < BYTES / 4; ++c) {
      uint32_t u = *reinterpret_cast<const uint32_t *>(src + 4 * c);
      __builtin_memcpy(dst + 4 * c, &u, 4);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) tmp[i] = p[i];
  }
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = f(tmp[i]);
}

// Store N floats as T at p, which is aligned to min(16, N * sizeof(T)) bytes.
template <typename T, int N>
__device__ __forceinline__ void store_vec(T *__restrict__ p, const float (&v)[N]) {
  constexpr int BYTES = N * (int)sizeof(T);
  T tmp[N];
#pragma unroll
  for (int i = 0; i < N; ++i) tmp[i] = to<T>(v[i]);
  const char *src = reinterpret_cast<const char *>(tmp);
  char *dst = reinterpret_cast<char *>(p);
  if constexpr (BYTES % 16 == 0) {
#pragma unroll
    for (int c = 0; c < BYTES / 16; ++c) {
      uint4 u;
      __builtin_memcpy(&u, src + 16 * c, 16);
      *reinterpret_cast<uint4 *>(dst + 16 * c) = u;
    }
  } else if constexpr (BYTES % 8 == 0) {
#pragma unroll
    for (int c = 0; c < BYTES / 8; ++c) {
      uint2 u;
      __builtin_memcpy(&u, src + 8 * c, 8);
      *reinterpret_cast<uint2 *>(dst + 8 * c) = u;
    }
  } else if constexpr (BYTES % 4 == 0) {
#pragma unroll
    for (int c = 0; c < BYTES / 4; ++c) {
      uint32_t u;
      __builtin_memcpy(&u, src + 4 * c, 4);
      *reinterpret_cast<uint32_t *>(dst + 4 * c) = u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) p[i] = tmp[i];
  }
}

// Streaming (non-temporal) variants for data touched exactly once: the
// accesses bypass the cache retention that would otherwise evict useful lines
// (measured: a 16 B/lane copy streams ~10% faster this way on gfx950).
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));

// Raw copy of N elements to registers; 16-byte non-temporal loads when the
// size and alignment allow, else the widest plain access `align` allows.
template <typename T, int N>
__device__ __forceinline__ void load_raw_nt(const T *__restrict__ p, int align, T (&out)[N]) {
  constexpr int BYTES = N * (int)sizeof(T);
  const char *src = reinterpret_cast<const char *>(p);
  char *dst = reinterpret_cast<char *>(out);
  if constexpr (BYTES % 16 == 0) {
    if (align >= 16) {
#pragma unroll
      for (int c = 0; c < BYTES / 16; ++c) {
        const u32x4_nt u = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(src + 16 * c));
        __builtin_memcpy(dst + 16 * c, &u, 16);
      }
      return;
    }
  }
  if constexpr (BYTES % 8 == 0) {
    if (align >= 8) {
#pragma unroll
      for (int c = 0; c < BYTES / 8; ++c) {
        const uint2 u = *reinterpret_cast<const uint2 *>(src + 8 * c);
        __builtin_memcpy(dst + 8 * c, &u, 8);
      }
      return;
    }
  }
  if constexpr (BYTES % 4 == 0) {
    if (align >= 4) {
#pragma unroll
      for (int c = 0; c < BYTES / 4; ++c) {
        const uint32_t u = *reinterpret_cast<const uint32_t *>(src + 4 * c);
        __builtin_memcpy(dst + 4 * c, &u, 4);
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = p[i];
}

template <typename T, int N>
__device__ __forceinline__ void load_vec_nt(const T *__restrict__ p, int align, float (&out)[N]) {
  T tmp[N];
  load_raw_nt<T, N>(p, align, tmp);
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = f(tmp[i]);
}

// Store N floats as T at p (aligned to min(16, N * sizeof(T)) bytes);
// non-temporal when the size is a multiple of 16 bytes.
template <typename T, int N>
__device__ __forceinline__ void store_vec_nt(T *__restrict__ p, const float (&v)[N]) {
  constexpr int BYTES = N * (int)sizeof(T);
  if constexpr (BYTES % 16 == 0) {
    T tmp[N];
#pragma unroll
    for (int i = 0; i < N; ++i) tmp[i] = to<T>(v[i]);
#pragma unroll
    for (int c = 0; c < BYTES / 16; ++c) {
      u32x4_nt u;
      __builtin_memcpy(&u, reinterpret_cast<const char *>(tmp) + 16 * c, 16);
      __builtin_nontemporal_store(u, reinterpret_cast<u32x4_nt *>(p) + c);
    }
  } else {
    store_vec<T, N>(p, v);
  }
}

// Round a float through T and back (the materialisation of a T value).
template <typename T> __device__ __forceinline__ float round_through(float x) {
  return f(to<T>(x));
}

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }

// x * sigmoid(x) as x * rcp(1 + exp(-x)) (hardware reciprocal, ~1 ulp,
// instead of a full IEEE division); for very negative x, exp(-x) overflows to
// inf, the reciprocal is 0 and the result is -0, the correctly signed limit.
__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// Sum over aligned groups of W lanes (W a power of two <= 64).
// Sum over aligned groups of W lanes (W = 2 .. 64), the result in every lane
// of the group. Groups up to 16 lanes use DPP lane permutations on the
// vector ALU (quad_perm xor 1, xor 2, then row_half_mirror, row_mirror), with
// no LDS round trip; the steps across 16-lane rows use ds_bpermute.
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int W> __device__ __forceinline__ float lane_sum(float v) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "group width");
  v += dpp_f<0xB1>(v);                      // quad_perm [1, 0, 3, 2]
  if constexpr (W >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  if constexpr (W >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
  if constexpr (W >= 16) v += dpp_f<0x140>(v); // row_mirror
  if constexpr (W >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (W >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

template <int W> __device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Bytes every address p + k*stride_bytes (k >= 0) is aligned to, capped at 16.
__host__ __device__ inline int align_of(uint64_t addr) {
  int a = 16;
  while (a > 1 && (addr % (uint64_t)a) != 0) a >>= 1;
  return a;
}

}  // namespace gdn
