// Device helpers shared by the chunk-rule kernels on gfx950: MFMA operand
// types (16x16x32 and 16x16x16 BF16/FP16), fragments of XOR-swizzled q/k
// tiles in LDS, LDS barriers and fences, and LDS DMA copies.
//
// Operand layouts. With v_mfma_f32_16x16x32, lane l = 16 g + c supplies 8 k
// values; an accumulator tile holds rows 4 g + i (i < 4) of column c. Two
// accumulator tiles (rows 16 t .. 16 t + 15, t = 2q, 2q + 1) therefore form
// one B operand whose k slots are {32q + 4g + i} then {32q + 16 + 4g + i}, and
// every A operand used against it is read in that k order. q/k tiles are
// stored row-major with the 16-byte chunks of each row XOR-swizzled by the
// row index, which keeps fragment reads and the ds_read_b64_tr_b16
// transposing reads (K^T fragments) free of bank conflicts.
#pragma once
#include "device_common.h"

namespace gdn {
namespace {

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

template <typename T> struct M2;
template <> struct M2<bf16> {
  typedef bf16x8 f8;
  typedef bf16x4 v4;
  typedef s16x4 f4;  // K16 operand
  static __device__ __forceinline__ f32x4 k32(f8 a, f8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 k16(f4 a, f4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f4 as_f4(v4 x) { return __builtin_bit_cast(s16x4, x); }
};
template <> struct M2<f16> {
  typedef f16x8 f8;
  typedef f16x4 v4;
  typedef f16x4 f4;
  static __device__ __forceinline__ f32x4 k32(f8 a, f8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 k16(f4 a, f4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f4 as_f4(v4 x) { return x; }
};

// Workgroup barrier for LDS hand-offs only: each wave waits for its own LDS
// accesses (lgkmcnt 0) and meets the others; global stores stay in flight.
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Orders LDS accesses of the lanes of one wavefront: stores issued before it
// are complete, and the compiler moves no LDS access across it. Needed where
// lanes read what other lanes of the same wave stored (the per-thread memory
// model lets the compiler hoist such a read above the other lanes' stores).
__device__ __forceinline__ void lds_fence_wave() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Asynchronous global -> LDS copy of 16 bytes per lane (gfx950
// global_load_lds_dwordx4): lane i's bytes land at `lds + 16 i`. The compiler
// sets M0 and keeps the wait state an LDS DMA needs after an M0 write.
__device__ __forceinline__ void g2l16(const void *gptr, unsigned char *lds) {
  __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void *)(lds_u8 *)lds, 16, 0, 0);
}
// XOR swizzle of the 16-byte units of a q/k tile row (DK 16-bit values per
// row): row r's unit u is stored at unit u ^ kswz(r). For 256-byte rows (and
// 512-byte rows, which span the 64 banks twice, so that the map acts on each
// 256-byte half alike) the mask is a GF(2)-linear map of r mod 16 (images of rows 1, 2, 4, 8: 6, 13,
// 8, 9), chosen by timing every invertible map on gfx950: 16-byte fragment
// reads of 16 consecutive rows run without bank conflicts, and transposing
// reads of 4 rows x 4 units per 16 lanes at the two-way minimum that 8-byte
// reads of 32 lanes into one 16-byte column half allow.
template <int DK>
__device__ __forceinline__ constexpr int kswz(int r) {
  if constexpr (DK >= 128) return (int)((0xac7124f935e8bd60ull >> (4 * (r & 15))) & 15);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// s_waitcnt vmcnt(N): returns once at most N vector memory operations of this
// wave are outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <typename T>
__device__ __forceinline__ typename M2<T>::f8 cat8(typename M2<T>::v4 a, typename M2<T>::v4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <typename T>
__device__ __forceinline__ typename M2<T>::v4 cvt4(f32x4 x) {
  return __builtin_convertvector(x, typename M2<T>::v4);
}

// A/B fragment from a q/k tile: `off` is the lane's byte offset of row
// 16 mt + c, k-step pp, half h (see FragOffsets).
template <typename T>
__device__ __forceinline__ typename M2<T>::f8 frag_at(const unsigned char *tile, int off0, int off1) {
  using v4 = typename M2<T>::v4;
  return cat8<T>(*reinterpret_cast<const v4 *>(tile + off0), *reinterpret_cast<const v4 *>(tile + off1));
}

// Sum of squares of 8 packed 16-bit values (two-element dot products).
template <typename T>
__device__ __forceinline__ float sumsq8(typename M2<T>::f8 x, float acc) {
  if constexpr (sizeof(T) == 2 && __is_same(T, bf16)) {
    typedef __attribute__((ext_vector_type(2))) __bf16 b2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const b2 v = {x[2 * j], x[2 * j + 1]};
      acc = __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
    }
  } else {
    typedef __attribute__((ext_vector_type(2))) _Float16 h2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const h2 v = {x[2 * j], x[2 * j + 1]};
      acc = __builtin_amdgcn_fdot2(v, v, acc, false);
    }
  }
  return acc;
}

}  // namespace
}  // namespace gdn
