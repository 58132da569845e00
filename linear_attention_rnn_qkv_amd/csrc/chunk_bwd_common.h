// Chunk geometry shared by the chunk-rule backward kernels.
#pragma once
#include "gdn_internal.h"

namespace gdn {
namespace {

// Where chunk gc of the whole call lies: batch row, first token, rows.
struct ChunkPos {
  int64_t brow, t0;
  int nr;
  bool valid;
};

__device__ __forceinline__ ChunkPos chunk_pos(const ChunkBwdArgs &p, int64_t gc) {
  constexpr int C = 64;
  ChunkPos c;
  if (p.cu_seqlens) {
    const int32_t *cuc = p.cu_chunks;
    c.valid = gc < cuc[p.n_seqs];
    if (!c.valid) return c;
    int64_t lo = 0, hi = p.n_seqs;  // cuc[lo] <= gc < cuc[hi]
    while (hi - lo > 1) {
      const int64_t mid = (lo + hi) >> 1;
      if (cuc[mid] <= gc) lo = mid; else hi = mid;
    }
    const int64_t ch = gc - cuc[lo], bos = p.cu_seqlens[lo], L = p.cu_seqlens[lo + 1] - bos;
    c.brow = 0;
    c.t0 = bos + ch * C;
    c.nr = (int)(L - ch * C < C ? L - ch * C : C);
  } else {
    const int64_t nc = (p.T + C - 1) / C;
    c.valid = gc < p.B * nc;
    if (!c.valid) return c;
    c.brow = gc / nc;
    const int64_t ch = gc % nc;
    c.t0 = ch * C;
    c.nr = (int)(p.T - c.t0 < C ? p.T - c.t0 : C);
  }
  return c;
}

}  // namespace
}  // namespace gdn
