// Internal launch descriptors shared by the C-ABI layer (gdn_api.cpp) and the
// kernel translation units. Plain structs of device pointers, sizes and
// element strides, filled by the host after validation.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace gdn {

enum Dt : int32_t { kF32 = 0, kBF16 = 1, kF16 = 2, kI32 = 3 };

struct PrologueArgs {
  // Inputs. Strides in elements; the channel/head stride is 1.
  const void *xq, *xk, *xv;
  int64_t sxq_b, sxq_t, sxk_b, sxk_t, sxv_b, sxv_t;
  const void *conv_w;  // [C, 4] contiguous
  const void *conv_b;  // [C] or null
  int32_t w_dtype, b_dtype;
  int32_t w_align;     // bytes conv_w's base address is aligned to (<= 16)
  const void *a, *b;   // [B, T, Hv]
  int64_t sa_b, sa_t, sa_h, sb_b, sb_t, sb_h;
  const float *A_log, *dt_bias;
  const int32_t *cu_seqlens;  // null => dense
  int64_t n_seqs;
  // Geometry.
  int64_t B, T, Hqk, dk, Hv, dv, C;
  int32_t act;           // Dt
  int32_t vec;           // elements per vector access of x (1, 2, 4 or 8)
  int32_t caller_l2norm;
  float l2_eps;
  // Outputs (contiguous).
  void *qkv;             // [B, T, C]
  float *g, *beta;       // [B, T, Hv]
};

struct ChunkArgs {
  const void *q, *k, *v;
  int64_t sq_b, sq_t, sq_h, sk_b, sk_t, sk_h, sv_b, sv_t, sv_h;
  const float *g, *beta;
  int64_t sg_b, sg_t, sg_h, sbt_b, sbt_t, sbt_h;
  const int32_t *cu_seqlens;  // null => dense
  int64_t n_seqs;             // B when dense
  const float *init_state;    // [N, Hv, dv, dk] or null
  float *final_state;         // [N, Hv, dv, dk] or null
  void *o;
  int64_t so_b, so_t, so_h;
  int64_t B, T, Hqk, dk, Hv, dv;
  int32_t act;
  int32_t use_l2;
  int32_t rows16;  // q, k and v rows are all 16-byte aligned
  int32_t o8;      // o rows are 8-byte aligned
  float l2_eps, scale;
  // Two-kernel path (chunk prep + chunk state): caller workspace.
  unsigned char *ws_rec;  // [chunk_bound, Hv] records of kRecBytes, or null
  int32_t *cu_chunks;     // [n_seqs + 1] chunk offsets of packed sequences
  int64_t chunk_bound;    // number of record rows (>= total chunks)
};

// Per-(chunk, value head) record that the chunk-prep kernel writes and the
// chunk-state kernel reads (16-bit activations). The 64 x 64 matrices are
// stored as six MFMA A-operand fragments (lane l's 16 bytes at l * 16 within
// each 1 KB fragment), fragment f = (row tile mt, k pair q) in the order
// (0,0) (1,0) (2,0) (3,0) (2,1) (3,1); element e of lane 16 g + c is
// M[16 mt + c][32 q + 16 (e / 4) + 4 g + e % 4].
constexpr int64_t kRecT = 0;        // T' = (I + A)^-1 diag(beta), activation dtype
constexpr int64_t kRecP = 6144;     // P (scaled, decayed, masked q.k), act dtype
constexpr int64_t kRecF = 12288;    // FP32 row factors [4][64]: aa, cw, zc, beta; then e^{gamma_C}
constexpr int64_t kRecBytes = 14336;

// Row r of a [B, T, H] grid of rows as (b, t, h). While B T H < 2^32 the two
// divisions (by H, then by T) are multiplications by 32-bit magic numbers:
// n / d = (umulhi(n, m) + n) >> s with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1, exact for every 32-bit n (the sum is
// formed in 64 bits); else 64-bit division.
struct RowDiv {
  uint32_t h_m, h_s, t_m, t_s;
  int32_t small;
};
inline void udiv_magic(uint32_t d, uint32_t &m, uint32_t &s) {
  s = 0;
  while (((uint64_t)1 << s) < d) ++s;
  m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << s) - d)) / d + 1);
}
inline RowDiv row_div(int64_t B, int64_t T, int64_t H) {
  RowDiv r{};
  r.small = B * T * H < ((int64_t)1 << 32) ? 1 : 0;
  if (r.small) {
    udiv_magic((uint32_t)H, r.h_m, r.h_s);
    udiv_magic((uint32_t)T, r.t_m, r.t_s);
  }
  return r;
}
__device__ __forceinline__ uint32_t udiv32(uint32_t n, uint32_t m, uint32_t s) {
  return (uint32_t)((((uint64_t)n * m >> 32) + n) >> s);
}
__device__ __forceinline__ void split_row(const RowDiv &d, int64_t T, int64_t H, int64_t row, int64_t &b, int64_t &t,
                                          int64_t &h) {
  if (d.small) {
    const uint32_t r = (uint32_t)row, bt = udiv32(r, d.h_m, d.h_s), bb = udiv32(bt, d.t_m, d.t_s);
    h = r - bt * (uint32_t)H;
    t = bt - bb * (uint32_t)T;
    b = bb;
  } else {
    h = row % H;
    const int64_t bt = row / H;
    t = bt % T;
    b = bt / T;
  }
}

struct NormArgs {
  const void *o;
  int64_t so_b, so_t, so_h;
  const void *gate;
  int64_t sg_b, sg_t, sg_h;
  const void *w;
  void *out;  // contiguous
  int64_t B, T, H, dv;
  int32_t act, gate_dtype, w_dtype;
  int32_t o_align, gate_align;  // bytes guaranteed for every row start
  float eps;
  RowDiv rd;
};

// One decode step (a new token per sequence, conv cache and state updated in
// place).
struct DecodeArgs {
  const void *xq, *xk, *xv;     // [N, Hqk*dk], [N, Hqk*dk], [N, Hv*dv], act dtype
  int64_t sxq, sxk, sxv;        // row strides
  const void *conv_w;           // [C, 4] act dtype or F32, contiguous
  const void *conv_b;           // [C] or null
  int32_t w_dtype, b_dtype;
  int32_t w_align;              // bytes conv_w's base address is aligned to (<= 16)
  void *conv_state;             // [N, 3, C] act dtype, inner stride 1; oldest input first
  int64_t scs_n, scs_t;
  const void *a, *b;            // [N, Hv] act dtype
  int64_t sa, sb;
  const float *A_log, *dt_bias; // [Hv]
  float *state;                 // [N, Hv, dv, dk] F32, contiguous
  const void *gate;             // [N, Hv, dv] act dtype or F32, inner stride 1
  int64_t sgate_n, sgate_h;
  int32_t gate_dtype, nw_dtype;
  const void *norm_w;           // [dv], contiguous
  void *out;                    // [N, Hv, dv] act dtype, contiguous
  int64_t N, Hqk, dk, Hv, dv;
  int32_t act, use_l2;
  float scale, l2_eps, rms_eps;
};

// Backward of the gated norm.
struct NormBwdArgs {
  const void *o, *gate, *dout, *w;
  int64_t so_b, so_t, so_h, sg_b, sg_t, sg_h, sd_b, sd_t, sd_h;
  void *d_o, *d_gate;    // contiguous [B, T, H, dv]: o's dtype, gate's dtype
  float *d_w;            // [dv]
  float *part;           // workspace [nblocks][dv]
  float *mid;            // workspace [32][dv]
  int64_t nblocks;
  int64_t B, T, H, dv;
  int32_t act, gate_dtype, w_dtype;
  int32_t o_align, gate_align, dout_align;
  float eps;
  RowDiv rd;
};

// Backward of the prologue (conv + SiLU, beta and g).
struct PrologueBwdArgs {
  const void *xq, *xk, *xv;
  int64_t sxq_b, sxq_t, sxk_b, sxk_t, sxv_b, sxv_t;
  const void *conv_w, *conv_b;
  int32_t w_dtype, b_dtype;
  const void *a, *b;
  int64_t sa_b, sa_t, sb_b, sb_t;
  const float *A_log, *dt_bias;
  const int32_t *cu_seqlens;
  int64_t n_seqs;
  const void *dqkv;      // [B, T, C] contiguous, act dtype or F32
  int32_t dqkv_dtype;
  const float *d_g, *d_beta;  // [B, T, Hv] contiguous
  void *dxq, *dxk, *dxv;      // contiguous, act dtype
  float *d_conv_w, *d_conv_b; // [C, 4], [C] or null
  void *d_a, *d_b;            // [B, T, Hv] contiguous, act dtype
  float *d_A_log, *d_dt_bias; // [Hv]
  // workspace: partial sums per token tile, and the reduction scratch
  float *part_w;              // [ntiles][C][4]
  float *part_b;              // [ntiles][C]
  float *part_dt, *part_al;   // [nhtiles][Hv]
  float *mid;                 // [32][C * 4]
  int64_t ntiles, tile_tokens, nhtiles, head_tile;
  int64_t B, T, Hqk, dk, Hv, dv, C;
  int32_t act;
  int32_t vec4;              // 4 channels per thread (segments and rows allow it)
  int32_t x_flat;            // every x view has batch stride T times its token stride
  int32_t x_align, dq_align; // bytes guaranteed for x rows and d_qkv rows
};

// Backward of the chunked gated delta rule. Workspace arrays are FP32, per
// chunk row gc (chunk_bound of them) and head:
//   qn, kn [gc][Hqk][64][dk] unit q, k rows; rq, rk [gc][Hqk][64] inverse norms
//   gam [gc][Hv][64] running sum of g in the chunk; mm, pp [gc][Hv][64][64]
//   (I + A)^-1 and scale * masked decayed q.k; s0, ds [gc][Hv][dv][dk] state
//   entering the chunk and gradient of the state leaving it; rr, del, drp
//   [gc][Hv][64][dv] R, Delta and M^T dDelta.
struct ChunkBwdArgs {
  const void *q, *k, *v;
  int64_t sq_b, sq_t, sq_h, sk_b, sk_t, sk_h, sv_b, sv_t, sv_h;
  const float *g, *beta;
  int64_t sg_b, sg_t, sg_h, sbt_b, sbt_t, sbt_h;
  const void *d_o;
  int64_t sdo_b, sdo_t, sdo_h;
  const int32_t *cu_seqlens;  // null => dense
  int64_t n_seqs;             // B when dense
  const float *init_state;    // [N, Hv, dv, dk] or null
  const float *d_final;       // [N, Hv, dv, dk] or null
  void *dqq, *dkk, *dvv;       // [B, T, H, d], grad_dtype, head stride d, inner 1
  int64_t sdq_b, sdq_t, sdk_b, sdk_t, sdv_b, sdv_t;
  float *dg, *dbeta;          // [B, T, Hv] contiguous
  float *d_init;              // [N, Hv, dv, dk] or null
  int64_t B, T, Hqk, dk, Hv, dv;
  int32_t act, grad_dtype, use_l2;
  float l2_eps, scale;
  int32_t *cu_chunks;         // [n_seqs + 1] (packed sequences)
  int64_t chunk_bound;
  float *qn, *kn, *rq, *rk, *gam, *mm, *pp, *s0, *ds, *rr, *del, *drp;
  unsigned char *brec;        // [gc][Hv] records of kBrBytes for the matrix-core reverse pass
};

// Backward record per (chunk, value head), written by the backward prep for
// the matrix-core state passes: MFMA A-operand fragments of M, of M^T and of
// P'^T (M = (I + A)^-1, P' = scale * masked decayed q.k with its rows past the
// chunk's end zeroed), each as BF16 hi and lo parts (x = hi + lo), and FP32
// factor rows [8][64]: e^gamma, cw rk, beta, scale e^gamma rq (0 past the
// end), -e^gamma beta rk, e^{gamma_C} at [5][0], e^gamma rk. Fragment
// element e of lane 16 g + c of fragment (row tile mt, k pair q) is
// X[16 mt + c][32 q + 16 (e / 4) + 4 g + e % 4]; M (lower triangular) has
// fragments (0,0) (1,0) (2,0) (3,0) (2,1) (3,1), M^T and P'^T (upper) have
// (0,0) (1,0) (0,1) (1,1) (2,1) (3,1). The forward-state pass reads
// [0, kBrMtH), the reverse pass [kBrF, kBrBytes).
constexpr int64_t kBrMH = 0, kBrML = 6144, kBrF = 12288, kBrMtH = 14336, kBrMtL = 20480, kBrPH = 26624,
                  kBrPL = 32768;
constexpr int64_t kBrBytes = 38912;

// Each returns the HIP error of the launch (hipSuccess if queued).
hipError_t launch_prologue(const PrologueArgs &a, hipStream_t s);
hipError_t launch_chunk_rule(const ChunkArgs &a, hipStream_t s);
hipError_t launch_gated_norm(const NormArgs &a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);
bool decode_supported(int64_t dk, int64_t G, int64_t dv);
hipError_t launch_gated_norm_bwd(const NormBwdArgs &a, hipStream_t s);
hipError_t launch_prologue_bwd(const PrologueBwdArgs &a, hipStream_t s);

// Host-side capability query used by validation (no device calls).
bool chunk_rule_supported(int64_t dk, int32_t act);

// Two-kernel path: chunk prep (parallel over chunks and heads) then chunk
// state (serial over chunks). Needs a.ws_rec / a.cu_chunks.
bool chunk_split_supported(int64_t dk, int64_t dv, int32_t act);
hipError_t launch_chunk_split(const ChunkArgs &a, hipStream_t s);

// Backward of the chunk rule (dk 64, 128 or 256, dv a multiple of 16).
bool chunk_bwd_supported(int64_t dk, int64_t dv);
hipError_t launch_chunk_bwd(const ChunkBwdArgs &a, hipStream_t s);
// Its gradient kernel on the 16-bit matrix cores (BF16 or FP16 activations,
// dk 64 or 128, dv a multiple of 32, aligned rows); the FP32 kernel serves the
// rest.
bool chunk_bwd_grad_mma_supported(const ChunkBwdArgs &a);
hipError_t launch_chunk_bwd_grad_mma(const ChunkBwdArgs &a, hipStream_t s);
// Its forward-state and reverse state passes on the 16-bit matrix cores (BF16
// or FP16 activations, dk 64 or 128, 16-byte aligned q, k, v and d_o rows), in
// one launch; they need a.brec written by the prep.
bool chunk_bwd_state_mma_supported(const ChunkBwdArgs &a);
hipError_t launch_chunk_bwd_state_passes_mma(const ChunkBwdArgs &a, hipStream_t s);

// Device address of the static chunk scratch (GDN_NOALLOC_SCRATCH_BYTES) on
// the current device; looked up once per device.
hipError_t static_scratch(void **out);

// cuc[n] = sum over sequences m < n of ceil(len_m / 64), for n in [0, n_seqs].
hipError_t launch_chunk_index(const int32_t *cu, int64_t n_seqs, int32_t *cuc, hipStream_t s);

// Largest power-of-two alignment (bytes, <= 16) of an address or stride set.
inline int align_of_host(uint64_t addr) {
  int a = 16;
  while (a > 1 && (addr % (uint64_t)a) != 0) a >>= 1;
  return a;
}

}  // namespace gdn
