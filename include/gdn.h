/*
 * gdn.h - C ABI of the MI355X (gfx950) forward layer core of Gated DeltaNet.
 *
 * The layer core is three stages, each a hand-written HIP kernel, plus a call
 * that runs all three on one stream:
 *
 *   gdn_prologue_fwd    concatenated depthwise causal conv + SiLU over the
 *                       q|k|v channels, beta = sigmoid(b) and the log-decay
 *                       g = -exp(A_log) * softplus(a + dt_bias)
 *   gdn_chunk_rule_fwd  chunked gated delta rule (chunks of 64 tokens) with
 *                       q/k L2 normalisation folded in and the GQA head map
 *   gdn_gated_norm_fwd  output RMSNorm, materialised in the activation dtype,
 *                       then the FP32 SiLU-gate multiply
 *   gdn_layer_fwd       the three stages in order, in a caller workspace
 *   gdn_decode_fwd      one recurrent step per sequence (conv cache and FP32
 *                       state updated in place), all stages in one kernel
 *   gdn_gated_norm_bwd, gdn_prologue_bwd, gdn_chunk_rule_bwd
 *                       first-order gradients of the gated norm, of the
 *                       prologue and of the chunked gated delta rule
 *   gdn_layer_bwd       the gradients of gdn_layer_fwd: the forward stages
 *                       recomputed, then the three backward stages
 *   gdn_layer_bwd_saved the same gradients from the activations a
 *                       gdn_layer_fwd call left in the workspace
 *
 * Sources (web pages):
 *   [P1] Megatron-LM pull request "perf(gated_delta_net): fold q/k L2-norm
 *        into the gated_delta_rule kernel" - sections What, Why.
 *   [P2] Megatron Core developer guide "GDN Elementwise Fusion" - option
 *        table, "Post-GDR requirements", "Execution and numerical behavior".
 *   [P3] flash-linear-attention pull request fusing GatedDeltaNet's q/k/v
 *        short convolutions - Summary, Why, Risk / scope.
 *   The recurrence is not printed on the pages; it is the gated delta rule of
 *   Gated DeltaNet (Yang, Kautz and Hatamizadeh, ICLR 2025):
 *       S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *       o_t = scale * S_t q_t,   S is dv x dk, FP32.
 *
 * Conventions shared by every call
 *   - Tensors are described by gdn_tensor: a DEVICE pointer, a dtype, a shape
 *     and strides counted in elements. Strides may be arbitrary (views are
 *     read in place, never copied) except that the innermost (channel /
 *     head-dim) stride must be 1. Outputs that this ABI calls "contiguous"
 *     must have row-major strides.
 *   - All memory is owned by the caller. The library never allocates, frees
 *     or synchronises; every call only enqueues kernels on `stream` (a
 *     hipStream_t; NULL is the legacy default stream) and returns.
 *   - Every argument is checked from host metadata alone (shapes, strides,
 *     dtypes, pointer alignment and overlap) before anything is launched, so
 *     a call that returns an error has had no effect ([P2] Post-GDR
 *     requirements: unsupported inputs are rejected on every call, without a
 *     device synchronisation and without a silent fallback). Device contents
 *     (e.g. cu_seqlens values) are not validated.
 *   - An optional tensor is passed as a NULL descriptor pointer.
 *   - Calls are re-entrant and may run concurrently on different streams.
 *   - On error, gdn_last_error() returns a message for the calling thread.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_MAX_DIMS 5

typedef enum gdn_dtype {
  GDN_F32 = 0,
  GDN_BF16 = 1,
  GDN_F16 = 2,
  GDN_I32 = 3
} gdn_dtype;

typedef struct gdn_tensor {
  void *data;                    /* device pointer */
  int32_t dtype;                 /* gdn_dtype */
  int32_t ndim;                  /* 1 .. GDN_MAX_DIMS */
  int64_t shape[GDN_MAX_DIMS];
  int64_t stride[GDN_MAX_DIMS];  /* in elements */
} gdn_tensor;

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_INVALID_VALUE = 1,  /* shape/dtype/stride mismatch, empty input,
                                 non-power-of-two head dim, Hv % Hqk != 0,
                                 inner stride != 1, output overlapping an
                                 input, workspace too small */
  GDN_ERR_NOT_SUPPORTED = 2,  /* valid but not built: head dims outside the
                                 instantiated set, misaligned vectors */
  GDN_ERR_LAUNCH = 3          /* the HIP runtime refused a launch */
} gdn_status;

/* Head geometry: Hqk query/key heads of dimension dk, Hv value heads of
 * dimension dv. Hv must be a multiple of Hqk; value head h reads query/key
 * head h / (Hv / Hqk) ([P1] Why: normalisation is per head, so head
 * replication leaves the result unchanged). Supported: dk in {64, 128, 256},
 * dv in {64, 128, 256, 512}. */
typedef struct gdn_dims {
  int64_t Hqk, dk, Hv, dv;
} gdn_dims;

/* Message describing the last error on the calling thread ("" if none). */
const char *gdn_last_error(void);

/* Library version string. */
const char *gdn_version(void);

/*
 * gdn_prologue_fwd - [P3] Summary/Why; [P2] option table ("causal
 * convolution, SiLU, layout transforms, Q/K L2 normalization, head expansion,
 * beta and decay preparation").
 *
 * One depthwise causal conv1d of 4 taps over the concatenated channels
 * c in [0, C), C = 2*Hqk*dk + Hv*dv, ordered q | k | v:
 *     y[t, c] = bias[c] + sum_{j=0..3} w[c, j] * x[t - 3 + j, c]
 *     qkv[t, c] = silu(y[t, c])  (computed in FP32, stored in the act dtype)
 * with zero history before the start of every sequence. The conv is
 * depthwise, so this equals three separate q, k and v convolutions.
 * Also, per token and value head:
 *     beta = sigmoid(b),  g = -exp(A_log[h]) * softplus(a + dt_bias[h])
 * stored in FP32.
 *
 *   x_q, x_k   [B, T, Hqk*dk] act dtype (F32/BF16/F16), any strides, inner 1
 *   x_v        [B, T, Hv*dv]  act dtype
 *   conv_w     [C, 4] act dtype or F32, contiguous
 *   conv_b     [C] act dtype or F32, or NULL
 *   a, b       [B, T, Hv] act dtype, any strides, inner 1
 *   A_log, dt_bias [Hv] F32
 *   cu_seqlens [N+1] I32 or NULL. NULL: each of the B rows is one sequence.
 *              Given: B must be 1 and sequence n is tokens
 *              [cu_seqlens[n], cu_seqlens[n+1]) of the row; the offsets must
 *              be non-decreasing with cu_seqlens[0] = 0, cu_seqlens[N] = T
 *              (caller's contract, not checked).
 *   caller_l2norm  0: q/k stored as conv outputs (the in-kernel route).
 *              1: q and k are additionally L2-normalised per head over dk
 *              (x / sqrt(sum x^2 + l2_eps)) before being stored (the
 *              caller-side route of [P1]).
 *   out_qkv    [B, T, C] act dtype, contiguous; q, k, v are its channel
 *              ranges [0, Hqk*dk), [Hqk*dk, 2*Hqk*dk), [2*Hqk*dk, C), head h
 *              at offset h*d inside its range.
 *   out_g, out_beta [B, T, Hv] F32, contiguous.
 */
gdn_status gdn_prologue_fwd(const gdn_tensor *x_q, const gdn_tensor *x_k,
                            const gdn_tensor *x_v, const gdn_tensor *conv_w,
                            const gdn_tensor *conv_b, const gdn_tensor *a,
                            const gdn_tensor *b, const gdn_tensor *A_log,
                            const gdn_tensor *dt_bias,
                            const gdn_tensor *cu_seqlens, const gdn_dims *dims,
                            int32_t caller_l2norm, float l2_eps,
                            const gdn_tensor *out_qkv, const gdn_tensor *out_g,
                            const gdn_tensor *out_beta, void *stream);

/*
 * gdn_chunk_rule_fwd - the gated delta rule over chunks of 64 tokens ([P3]
 * Benchmark: FLA's chunk mode; [P1] What: q/k normalisation inside the
 * recurrence kernel). Per (sequence, value head h), starting from the given
 * initial state (or zero):
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t
 * where, with use_qk_l2norm_in_kernel = 1, q and k are first replaced by
 * x / sqrt(sum x^2 + l2_eps) over dk ([P1] Why: eps 1e-6 on both routes;
 * 0 is a no-op). Arithmetic: FP32 state and accumulation; MFMA operands in
 * the act dtype (FP32 MFMA for F32 inputs).
 *
 *   q, k       [B, T, Hqk, dk] act dtype, any strides, inner 1
 *   v          [B, T, Hv, dv]  act dtype, any strides, inner 1
 *   g, beta    [B, T, Hv] F32, any strides
 *   cu_seqlens [N+1] I32 or NULL (as in gdn_prologue_fwd); state and
 *              chunking restart at every sequence boundary
 *   initial_state [N, Hv, dv, dk] F32 contiguous, or NULL (zero state)
 *   out_o      [B, T, Hv, dv] act dtype, any strides, inner 1
 *   final_state   [N, Hv, dv, dk] F32 contiguous, or NULL; may alias
 *              initial_state (each state is read before it is written)
 *   workspace  device memory of gdn_chunk_rule_workspace_bytes(...) bytes,
 *              256-byte aligned, or NULL. With a workspace, BF16/FP16 inputs
 *              with dk 64 or 128 (dv a multiple of 16) or dk 256 (dv a
 *              multiple of 32), 16-byte aligned q/k/v rows and 8-byte
 *              aligned o rows run as two kernels: a chunk prep that is
 *              parallel over (chunk, value head) and writes T = (I + A)^-1,
 *              P and row factors of every chunk to the workspace, then the
 *              serial state pass. Without one (or where that path does not
 *              apply) a single kernel does both. The
 *              results agree to rounding. A workspace smaller than required
 *              is an error; the memory must not overlap any tensor argument
 *              and must not be used by any other call until this call's work
 *              on `stream` is done.
 * N = B without cu_seqlens.
 */
gdn_status gdn_chunk_rule_fwd(const gdn_tensor *q, const gdn_tensor *k,
                              const gdn_tensor *v, const gdn_tensor *g,
                              const gdn_tensor *beta, float scale,
                              int32_t use_qk_l2norm_in_kernel, float l2_eps,
                              const gdn_tensor *cu_seqlens,
                              const gdn_tensor *initial_state,
                              const gdn_tensor *out_o,
                              const gdn_tensor *final_state, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * gdn_chunk_rule_fwd_noalloc - gdn_chunk_rule_fwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, arguments and
 * results as gdn_chunk_rule_fwd with a workspace, except that the chunk
 * records live in a static device array of GDN_NOALLOC_SCRATCH_BYTES that the
 * library owns on every device it runs on (from the first call on a device
 * until the process ends), not in a caller workspace. The call allocates and
 * frees nothing.
 *
 * Limit: gdn_chunk_rule_workspace_bytes(...) for the call's shape must be at
 * most GDN_NOALLOC_SCRATCH_BYTES (64 MiB: for example 4096 (chunk, value
 * head) records, 8192 tokens of 32 value heads); a larger call is rejected
 * with GDN_ERR_INVALID_VALUE before anything is launched (split the sequence
 * with initial_state / final_state, or pass a workspace to
 * gdn_chunk_rule_fwd). Where the two-kernel path does not apply (see
 * gdn_chunk_rule_fwd), the single recurrence kernel runs and no scratch is
 * used.
 *
 * Every call on one device shares that device's scratch: calls whose work
 * overlaps on one device (different streams, different host threads) race
 * and must be serialised by the caller. The scratch holds no state between
 * calls (every call writes what it reads). `stream` must belong to the
 * current device. A failure to look up the scratch's device address is
 * GDN_ERR_LAUNCH.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gdn_status gdn_chunk_rule_fwd_noalloc(const gdn_tensor *q, const gdn_tensor *k,
                                      const gdn_tensor *v, const gdn_tensor *g,
                                      const gdn_tensor *beta, float scale,
                                      int32_t use_qk_l2norm_in_kernel,
                                      float l2_eps,
                                      const gdn_tensor *cu_seqlens,
                                      const gdn_tensor *initial_state,
                                      const gdn_tensor *out_o,
                                      const gdn_tensor *final_state,
                                      void *stream);

/* Bytes of chunk workspace for B*T tokens (n_seqs = number of packed
 * sequences with cu_seqlens, 0 without): 4*(N+1) rounded to 256, plus
 * (ceil(T/64) + n_seqs, or B*ceil(T/64)) * Hv records of 14336 bytes.
 * Returns 0 where the two-kernel path does not apply (F32 inputs; dk 256
 * with dv not a multiple of 32) and for invalid arguments. */
size_t gdn_chunk_rule_workspace_bytes(int64_t B, int64_t T, int64_t n_seqs,
                                      const gdn_dims *dims, int32_t act_dtype);

/*
 * gdn_gated_norm_fwd - [P2] option table (output RMSNorm and SiLU gating),
 * Post-GDR requirements and Execution and numerical behavior. Per
 * (token, head) row of length dv:
 *     r   = 1 / sqrt(mean(o^2) + eps)
 *     y   = round_act(o * r * weight)          (RMSNorm in the act dtype)
 *     out = round_act(float(y) * silu(float(gate)))   (FP32 gate multiply)
 *
 *   o       [B, T, H, dv] F32/BF16/F16, any strides, inner 1, nonempty,
 *           dv a power of two
 *   gate    [B, T, H, dv] o's dtype or F32, any strides (separate batch and
 *           sequence strides, e.g. a view into a projection buffer), inner 1
 *   weight  [dv] F32/BF16/F16, contiguous
 *   out     [B, T, H, dv] o's dtype, contiguous
 */
gdn_status gdn_gated_norm_fwd(const gdn_tensor *o, const gdn_tensor *gate,
                              const gdn_tensor *weight, float eps,
                              const gdn_tensor *out, void *stream);

/* Bytes of workspace gdn_layer_fwd needs for B*T tokens (a multiple of 256):
 * qkv [B,T,C] act dtype, g and beta [B,T,Hv] F32, o [B,T,Hv,dv] act dtype,
 * each 256-byte aligned, then the chunk workspace
 * (gdn_chunk_rule_workspace_bytes). n_seqs: number of packed sequences when
 * cu_seqlens is given, else 0. Returns 0 for invalid arguments. */
size_t gdn_layer_workspace_bytes(int64_t B, int64_t T, int64_t n_seqs,
                                 const gdn_dims *dims, int32_t act_dtype);

/*
 * gdn_layer_fwd - the layer core ([P2] Execution: the pre-recurrence stage,
 * the recurrence and the gated norm; the output projection is not part of
 * it). Runs gdn_prologue_fwd (caller_l2norm = 0), gdn_chunk_rule_fwd on the
 * q/k/v channel views of its output, and gdn_gated_norm_fwd, on one stream.
 * Arguments are those of the three stages; `workspace` is device memory of
 * at least gdn_layer_workspace_bytes(...) bytes, 256-byte aligned, owned by
 * the caller and not used by any other call until this call's work on
 * `stream` is done. `out` is [B, T, Hv, dv] act dtype, contiguous.
 */
gdn_status gdn_layer_fwd(const gdn_tensor *x_q, const gdn_tensor *x_k,
                         const gdn_tensor *x_v, const gdn_tensor *conv_w,
                         const gdn_tensor *conv_b, const gdn_tensor *a,
                         const gdn_tensor *b, const gdn_tensor *A_log,
                         const gdn_tensor *dt_bias, const gdn_tensor *gate,
                         const gdn_tensor *norm_w,
                         const gdn_tensor *cu_seqlens, const gdn_dims *dims,
                         float scale, int32_t use_qk_l2norm_in_kernel,
                         float l2_eps, float rms_eps, void *workspace,
                         size_t workspace_bytes, const gdn_tensor *out,
                         void *stream);

/*
 * gdn_decode_fwd - one recurrent decode step of the layer core: a new token
 * for each of N independent sequences, each carrying a conv cache and a
 * state. It is the recurrent form of the same layer (the gated delta rule of
 * Gated DeltaNet for one token, the conv of [P3] Summary at the newest token,
 * the gated norm of [P2] Execution and numerical behavior). Per sequence n:
 *     window = (cache[n, 0], cache[n, 1], cache[n, 2], x[n])  per channel
 *     z      = round_act(silu(bias + sum_j conv_w[:, j] * window[j]))
 *     cache[n] <- (window[1], window[2], window[3])   (exact copies)
 *     beta, g as in gdn_prologue_fwd; q, k L2-normalised if requested
 *     S[n, h] <- e^g S (I - beta k k^T) + beta v k^T;  o = scale S q
 *     out[n, h] = gdn_gated_norm_fwd of round_act(o)
 * A sequence that starts from a zero cache and a zero state and takes T
 * steps produces what gdn_layer_fwd produces for those T tokens, and its
 * state is gdn_chunk_rule_fwd's final state.
 *
 *   x_q, x_k     [N, Hqk*dk] F32/BF16/F16 (the activation dtype), row stride
 *                free, inner 1
 *   x_v          [N, Hv*dv] act dtype, inner 1
 *   conv_w       [C, 4] act dtype or F32, contiguous, C = 2 Hqk dk + Hv dv
 *   conv_b       [C] act dtype or F32, contiguous, or NULL
 *   conv_state   [N, 3, C] act dtype, inner 1: the last three inputs of every
 *                channel, oldest first (zeros for a fresh sequence). Read and
 *                updated in place.
 *   a, b         [N, Hv] act dtype, inner 1
 *   A_log, dt_bias [Hv] F32, contiguous
 *   state        [N, Hv, dv, dk] F32, contiguous, 16-byte aligned (zeros for
 *                a fresh sequence). Read and updated in place.
 *   gate         [N, Hv, dv] act dtype or F32, inner 1
 *   norm_w       [dv] F32/BF16/F16, contiguous
 *   out          [N, Hv, dv] act dtype, contiguous
 * conv_state, state and out must not overlap one another or any input.
 * Supported: dk in {64, 128, 256}, 64 <= dv <= 512, Hv / Hqk <= 64,
 * (Hv / Hqk) * dv <= 8192, N <= 65535 (else GDN_ERR_NOT_SUPPORTED).
 */
gdn_status gdn_decode_fwd(const gdn_tensor *x_q, const gdn_tensor *x_k,
                          const gdn_tensor *x_v, const gdn_tensor *conv_w,
                          const gdn_tensor *conv_b,
                          const gdn_tensor *conv_state, const gdn_tensor *a,
                          const gdn_tensor *b, const gdn_tensor *A_log,
                          const gdn_tensor *dt_bias, const gdn_tensor *state,
                          const gdn_dims *dims, float scale,
                          int32_t use_qk_l2norm_in_kernel, float l2_eps,
                          const gdn_tensor *gate, const gdn_tensor *norm_w,
                          float rms_eps, const gdn_tensor *out, void *stream);

/*
 * Backward (first-order gradients). The Megatron Core page "GDN Elementwise
 * Fusion" (Execution and numerical behavior) gives the fused stages
 * first-order autograd; the Megatron-LM L2-fold pull request (Validation) and
 * the flash-linear-attention fused-conv pull request (Test plan) check input
 * and parameter gradients. The gradients are those of the stage's exact
 * function (the forward's activation-dtype roundings taken as the identity),
 * computed in FP32. Parameter gradients are sums over tokens; each call adds
 * them up in a fixed order (deterministic), using a caller workspace for the
 * partial sums (256-byte aligned, at least the size the matching
 * *_workspace_bytes call returns, not used by another call until this one's
 * work on `stream` is done).
 *
 * gdn_gated_norm_bwd - with r, n = o r, y = n weight, out = y silu(gate) as
 * in gdn_gated_norm_fwd, for the gradient dout of out:
 *     d_gate = dout y silu'(gate),  dn = dout silu(gate) weight,
 *     d_o = r (dn - n mean(dn n)),  d_weight = sum over rows of
 *     dout silu(gate) n
 *   o, gate, weight, eps  as in gdn_gated_norm_fwd
 *   dout      [B, T, H, dv] o's dtype, any strides, inner 1
 *   d_o       [B, T, H, dv] o's dtype, contiguous, 16-byte aligned
 *   d_gate    [B, T, H, dv] gate's dtype, contiguous, 16-byte aligned
 *   d_weight  [dv] F32 (written, not accumulated)
 */
size_t gdn_gated_norm_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H,
                                          int64_t dv);
gdn_status gdn_gated_norm_bwd(const gdn_tensor *o, const gdn_tensor *gate,
                              const gdn_tensor *weight, float eps,
                              const gdn_tensor *dout, const gdn_tensor *d_o,
                              const gdn_tensor *d_gate,
                              const gdn_tensor *d_weight, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * gdn_prologue_bwd - gradients of the prologue (gdn_prologue_fwd with
 * caller_l2norm = 0) for the gradients d_qkv of its conv output, d_g of g and
 * d_beta of beta. Per channel c of each sequence, y_t = bias + sum_j
 * w_j x_{t-3+j}, z_t = silu(y_t), e_t = d_qkv_t silu'(y_t):
 *     dx_t = sum_j w_j e_{t+3-j} (tokens of the same sequence),
 *     d_conv_w[c, j] = sum_t e_t x_{t-3+j},  d_conv_b[c] = sum_t e_t
 *     d_b = d_beta beta (1 - beta),
 *     d_a = -d_g exp(A_log) sigmoid(a + dt_bias)  (1 above softplus's 20),
 *     d_dt_bias = sum of d_a,  d_A_log = sum of d_g g
 *   x_q .. cu_seqlens, dims  as in gdn_prologue_fwd
 *   d_qkv     [B, T, C] act dtype or F32, contiguous
 *   d_g, d_beta  [B, T, Hv] F32, contiguous
 *   dx_q, dx_k [B, T, Hqk*dk], dx_v [B, T, Hv*dv]  act dtype, contiguous
 *   d_conv_w  [C, 4] F32;  d_conv_b [C] F32, given exactly when conv_b is
 *   d_a, d_b  [B, T, Hv] act dtype, contiguous
 *   d_A_log, d_dt_bias [Hv] F32
 */
size_t gdn_prologue_bwd_workspace_bytes(int64_t B, int64_t T,
                                        const gdn_dims *dims);
gdn_status gdn_prologue_bwd(const gdn_tensor *x_q, const gdn_tensor *x_k,
                            const gdn_tensor *x_v, const gdn_tensor *conv_w,
                            const gdn_tensor *conv_b, const gdn_tensor *a,
                            const gdn_tensor *b, const gdn_tensor *A_log,
                            const gdn_tensor *dt_bias,
                            const gdn_tensor *cu_seqlens, const gdn_dims *dims,
                            const gdn_tensor *d_qkv, const gdn_tensor *d_g,
                            const gdn_tensor *d_beta, const gdn_tensor *dx_q,
                            const gdn_tensor *dx_k, const gdn_tensor *dx_v,
                            const gdn_tensor *d_conv_w,
                            const gdn_tensor *d_conv_b, const gdn_tensor *d_a,
                            const gdn_tensor *d_b, const gdn_tensor *d_A_log,
                            const gdn_tensor *d_dt_bias, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * gdn_chunk_rule_bwd - first-order gradients of gdn_chunk_rule_fwd ([P2]
 * Execution and numerical behavior: the fused stages support first-order
 * autograd; [P1] Validation checks q/k gradients through the L2 fold).
 * Gradients of L = sum(d_o * o) + sum(d_final_state * final_state) with
 * respect to q, k, v, g, beta and the initial state, where o and the final
 * state are the exact function the forward computes (its activation-dtype
 * roundings treated as the identity). Arithmetic is FP32; the chunk's state
 * entering every chunk is recomputed into the workspace, so the forward's
 * output is not needed.
 *
 *   q, k, v, g, beta, scale, use_qk_l2norm_in_kernel, l2_eps, cu_seqlens,
 *   initial_state   as in gdn_chunk_rule_fwd (initial_state NULL: zero)
 *   d_o             [B, T, Hv, dv] act dtype, any strides, inner 1
 *   d_final_state   [N, Hv, dv, dk] F32 contiguous, or NULL (zero)
 *   dq, dk          [B, T, Hqk, dk] contiguous, act dtype or F32 (dq, dk and
 *                   dv share one dtype); dq and dk sum over the value heads
 *                   of each GQA group
 *   dv              [B, T, Hv, dv] contiguous
 *   dg, dbeta       [B, T, Hv] F32 contiguous
 *   d_initial_state [N, Hv, dv, dk] F32 contiguous, or NULL (not written);
 *                   for an empty packed sequence it equals d_final_state
 *   workspace       device memory of gdn_chunk_rule_bwd_workspace_bytes(...)
 *                   bytes, 256-byte aligned, required; it must not overlap
 *                   any tensor argument or be used by another call until
 *                   this call's work on `stream` is done
 * Outputs must not overlap inputs or each other. Supported: dk 64, 128 or
 * 256, dv a multiple of 16 (GDN_ERR_NOT_SUPPORTED otherwise).
 */
gdn_status gdn_chunk_rule_bwd(const gdn_tensor *q, const gdn_tensor *k,
                              const gdn_tensor *v, const gdn_tensor *g,
                              const gdn_tensor *beta, float scale,
                              int32_t use_qk_l2norm_in_kernel, float l2_eps,
                              const gdn_tensor *cu_seqlens,
                              const gdn_tensor *initial_state,
                              const gdn_tensor *d_o,
                              const gdn_tensor *d_final_state,
                              const gdn_tensor *dq, const gdn_tensor *dk,
                              const gdn_tensor *dv, const gdn_tensor *dg,
                              const gdn_tensor *dbeta,
                              const gdn_tensor *d_initial_state,
                              void *workspace, size_t workspace_bytes,
                              void *stream);

/* Bytes of workspace gdn_chunk_rule_bwd needs (n_seqs as in
 * gdn_chunk_rule_workspace_bytes). With C = number of chunk rows
 * (ceil(T/64) + n_seqs packed, B*ceil(T/64) dense), about
 * 4 C (2 Hqk 64 dk + 2 Hv 64 64 + 2 Hv dv dk + 3 Hv 64 dv) bytes. 0 for
 * invalid or unsupported geometry. */
size_t gdn_chunk_rule_bwd_workspace_bytes(int64_t B, int64_t T, int64_t n_seqs,
                                          const gdn_dims *dims);

/*
 * gdn_layer_bwd - first-order gradients of gdn_layer_fwd ([P2] Execution and
 * numerical behavior: the fused stages support first-order autograd; [P3]
 * Test plan: input and parameter gradients of the fused layer checked).
 * Gradients of L = sum(d_out * out) with respect to every input and
 * parameter of gdn_layer_fwd. On `stream`, in a caller workspace: the
 * prologue and the chunk rule are recomputed (qkv, g, beta and o as
 * gdn_layer_fwd materialises them), then gdn_gated_norm_bwd (d_o in the act
 * dtype), gdn_chunk_rule_bwd (dq, dk, dv into one [B, T, C] buffer of the
 * act dtype, dg, dbeta) and gdn_prologue_bwd run. Each stage's gradient is evaluated at
 * the stored values of its inputs, the roundings taken as the identity.
 *
 *   inputs          as in gdn_layer_fwd (initial state: none)
 *   d_out           [B, T, Hv, dv] act dtype, any strides, inner 1
 *   dx_q, dx_k, dx_v, d_conv_w, d_conv_b (NULL when conv_b is NULL), d_a,
 *   d_b, d_A_log, d_dt_bias   as the outputs of gdn_prologue_bwd
 *   d_gate          [B, T, Hv, dv] gate's dtype, contiguous
 *   d_norm_w        [dv] F32
 *   workspace       gdn_layer_bwd_workspace_bytes(...) bytes, 256-byte
 *                   aligned, owned by the caller and not used by any other
 *                   call until this call's work on `stream` is done
 * Outputs must not overlap inputs, each other or the workspace. Supported:
 * the geometries of gdn_chunk_rule_bwd.
 */
gdn_status gdn_layer_bwd(const gdn_tensor *x_q, const gdn_tensor *x_k,
                         const gdn_tensor *x_v, const gdn_tensor *conv_w,
                         const gdn_tensor *conv_b, const gdn_tensor *a,
                         const gdn_tensor *b, const gdn_tensor *A_log,
                         const gdn_tensor *dt_bias, const gdn_tensor *gate,
                         const gdn_tensor *norm_w,
                         const gdn_tensor *cu_seqlens, const gdn_dims *dims,
                         float scale, int32_t use_qk_l2norm_in_kernel,
                         float l2_eps, float rms_eps,
                         const gdn_tensor *d_out, const gdn_tensor *dx_q,
                         const gdn_tensor *dx_k, const gdn_tensor *dx_v,
                         const gdn_tensor *d_conv_w,
                         const gdn_tensor *d_conv_b, const gdn_tensor *d_a,
                         const gdn_tensor *d_b, const gdn_tensor *d_A_log,
                         const gdn_tensor *d_dt_bias,
                         const gdn_tensor *d_gate, const gdn_tensor *d_norm_w,
                         void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * gdn_layer_bwd_saved - gdn_layer_bwd for callers that keep the forward's
 * activations (the same gradients, [P2] Execution and numerical behavior):
 * the prologue and the chunk rule are not recomputed. `workspace` must hold
 * what a gdn_layer_fwd call with the same inputs and arguments wrote into
 * its first gdn_layer_workspace_bytes(...) bytes (qkv, g, beta and o sit at
 * the same offsets in both layouts), and nothing may have written to it
 * since; it is gdn_layer_bwd_workspace_bytes(...) bytes, so the forward call
 * is given the same buffer. The outputs are then bit for bit those of
 * gdn_layer_bwd (the kernels are deterministic); with other contents they are
 * the gradients at whatever the workspace holds, and no error is reported.
 * Arguments, validation and errors otherwise as gdn_layer_bwd.
 */
gdn_status gdn_layer_bwd_saved(const gdn_tensor *x_q, const gdn_tensor *x_k,
                               const gdn_tensor *x_v, const gdn_tensor *conv_w,
                               const gdn_tensor *conv_b, const gdn_tensor *a,
                               const gdn_tensor *b, const gdn_tensor *A_log,
                               const gdn_tensor *dt_bias, const gdn_tensor *gate,
                               const gdn_tensor *norm_w,
                               const gdn_tensor *cu_seqlens, const gdn_dims *dims,
                               float scale, int32_t use_qk_l2norm_in_kernel,
                               float l2_eps, float rms_eps,
                               const gdn_tensor *d_out, const gdn_tensor *dx_q,
                               const gdn_tensor *dx_k, const gdn_tensor *dx_v,
                               const gdn_tensor *d_conv_w,
                               const gdn_tensor *d_conv_b, const gdn_tensor *d_a,
                               const gdn_tensor *d_b, const gdn_tensor *d_A_log,
                               const gdn_tensor *d_dt_bias,
                               const gdn_tensor *d_gate, const gdn_tensor *d_norm_w,
                               void *workspace, size_t workspace_bytes,
                               void *stream);

/* Bytes of workspace gdn_layer_bwd needs (n_seqs as in
 * gdn_layer_workspace_bytes): the forward stage outputs and the chunk
 * forward's workspace, d_o, d_qkv (act dtype), dg and dbeta, and the three
 * backward stages' workspaces, each 256-byte aligned. 0 for invalid or
 * unsupported geometry. */
size_t gdn_layer_bwd_workspace_bytes(int64_t B, int64_t T, int64_t n_seqs,
                                     const gdn_dims *dims, int32_t act_dtype);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
