// C ABI of the GDN layer core: argument validation from host metadata only,
// launch planning, and the composition of the three stages.
//
// Validation follows the Megatron Core "GDN Elementwise Fusion" guide (Post-
// GDR requirements): every call checks its inputs from tensor metadata, with
// no device synchronisation, and rejects what it does not support with an
// error instead of falling back to another path. Nothing here touches the
// device before all checks have passed, so a rejected call has no effect.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace {

thread_local std::string g_error;

gdn_status fail(gdn_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

int64_t elem_size(int32_t dt) {
  switch (dt) {
    case GDN_F32: return 4;
    case GDN_BF16: return 2;
    case GDN_F16: return 2;
    case GDN_I32: return 4;
  }
  return 0;
}

const char *dt_name(int32_t dt) {
  switch (dt) {
    case GDN_F32: return "F32";
    case GDN_BF16: return "BF16";
    case GDN_F16: return "F16";
    case GDN_I32: return "I32";
  }
  return "?";
}

bool is_act(int32_t dt) { return dt == GDN_F32 || dt == GDN_BF16 || dt == GDN_F16; }

bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Byte range [lo, hi) covered by a tensor with non-negative strides.
struct Range {
  uintptr_t lo, hi;
};

Range range_of(const gdn_tensor *t) {
  int64_t last = 0;
  for (int i = 0; i < t->ndim; ++i) {
    if (t->shape[i] == 0) return {0, 0};
    last += (t->shape[i] - 1) * t->stride[i];
  }
  const uintptr_t lo = (uintptr_t)t->data;
  return {lo, lo + (uintptr_t)((last + 1) * elem_size(t->dtype))};
}

bool overlaps(const gdn_tensor *a, const gdn_tensor *b) {
  if (!a || !b) return false;
  const Range x = range_of(a), y = range_of(b);
  if (x.lo == x.hi || y.lo == y.hi) return false;
  return x.lo < y.hi && y.lo < x.hi;
}

// Basic descriptor sanity: non-null, data non-null, rank, dtype, shape.
gdn_status check(const gdn_tensor *t, const char *name, int ndim, const int64_t *shape) {
  if (!t) return fail(GDN_ERR_INVALID_VALUE, "%s: descriptor is NULL", name);
  if (t->ndim != ndim)
    return fail(GDN_ERR_INVALID_VALUE, "%s: expected %d dims, got %d", name, ndim, t->ndim);
  if (!elem_size(t->dtype)) return fail(GDN_ERR_INVALID_VALUE, "%s: unknown dtype %d", name, t->dtype);
  for (int i = 0; i < ndim; ++i) {
    if (t->shape[i] != shape[i])
      return fail(GDN_ERR_INVALID_VALUE, "%s: dim %d is %lld, expected %lld", name, i,
                  (long long)t->shape[i], (long long)shape[i]);
    if (t->stride[i] < 0) return fail(GDN_ERR_INVALID_VALUE, "%s: negative stride", name);
  }
  if (!t->data) return fail(GDN_ERR_INVALID_VALUE, "%s: data pointer is NULL", name);
  if ((uintptr_t)t->data % (uintptr_t)elem_size(t->dtype))
    return fail(GDN_ERR_INVALID_VALUE, "%s: data not aligned to its element size", name);
  return GDN_OK;
}

gdn_status check_dtype(const gdn_tensor *t, const char *name, int32_t want) {
  if (t->dtype != want)
    return fail(GDN_ERR_INVALID_VALUE, "%s: dtype %s, expected %s", name, dt_name(t->dtype), dt_name(want));
  return GDN_OK;
}

gdn_status check_inner(const gdn_tensor *t, const char *name) {
  if (t->shape[t->ndim - 1] > 1 && t->stride[t->ndim - 1] != 1)
    return fail(GDN_ERR_INVALID_VALUE, "%s: innermost stride must be 1", name);
  return GDN_OK;
}

bool contiguous(const gdn_tensor *t) {
  int64_t expect = 1;
  for (int i = t->ndim - 1; i >= 0; --i) {
    if (t->shape[i] != 1 && t->stride[i] != expect) return false;
    expect *= t->shape[i];
  }
  return true;
}

gdn_status check_contig(const gdn_tensor *t, const char *name) {
  if (!contiguous(t)) return fail(GDN_ERR_INVALID_VALUE, "%s: must be contiguous", name);
  return GDN_OK;
}

// Largest power-of-two byte alignment (<= 16) shared by the base address and
// every stride (in bytes) of the leading `nd` dims.
int row_align(const gdn_tensor *t, int nd) {
  uint64_t acc = (uint64_t)(uintptr_t)t->data;
  const int64_t es = elem_size(t->dtype);
  for (int i = 0; i < nd; ++i)
    if (t->shape[i] > 1) acc |= (uint64_t)(t->stride[i] * es);
  return gdn::align_of_host(acc);
}

#define TRY(x)                        \
  do {                                \
    gdn_status _st = (x);             \
    if (_st != GDN_OK) return _st;    \
  } while (0)

gdn_status check_dims(const gdn_dims *d) {
  if (!d) return fail(GDN_ERR_INVALID_VALUE, "dims is NULL");
  if (d->Hqk <= 0 || d->dk <= 0 || d->Hv <= 0 || d->dv <= 0)
    return fail(GDN_ERR_INVALID_VALUE, "dims must be positive");
  if (d->Hv % d->Hqk)
    return fail(GDN_ERR_INVALID_VALUE, "Hv (%lld) must be a multiple of Hqk (%lld)", (long long)d->Hv,
                (long long)d->Hqk);
  if (!pow2(d->dk) || !pow2(d->dv))
    return fail(GDN_ERR_INVALID_VALUE, "head dims must be powers of two (dk=%lld, dv=%lld)",
                (long long)d->dk, (long long)d->dv);
  return GDN_OK;
}

gdn_status check_cu(const gdn_tensor *cu, int64_t B, int64_t *n_seqs) {
  if (!cu) {
    *n_seqs = B;
    return GDN_OK;
  }
  if (cu->ndim != 1 || cu->shape[0] < 2)
    return fail(GDN_ERR_INVALID_VALUE, "cu_seqlens: expected shape [N+1] with N >= 1");
  TRY(check(cu, "cu_seqlens", 1, cu->shape));
  TRY(check_dtype(cu, "cu_seqlens", GDN_I32));
  TRY(check_contig(cu, "cu_seqlens"));
  if (B != 1) return fail(GDN_ERR_INVALID_VALUE, "cu_seqlens requires B == 1 (got B=%lld)", (long long)B);
  *n_seqs = cu->shape[0] - 1;
  return GDN_OK;
}

gdn_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return GDN_OK;
}

// ---------------------------------------------------------------------------
// Planning of each stage (validation + argument packing, no device calls).
// ---------------------------------------------------------------------------
gdn_status plan_prologue(const gdn_tensor *x_q, const gdn_tensor *x_k, const gdn_tensor *x_v,
                         const gdn_tensor *conv_w, const gdn_tensor *conv_b, const gdn_tensor *a,
                         const gdn_tensor *b, const gdn_tensor *A_log, const gdn_tensor *dt_bias,
                         const gdn_tensor *cu_seqlens, const gdn_dims *dims, int32_t caller_l2norm,
                         float l2_eps, const gdn_tensor *out_qkv, const gdn_tensor *out_g,
                         const gdn_tensor *out_beta, gdn::PrologueArgs *P) {
  TRY(check_dims(dims));
  if (!x_q) return fail(GDN_ERR_INVALID_VALUE, "x_q: descriptor is NULL");
  if (x_q->ndim != 3) return fail(GDN_ERR_INVALID_VALUE, "x_q: expected [B, T, Hqk*dk]");
  const int64_t B = x_q->shape[0], T = x_q->shape[1];
  const int64_t nq = dims->Hqk * dims->dk, nv = dims->Hv * dims->dv, C = 2 * nq + nv;
  const int64_t sq[3] = {B, T, nq}, sv[3] = {B, T, nv}, sw[2] = {C, 4}, sc[1] = {C};
  const int64_t sab[3] = {B, T, dims->Hv}, sh[1] = {dims->Hv}, so[3] = {B, T, C};
  if (B * T == 0) return fail(GDN_ERR_INVALID_VALUE, "empty input (B*T == 0)");
  TRY(check(x_q, "x_q", 3, sq));
  const int32_t act = x_q->dtype;
  if (!is_act(act)) return fail(GDN_ERR_INVALID_VALUE, "x_q: dtype must be F32, BF16 or F16");
  TRY(check(x_k, "x_k", 3, sq));
  TRY(check(x_v, "x_v", 3, sv));
  TRY(check_dtype(x_k, "x_k", act));
  TRY(check_dtype(x_v, "x_v", act));
  TRY(check_inner(x_q, "x_q"));
  TRY(check_inner(x_k, "x_k"));
  TRY(check_inner(x_v, "x_v"));
  TRY(check(conv_w, "conv_w", 2, sw));
  if (conv_w->dtype != act && conv_w->dtype != GDN_F32)
    return fail(GDN_ERR_INVALID_VALUE, "conv_w: dtype must be the activation dtype or F32");
  TRY(check_contig(conv_w, "conv_w"));
  if (conv_b) {
    TRY(check(conv_b, "conv_b", 1, sc));
    if (conv_b->dtype != act && conv_b->dtype != GDN_F32)
      return fail(GDN_ERR_INVALID_VALUE, "conv_b: dtype must be the activation dtype or F32");
    TRY(check_contig(conv_b, "conv_b"));
  }
  TRY(check(a, "a", 3, sab));
  TRY(check(b, "b", 3, sab));
  TRY(check_dtype(a, "a", act));
  TRY(check_dtype(b, "b", act));
  TRY(check(A_log, "A_log", 1, sh));
  TRY(check(dt_bias, "dt_bias", 1, sh));
  TRY(check_dtype(A_log, "A_log", GDN_F32));
  TRY(check_dtype(dt_bias, "dt_bias", GDN_F32));
  TRY(check_contig(A_log, "A_log"));
  TRY(check_contig(dt_bias, "dt_bias"));
  int64_t n_seqs = 0;
  TRY(check_cu(cu_seqlens, B, &n_seqs));
  TRY(check(out_qkv, "out_qkv", 3, so));
  TRY(check_dtype(out_qkv, "out_qkv", act));
  TRY(check_contig(out_qkv, "out_qkv"));
  TRY(check(out_g, "out_g", 3, sab));
  TRY(check(out_beta, "out_beta", 3, sab));
  TRY(check_dtype(out_g, "out_g", GDN_F32));
  TRY(check_dtype(out_beta, "out_beta", GDN_F32));
  TRY(check_contig(out_g, "out_g"));
  TRY(check_contig(out_beta, "out_beta"));
  const gdn_tensor *ins[] = {x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, cu_seqlens};
  const gdn_tensor *outs[] = {out_qkv, out_g, out_beta};
  for (auto *o : outs)
    for (auto *i : ins)
      if (overlaps(o, i)) return fail(GDN_ERR_INVALID_VALUE, "an output overlaps an input");
  if (overlaps(out_qkv, out_g) || overlaps(out_qkv, out_beta) || overlaps(out_g, out_beta))
    return fail(GDN_ERR_INVALID_VALUE, "outputs overlap each other");
  if (!(l2_eps >= 0.f) || !std::isfinite(l2_eps)) return fail(GDN_ERR_INVALID_VALUE, "l2_eps must be finite and >= 0");

  const int64_t es = elem_size(act);
  int al = 16;
  for (const gdn_tensor *x : {x_q, x_k, x_v}) {
    const int r = row_align(x, 2);
    al = r < al ? r : al;
  }
  int vec = (int)(al / es);
  if (vec > 8) vec = 8;
  while (vec > 1 && (nq % vec || nv % vec)) vec >>= 1;
  if (vec < 1) return fail(GDN_ERR_INVALID_VALUE, "x: misaligned rows");
  if (caller_l2norm && (dims->dk % vec || dims->dk / vec > 64))
    return fail(GDN_ERR_NOT_SUPPORTED,
                "caller-side L2 norm needs rows aligned to at least %lld bytes", (long long)(dims->dk / 64 * es));

  if (B > 65535 || (C + 255) / 256 + 1 > 65535 || (T + 127) / 128 > 0x7fffffff)
    return fail(GDN_ERR_NOT_SUPPORTED, "prologue: grid too large (B=%lld, T=%lld, C=%lld)", (long long)B,
                (long long)T, (long long)C);

  gdn::PrologueArgs &p = *P;
  memset(&p, 0, sizeof p);
  p.xq = x_q->data; p.xk = x_k->data; p.xv = x_v->data;
  p.sxq_b = x_q->stride[0]; p.sxq_t = x_q->stride[1];
  p.sxk_b = x_k->stride[0]; p.sxk_t = x_k->stride[1];
  p.sxv_b = x_v->stride[0]; p.sxv_t = x_v->stride[1];
  p.conv_w = conv_w->data; p.w_dtype = conv_w->dtype;
  p.w_align = gdn::align_of_host((uint64_t)(uintptr_t)conv_w->data);
  p.conv_b = conv_b ? conv_b->data : nullptr; p.b_dtype = conv_b ? conv_b->dtype : act;
  p.a = a->data; p.b = b->data;
  p.sa_b = a->stride[0]; p.sa_t = a->stride[1]; p.sa_h = a->stride[2];
  p.sb_b = b->stride[0]; p.sb_t = b->stride[1]; p.sb_h = b->stride[2];
  p.A_log = static_cast<const float *>(A_log->data);
  p.dt_bias = static_cast<const float *>(dt_bias->data);
  p.cu_seqlens = cu_seqlens ? static_cast<const int32_t *>(cu_seqlens->data) : nullptr;
  p.n_seqs = n_seqs;
  p.B = B; p.T = T; p.Hqk = dims->Hqk; p.dk = dims->dk; p.Hv = dims->Hv; p.dv = dims->dv; p.C = C;
  p.act = act; p.vec = vec; p.caller_l2norm = caller_l2norm ? 1 : 0; p.l2_eps = l2_eps;
  p.qkv = out_qkv->data;
  p.g = static_cast<float *>(out_g->data);
  p.beta = static_cast<float *>(out_beta->data);
  return GDN_OK;
}

gdn_status plan_chunk(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v, const gdn_tensor *g,
                      const gdn_tensor *beta, float scale, int32_t use_l2, float l2_eps,
                      const gdn_tensor *cu_seqlens, const gdn_tensor *initial_state, const gdn_tensor *out_o,
                      const gdn_tensor *final_state, gdn::ChunkArgs *P) {
  if (!q || q->ndim != 4) return fail(GDN_ERR_INVALID_VALUE, "q: expected [B, T, Hqk, dk]");
  if (!v || v->ndim != 4) return fail(GDN_ERR_INVALID_VALUE, "v: expected [B, T, Hv, dv]");
  const int64_t B = q->shape[0], T = q->shape[1], Hqk = q->shape[2], dk = q->shape[3];
  const int64_t Hv = v->shape[2], dv = v->shape[3];
  if (B * T == 0) return fail(GDN_ERR_INVALID_VALUE, "empty input (B*T == 0)");
  const gdn_dims d = {Hqk, dk, Hv, dv};
  TRY(check_dims(&d));
  const int64_t sq[4] = {B, T, Hqk, dk}, svv[4] = {B, T, Hv, dv}, sg[3] = {B, T, Hv};
  TRY(check(q, "q", 4, sq));
  const int32_t act = q->dtype;
  if (!is_act(act)) return fail(GDN_ERR_INVALID_VALUE, "q: dtype must be F32, BF16 or F16");
  TRY(check(k, "k", 4, sq));
  TRY(check(v, "v", 4, svv));
  TRY(check_dtype(k, "k", act));
  TRY(check_dtype(v, "v", act));
  TRY(check_inner(q, "q"));
  TRY(check_inner(k, "k"));
  TRY(check_inner(v, "v"));
  TRY(check(g, "g", 3, sg));
  TRY(check(beta, "beta", 3, sg));
  TRY(check_dtype(g, "g", GDN_F32));
  TRY(check_dtype(beta, "beta", GDN_F32));
  int64_t n_seqs = 0;
  TRY(check_cu(cu_seqlens, B, &n_seqs));
  const int64_t ss[4] = {n_seqs, Hv, dv, dk};
  if (initial_state) {
    TRY(check(initial_state, "initial_state", 4, ss));
    TRY(check_dtype(initial_state, "initial_state", GDN_F32));
    TRY(check_contig(initial_state, "initial_state"));
  }
  if (final_state) {
    TRY(check(final_state, "final_state", 4, ss));
    TRY(check_dtype(final_state, "final_state", GDN_F32));
    TRY(check_contig(final_state, "final_state"));
  }
  TRY(check(out_o, "out_o", 4, svv));
  TRY(check_dtype(out_o, "out_o", act));
  TRY(check_inner(out_o, "out_o"));
  if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_VALUE, "scale must be finite");
  if (!(l2_eps >= 0.f) || !std::isfinite(l2_eps)) return fail(GDN_ERR_INVALID_VALUE, "l2_eps must be finite and >= 0");
  const gdn_tensor *ins[] = {q, k, v, g, beta, cu_seqlens, initial_state};
  for (auto *i : ins) {
    if (overlaps(out_o, i)) return fail(GDN_ERR_INVALID_VALUE, "out_o overlaps an input");
    if (i != initial_state && overlaps(final_state, i))
      return fail(GDN_ERR_INVALID_VALUE, "final_state overlaps an input");
  }
  if (overlaps(out_o, final_state)) return fail(GDN_ERR_INVALID_VALUE, "out_o overlaps final_state");
  if (initial_state && final_state && overlaps(initial_state, final_state) &&
      initial_state->data != final_state->data)
    return fail(GDN_ERR_INVALID_VALUE, "final_state partially overlaps initial_state");
  if (!gdn::chunk_rule_supported(dk, act) || dv % 16)
    return fail(GDN_ERR_NOT_SUPPORTED, "chunk rule: dk=%lld dv=%lld %s is not instantiated", (long long)dk,
                (long long)dv, dt_name(act));
  if (n_seqs > 65535 || Hv > 65535)
    return fail(GDN_ERR_NOT_SUPPORTED, "chunk rule: at most 65535 sequences and heads");
  const int64_t es = elem_size(act);
  if (row_align(q, 3) < 16 || row_align(k, 3) < 16)
    return fail(GDN_ERR_NOT_SUPPORTED, "q/k rows must be 16-byte aligned");
  if (row_align(v, 3) < 4 * es) return fail(GDN_ERR_NOT_SUPPORTED, "v rows must be %lld-byte aligned", (long long)(4 * es));

  gdn::ChunkArgs &p = *P;
  memset(&p, 0, sizeof p);
  p.q = q->data; p.k = k->data; p.v = v->data;
  p.sq_b = q->stride[0]; p.sq_t = q->stride[1]; p.sq_h = q->stride[2];
  p.sk_b = k->stride[0]; p.sk_t = k->stride[1]; p.sk_h = k->stride[2];
  p.sv_b = v->stride[0]; p.sv_t = v->stride[1]; p.sv_h = v->stride[2];
  p.g = static_cast<const float *>(g->data);
  p.beta = static_cast<const float *>(beta->data);
  p.sg_b = g->stride[0]; p.sg_t = g->stride[1]; p.sg_h = g->stride[2];
  p.sbt_b = beta->stride[0]; p.sbt_t = beta->stride[1]; p.sbt_h = beta->stride[2];
  p.cu_seqlens = cu_seqlens ? static_cast<const int32_t *>(cu_seqlens->data) : nullptr;
  p.n_seqs = n_seqs;
  p.init_state = initial_state ? static_cast<const float *>(initial_state->data) : nullptr;
  p.final_state = final_state ? static_cast<float *>(final_state->data) : nullptr;
  p.o = out_o->data;
  p.so_b = out_o->stride[0]; p.so_t = out_o->stride[1]; p.so_h = out_o->stride[2];
  p.B = B; p.T = T; p.Hqk = Hqk; p.dk = dk; p.Hv = Hv; p.dv = dv;
  p.act = act; p.use_l2 = use_l2 ? 1 : 0; p.l2_eps = l2_eps; p.scale = scale;
  p.rows16 = row_align(v, 3) >= 16 ? 1 : 0;
  p.o8 = row_align(out_o, 3) >= 8 ? 1 : 0;
  return GDN_OK;
}

gdn_status plan_norm(const gdn_tensor *o, const gdn_tensor *gate, const gdn_tensor *weight, float eps,
                     const gdn_tensor *out, gdn::NormArgs *P) {
  if (!o || o->ndim != 4) return fail(GDN_ERR_INVALID_VALUE, "o: expected [B, T, H, dv]");
  const int64_t B = o->shape[0], T = o->shape[1], H = o->shape[2], dv = o->shape[3];
  if (B * T * H * dv == 0) return fail(GDN_ERR_INVALID_VALUE, "o: empty tensor");
  if (!pow2(dv)) return fail(GDN_ERR_INVALID_VALUE, "head dim %lld is not a power of two", (long long)dv);
  const int64_t so[4] = {B, T, H, dv}, sw[1] = {dv};
  TRY(check(o, "o", 4, so));
  const int32_t act = o->dtype;
  if (!is_act(act)) return fail(GDN_ERR_INVALID_VALUE, "o: dtype must be F32, BF16 or F16");
  TRY(check_inner(o, "o"));
  TRY(check(gate, "gate", 4, so));
  if (gate->dtype != act && gate->dtype != GDN_F32)
    return fail(GDN_ERR_INVALID_VALUE, "gate: dtype must be o's dtype or F32");
  TRY(check_inner(gate, "gate"));
  TRY(check(weight, "weight", 1, sw));
  if (!is_act(weight->dtype)) return fail(GDN_ERR_INVALID_VALUE, "weight: dtype must be F32, BF16 or F16");
  TRY(check_contig(weight, "weight"));
  TRY(check(out, "out", 4, so));
  TRY(check_dtype(out, "out", act));
  TRY(check_contig(out, "out"));
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(GDN_ERR_INVALID_VALUE, "eps must be finite and >= 0");
  if (overlaps(out, o) || overlaps(out, gate) || overlaps(out, weight))
    return fail(GDN_ERR_INVALID_VALUE, "out overlaps an input");
  if (dv < 64 || dv > 512)
    return fail(GDN_ERR_NOT_SUPPORTED, "gated norm: head dim %lld is not instantiated (64..512)", (long long)dv);
  if ((uintptr_t)weight->data % 16 || (uintptr_t)out->data % 16)
    return fail(GDN_ERR_NOT_SUPPORTED, "weight and out must be 16-byte aligned");
  gdn::NormArgs &p = *P;
  memset(&p, 0, sizeof p);
  p.o = o->data; p.so_b = o->stride[0]; p.so_t = o->stride[1]; p.so_h = o->stride[2];
  p.gate = gate->data; p.sg_b = gate->stride[0]; p.sg_t = gate->stride[1]; p.sg_h = gate->stride[2];
  p.w = weight->data; p.out = out->data;
  p.B = B; p.T = T; p.H = H; p.dv = dv;
  p.act = act; p.gate_dtype = gate->dtype; p.w_dtype = weight->dtype;
  p.o_align = row_align(o, 3);
  p.gate_align = row_align(gate, 3);
  p.eps = eps;
  p.rd = gdn::row_div(B, T, H);
  return GDN_OK;
}

gdn_status plan_decode(const gdn_tensor *x_q, const gdn_tensor *x_k, const gdn_tensor *x_v,
                       const gdn_tensor *conv_w, const gdn_tensor *conv_b, const gdn_tensor *conv_state,
                       const gdn_tensor *a, const gdn_tensor *b, const gdn_tensor *A_log,
                       const gdn_tensor *dt_bias, const gdn_tensor *state, const gdn_tensor *gate,
                       const gdn_tensor *norm_w, const gdn_dims *dims, float scale, int32_t use_l2, float l2_eps,
                       float rms_eps, const gdn_tensor *out, gdn::DecodeArgs *P) {
  TRY(check_dims(dims));
  if (!x_q) return fail(GDN_ERR_INVALID_VALUE, "x_q: descriptor is NULL");
  if (x_q->ndim != 2) return fail(GDN_ERR_INVALID_VALUE, "x_q: expected [N, Hqk*dk]");
  const int64_t N = x_q->shape[0], Hv = dims->Hv, dv = dims->dv, dk = dims->dk;
  const int64_t nq = dims->Hqk * dk, nv = Hv * dv, C = 2 * nq + nv;
  if (N == 0) return fail(GDN_ERR_INVALID_VALUE, "empty input (N == 0)");
  const int64_t sq[2] = {N, nq}, sv[2] = {N, nv}, sw[2] = {C, 4}, sc[1] = {C}, scs[3] = {N, 3, C};
  const int64_t sab[2] = {N, Hv}, sh[1] = {Hv}, sst[4] = {N, Hv, dv, dk}, so[3] = {N, Hv, dv}, sn[1] = {dv};
  TRY(check(x_q, "x_q", 2, sq));
  const int32_t act = x_q->dtype;
  if (!is_act(act)) return fail(GDN_ERR_INVALID_VALUE, "x_q: dtype must be F32, BF16 or F16");
  TRY(check(x_k, "x_k", 2, sq));
  TRY(check(x_v, "x_v", 2, sv));
  TRY(check_dtype(x_k, "x_k", act));
  TRY(check_dtype(x_v, "x_v", act));
  TRY(check_inner(x_q, "x_q"));
  TRY(check_inner(x_k, "x_k"));
  TRY(check_inner(x_v, "x_v"));
  TRY(check(conv_w, "conv_w", 2, sw));
  if (conv_w->dtype != act && conv_w->dtype != GDN_F32)
    return fail(GDN_ERR_INVALID_VALUE, "conv_w: dtype must be the activation dtype or F32");
  TRY(check_contig(conv_w, "conv_w"));
  if (conv_b) {
    TRY(check(conv_b, "conv_b", 1, sc));
    if (conv_b->dtype != act && conv_b->dtype != GDN_F32)
      return fail(GDN_ERR_INVALID_VALUE, "conv_b: dtype must be the activation dtype or F32");
    TRY(check_contig(conv_b, "conv_b"));
  }
  TRY(check(conv_state, "conv_state", 3, scs));
  TRY(check_dtype(conv_state, "conv_state", act));
  TRY(check_inner(conv_state, "conv_state"));
  TRY(check(a, "a", 2, sab));
  TRY(check(b, "b", 2, sab));
  TRY(check_dtype(a, "a", act));
  TRY(check_dtype(b, "b", act));
  TRY(check_inner(a, "a"));
  TRY(check_inner(b, "b"));
  TRY(check(A_log, "A_log", 1, sh));
  TRY(check(dt_bias, "dt_bias", 1, sh));
  TRY(check_dtype(A_log, "A_log", GDN_F32));
  TRY(check_dtype(dt_bias, "dt_bias", GDN_F32));
  TRY(check_contig(A_log, "A_log"));
  TRY(check_contig(dt_bias, "dt_bias"));
  TRY(check(state, "state", 4, sst));
  TRY(check_dtype(state, "state", GDN_F32));
  TRY(check_contig(state, "state"));
  TRY(check(gate, "gate", 3, so));
  if (gate->dtype != act && gate->dtype != GDN_F32)
    return fail(GDN_ERR_INVALID_VALUE, "gate: dtype must be the activation dtype or F32");
  TRY(check_inner(gate, "gate"));
  TRY(check(norm_w, "norm_w", 1, sn));
  if (!is_act(norm_w->dtype)) return fail(GDN_ERR_INVALID_VALUE, "norm_w: dtype must be F32, BF16 or F16");
  TRY(check_contig(norm_w, "norm_w"));
  TRY(check(out, "out", 3, so));
  TRY(check_dtype(out, "out", act));
  TRY(check_contig(out, "out"));
  if (!(l2_eps >= 0.f) || !std::isfinite(l2_eps)) return fail(GDN_ERR_INVALID_VALUE, "l2_eps must be finite and >= 0");
  if (!(rms_eps >= 0.f) || !std::isfinite(rms_eps))
    return fail(GDN_ERR_INVALID_VALUE, "rms_eps must be finite and >= 0");
  if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_VALUE, "scale must be finite");
  // conv_state and state are updated in place; nothing else may alias them or out
  const gdn_tensor *ins[] = {x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, gate, norm_w};
  const gdn_tensor *outs[] = {conv_state, state, out};
  for (auto *o : outs)
    for (auto *i : ins)
      if (overlaps(o, i)) return fail(GDN_ERR_INVALID_VALUE, "an output or cache overlaps an input");
  if (overlaps(conv_state, state) || overlaps(conv_state, out) || overlaps(state, out))
    return fail(GDN_ERR_INVALID_VALUE, "conv_state, state and out must not overlap");
  const int64_t G = Hv / dims->Hqk;
  if (!gdn::decode_supported(dk, G, dv))
    return fail(GDN_ERR_NOT_SUPPORTED, "decode: dk %lld, dv %lld, group size %lld not instantiated", (long long)dk,
                (long long)dv, (long long)G);
  if ((uintptr_t)state->data % 16) return fail(GDN_ERR_NOT_SUPPORTED, "state must be 16-byte aligned");
  if (N > 65535 || dims->Hqk > 0x7fffffff) return fail(GDN_ERR_NOT_SUPPORTED, "decode: grid too large");

  gdn::DecodeArgs &p = *P;
  memset(&p, 0, sizeof p);
  p.xq = x_q->data; p.xk = x_k->data; p.xv = x_v->data;
  p.sxq = x_q->stride[0]; p.sxk = x_k->stride[0]; p.sxv = x_v->stride[0];
  p.conv_w = conv_w->data; p.w_dtype = conv_w->dtype;
  p.w_align = gdn::align_of_host((uint64_t)(uintptr_t)conv_w->data);
  p.conv_b = conv_b ? conv_b->data : nullptr; p.b_dtype = conv_b ? conv_b->dtype : act;
  p.conv_state = conv_state->data; p.scs_n = conv_state->stride[0]; p.scs_t = conv_state->stride[1];
  p.a = a->data; p.b = b->data; p.sa = a->stride[0]; p.sb = b->stride[0];
  p.A_log = static_cast<const float *>(A_log->data);
  p.dt_bias = static_cast<const float *>(dt_bias->data);
  p.state = static_cast<float *>(state->data);
  p.gate = gate->data; p.sgate_n = gate->stride[0]; p.sgate_h = gate->stride[1]; p.gate_dtype = gate->dtype;
  p.norm_w = norm_w->data; p.nw_dtype = norm_w->dtype;
  p.out = out->data;
  p.N = N; p.Hqk = dims->Hqk; p.dk = dk; p.Hv = Hv; p.dv = dv;
  p.act = act; p.use_l2 = use_l2 ? 1 : 0;
  p.scale = scale; p.l2_eps = l2_eps; p.rms_eps = rms_eps;
  return GDN_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ------------------------------------------------------------- backward
int64_t norm_bwd_blocks(int64_t rows, int64_t dv) {
  const int64_t rpb = 2 * 2048 / dv;  // rows per block and pass (4 waves, dv / 8 lanes per row, 2 rows)
  const int64_t nb = (rows + rpb - 1) / rpb;
  return nb < 8192 ? nb : 8192;
}

gdn_status plan_norm_bwd(const gdn_tensor *o, const gdn_tensor *gate, const gdn_tensor *weight, float eps,
                         const gdn_tensor *dout, const gdn_tensor *d_o, const gdn_tensor *d_gate,
                         const gdn_tensor *d_weight, void *ws, size_t ws_bytes, gdn::NormBwdArgs *P) {
  gdn::NormArgs f;
  // o, gate, weight and eps as in the forward; d_o stands in for its output
  TRY(plan_norm(o, gate, weight, eps, d_o, &f));
  const int64_t so[4] = {f.B, f.T, f.H, f.dv}, sw[1] = {f.dv};
  TRY(check(dout, "dout", 4, so));
  TRY(check_dtype(dout, "dout", f.act));
  TRY(check_inner(dout, "dout"));
  TRY(check(d_gate, "d_gate", 4, so));
  TRY(check_dtype(d_gate, "d_gate", gate->dtype));
  TRY(check_contig(d_gate, "d_gate"));
  TRY(check(d_weight, "d_weight", 1, sw));
  TRY(check_dtype(d_weight, "d_weight", GDN_F32));
  TRY(check_contig(d_weight, "d_weight"));
  const gdn_tensor *ins[] = {o, gate, weight, dout};
  const gdn_tensor *outs[] = {d_o, d_gate, d_weight};
  for (auto *x : outs)
    for (auto *i : ins)
      if (overlaps(x, i)) return fail(GDN_ERR_INVALID_VALUE, "an output overlaps an input");
  if (overlaps(d_o, d_gate) || overlaps(d_o, d_weight) || overlaps(d_gate, d_weight))
    return fail(GDN_ERR_INVALID_VALUE, "outputs overlap each other");
  if ((uintptr_t)d_gate->data % 16) return fail(GDN_ERR_NOT_SUPPORTED, "d_gate must be 16-byte aligned");
  const int64_t nb = norm_bwd_blocks(f.B * f.T * f.H, f.dv);
  const size_t need = align256((size_t)nb * (size_t)f.dv * 4) + align256((size_t)32 * f.dv * 4);
  if (!ws || ws_bytes < need)
    return fail(GDN_ERR_INVALID_VALUE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  if ((uintptr_t)ws % 256) return fail(GDN_ERR_INVALID_VALUE, "workspace must be 256-byte aligned");
  gdn::NormBwdArgs &p = *P;
  memset(&p, 0, sizeof p);
  p.o = f.o; p.so_b = f.so_b; p.so_t = f.so_t; p.so_h = f.so_h;
  p.gate = f.gate; p.sg_b = f.sg_b; p.sg_t = f.sg_t; p.sg_h = f.sg_h;
  p.dout = dout->data; p.sd_b = dout->stride[0]; p.sd_t = dout->stride[1]; p.sd_h = dout->stride[2];
  p.w = f.w; p.d_o = d_o->data; p.d_gate = d_gate->data;
  p.d_w = static_cast<float *>(d_weight->data);
  p.part = static_cast<float *>(ws);
  p.mid = reinterpret_cast<float *>(static_cast<char *>(ws) + align256((size_t)nb * (size_t)f.dv * 4));
  p.nblocks = nb;
  p.B = f.B; p.T = f.T; p.H = f.H; p.dv = f.dv;
  p.act = f.act; p.gate_dtype = f.gate_dtype; p.w_dtype = f.w_dtype;
  p.o_align = f.o_align; p.gate_align = f.gate_align; p.dout_align = row_align(dout, 3);
  p.eps = eps;
  p.rd = f.rd;
  return GDN_OK;
}

// Tokens per tile of the prologue backward: 128, halved down to 32 while the
// conv launch (one 256-thread block per 1024 channels and tile) would have
// fewer than 2048 blocks, eight per CU. Measured at 131072 tokens of 16 + 16 +
// 32 heads (C = 8192): 512-token tiles 2.04 ms, 256 1.77 ms, 128 1.62 ms, 64
// 1.63 ms, 32 1.82 ms (more, shorter blocks keep more loads in flight until
// the partial sums, one [C][5] row per tile, start to cost).
int64_t prologue_bwd_tile(int64_t ntok, int64_t C) {
  const int64_t chb = (C / 4 + 255) / 256;
  int64_t tile = 128;
  while (tile > 32 && ((ntok + tile - 1) / tile) * chb < 2048) tile /= 2;
  return tile;
}

// Workspace of the prologue backward: per token tile, partial sums of d_conv_w
// [C][4] and d_conv_b [C]; per head tile (4096 / Hv tokens), of d_dt_bias and
// d_A_log [Hv]; then the reduction scratch [32][C * 4].
struct ProBwdWs {
  int64_t tile, ntiles, head_tile, nhtiles;
  size_t w, b, h, mid;  // byte sizes of the regions, each 256-byte aligned
  size_t total() const { return w + b + 2 * h + mid; }
};
ProBwdWs prologue_bwd_layout(int64_t B, int64_t T, const gdn_dims *d) {
  ProBwdWs L;
  const int64_t ntok = B * T, C = 2 * d->Hqk * d->dk + d->Hv * d->dv;
  L.tile = prologue_bwd_tile(ntok, C);
  L.ntiles = (ntok + L.tile - 1) / L.tile;
  L.head_tile = d->Hv <= 4096 ? 4096 / d->Hv : 1;
  L.nhtiles = (ntok + L.head_tile - 1) / L.head_tile;
  L.w = align256((size_t)(L.ntiles * C * 4 * 4));
  L.b = align256((size_t)(L.ntiles * C * 4));
  L.h = align256((size_t)(L.nhtiles * d->Hv * 4));
  L.mid = align256((size_t)(32 * C * 4 * 4));
  return L;
}
size_t prologue_bwd_ws(int64_t B, int64_t T, const gdn_dims *d) { return prologue_bwd_layout(B, T, d).total(); }

gdn_status plan_prologue_bwd(const gdn_tensor *x_q, const gdn_tensor *x_k, const gdn_tensor *x_v,
                             const gdn_tensor *conv_w, const gdn_tensor *conv_b, const gdn_tensor *a,
                             const gdn_tensor *b, const gdn_tensor *A_log, const gdn_tensor *dt_bias,
                             const gdn_tensor *cu_seqlens, const gdn_dims *dims, const gdn_tensor *d_qkv,
                             const gdn_tensor *d_g, const gdn_tensor *d_beta, const gdn_tensor *dx_q,
                             const gdn_tensor *dx_k, const gdn_tensor *dx_v, const gdn_tensor *d_conv_w,
                             const gdn_tensor *d_conv_b, const gdn_tensor *d_a, const gdn_tensor *d_b,
                             const gdn_tensor *d_A_log, const gdn_tensor *d_dt_bias, void *ws, size_t ws_bytes,
                             gdn::PrologueBwdArgs *P) {
  TRY(check_dims(dims));
  if (!x_q) return fail(GDN_ERR_INVALID_VALUE, "x_q: descriptor is NULL");
  if (x_q->ndim != 3) return fail(GDN_ERR_INVALID_VALUE, "x_q: expected [B, T, Hqk*dk]");
  const int64_t B = x_q->shape[0], T = x_q->shape[1], Hv = dims->Hv;
  const int64_t nq = dims->Hqk * dims->dk, nv = Hv * dims->dv, C = 2 * nq + nv;
  const int64_t sq[3] = {B, T, nq}, sv[3] = {B, T, nv}, sw[2] = {C, 4}, sc[1] = {C};
  const int64_t sab[3] = {B, T, Hv}, sh[1] = {Hv}, so[3] = {B, T, C};
  if (B * T == 0) return fail(GDN_ERR_INVALID_VALUE, "empty input (B*T == 0)");
  TRY(check(x_q, "x_q", 3, sq));
  const int32_t act = x_q->dtype;
  if (!is_act(act)) return fail(GDN_ERR_INVALID_VALUE, "x_q: dtype must be F32, BF16 or F16");
  TRY(check(x_k, "x_k", 3, sq));
  TRY(check(x_v, "x_v", 3, sv));
  TRY(check_dtype(x_k, "x_k", act));
  TRY(check_dtype(x_v, "x_v", act));
  TRY(check_inner(x_q, "x_q"));
  TRY(check_inner(x_k, "x_k"));
  TRY(check_inner(x_v, "x_v"));
  TRY(check(conv_w, "conv_w", 2, sw));
  if (conv_w->dtype != act && conv_w->dtype != GDN_F32)
    return fail(GDN_ERR_INVALID_VALUE, "conv_w: dtype must be the activation dtype or F32");
  TRY(check_contig(conv_w, "conv_w"));
  if (conv_b) {
    TRY(check(conv_b, "conv_b", 1, sc));
    if (conv_b->dtype != act && conv_b->dtype != GDN_F32)
      return fail(GDN_ERR_INVALID_VALUE, "conv_b: dtype must be the activation dtype or F32");
    TRY(check_contig(conv_b, "conv_b"));
  }
  TRY(check(a, "a", 3, sab));
  TRY(check(b, "b", 3, sab));
  TRY(check_dtype(a, "a", act));
  TRY(check_dtype(b, "b", act));
  TRY(check_inner(a, "a"));
  TRY(check_inner(b, "b"));
  TRY(check(A_log, "A_log", 1, sh));
  TRY(check(dt_bias, "dt_bias", 1, sh));
  TRY(check_dtype(A_log, "A_log", GDN_F32));
  TRY(check_dtype(dt_bias, "dt_bias", GDN_F32));
  TRY(check_contig(A_log, "A_log"));
  TRY(check_contig(dt_bias, "dt_bias"));
  int64_t n_seqs = 0;
  TRY(check_cu(cu_seqlens, B, &n_seqs));
  TRY(check(d_qkv, "d_qkv", 3, so));
  if (d_qkv->dtype != act && d_qkv->dtype != GDN_F32)
    return fail(GDN_ERR_INVALID_VALUE, "d_qkv: dtype must be the activation dtype or F32");
  TRY(check_contig(d_qkv, "d_qkv"));
  TRY(check(d_g, "d_g", 3, sab));
  TRY(check(d_beta, "d_beta", 3, sab));
  TRY(check_dtype(d_g, "d_g", GDN_F32));
  TRY(check_dtype(d_beta, "d_beta", GDN_F32));
  TRY(check_contig(d_g, "d_g"));
  TRY(check_contig(d_beta, "d_beta"));
  TRY(check(dx_q, "dx_q", 3, sq));
  TRY(check(dx_k, "dx_k", 3, sq));
  TRY(check(dx_v, "dx_v", 3, sv));
  TRY(check(d_a, "d_a", 3, sab));
  TRY(check(d_b, "d_b", 3, sab));
  for (const gdn_tensor *t : {dx_q, dx_k, dx_v, d_a, d_b}) {
    TRY(check_dtype(t, "gradient", act));
    TRY(check_contig(t, "gradient"));
  }
  TRY(check(d_conv_w, "d_conv_w", 2, sw));
  TRY(check_dtype(d_conv_w, "d_conv_w", GDN_F32));
  TRY(check_contig(d_conv_w, "d_conv_w"));
  if (!conv_b != !d_conv_b) return fail(GDN_ERR_INVALID_VALUE, "d_conv_b must be given exactly when conv_b is");
  if (d_conv_b) {
    TRY(check(d_conv_b, "d_conv_b", 1, sc));
    TRY(check_dtype(d_conv_b, "d_conv_b", GDN_F32));
    TRY(check_contig(d_conv_b, "d_conv_b"));
  }
  TRY(check(d_A_log, "d_A_log", 1, sh));
  TRY(check(d_dt_bias, "d_dt_bias", 1, sh));
  TRY(check_dtype(d_A_log, "d_A_log", GDN_F32));
  TRY(check_dtype(d_dt_bias, "d_dt_bias", GDN_F32));
  const gdn_tensor *ins[] = {x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, cu_seqlens, d_qkv, d_g, d_beta};
  const gdn_tensor *outs[] = {dx_q, dx_k, dx_v, d_conv_w, d_conv_b, d_a, d_b, d_A_log, d_dt_bias};
  for (auto *x : outs)
    for (auto *i : ins)
      if (overlaps(x, i)) return fail(GDN_ERR_INVALID_VALUE, "an output overlaps an input");
  for (size_t i = 0; i < 9; ++i)
    for (size_t j = i + 1; j < 9; ++j)
      if (overlaps(outs[i], outs[j])) return fail(GDN_ERR_INVALID_VALUE, "outputs overlap each other");
  const size_t need = prologue_bwd_ws(B, T, dims);
  if (!ws || ws_bytes < need)
    return fail(GDN_ERR_INVALID_VALUE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  if ((uintptr_t)ws % 256) return fail(GDN_ERR_INVALID_VALUE, "workspace must be 256-byte aligned");
  if (C > 0x7fffffff / 5) return fail(GDN_ERR_NOT_SUPPORTED, "too many channels");
  if (Hv > 4096) return fail(GDN_ERR_NOT_SUPPORTED, "prologue backward: more than 4096 value heads");

  gdn::PrologueBwdArgs &p = *P;
  memset(&p, 0, sizeof p);
  p.xq = x_q->data; p.xk = x_k->data; p.xv = x_v->data;
  p.sxq_b = x_q->stride[0]; p.sxq_t = x_q->stride[1];
  p.sxk_b = x_k->stride[0]; p.sxk_t = x_k->stride[1];
  p.sxv_b = x_v->stride[0]; p.sxv_t = x_v->stride[1];
  p.conv_w = conv_w->data; p.w_dtype = conv_w->dtype;
  p.conv_b = conv_b ? conv_b->data : nullptr; p.b_dtype = conv_b ? conv_b->dtype : act;
  p.a = a->data; p.b = b->data;
  p.sa_b = a->stride[0]; p.sa_t = a->stride[1]; p.sb_b = b->stride[0]; p.sb_t = b->stride[1];
  p.A_log = static_cast<const float *>(A_log->data);
  p.dt_bias = static_cast<const float *>(dt_bias->data);
  p.cu_seqlens = cu_seqlens ? static_cast<const int32_t *>(cu_seqlens->data) : nullptr;
  p.n_seqs = n_seqs;
  p.dqkv = d_qkv->data; p.dqkv_dtype = d_qkv->dtype;
  p.d_g = static_cast<const float *>(d_g->data);
  p.d_beta = static_cast<const float *>(d_beta->data);
  p.dxq = dx_q->data; p.dxk = dx_k->data; p.dxv = dx_v->data;
  p.d_conv_w = static_cast<float *>(d_conv_w->data);
  p.d_conv_b = d_conv_b ? static_cast<float *>(d_conv_b->data) : nullptr;
  p.d_a = d_a->data; p.d_b = d_b->data;
  p.d_A_log = static_cast<float *>(d_A_log->data);
  p.d_dt_bias = static_cast<float *>(d_dt_bias->data);
  const ProBwdWs L = prologue_bwd_layout(B, T, dims);
  p.tile_tokens = L.tile;
  p.ntiles = L.ntiles;
  p.head_tile = L.head_tile;
  p.nhtiles = L.nhtiles;
  char *w = static_cast<char *>(ws);
  p.part_w = reinterpret_cast<float *>(w);
  p.part_b = reinterpret_cast<float *>(w + L.w);
  p.part_dt = reinterpret_cast<float *>(w + L.w + L.b);
  p.part_al = reinterpret_cast<float *>(w + L.w + L.b + L.h);
  p.mid = reinterpret_cast<float *>(w + L.w + L.b + 2 * L.h);
  p.B = B; p.T = T; p.Hqk = dims->Hqk; p.dk = dims->dk; p.Hv = Hv; p.dv = dims->dv; p.C = C;
  p.act = act;
  int xa = 16;
  for (const gdn_tensor *x : {x_q, x_k, x_v}) {
    const int r = row_align(x, 2);
    xa = r < xa ? r : xa;
  }
  p.x_align = xa;
  p.dq_align = row_align(d_qkv, 2);
  const int64_t es = elem_size(act), eq = elem_size(d_qkv->dtype);
  int oa = 16;
  for (const gdn_tensor *x : {dx_q, dx_k, dx_v}) {
    const int r = row_align(x, 2);
    oa = r < oa ? r : oa;
  }
  // four channels per thread: the q/k/v segments split at multiples of 4 and
  // every row start is aligned to a 4-element access
  p.vec4 = nq % 4 == 0 && nv % 4 == 0 && xa >= 4 * es && p.dq_align >= 4 * eq && oa >= (4 * es < 16 ? 4 * es : 16);
  p.x_flat = 1;
  for (const gdn_tensor *x : {x_q, x_k, x_v})
    if (B > 1 && x->stride[0] != T * x->stride[1]) p.x_flat = 0;
  return GDN_OK;
}



// Workspace of the two-kernel chunk path: chunk offsets of packed sequences,
// then one record per (chunk, value head). 0 when that path does not apply.
int64_t chunk_bound_of(int64_t B, int64_t T, int64_t n_seqs) {
  const int64_t nc = (T + 63) / 64;
  return n_seqs > 0 ? nc + n_seqs : B * nc;
}
size_t chunk_ws_bytes(int64_t B, int64_t T, int64_t n_seqs, int64_t dk, int64_t Hv, int64_t dv, int32_t act) {
  if (!gdn::chunk_split_supported(dk, dv, act)) return 0;
  const int64_t N = n_seqs > 0 ? n_seqs : B;
  return align256((size_t)(N + 1) * 4) + (size_t)chunk_bound_of(B, T, n_seqs) * (size_t)Hv * (size_t)gdn::kRecBytes;
}

// Attach a caller workspace to a planned chunk call (validated, no launch).
gdn_status attach_chunk_ws(gdn::ChunkArgs *p, void *ws, size_t ws_bytes) {
  p->ws_rec = nullptr;
  p->cu_chunks = nullptr;
  p->chunk_bound = 0;
  if (!ws) return GDN_OK;
  if (!gdn::chunk_split_supported(p->dk, p->dv, p->act) || !p->rows16 || !p->o8) return GDN_OK;  // not used
  const int64_t ns = p->cu_seqlens ? p->n_seqs : 0;
  const size_t need = chunk_ws_bytes(p->B, p->T, ns, p->dk, p->Hv, p->dv, p->act);
  if (ws_bytes < need)
    return fail(GDN_ERR_INVALID_VALUE, "chunk workspace too small: %zu < %zu bytes", ws_bytes, need);
  if ((uintptr_t)ws % 256) return fail(GDN_ERR_INVALID_VALUE, "chunk workspace must be 256-byte aligned");
  char *w = static_cast<char *>(ws);
  p->cu_chunks = reinterpret_cast<int32_t *>(w);
  p->ws_rec = reinterpret_cast<unsigned char *>(w + align256((size_t)(p->n_seqs + 1) * 4));
  p->chunk_bound = chunk_bound_of(p->B, p->T, ns);
  return GDN_OK;
}

// Workspace of the chunk-rule backward (offsets in bytes, each 256-aligned).
struct ChunkBwdWs {
  size_t cu, qn, kn, rq, rk, gam, mm, pp, s0, ds, rr, del, drp, brec, total;
};
ChunkBwdWs chunk_bwd_layout(int64_t B, int64_t T, int64_t n_seqs, const gdn_dims *d) {
  ChunkBwdWs w;
  const size_t N = (size_t)(n_seqs > 0 ? n_seqs : B), cb = (size_t)chunk_bound_of(B, T, n_seqs);
  const size_t Hqk = (size_t)d->Hqk, Hv = (size_t)d->Hv, dk = (size_t)d->dk, dv = (size_t)d->dv;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  w.cu = take((N + 1) * 4);
  w.qn = take(cb * Hqk * 64 * dk * 4);
  w.kn = take(cb * Hqk * 64 * dk * 4);
  w.rq = take(cb * Hqk * 64 * 4);
  w.rk = take(cb * Hqk * 64 * 4);
  w.gam = take(cb * Hv * 64 * 4);
  w.mm = take(cb * Hv * 64 * 64 * 4);
  w.pp = take(cb * Hv * 64 * 64 * 4);
  w.s0 = take(cb * Hv * dv * dk * 4);
  w.ds = take(cb * Hv * dv * dk * 4);
  w.rr = take(cb * Hv * 64 * dv * 4);
  w.del = take(cb * Hv * 64 * dv * 4);
  w.drp = take(cb * Hv * 64 * dv * 4);
  w.brec = take(cb * Hv * (size_t)gdn::kBrBytes);
  w.total = o;
  return w;
}

gdn_status plan_chunk_bwd(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v, const gdn_tensor *g,
                          const gdn_tensor *beta, float scale, int32_t use_l2, float l2_eps,
                          const gdn_tensor *cu_seqlens, const gdn_tensor *initial_state, const gdn_tensor *d_o,
                          const gdn_tensor *d_final, const gdn_tensor *dq, const gdn_tensor *dk,
                          const gdn_tensor *dv, const gdn_tensor *dg, const gdn_tensor *dbeta,
                          const gdn_tensor *d_init, void *ws, size_t ws_bytes, gdn::ChunkBwdArgs *P,
                          bool grad_views = false) {
  // grad_views (the layer backward): dq, dk, dv may be channel views of one
  // [B, T, C] buffer (head stride d, inner stride 1) instead of contiguous
  // tensors; they then share a byte range without sharing an element.
  if (!q || q->ndim != 4) return fail(GDN_ERR_INVALID_VALUE, "q: expected [B, T, Hqk, dk]");
  if (!v || v->ndim != 4) return fail(GDN_ERR_INVALID_VALUE, "v: expected [B, T, Hv, dv]");
  const int64_t B = q->shape[0], T = q->shape[1], Hqk = q->shape[2], dkn = q->shape[3];
  const int64_t Hv = v->shape[2], dvn = v->shape[3];
  if (B * T == 0) return fail(GDN_ERR_INVALID_VALUE, "empty input (B*T == 0)");
  const gdn_dims d = {Hqk, dkn, Hv, dvn};
  TRY(check_dims(&d));
  const int64_t sq[4] = {B, T, Hqk, dkn}, svv[4] = {B, T, Hv, dvn}, sg[3] = {B, T, Hv};
  TRY(check(q, "q", 4, sq));
  const int32_t act = q->dtype;
  if (!is_act(act)) return fail(GDN_ERR_INVALID_VALUE, "q: dtype must be F32, BF16 or F16");
  TRY(check(k, "k", 4, sq));
  TRY(check(v, "v", 4, svv));
  TRY(check(d_o, "d_o", 4, svv));
  TRY(check_dtype(k, "k", act));
  TRY(check_dtype(v, "v", act));
  TRY(check_dtype(d_o, "d_o", act));
  TRY(check_inner(q, "q"));
  TRY(check_inner(k, "k"));
  TRY(check_inner(v, "v"));
  TRY(check_inner(d_o, "d_o"));
  TRY(check(g, "g", 3, sg));
  TRY(check(beta, "beta", 3, sg));
  TRY(check_dtype(g, "g", GDN_F32));
  TRY(check_dtype(beta, "beta", GDN_F32));
  int64_t n_seqs = 0;
  TRY(check_cu(cu_seqlens, B, &n_seqs));
  const int64_t ss[4] = {n_seqs, Hv, dvn, dkn};
  const gdn_tensor *states[] = {initial_state, d_final, d_init};
  const char *snames[] = {"initial_state", "d_final_state", "d_initial_state"};
  for (int i = 0; i < 3; ++i)
    if (states[i]) {
      TRY(check(states[i], snames[i], 4, ss));
      TRY(check_dtype(states[i], snames[i], GDN_F32));
      TRY(check_contig(states[i], snames[i]));
    }
  TRY(check(dq, "dq", 4, sq));
  const int32_t gdt = dq->dtype;
  if (gdt != act && gdt != GDN_F32) return fail(GDN_ERR_INVALID_VALUE, "dq: dtype must be q's or F32");
  TRY(check(dk, "dk", 4, sq));
  TRY(check(dv, "dv", 4, svv));
  TRY(check_dtype(dk, "dk", gdt));
  TRY(check_dtype(dv, "dv", gdt));
  TRY(check(dg, "dg", 3, sg));
  TRY(check(dbeta, "dbeta", 3, sg));
  TRY(check_dtype(dg, "dg", GDN_F32));
  TRY(check_dtype(dbeta, "dbeta", GDN_F32));
  const gdn_tensor *outs[] = {dq, dk, dv, dg, dbeta, d_init};
  const char *onames[] = {"dq", "dk", "dv", "dg", "dbeta", "d_initial_state"};
  for (int i = 0; i < 5; ++i) {
    if (grad_views && i < 3) {
      if (outs[i]->stride[3] != 1 || outs[i]->stride[2] != outs[i]->shape[3])
        return fail(GDN_ERR_INVALID_VALUE, "%s: head stride must be the head dim, inner stride 1", onames[i]);
      continue;
    }
    TRY(check_contig(outs[i], onames[i]));
  }
  if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_VALUE, "scale must be finite");
  if (!(l2_eps >= 0.f) || !std::isfinite(l2_eps)) return fail(GDN_ERR_INVALID_VALUE, "l2_eps must be finite and >= 0");
  if (!gdn::chunk_bwd_supported(dkn, dvn))
    return fail(GDN_ERR_NOT_SUPPORTED,
                "chunk rule backward: dk=%lld dv=%lld is not instantiated (dk 64, 128 or 256; dv a multiple of 16)",
                (long long)dkn, (long long)dvn);
  if (n_seqs > 65535 || Hv > 65535 || Hqk > 65535)
    return fail(GDN_ERR_NOT_SUPPORTED, "chunk rule backward: at most 65535 sequences and heads");
  const int64_t ns = cu_seqlens ? n_seqs : 0;
  const ChunkBwdWs L = chunk_bwd_layout(B, T, ns, &d);
  if (!ws) return fail(GDN_ERR_INVALID_VALUE, "chunk rule backward: a workspace is required");
  if (ws_bytes < L.total)
    return fail(GDN_ERR_INVALID_VALUE, "chunk backward workspace too small: %zu < %zu bytes", ws_bytes, L.total);
  if ((uintptr_t)ws % 256) return fail(GDN_ERR_INVALID_VALUE, "workspace must be 256-byte aligned");
  const gdn_tensor wsd = {ws, GDN_BF16, 1, {(int64_t)(ws_bytes / 2)}, {1}};
  const gdn_tensor *ins[] = {q, k, v, g, beta, cu_seqlens, initial_state, d_o, d_final};
  for (int i = 0; i < 6; ++i) {
    if (!outs[i]) continue;
    for (auto *t : ins)
      if (overlaps(outs[i], t)) return fail(GDN_ERR_INVALID_VALUE, "%s overlaps an input", onames[i]);
    for (int j = i + 1; j < 6; ++j)
      if (!(grad_views && j < 3) && overlaps(outs[i], outs[j]))
        return fail(GDN_ERR_INVALID_VALUE, "%s overlaps %s", onames[i], onames[j]);
    if (overlaps(&wsd, outs[i])) return fail(GDN_ERR_INVALID_VALUE, "workspace overlaps %s", onames[i]);
  }
  for (auto *t : ins)
    if (overlaps(&wsd, t)) return fail(GDN_ERR_INVALID_VALUE, "workspace overlaps an input");

  gdn::ChunkBwdArgs &p = *P;
  memset(&p, 0, sizeof p);
  p.q = q->data; p.k = k->data; p.v = v->data;
  p.sq_b = q->stride[0]; p.sq_t = q->stride[1]; p.sq_h = q->stride[2];
  p.sk_b = k->stride[0]; p.sk_t = k->stride[1]; p.sk_h = k->stride[2];
  p.sv_b = v->stride[0]; p.sv_t = v->stride[1]; p.sv_h = v->stride[2];
  p.g = static_cast<const float *>(g->data);
  p.beta = static_cast<const float *>(beta->data);
  p.sg_b = g->stride[0]; p.sg_t = g->stride[1]; p.sg_h = g->stride[2];
  p.sbt_b = beta->stride[0]; p.sbt_t = beta->stride[1]; p.sbt_h = beta->stride[2];
  p.d_o = d_o->data;
  p.sdo_b = d_o->stride[0]; p.sdo_t = d_o->stride[1]; p.sdo_h = d_o->stride[2];
  p.cu_seqlens = cu_seqlens ? static_cast<const int32_t *>(cu_seqlens->data) : nullptr;
  p.n_seqs = n_seqs;
  p.init_state = initial_state ? static_cast<const float *>(initial_state->data) : nullptr;
  p.d_final = d_final ? static_cast<const float *>(d_final->data) : nullptr;
  p.dqq = dq->data; p.dkk = dk->data; p.dvv = dv->data;
  p.sdq_b = dq->stride[0]; p.sdq_t = dq->stride[1];
  p.sdk_b = dk->stride[0]; p.sdk_t = dk->stride[1];
  p.sdv_b = dv->stride[0]; p.sdv_t = dv->stride[1];
  p.dg = static_cast<float *>(dg->data);
  p.dbeta = static_cast<float *>(dbeta->data);
  p.d_init = d_init ? static_cast<float *>(d_init->data) : nullptr;
  p.B = B; p.T = T; p.Hqk = Hqk; p.dk = dkn; p.Hv = Hv; p.dv = dvn;
  p.act = act; p.grad_dtype = gdt; p.use_l2 = use_l2 ? 1 : 0; p.l2_eps = l2_eps; p.scale = scale;
  char *w = static_cast<char *>(ws);
  auto fp = [&](size_t off) { return reinterpret_cast<float *>(w + off); };
  p.cu_chunks = reinterpret_cast<int32_t *>(w + L.cu);
  p.chunk_bound = chunk_bound_of(B, T, ns);
  p.qn = fp(L.qn); p.kn = fp(L.kn); p.rq = fp(L.rq); p.rk = fp(L.rk); p.gam = fp(L.gam);
  p.mm = fp(L.mm); p.pp = fp(L.pp); p.s0 = fp(L.s0); p.ds = fp(L.ds);
  p.rr = fp(L.rr); p.del = fp(L.del); p.drp = fp(L.drp);
  p.brec = reinterpret_cast<unsigned char *>(w + L.brec);
  return GDN_OK;
}

// Workspace of the layer backward (byte offsets, each 256-aligned): the
// recomputed forward stage outputs, the chunk forward's workspace, d_o and the
// gated-norm backward's partials, d_qkv (activation dtype) with dg and dbeta, then the
// chunk-rule and prologue backward workspaces.
struct LayerBwdWs {
  size_t qkv, g, beta, o, cfw, d_o, nbw, dqkv, dg, dbeta, cbw, pbw, total;
  size_t cfw_n, nbw_n, cbw_n, pbw_n;
};
LayerBwdWs layer_bwd_layout(int64_t B, int64_t T, int64_t n_seqs, const gdn_dims *d, int32_t act) {
  LayerBwdWs w;
  const size_t n = (size_t)(B * T), es = (size_t)elem_size(act);
  const size_t C = (size_t)(2 * d->Hqk * d->dk + d->Hv * d->dv), Hv = (size_t)d->Hv, HD = (size_t)(d->Hv * d->dv);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  w.cfw_n = chunk_ws_bytes(B, T, n_seqs, d->dk, d->Hv, d->dv, act);
  w.nbw_n = (size_t)align256((size_t)norm_bwd_blocks(B * T * d->Hv, d->dv) * (size_t)d->dv * 4) +
            align256((size_t)32 * d->dv * 4);
  w.cbw_n = chunk_bwd_layout(B, T, n_seqs, d).total;
  w.pbw_n = prologue_bwd_ws(B, T, d);
  w.qkv = take(n * C * es);
  w.g = take(n * Hv * 4);
  w.beta = take(n * Hv * 4);
  w.o = take(n * HD * es);
  w.cfw = take(w.cfw_n);
  w.d_o = take(n * HD * es);
  w.nbw = take(w.nbw_n);
  w.dqkv = take(n * C * es);
  w.dg = take(n * Hv * 4);
  w.dbeta = take(n * Hv * 4);
  w.cbw = take(w.cbw_n);
  w.pbw = take(w.pbw_n);
  w.total = o;
  return w;
}

// The layer backward; with recompute false the workspace already holds the
// forward stage outputs (qkv, g, beta, o) that gdn_layer_fwd wrote at the
// same offsets, and the prologue and chunk rule are planned (validated) but
// not launched.
gdn_status layer_bwd(const gdn_tensor *x_q, const gdn_tensor *x_k, const gdn_tensor *x_v,
                     const gdn_tensor *conv_w, const gdn_tensor *conv_b, const gdn_tensor *a, const gdn_tensor *b,
                     const gdn_tensor *A_log, const gdn_tensor *dt_bias, const gdn_tensor *gate,
                     const gdn_tensor *norm_w, const gdn_tensor *cu_seqlens, const gdn_dims *dims, float scale,
                     int32_t use_qk_l2norm_in_kernel, float l2_eps, float rms_eps, const gdn_tensor *d_out,
                     const gdn_tensor *dx_q, const gdn_tensor *dx_k, const gdn_tensor *dx_v,
                     const gdn_tensor *d_conv_w, const gdn_tensor *d_conv_b, const gdn_tensor *d_a,
                     const gdn_tensor *d_b, const gdn_tensor *d_A_log, const gdn_tensor *d_dt_bias,
                     const gdn_tensor *d_gate, const gdn_tensor *d_norm_w, void *workspace, size_t workspace_bytes,
                     void *stream, bool recompute) {
  g_error.clear();
  TRY(check_dims(dims));
  if (!x_q || x_q->ndim != 3) return fail(GDN_ERR_INVALID_VALUE, "x_q: expected [B, T, Hqk*dk]");
  const int64_t B = x_q->shape[0], T = x_q->shape[1];
  const int32_t act = x_q->dtype;
  if (!is_act(act)) return fail(GDN_ERR_INVALID_VALUE, "x_q: dtype must be F32, BF16 or F16");
  if (B * T == 0) return fail(GDN_ERR_INVALID_VALUE, "empty input (B*T == 0)");
  int64_t n_seqs = 0;
  if (cu_seqlens) {
    if (cu_seqlens->ndim != 1 || cu_seqlens->shape[0] < 1)
      return fail(GDN_ERR_INVALID_VALUE, "cu_seqlens: expected [N+1]");
    n_seqs = cu_seqlens->shape[0] - 1;
  }
  if (!gdn::chunk_bwd_supported(dims->dk, dims->dv))
    return fail(GDN_ERR_NOT_SUPPORTED, "layer backward: dk=%lld dv=%lld is not instantiated", (long long)dims->dk,
                (long long)dims->dv);
  const LayerBwdWs L = layer_bwd_layout(B, T, n_seqs, dims, act);
  if (!workspace) return fail(GDN_ERR_INVALID_VALUE, "workspace is NULL");
  if (workspace_bytes < L.total)
    return fail(GDN_ERR_INVALID_VALUE, "workspace too small: %zu < %zu bytes", workspace_bytes, L.total);
  if ((uintptr_t)workspace % 256) return fail(GDN_ERR_INVALID_VALUE, "workspace must be 256-byte aligned");

  const int64_t Hqk = dims->Hqk, dk = dims->dk, Hv = dims->Hv, dv = dims->dv;
  const int64_t nq = Hqk * dk, C = 2 * nq + Hv * dv, es = elem_size(act);
  char *w = static_cast<char *>(workspace);
  gdn_tensor qkv = {w + L.qkv, act, 3, {B, T, C}, {T * C, C, 1}};
  gdn_tensor gt = {w + L.g, GDN_F32, 3, {B, T, Hv}, {T * Hv, Hv, 1}};
  gdn_tensor bt = {w + L.beta, GDN_F32, 3, {B, T, Hv}, {T * Hv, Hv, 1}};
  gdn_tensor ot = {w + L.o, act, 4, {B, T, Hv, dv}, {T * Hv * dv, Hv * dv, dv, 1}};
  gdn_tensor dot = {w + L.d_o, act, 4, {B, T, Hv, dv}, {T * Hv * dv, Hv * dv, dv, 1}};
  gdn_tensor dqkv = {w + L.dqkv, act, 3, {B, T, C}, {T * C, C, 1}};
  gdn_tensor dgt = {w + L.dg, GDN_F32, 3, {B, T, Hv}, {T * Hv, Hv, 1}};
  gdn_tensor dbt = {w + L.dbeta, GDN_F32, 3, {B, T, Hv}, {T * Hv, Hv, 1}};
  char *qb = w + L.qkv, *db = w + L.dqkv;
  gdn_tensor qv = {qb, act, 4, {B, T, Hqk, dk}, {T * C, C, dk, 1}};
  gdn_tensor kv = {qb + nq * es, act, 4, {B, T, Hqk, dk}, {T * C, C, dk, 1}};
  gdn_tensor vv = {qb + 2 * nq * es, act, 4, {B, T, Hv, dv}, {T * C, C, dv, 1}};
  gdn_tensor dqv = {db, act, 4, {B, T, Hqk, dk}, {T * C, C, dk, 1}};
  gdn_tensor dkv = {db + nq * es, act, 4, {B, T, Hqk, dk}, {T * C, C, dk, 1}};
  gdn_tensor dvv = {db + 2 * nq * es, act, 4, {B, T, Hv, dv}, {T * C, C, dv, 1}};
  gdn_tensor wsd = {workspace, GDN_BF16, 1, {(int64_t)(L.total / 2)}, {1}};

  // Plan every stage before launching anything.
  gdn::PrologueArgs PP;
  gdn::ChunkArgs PC;
  gdn::NormBwdArgs PN;
  gdn::ChunkBwdArgs PB;
  gdn::PrologueBwdArgs PR;
  TRY(plan_prologue(x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, cu_seqlens, dims, 0, l2_eps, &qkv, &gt,
                    &bt, &PP));
  TRY(plan_chunk(&qv, &kv, &vv, &gt, &bt, scale, use_qk_l2norm_in_kernel, l2_eps, cu_seqlens, nullptr, &ot,
                 nullptr, &PC));
  TRY(attach_chunk_ws(&PC, L.cfw_n ? w + L.cfw : nullptr, L.cfw_n));
  TRY(plan_norm_bwd(&ot, gate, norm_w, rms_eps, d_out, &dot, d_gate, d_norm_w, w + L.nbw, L.nbw_n, &PN));
  TRY(plan_chunk_bwd(&qv, &kv, &vv, &gt, &bt, scale, use_qk_l2norm_in_kernel, l2_eps, cu_seqlens, nullptr, &dot,
                     nullptr, &dqv, &dkv, &dvv, &dgt, &dbt, nullptr, w + L.cbw, L.cbw_n, &PB, true));
  TRY(plan_prologue_bwd(x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, cu_seqlens, dims, &dqkv, &dgt, &dbt,
                        dx_q, dx_k, dx_v, d_conv_w, d_conv_b, d_a, d_b, d_A_log, d_dt_bias, w + L.pbw, L.pbw_n,
                        &PR));
  const gdn_tensor *ins[] = {x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, gate, norm_w, cu_seqlens, d_out};
  const gdn_tensor *outs[] = {dx_q, dx_k, dx_v, d_conv_w, d_conv_b, d_a, d_b, d_A_log, d_dt_bias, d_gate, d_norm_w};
  for (auto *t : ins)
    if (overlaps(&wsd, t)) return fail(GDN_ERR_INVALID_VALUE, "workspace overlaps an input");
  for (size_t i = 0; i < sizeof outs / sizeof outs[0]; ++i) {
    if (overlaps(&wsd, outs[i])) return fail(GDN_ERR_INVALID_VALUE, "workspace overlaps an output");
    for (auto *t : ins)
      if (overlaps(outs[i], t)) return fail(GDN_ERR_INVALID_VALUE, "an output overlaps an input");
    for (size_t j = i + 1; j < sizeof outs / sizeof outs[0]; ++j)
      if (overlaps(outs[i], outs[j])) return fail(GDN_ERR_INVALID_VALUE, "two outputs overlap");
  }

  hipStream_t s = (hipStream_t)stream;
  if (recompute) {
    TRY(launched(gdn::launch_prologue(PP, s), "prologue"));
    TRY(launched(gdn::launch_chunk_rule(PC, s), "chunk rule"));
  }
  TRY(launched(gdn::launch_gated_norm_bwd(PN, s), "gated norm backward"));
  TRY(launched(gdn::launch_chunk_bwd(PB, s), "chunk rule backward"));
  return launched(gdn::launch_prologue_bwd(PR, s), "prologue backward");
}

}  // namespace

extern "C" {

const char *gdn_last_error(void) { return g_error.c_str(); }

const char *gdn_version(void) { return "gdn-mi355x 0.1.0 (gfx950)"; }

gdn_status gdn_prologue_fwd(const gdn_tensor *x_q, const gdn_tensor *x_k, const gdn_tensor *x_v,
                            const gdn_tensor *conv_w, const gdn_tensor *conv_b, const gdn_tensor *a,
                            const gdn_tensor *b, const gdn_tensor *A_log, const gdn_tensor *dt_bias,
                            const gdn_tensor *cu_seqlens, const gdn_dims *dims, int32_t caller_l2norm,
                            float l2_eps, const gdn_tensor *out_qkv, const gdn_tensor *out_g,
                            const gdn_tensor *out_beta, void *stream) {
  g_error.clear();
  gdn::PrologueArgs P;
  TRY(plan_prologue(x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, cu_seqlens, dims, caller_l2norm,
                    l2_eps, out_qkv, out_g, out_beta, &P));
  return launched(gdn::launch_prologue(P, (hipStream_t)stream), "prologue");
}

gdn_status gdn_chunk_rule_fwd(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v,
                              const gdn_tensor *g, const gdn_tensor *beta, float scale,
                              int32_t use_qk_l2norm_in_kernel, float l2_eps, const gdn_tensor *cu_seqlens,
                              const gdn_tensor *initial_state, const gdn_tensor *out_o,
                              const gdn_tensor *final_state, void *workspace, size_t workspace_bytes,
                              void *stream) {
  g_error.clear();
  gdn::ChunkArgs P;
  TRY(plan_chunk(q, k, v, g, beta, scale, use_qk_l2norm_in_kernel, l2_eps, cu_seqlens, initial_state, out_o,
                 final_state, &P));
  TRY(attach_chunk_ws(&P, workspace, workspace_bytes));
  if (P.ws_rec) {
    const gdn_tensor wsd = {workspace, GDN_BF16, 1, {(int64_t)(workspace_bytes / 2)}, {1}};
    const gdn_tensor *all[] = {q, k, v, g, beta, cu_seqlens, initial_state, out_o, final_state};
    for (auto *t : all)
      if (overlaps(&wsd, t)) return fail(GDN_ERR_INVALID_VALUE, "workspace overlaps a tensor argument");
  }
  return launched(gdn::launch_chunk_rule(P, (hipStream_t)stream), "chunk rule");
}

gdn_status gdn_chunk_rule_fwd_noalloc(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v,
                                      const gdn_tensor *g, const gdn_tensor *beta, float scale,
                                      int32_t use_qk_l2norm_in_kernel, float l2_eps,
                                      const gdn_tensor *cu_seqlens, const gdn_tensor *initial_state,
                                      const gdn_tensor *out_o, const gdn_tensor *final_state, void *stream) {
  g_error.clear();
  gdn::ChunkArgs P;
  TRY(plan_chunk(q, k, v, g, beta, scale, use_qk_l2norm_in_kernel, l2_eps, cu_seqlens, initial_state, out_o,
                 final_state, &P));
  const int64_t ns = P.cu_seqlens ? P.n_seqs : 0;
  const size_t need = chunk_ws_bytes(P.B, P.T, ns, P.dk, P.Hv, P.dv, P.act);
  if (need > 0 && P.rows16 && P.o8) {  // the two-kernel path applies: records in the static scratch
    if (need > GDN_NOALLOC_SCRATCH_BYTES)
      return fail(GDN_ERR_INVALID_VALUE,
                  "chunk records need %zu bytes, more than the %zu bytes of static scratch; split the "
                  "sequence (initial_state / final_state) or call gdn_chunk_rule_fwd with a workspace",
                  need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
    void *scr = nullptr;
    const hipError_t e = gdn::static_scratch(&scr);
    if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "static scratch: %s", hipGetErrorString(e));
    TRY(attach_chunk_ws(&P, scr, (size_t)GDN_NOALLOC_SCRATCH_BYTES));
  }
  return launched(gdn::launch_chunk_rule(P, (hipStream_t)stream), "chunk rule");
}

size_t gdn_chunk_rule_workspace_bytes(int64_t B, int64_t T, int64_t n_seqs, const gdn_dims *dims,
                                      int32_t act_dtype) {
  if (!dims || B < 0 || T < 0 || n_seqs < 0 || !is_act(act_dtype)) return 0;
  if (dims->Hqk <= 0 || dims->dk <= 0 || dims->Hv <= 0 || dims->dv <= 0) return 0;
  return chunk_ws_bytes(B, T, n_seqs, dims->dk, dims->Hv, dims->dv, act_dtype);
}

gdn_status gdn_gated_norm_fwd(const gdn_tensor *o, const gdn_tensor *gate, const gdn_tensor *weight, float eps,
                              const gdn_tensor *out, void *stream) {
  g_error.clear();
  gdn::NormArgs P;
  TRY(plan_norm(o, gate, weight, eps, out, &P));
  return launched(gdn::launch_gated_norm(P, (hipStream_t)stream), "gated norm");
}

gdn_status gdn_decode_fwd(const gdn_tensor *x_q, const gdn_tensor *x_k, const gdn_tensor *x_v,
                          const gdn_tensor *conv_w, const gdn_tensor *conv_b, const gdn_tensor *conv_state,
                          const gdn_tensor *a, const gdn_tensor *b, const gdn_tensor *A_log,
                          const gdn_tensor *dt_bias, const gdn_tensor *state, const gdn_dims *dims, float scale,
                          int32_t use_qk_l2norm_in_kernel, float l2_eps, const gdn_tensor *gate,
                          const gdn_tensor *norm_w, float rms_eps, const gdn_tensor *out, void *stream) {
  g_error.clear();
  gdn::DecodeArgs p;
  TRY(plan_decode(x_q, x_k, x_v, conv_w, conv_b, conv_state, a, b, A_log, dt_bias, state, gate, norm_w, dims,
                  scale, use_qk_l2norm_in_kernel, l2_eps, rms_eps, out, &p));
  return launched(gdn::launch_decode(p, static_cast<hipStream_t>(stream)), "decode");
}

size_t gdn_gated_norm_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dv) {
  if (B < 0 || T < 0 || H < 0 || dv < 64 || dv > 512 || !pow2(dv)) return 0;
  return align256((size_t)norm_bwd_blocks(B * T * H, dv) * (size_t)dv * 4) + align256((size_t)32 * dv * 4);
}

gdn_status gdn_gated_norm_bwd(const gdn_tensor *o, const gdn_tensor *gate, const gdn_tensor *weight, float eps,
                              const gdn_tensor *dout, const gdn_tensor *d_o, const gdn_tensor *d_gate,
                              const gdn_tensor *d_weight, void *workspace, size_t workspace_bytes, void *stream) {
  g_error.clear();
  gdn::NormBwdArgs p;
  TRY(plan_norm_bwd(o, gate, weight, eps, dout, d_o, d_gate, d_weight, workspace, workspace_bytes, &p));
  return launched(gdn::launch_gated_norm_bwd(p, static_cast<hipStream_t>(stream)), "gated norm backward");
}

size_t gdn_prologue_bwd_workspace_bytes(int64_t B, int64_t T, const gdn_dims *dims) {
  if (!dims || B < 0 || T < 0 || dims->Hqk <= 0 || dims->dk <= 0 || dims->Hv <= 0 || dims->dv <= 0) return 0;
  return prologue_bwd_ws(B, T, dims);
}

gdn_status gdn_prologue_bwd(const gdn_tensor *x_q, const gdn_tensor *x_k, const gdn_tensor *x_v,
                            const gdn_tensor *conv_w, const gdn_tensor *conv_b, const gdn_tensor *a,
                            const gdn_tensor *b, const gdn_tensor *A_log, const gdn_tensor *dt_bias,
                            const gdn_tensor *cu_seqlens, const gdn_dims *dims, const gdn_tensor *d_qkv,
                            const gdn_tensor *d_g, const gdn_tensor *d_beta, const gdn_tensor *dx_q,
                            const gdn_tensor *dx_k, const gdn_tensor *dx_v, const gdn_tensor *d_conv_w,
                            const gdn_tensor *d_conv_b, const gdn_tensor *d_a, const gdn_tensor *d_b,
                            const gdn_tensor *d_A_log, const gdn_tensor *d_dt_bias, void *workspace,
                            size_t workspace_bytes, void *stream) {
  g_error.clear();
  gdn::PrologueBwdArgs p;
  TRY(plan_prologue_bwd(x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, cu_seqlens, dims, d_qkv, d_g, d_beta,
                        dx_q, dx_k, dx_v, d_conv_w, d_conv_b, d_a, d_b, d_A_log, d_dt_bias, workspace,
                        workspace_bytes, &p));
  return launched(gdn::launch_prologue_bwd(p, static_cast<hipStream_t>(stream)), "prologue backward");
}

size_t gdn_chunk_rule_bwd_workspace_bytes(int64_t B, int64_t T, int64_t n_seqs, const gdn_dims *dims) {
  if (!dims || B <= 0 || T <= 0 || n_seqs < 0) return 0;
  if (dims->Hqk <= 0 || dims->dk <= 0 || dims->Hv <= 0 || dims->dv <= 0) return 0;
  if (!gdn::chunk_bwd_supported(dims->dk, dims->dv)) return 0;
  return chunk_bwd_layout(B, T, n_seqs, dims).total;
}

gdn_status gdn_chunk_rule_bwd(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v, const gdn_tensor *g,
                              const gdn_tensor *beta, float scale, int32_t use_qk_l2norm_in_kernel, float l2_eps,
                              const gdn_tensor *cu_seqlens, const gdn_tensor *initial_state,
                              const gdn_tensor *d_o, const gdn_tensor *d_final_state, const gdn_tensor *dq,
                              const gdn_tensor *dk, const gdn_tensor *dv, const gdn_tensor *dg,
                              const gdn_tensor *dbeta, const gdn_tensor *d_initial_state, void *workspace,
                              size_t workspace_bytes, void *stream) {
  g_error.clear();
  gdn::ChunkBwdArgs P;
  TRY(plan_chunk_bwd(q, k, v, g, beta, scale, use_qk_l2norm_in_kernel, l2_eps, cu_seqlens, initial_state, d_o,
                     d_final_state, dq, dk, dv, dg, dbeta, d_initial_state, workspace, workspace_bytes, &P));
  return launched(gdn::launch_chunk_bwd(P, (hipStream_t)stream), "chunk rule backward");
}

size_t gdn_layer_bwd_workspace_bytes(int64_t B, int64_t T, int64_t n_seqs, const gdn_dims *dims,
                                     int32_t act_dtype) {
  if (!dims || B <= 0 || T <= 0 || n_seqs < 0 || !is_act(act_dtype)) return 0;
  if (dims->Hqk <= 0 || dims->dk <= 0 || dims->Hv <= 0 || dims->dv < 64 || dims->dv > 512 || !pow2(dims->dv))
    return 0;
  if (!gdn::chunk_bwd_supported(dims->dk, dims->dv)) return 0;
  return layer_bwd_layout(B, T, n_seqs, dims, act_dtype).total;
}

gdn_status gdn_layer_bwd(const gdn_tensor *x_q, const gdn_tensor *x_k, const gdn_tensor *x_v,
                         const gdn_tensor *conv_w, const gdn_tensor *conv_b, const gdn_tensor *a,
                         const gdn_tensor *b, const gdn_tensor *A_log, const gdn_tensor *dt_bias,
                         const gdn_tensor *gate, const gdn_tensor *norm_w, const gdn_tensor *cu_seqlens,
                         const gdn_dims *dims, float scale, int32_t use_qk_l2norm_in_kernel, float l2_eps,
                         float rms_eps, const gdn_tensor *d_out, const gdn_tensor *dx_q, const gdn_tensor *dx_k,
                         const gdn_tensor *dx_v, const gdn_tensor *d_conv_w, const gdn_tensor *d_conv_b,
                         const gdn_tensor *d_a, const gdn_tensor *d_b, const gdn_tensor *d_A_log,
                         const gdn_tensor *d_dt_bias, const gdn_tensor *d_gate, const gdn_tensor *d_norm_w,
                         void *workspace, size_t workspace_bytes, void *stream) {
  return layer_bwd(x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, gate, norm_w, cu_seqlens, dims, scale,
                   use_qk_l2norm_in_kernel, l2_eps, rms_eps, d_out, dx_q, dx_k, dx_v, d_conv_w, d_conv_b, d_a, d_b,
                   d_A_log, d_dt_bias, d_gate, d_norm_w, workspace, workspace_bytes, stream, true);
}

gdn_status gdn_layer_bwd_saved(const gdn_tensor *x_q, const gdn_tensor *x_k, const gdn_tensor *x_v,
                               const gdn_tensor *conv_w, const gdn_tensor *conv_b, const gdn_tensor *a,
                               const gdn_tensor *b, const gdn_tensor *A_log, const gdn_tensor *dt_bias,
                               const gdn_tensor *gate, const gdn_tensor *norm_w, const gdn_tensor *cu_seqlens,
                               const gdn_dims *dims, float scale, int32_t use_qk_l2norm_in_kernel, float l2_eps,
                               float rms_eps, const gdn_tensor *d_out, const gdn_tensor *dx_q,
                               const gdn_tensor *dx_k, const gdn_tensor *dx_v, const gdn_tensor *d_conv_w,
                               const gdn_tensor *d_conv_b, const gdn_tensor *d_a, const gdn_tensor *d_b,
                               const gdn_tensor *d_A_log, const gdn_tensor *d_dt_bias, const gdn_tensor *d_gate,
                               const gdn_tensor *d_norm_w, void *workspace, size_t workspace_bytes,
                               void *stream) {
  return layer_bwd(x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, gate, norm_w, cu_seqlens, dims, scale,
                   use_qk_l2norm_in_kernel, l2_eps, rms_eps, d_out, dx_q, dx_k, dx_v, d_conv_w, d_conv_b, d_a, d_b,
                   d_A_log, d_dt_bias, d_gate, d_norm_w, workspace, workspace_bytes, stream, false);
}

size_t gdn_layer_workspace_bytes(int64_t B, int64_t T, int64_t n_seqs, const gdn_dims *dims,
                                 int32_t act_dtype) {
  if (!dims || B < 0 || T < 0 || n_seqs < 0 || !is_act(act_dtype)) return 0;
  if (dims->Hqk <= 0 || dims->dk <= 0 || dims->Hv <= 0 || dims->dv <= 0) return 0;
  const size_t es = (size_t)elem_size(act_dtype), n = (size_t)(B * T);
  const size_t C = (size_t)(2 * dims->Hqk * dims->dk + dims->Hv * dims->dv);
  return align256(n * C * es) + 2 * align256(n * (size_t)dims->Hv * 4) +
         align256(n * (size_t)(dims->Hv * dims->dv) * es) +
         chunk_ws_bytes(B, T, n_seqs, dims->dk, dims->Hv, dims->dv, act_dtype);
}

gdn_status gdn_layer_fwd(const gdn_tensor *x_q, const gdn_tensor *x_k, const gdn_tensor *x_v,
                         const gdn_tensor *conv_w, const gdn_tensor *conv_b, const gdn_tensor *a,
                         const gdn_tensor *b, const gdn_tensor *A_log, const gdn_tensor *dt_bias,
                         const gdn_tensor *gate, const gdn_tensor *norm_w, const gdn_tensor *cu_seqlens,
                         const gdn_dims *dims, float scale, int32_t use_qk_l2norm_in_kernel, float l2_eps,
                         float rms_eps, void *workspace, size_t workspace_bytes, const gdn_tensor *out,
                         void *stream) {
  g_error.clear();
  TRY(check_dims(dims));
  if (!x_q || x_q->ndim != 3) return fail(GDN_ERR_INVALID_VALUE, "x_q: expected [B, T, Hqk*dk]");
  const int64_t B = x_q->shape[0], T = x_q->shape[1];
  const int32_t act = x_q->dtype;
  if (!is_act(act)) return fail(GDN_ERR_INVALID_VALUE, "x_q: dtype must be F32, BF16 or F16");
  int64_t n_seqs = 0;
  if (cu_seqlens) {
    if (cu_seqlens->ndim != 1 || cu_seqlens->shape[0] < 1)
      return fail(GDN_ERR_INVALID_VALUE, "cu_seqlens: expected [N+1]");
    n_seqs = cu_seqlens->shape[0] - 1;
  }
  const size_t need = gdn_layer_workspace_bytes(B, T, n_seqs, dims, act);
  if (!workspace) return fail(GDN_ERR_INVALID_VALUE, "workspace is NULL");
  if (workspace_bytes < need)
    return fail(GDN_ERR_INVALID_VALUE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
  if ((uintptr_t)workspace % 256) return fail(GDN_ERR_INVALID_VALUE, "workspace must be 256-byte aligned");

  const int64_t Hqk = dims->Hqk, dk = dims->dk, Hv = dims->Hv, dv = dims->dv;
  const int64_t nq = Hqk * dk, C = 2 * nq + Hv * dv, es = elem_size(act);
  char *ws = static_cast<char *>(workspace);
  const size_t n = (size_t)(B * T);
  gdn_tensor qkv = {ws, act, 3, {B, T, C}, {T * C, C, 1}};
  ws += align256(n * (size_t)C * (size_t)es);
  gdn_tensor gt = {ws, GDN_F32, 3, {B, T, Hv}, {T * Hv, Hv, 1}};
  ws += align256(n * (size_t)Hv * 4);
  gdn_tensor bt = {ws, GDN_F32, 3, {B, T, Hv}, {T * Hv, Hv, 1}};
  ws += align256(n * (size_t)Hv * 4);
  gdn_tensor ot = {ws, act, 4, {B, T, Hv, dv}, {T * Hv * dv, Hv * dv, dv, 1}};
  ws += align256(n * (size_t)(Hv * dv) * (size_t)es);
  const size_t chunk_ws = chunk_ws_bytes(B, T, n_seqs, dk, Hv, dv, act);
  char *qkv_base = static_cast<char *>(qkv.data);
  gdn_tensor qv = {qkv_base, act, 4, {B, T, Hqk, dk}, {T * C, C, dk, 1}};
  gdn_tensor kv = {qkv_base + nq * es, act, 4, {B, T, Hqk, dk}, {T * C, C, dk, 1}};
  gdn_tensor vv = {qkv_base + 2 * nq * es, act, 4, {B, T, Hv, dv}, {T * C, C, dv, 1}};
  gdn_tensor wsd = {workspace, GDN_BF16, 1, {(int64_t)(need / 2)}, {1}};

  // Plan all three stages before launching anything.
  gdn::PrologueArgs PP;
  gdn::ChunkArgs PC;
  gdn::NormArgs PN;
  TRY(plan_prologue(x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, cu_seqlens, dims, 0, l2_eps, &qkv, &gt,
                    &bt, &PP));
  TRY(plan_chunk(&qv, &kv, &vv, &gt, &bt, scale, use_qk_l2norm_in_kernel, l2_eps, cu_seqlens, nullptr, &ot,
                 nullptr, &PC));
  TRY(attach_chunk_ws(&PC, chunk_ws ? ws : nullptr, chunk_ws));
  TRY(plan_norm(&ot, gate, norm_w, rms_eps, out, &PN));
  if (out->dtype != act) return fail(GDN_ERR_INVALID_VALUE, "out: dtype must be the activation dtype");
  const gdn_tensor *ins[] = {x_q, x_k, x_v, conv_w, conv_b, a, b, A_log, dt_bias, gate, norm_w, cu_seqlens};
  for (auto *i : ins)
    if (overlaps(&wsd, i)) return fail(GDN_ERR_INVALID_VALUE, "workspace overlaps an input");
  if (overlaps(&wsd, out)) return fail(GDN_ERR_INVALID_VALUE, "workspace overlaps out");
  for (auto *i : ins)
    if (overlaps(out, i)) return fail(GDN_ERR_INVALID_VALUE, "out overlaps an input");

  hipStream_t s = (hipStream_t)stream;
  TRY(launched(gdn::launch_prologue(PP, s), "prologue"));
  TRY(launched(gdn::launch_chunk_rule(PC, s), "chunk rule"));
  return launched(gdn::launch_gated_norm(PN, s), "gated norm");
}

}  // extern "C"
