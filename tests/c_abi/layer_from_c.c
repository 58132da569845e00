/*
 * Drives the C ABI of libgdn.so from C with the HIP runtime alone (no Python,
 * no PyTorch): reads a little-endian input file, copies the tensors to device
 * memory, runs gdn_layer_fwd (BF16, dense, caller workspace) and
 * gdn_decode_fwd on the first token, and writes the outputs back to a file.
 *
 * usage: layer_from_c <input.bin> <output.bin>
 * input:  int64 B, T, Hqk, dk, Hv, dv; float scale; then, as raw bfloat16
 *         bits: x_q [B,T,Hqk*dk], x_k, x_v [B,T,Hv*dv], conv_w [C,4],
 *         a, b [B,T,Hv], gate [B,T,Hv,dv], norm_w [dv]; then float32 A_log,
 *         dt_bias [Hv]
 * output: out [B,T,Hv,dv] bfloat16 bits, then the decode output of token 0
 *         [B,Hv,dv] bfloat16 bits and the state after it [B,Hv,dv,dk] float32
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gdn.h"

#define HIPCHECK(x)                                                        \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "%s:%d %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      exit(2);                                                             \
    }                                                                      \
  } while (0)
#define GDNCHECK(x)                                                        \
  do {                                                                     \
    gdn_status s_ = (x);                                                   \
    if (s_ != GDN_OK) {                                                    \
      fprintf(stderr, "gdn status %d: %s\n", (int)s_, gdn_last_error());  \
      exit(3);                                                             \
    }                                                                      \
  } while (0)

static void *dev_from(FILE *f, size_t bytes) {
  void *h = malloc(bytes), *d = NULL;
  if (!h || fread(h, 1, bytes, f) != bytes) {
    fprintf(stderr, "short input\n");
    exit(4);
  }
  HIPCHECK(hipMalloc(&d, bytes ? bytes : 1));
  HIPCHECK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  free(h);
  return d;
}

static gdn_tensor desc(void *p, int32_t dt, int nd, const int64_t *shape) {
  gdn_tensor t;
  memset(&t, 0, sizeof t);
  t.data = p;
  t.dtype = dt;
  t.ndim = nd;
  int64_t st = 1;
  for (int i = nd - 1; i >= 0; --i) {
    t.shape[i] = shape[i];
    t.stride[i] = st;
    st *= shape[i];
  }
  return t;
}

int main(int argc, char **argv) {
  if (argc != 3) return 1;
  FILE *f = fopen(argv[1], "rb");
  if (!f) return 1;
  int64_t hdr[6];
  float scale;
  if (fread(hdr, 8, 6, f) != 6 || fread(&scale, 4, 1, f) != 1) return 4;
  const int64_t B = hdr[0], T = hdr[1], Hqk = hdr[2], dk = hdr[3], Hv = hdr[4], dv = hdr[5];
  const int64_t nq = Hqk * dk, nv = Hv * dv, C = 2 * nq + nv;
  void *xq = dev_from(f, (size_t)(B * T * nq * 2)), *xk = dev_from(f, (size_t)(B * T * nq * 2));
  void *xv = dev_from(f, (size_t)(B * T * nv * 2)), *w = dev_from(f, (size_t)(C * 4 * 2));
  void *a = dev_from(f, (size_t)(B * T * Hv * 2)), *b = dev_from(f, (size_t)(B * T * Hv * 2));
  void *gate = dev_from(f, (size_t)(B * T * nv * 2)), *nw = dev_from(f, (size_t)(dv * 2));
  void *alog = dev_from(f, (size_t)(Hv * 4)), *dtb = dev_from(f, (size_t)(Hv * 4));
  fclose(f);

  const int64_t s_q[3] = {B, T, nq}, s_v[3] = {B, T, nv}, s_w[2] = {C, 4}, s_ab[3] = {B, T, Hv};
  const int64_t s_g[4] = {B, T, Hv, dv}, s_n[1] = {dv}, s_h[1] = {Hv};
  gdn_tensor tq = desc(xq, GDN_BF16, 3, s_q), tk = desc(xk, GDN_BF16, 3, s_q), tv = desc(xv, GDN_BF16, 3, s_v);
  gdn_tensor tw = desc(w, GDN_BF16, 2, s_w), ta = desc(a, GDN_BF16, 3, s_ab), tb = desc(b, GDN_BF16, 3, s_ab);
  gdn_tensor tg = desc(gate, GDN_BF16, 4, s_g), tn = desc(nw, GDN_BF16, 1, s_n);
  gdn_tensor tal = desc(alog, GDN_F32, 1, s_h), tdt = desc(dtb, GDN_F32, 1, s_h);
  gdn_dims dims = {Hqk, dk, Hv, dv};

  hipStream_t stream;
  HIPCHECK(hipStreamCreate(&stream));
  const size_t wsb = gdn_layer_workspace_bytes(B, T, 0, &dims, GDN_BF16);
  void *ws = NULL, *out = NULL;
  HIPCHECK(hipMalloc(&ws, wsb));
  HIPCHECK(hipMalloc(&out, (size_t)(B * T * nv * 2)));
  gdn_tensor to = desc(out, GDN_BF16, 4, s_g);
  GDNCHECK(gdn_layer_fwd(&tq, &tk, &tv, &tw, NULL, &ta, &tb, &tal, &tdt, &tg, &tn, NULL, &dims, scale, 1, 1e-6f,
                         1e-5f, ws, wsb, &to, stream));

  /* decode of token 0 of every row from a zero cache and state: token 0's
     rows are views with row stride T * width */
  gdn_tensor dq, dkk, dvv, da, db, dg;
  const int64_t sq2[2] = {B, nq}, sv2[2] = {B, nv}, sab2[2] = {B, Hv}, sg3[3] = {B, Hv, dv};
  dq = desc(xq, GDN_BF16, 2, sq2); dq.stride[0] = T * nq;
  dkk = desc(xk, GDN_BF16, 2, sq2); dkk.stride[0] = T * nq;
  dvv = desc(xv, GDN_BF16, 2, sv2); dvv.stride[0] = T * nv;
  da = desc(a, GDN_BF16, 2, sab2); da.stride[0] = T * Hv;
  db = desc(b, GDN_BF16, 2, sab2); db.stride[0] = T * Hv;
  dg = desc(gate, GDN_BF16, 3, sg3); dg.stride[0] = T * nv;
  void *cs = NULL, *st = NULL, *dout = NULL;
  const size_t cs_b = (size_t)(B * 3 * C * 2), st_b = (size_t)(B * Hv * dv * dk * 4);
  HIPCHECK(hipMalloc(&cs, cs_b));
  HIPCHECK(hipMalloc(&st, st_b));
  HIPCHECK(hipMalloc(&dout, (size_t)(B * nv * 2)));
  HIPCHECK(hipMemsetAsync(cs, 0, cs_b, stream));
  HIPCHECK(hipMemsetAsync(st, 0, st_b, stream));
  const int64_t s_cs[3] = {B, 3, C}, s_st[4] = {B, Hv, dv, dk};
  gdn_tensor tcs = desc(cs, GDN_BF16, 3, s_cs), tst = desc(st, GDN_F32, 4, s_st), tdo = desc(dout, GDN_BF16, 3, sg3);
  GDNCHECK(gdn_decode_fwd(&dq, &dkk, &dvv, &tw, NULL, &tcs, &da, &db, &tal, &tdt, &tst, &dims, scale, 1, 1e-6f,
                          &dg, &tn, 1e-5f, &tdo, stream));
  HIPCHECK(hipStreamSynchronize(stream));

  FILE *g = fopen(argv[2], "wb");
  if (!g) return 1;
  const size_t ob = (size_t)(B * T * nv * 2), db_ = (size_t)(B * nv * 2);
  void *h = malloc(ob > st_b ? ob : st_b);
  HIPCHECK(hipMemcpy(h, out, ob, hipMemcpyDeviceToHost));
  fwrite(h, 1, ob, g);
  HIPCHECK(hipMemcpy(h, dout, db_, hipMemcpyDeviceToHost));
  fwrite(h, 1, db_, g);
  HIPCHECK(hipMemcpy(h, st, st_b, hipMemcpyDeviceToHost));
  fwrite(h, 1, st_b, g);
  fclose(g);
  free(h);
  printf("layer_from_c: %s, %lld x %lld tokens, workspace %zu bytes\n", gdn_version(), (long long)B, (long long)T, wsb);
  return 0;
}
