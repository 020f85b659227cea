/* A plain C99 client of libdfa's device calls, built and run by
 * tests/test_c_gpu_client.py on a GPU: no torch, no C++ -- the HIP runtime's
 * C API for memory and the stream, libdfa for the rest.  It reads bf16 q, k,
 * v, dO (contiguous [1][N][H][128]) from files, runs the folded schedule's
 * fused forward and backward, and writes o, lse, dq, dk, dv back to files.
 *   usage: c_gpu_client <dir> <N> <P> <Hq> <Hkv>
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dfa.h"

#define HIPCHECK(x)                                                    \
  do {                                                                 \
    hipError_t e_ = (x);                                               \
    if (e_ != hipSuccess) {                                            \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));   \
      return 2;                                                        \
    }                                                                  \
  } while (0)
#define DFACHECK(x)                                                        \
  do {                                                                     \
    dfa_status s_ = (x);                                                   \
    if (s_ != DFA_OK) {                                                    \
      fprintf(stderr, "%s failed: %s\n", #x, dfa_status_string(s_));       \
      return 3;                                                            \
    }                                                                      \
  } while (0)

static void *read_file(const char *dir, const char *name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) return NULL;
  void *p = malloc(bytes);
  size_t got = p ? fread(p, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static int write_file(const char *dir, const char *name, const void *p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "wb");
  if (!f) return 0;
  size_t put = fwrite(p, 1, bytes, f);
  fclose(f);
  return put == bytes;
}

int main(int argc, char **argv) {
  if (argc != 6) return 1;
  const char *dir = argv[1];
  const int64_t n = atoll(argv[2]);
  const int32_t p = atoi(argv[3]), hq = atoi(argv[4]), hkv = atoi(argv[5]);
  const int32_t hd = 128;
  const size_t qbytes = (size_t)n * hq * hd * 2, kbytes = (size_t)n * hkv * hd * 2;
  const size_t lbytes = (size_t)hq * n * sizeof(float);

  int64_t nb = 0;
  DFACHECK(dfa_schedule_build(DFA_SCHED_BALANCED, n, p, NULL, 0, &nb));
  dfa_block *blocks = (dfa_block *)malloc((size_t)nb * sizeof(dfa_block));
  if (!blocks) return 1;
  DFACHECK(dfa_schedule_build(DFA_SCHED_BALANCED, n, p, blocks, nb, &nb));

  dfa_attn_desc d;
  memset(&d, 0, sizeof d);
  d.dtype = DFA_BF16;
  d.batch = 1;
  d.heads_q = hq;
  d.heads_kv = hkv;
  d.head_dim = hd;
  d.softmax_scale = 0.08838834764831845f; /* 1/sqrt(128) */
  d.seqlen = n;
  const int64_t qs[3] = {n * hq * hd, hq * hd, hd}, ks[3] = {n * hkv * hd, hkv * hd, hd};
  for (int i = 0; i < 3; ++i) {
    d.q_strides[i] = qs[i];
    d.o_strides[i] = qs[i];
    d.k_strides[i] = ks[i];
    d.v_strides[i] = ks[i];
  }
  size_t ws_f = 0, ws_b = 0;
  DFACHECK(dfa_workspace_size(&d, blocks, nb, DFA_OP_FWD_FUSED, &ws_f));
  DFACHECK(dfa_workspace_size(&d, blocks, nb, DFA_OP_BWD, &ws_b));
  const size_t ws_bytes = ws_f > ws_b ? ws_f : ws_b;

  void *hq_ = read_file(dir, "q.bin", qbytes), *hk = read_file(dir, "k.bin", kbytes);
  void *hv = read_file(dir, "v.bin", kbytes), *hdo = read_file(dir, "do.bin", qbytes);
  if (!hq_ || !hk || !hv || !hdo) {
    fprintf(stderr, "input files missing or short\n");
    return 1;
  }
  void *q, *k, *v, *o, *dO, *dq, *dk, *dv, *ws;
  float *lse;
  HIPCHECK(hipMalloc(&q, qbytes));
  HIPCHECK(hipMalloc(&k, kbytes));
  HIPCHECK(hipMalloc(&v, kbytes));
  HIPCHECK(hipMalloc(&o, qbytes));
  HIPCHECK(hipMalloc(&dO, qbytes));
  HIPCHECK(hipMalloc(&dq, qbytes));
  HIPCHECK(hipMalloc(&dk, kbytes));
  HIPCHECK(hipMalloc(&dv, kbytes));
  HIPCHECK(hipMalloc((void **)&lse, lbytes));
  HIPCHECK(hipMalloc(&ws, ws_bytes > 0 ? ws_bytes : 256));
  HIPCHECK(hipMemcpy(q, hq_, qbytes, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(k, hk, kbytes, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(v, hv, kbytes, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(dO, hdo, qbytes, hipMemcpyHostToDevice));
  hipStream_t s;
  HIPCHECK(hipStreamCreate(&s));

  DFACHECK(dfa_attn_fwd(&d, blocks, nb, DFA_FWD_FUSED, q, k, v, o, lse, ws, ws_bytes, s));
  DFACHECK(dfa_attn_bwd(&d, blocks, nb, q, k, v, o, dO, lse, dq, dk, dv, ws, ws_bytes, s));
  HIPCHECK(hipStreamSynchronize(s));

  void *ho = malloc(qbytes), *hlse = malloc(lbytes), *hdq = malloc(qbytes);
  void *hdk = malloc(kbytes), *hdv = malloc(kbytes);
  if (!ho || !hlse || !hdq || !hdk || !hdv) return 1;
  HIPCHECK(hipMemcpy(ho, o, qbytes, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(hlse, lse, lbytes, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(hdq, dq, qbytes, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(hdk, dk, kbytes, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(hdv, dv, kbytes, hipMemcpyDeviceToHost));
  if (!write_file(dir, "o.bin", ho, qbytes) || !write_file(dir, "lse.bin", hlse, lbytes) ||
      !write_file(dir, "dq.bin", hdq, qbytes) || !write_file(dir, "dk.bin", hdk, kbytes) ||
      !write_file(dir, "dv.bin", hdv, kbytes))
    return 1;
  HIPCHECK(hipStreamDestroy(s));
  HIPCHECK(hipFree(q));
  HIPCHECK(hipFree(k));
  HIPCHECK(hipFree(v));
  HIPCHECK(hipFree(o));
  HIPCHECK(hipFree(dO));
  HIPCHECK(hipFree(dq));
  HIPCHECK(hipFree(dk));
  HIPCHECK(hipFree(dv));
  HIPCHECK(hipFree(lse));
  HIPCHECK(hipFree(ws));
  printf("c client: %lld blocks, workspace %zu bytes\n", (long long)nb, ws_bytes);
  return 0;
}
