/*
 * A plain C client of libs2attn: the forward and the backward through the C ABI
 * of include/s2attn.h, with device memory from the HIP runtime and no Python.
 *
 *   c_abi_client IN OUT B H Hkv N d G shift_heads wrap
 *
 * IN holds q, k, v, dO as raw bfloat16 ([B,N,H,d], [B,N,Hkv,d], [B,N,Hkv,d],
 * [B,N,H,d], in that order); OUT receives o (bf16), lse (fp32 [B,H,N]), dq, dk,
 * dv (bf16), in that order.  Exit status 0 on success; otherwise the failing
 * call and its status string are printed.  tests/test_gpu_parity.py feeds it
 * seeded inputs and checks OUT against the float64 oracle.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>

#include "s2attn.h"

#define HIP_CHECK(x)                                                            \
  do {                                                                          \
    hipError_t e_ = (x);                                                        \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));           \
      return 2;                                                                 \
    }                                                                           \
  } while (0)

#define S2_CHECK(x)                                                             \
  do {                                                                          \
    int s_ = (x);                                                               \
    if (s_ != S2ATTN_OK) {                                                      \
      fprintf(stderr, "%s failed: %s\n", #x, s2attn_status_str(s_));           \
      return 3;                                                                 \
    }                                                                           \
  } while (0)

static int read_exact(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }
static int write_exact(FILE* f, const void* p, size_t n) { return fwrite(p, 1, n, f) == n; }

int main(int argc, char** argv) {
  if (argc != 11) {
    fprintf(stderr, "usage: %s IN OUT B H Hkv N d G shift_heads wrap\n", argv[0]);
    return 1;
  }
  const int B = atoi(argv[3]), H = atoi(argv[4]), Hkv = atoi(argv[5]), N = atoi(argv[6]);
  const int d = atoi(argv[7]), G = atoi(argv[8]), S = atoi(argv[9]), wrap = atoi(argv[10]);
  const size_t nq = (size_t)B * N * H * d * 2, nkv = (size_t)B * N * Hkv * d * 2;
  const size_t nlse = (size_t)B * H * N * sizeof(float);

  /* host images of the inputs and outputs */
  char* host = malloc(2 * nq + 2 * nkv);
  char* out = malloc(3 * nq + 2 * nkv + nlse);
  if (!host || !out) return 1;
  FILE* fi = fopen(argv[1], "rb");
  if (!fi || !read_exact(fi, host, 2 * nq + 2 * nkv)) {
    fprintf(stderr, "cannot read %s\n", argv[1]);
    return 1;
  }
  fclose(fi);

  void *q, *k, *v, *dO, *o, *dq, *dk, *dv, *qr, *ws = NULL;
  float* lse;
  HIP_CHECK(hipMalloc(&q, nq));
  HIP_CHECK(hipMalloc(&k, nkv));
  HIP_CHECK(hipMalloc(&v, nkv));
  HIP_CHECK(hipMalloc(&dO, nq));
  HIP_CHECK(hipMalloc(&o, nq));
  HIP_CHECK(hipMalloc((void**)&lse, nlse));
  HIP_CHECK(hipMalloc(&dq, nq));
  HIP_CHECK(hipMalloc(&dk, nkv));
  HIP_CHECK(hipMalloc(&dv, nkv));
  HIP_CHECK(hipMalloc(&qr, nq));
  const size_t wsb = s2attn_bwd_workspace_bytes(B, H, Hkv, N, d, G, S, S2ATTN_BF16);
  if (wsb == 0) {
    fprintf(stderr, "s2attn_bwd_workspace_bytes rejected the problem\n");
    return 3;
  }
  HIP_CHECK(hipMalloc(&ws, wsb));   /* hipMalloc returns at least 256-byte alignment */
  HIP_CHECK(hipMemcpy(q, host, nq, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(k, host + nq, nkv, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(v, host + nq + nkv, nkv, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(dO, host + nq + 2 * nkv, nq, hipMemcpyHostToDevice));

  hipStream_t stream;
  HIP_CHECK(hipStreamCreate(&stream));
  S2_CHECK(s2attn_fwd_ex(q, k, v, o, lse, B, H, Hkv, N, d, G, S, wrap, S2ATTN_BF16, stream));
  S2_CHECK(s2attn_bwd_ex(q, k, v, o, lse, dO, dq, dk, dv, ws, wsb, B, H, Hkv, N, d, G, S, wrap, S2ATTN_BF16,
                         stream));
  /* rotary embedding of q with Position Interpolation by 1/4, base 10000 */
  S2_CHECK(s2attn_rope(q, qr, B, N, H, d, 0.25, 10000.0, 0, S2ATTN_BF16, stream));
  HIP_CHECK(hipStreamSynchronize(stream));

  char* p = out;
  HIP_CHECK(hipMemcpy(p, o, nq, hipMemcpyDeviceToHost));
  p += nq;
  HIP_CHECK(hipMemcpy(p, lse, nlse, hipMemcpyDeviceToHost));
  p += nlse;
  HIP_CHECK(hipMemcpy(p, dq, nq, hipMemcpyDeviceToHost));
  p += nq;
  HIP_CHECK(hipMemcpy(p, dk, nkv, hipMemcpyDeviceToHost));
  p += nkv;
  HIP_CHECK(hipMemcpy(p, dv, nkv, hipMemcpyDeviceToHost));
  p += nkv;
  HIP_CHECK(hipMemcpy(p, qr, nq, hipMemcpyDeviceToHost));
  FILE* fo = fopen(argv[2], "wb");
  if (!fo || !write_exact(fo, out, 3 * nq + 2 * nkv + nlse)) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(fo);

  HIP_CHECK(hipStreamDestroy(stream));
  void* bufs[] = {q, k, v, dO, o, lse, dq, dk, dv, qr, ws};
  for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) HIP_CHECK(hipFree(bufs[i]));
  free(host);
  free(out);
  printf("ok\n");
  return 0;
}
