/*
 * A plain C caller of the decode-attention C ABI (include/fd_decode.h): no
 * Python, no torch. Used by the tests to show the boundary works from C.
 *
 *   decode_demo host
 *     Host-only calls (no device needed): plans splits for a 64K history,
 *     sizes the workspace, prints the results and the status strings.
 *   decode_demo run IN OUT
 *     Reads a problem from IN, allocates device buffers with HIP, runs
 *     fd_decode_attn at the planned split count and writes out / lse to OUT.
 *
 * IN layout (little-endian): int32 batch, num_q_heads, num_kv_heads,
 * head_dim, max_seq_len; then q bf16 [B,Hq,D], k bf16 [B,Hkv,L,D],
 * v bf16 [B,Hkv,L,D], seq_lens int32 [B]. OUT: int32 num_splits, then
 * out fp32 [B,Hq,D], lse fp32 [B,Hq].
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fd_decode.h"

#define CHECK_HIP(x)                                                       \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_),  \
              __LINE__);                                                   \
      return 3;                                                            \
    }                                                                      \
  } while (0)

static int host_only(void) {
  fd_shape s;
  int splits = 0;
  size_t bytes = 0;
  memset(&s, 0, sizeof s);
  s.batch = 1;
  s.num_q_heads = 16;
  s.num_kv_heads = 2;
  s.head_dim = 128;
  s.max_seq_len = 65536;
  s.dtype = FD_DTYPE_BF16;
  if (fd_plan_splits(&s, 256, -1, &splits) != FD_OK) return 1;
  if (fd_workspace_size(&s, splits, &bytes) != FD_OK) return 1;
  printf("splits %d workspace %zu version %d\n", splits, bytes, fd_version());
  printf("status %s | %s\n", fd_status_str(FD_OK),
         fd_status_str(FD_ERR_WORKSPACE));
  s.head_dim = 96;
  printf("head_dim 96 -> %d\n", fd_plan_splits(&s, 256, -1, &splits));
  return 0;
}

static void* read_exact(FILE* f, size_t n) {
  void* p = malloc(n ? n : 1);
  if (p && n && fread(p, 1, n, f) != n) {
    free(p);
    return NULL;
  }
  return p;
}

static int run(const char* in_path, const char* out_path) {
  FILE* f = fopen(in_path, "rb");
  int32_t hdr[5];
  if (!f || fread(hdr, sizeof hdr, 1, f) != 1) return 2;
  fd_shape s;
  memset(&s, 0, sizeof s);
  s.batch = hdr[0];
  s.num_q_heads = hdr[1];
  s.num_kv_heads = hdr[2];
  s.head_dim = hdr[3];
  s.max_seq_len = hdr[4];
  s.dtype = FD_DTYPE_BF16;
  const size_t nq = (size_t)s.batch * s.num_q_heads * s.head_dim;
  const size_t nkv = (size_t)s.batch * s.num_kv_heads * s.max_seq_len *
                     s.head_dim;
  void* hq = read_exact(f, nq * 2);
  void* hk = read_exact(f, nkv * 2);
  void* hv = read_exact(f, nkv * 2);
  void* hl = read_exact(f, (size_t)s.batch * 4);
  fclose(f);
  if (!hq || !hk || !hv || !hl) return 2;

  int splits = 0;
  size_t ws_bytes = 0;
  int64_t sum = 0;
  for (int b = 0; b < s.batch; ++b) sum += ((const int32_t*)hl)[b];
  int device_cus = 0;
  CHECK_HIP(hipDeviceGetAttribute(&device_cus,
                                  hipDeviceAttributeMultiprocessorCount, 0));
  int st = fd_plan_splits(&s, device_cus, sum, &splits);
  if (st == FD_OK) st = fd_workspace_size(&s, splits, &ws_bytes);
  if (st != FD_OK) {
    fprintf(stderr, "%s\n", fd_status_str(st));
    return 1;
  }

  void *dq, *dk, *dv, *dl, *dws = NULL;
  float *dout, *dlse;
  CHECK_HIP(hipMalloc(&dq, nq * 2));
  CHECK_HIP(hipMalloc(&dk, nkv * 2));
  CHECK_HIP(hipMalloc(&dv, nkv * 2));
  CHECK_HIP(hipMalloc(&dl, (size_t)s.batch * 4));
  CHECK_HIP(hipMalloc((void**)&dout, nq * 4));
  CHECK_HIP(hipMalloc((void**)&dlse, (size_t)s.batch * s.num_q_heads * 4));
  if (ws_bytes) CHECK_HIP(hipMalloc(&dws, ws_bytes));
  CHECK_HIP(hipMemcpy(dq, hq, nq * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dk, hk, nkv * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dv, hv, nkv * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dl, hl, (size_t)s.batch * 4, hipMemcpyHostToDevice));

  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  st = fd_decode_attn(&s, dq, dk, dv, NULL, (const int32_t*)dl, splits, dws,
                      ws_bytes, dout, dlse, (void*)stream);
  if (st != FD_OK) {
    fprintf(stderr, "fd_decode_attn: %s\n", fd_status_str(st));
    return 1;
  }
  CHECK_HIP(hipStreamSynchronize(stream));

  float* hout = (float*)malloc(nq * 4);
  float* hlse = (float*)malloc((size_t)s.batch * s.num_q_heads * 4);
  if (!hout || !hlse) return 2;
  CHECK_HIP(hipMemcpy(hout, dout, nq * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hlse, dlse, (size_t)s.batch * s.num_q_heads * 4,
                      hipMemcpyDeviceToHost));
  FILE* o = fopen(out_path, "wb");
  if (!o) return 2;
  int32_t sp = splits;
  fwrite(&sp, 4, 1, o);
  fwrite(hout, 4, nq, o);
  fwrite(hlse, 4, (size_t)s.batch * s.num_q_heads, o);
  fclose(o);
  CHECK_HIP(hipStreamDestroy(stream));
  hipFree(dq);
  hipFree(dk);
  hipFree(dv);
  hipFree(dl);
  hipFree(dout);
  hipFree(dlse);
  if (dws) hipFree(dws);
  free(hq);
  free(hk);
  free(hv);
  free(hl);
  free(hout);
  free(hlse);
  return 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "host") == 0) return host_only();
  if (argc >= 4 && strcmp(argv[1], "run") == 0) return run(argv[2], argv[3]);
  fprintf(stderr, "usage: decode_demo host | run IN OUT\n");
  return 2;
}
