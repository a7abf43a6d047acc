/*
 * A plain C (C99) client of libfa.so: shows that the C ABI of include/fa.h is
 * usable without Python or torch, and lets a GPU test compare it with the
 * binding and the oracle.
 *
 *   fa_c_client --abi
 *       prints FA_ABI_VERSION of the loaded library and a status string
 *       (host only, no GPU needed).
 *   fa_c_client IN OUT BH N D CAUSAL [WINDOW FUSED]
 *       reads q, k, v, dO (bf16, each BH * N * D values, raw, in that order)
 *       from IN, runs fa_fwd, fa_bwd_preprocess, fa_bwd_dkdv and fa_bwd_dq on
 *       the default stream with the default tilings and scale 1/sqrt(D), and
 *       writes o (bf16), lse (float32, BH * N), dq, dk, dv (bf16) and delta
 *       (float32) to OUT.  WINDOW > 0 runs the *_rect calls with that causal
 *       window; FUSED = 1 replaces fa_bwd_dkdv and fa_bwd_dq by
 *       fa_bwd_fused with a workspace of fa_bwd_fused_workspace_bytes.  Also
 *       checks that an unsupported head dim is rejected before any launch.
 *       Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fa.h"

#define HIP_OK(call)                                                            \
  do {                                                                          \
    hipError_t e_ = (call);                                                     \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));        \
      return 2;                                                                 \
    }                                                                           \
  } while (0)

#define FA_OK_OR_FAIL(call)                                                     \
  do {                                                                          \
    fa_status s_ = (call);                                                      \
    if (s_ != FA_OK) {                                                          \
      fprintf(stderr, "%s failed: %s\n", #call, fa_status_str(s_));            \
      return 3;                                                                 \
    }                                                                           \
  } while (0)

static int read_all(const char* path, void* buf, size_t bytes) {
  FILE* f = fopen(path, "rb");
  if (!f) return -1;
  size_t got = fread(buf, 1, bytes, f);
  fclose(f);
  return got == bytes ? 0 : -1;
}

int main(int argc, char** argv) {
  if (argc == 2 && strcmp(argv[1], "--abi") == 0) {
    printf("abi %d %s\n", fa_abi_version(), fa_status_str(FA_ERR_UNSUPPORTED));
    return fa_abi_version() == FA_ABI_VERSION ? 0 : 1;
  }
  if (argc != 7 && argc != 9) {
    fprintf(stderr, "usage: %s --abi | IN OUT BH N D CAUSAL [WINDOW FUSED]\n", argv[0]);
    return 1;
  }
  const int bh = atoi(argv[3]), n = atoi(argv[4]), d = atoi(argv[5]), causal = atoi(argv[6]);
  const int window = argc == 9 ? atoi(argv[7]) : 0, fused = argc == 9 ? atoi(argv[8]) : 0;
  if (bh <= 0 || n <= 0 || d <= 0) return 1;
  const size_t elems = (size_t)bh * n * d, rows = (size_t)bh * n;
  const size_t tb = elems * sizeof(uint16_t), rb = rows * sizeof(float);

  uint16_t* host_in = (uint16_t*)malloc(4 * tb);
  unsigned char* host_out = (unsigned char*)malloc(4 * tb + 2 * rb);
  if (!host_in || !host_out) return 2;
  if (read_all(argv[1], host_in, 4 * tb) != 0) {
    fprintf(stderr, "cannot read %zu bytes from %s\n", 4 * tb, argv[1]);
    return 1;
  }

  void *q, *k, *v, *dO, *o, *dq, *dk, *dv;
  float *lse, *delta;
  HIP_OK(hipMalloc(&q, tb));
  HIP_OK(hipMalloc(&k, tb));
  HIP_OK(hipMalloc(&v, tb));
  HIP_OK(hipMalloc(&dO, tb));
  HIP_OK(hipMalloc(&o, tb));
  HIP_OK(hipMalloc(&dq, tb));
  HIP_OK(hipMalloc(&dk, tb));
  HIP_OK(hipMalloc(&dv, tb));
  HIP_OK(hipMalloc((void**)&lse, rb));
  HIP_OK(hipMalloc((void**)&delta, rb));
  HIP_OK(hipMemcpy(q, host_in, tb, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, host_in + elems, tb, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, host_in + 2 * elems, tb, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dO, host_in + 3 * elems, tb, hipMemcpyHostToDevice));

  /* an unsupported head dim is rejected on the host, before any launch */
  if (fa_fwd(q, k, v, o, lse, bh, n, 96, FA_BF16, 0.1f, causal, 0, 0, NULL) != FA_ERR_UNSUPPORTED) {
    fprintf(stderr, "head dim 96 was not rejected\n");
    return 4;
  }

  const float scale = 1.0f / sqrtf((float)d);
  if (window > 0)
    FA_OK_OR_FAIL(fa_fwd_rect(q, k, v, o, lse, bh, n, n, d, FA_BF16, scale, causal, window, 0, 0, NULL));
  else
    FA_OK_OR_FAIL(fa_fwd(q, k, v, o, lse, bh, n, d, FA_BF16, scale, causal, 0, 0, NULL));
  FA_OK_OR_FAIL(fa_bwd_preprocess(o, dO, delta, bh, n, d, FA_BF16, NULL));
  void* ws = NULL;
  if (fused) {
    HIP_OK(hipMalloc(&ws, fa_bwd_fused_workspace_bytes(bh, n, d, FA_BF16)));
    FA_OK_OR_FAIL(fa_bwd_fused(q, k, v, dO, lse, delta, dq, dk, dv, (float*)ws, bh, n, n, d, FA_BF16,
                               scale, causal, window, 0, 0, NULL));
  } else if (window > 0) {
    FA_OK_OR_FAIL(fa_bwd_dkdv_rect(q, k, v, dO, lse, delta, dk, dv, bh, n, n, d, FA_BF16, scale, causal,
                                   window, 0, 0, NULL));
    FA_OK_OR_FAIL(fa_bwd_dq_rect(q, k, v, dO, lse, delta, dq, bh, n, n, d, FA_BF16, scale, causal,
                                 window, 0, 0, NULL));
  } else {
    FA_OK_OR_FAIL(fa_bwd_dkdv(q, k, v, dO, lse, delta, dk, dv, bh, n, d, FA_BF16, scale, causal, 0, 0, NULL));
    FA_OK_OR_FAIL(fa_bwd_dq(q, k, v, dO, lse, delta, dq, bh, n, d, FA_BF16, scale, causal, 0, 0, NULL));
  }
  HIP_OK(hipDeviceSynchronize());
  if (ws) HIP_OK(hipFree(ws));

  unsigned char* p = host_out;
  HIP_OK(hipMemcpy(p, o, tb, hipMemcpyDeviceToHost));
  p += tb;
  HIP_OK(hipMemcpy(p, lse, rb, hipMemcpyDeviceToHost));
  p += rb;
  HIP_OK(hipMemcpy(p, dq, tb, hipMemcpyDeviceToHost));
  p += tb;
  HIP_OK(hipMemcpy(p, dk, tb, hipMemcpyDeviceToHost));
  p += tb;
  HIP_OK(hipMemcpy(p, dv, tb, hipMemcpyDeviceToHost));
  p += tb;
  HIP_OK(hipMemcpy(p, delta, rb, hipMemcpyDeviceToHost));

  FILE* f = fopen(argv[2], "wb");
  if (!f || fwrite(host_out, 1, 4 * tb + 2 * rb, f) != 4 * tb + 2 * rb) return 2;
  fclose(f);

  void* bufs[] = {q, k, v, dO, o, dq, dk, dv, lse, delta};
  for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) HIP_OK(hipFree(bufs[i]));
  free(host_in);
  free(host_out);
  printf("ok bh=%d n=%d d=%d causal=%d window=%d fused=%d\n", bh, n, d, causal, window, fused);
  return 0;
}
