/*
 * A plain C (C11) consumer of the library's C ABI, built with gcc against
 * include/paged_attn.h and the HIP runtime's C API only (no C++, no Python).
 * It allocates device memory with hipMalloc, runs paged_attn_decode on a
 * small fp32 batch (shuffled block table, unused table entries pointing at a
 * NaN-filled block, a materialised bias, with and without a sliding window),
 * and compares each result with the float64 oracle (liboracle, test
 * infrastructure) called on the same host arrays. It also checks that an
 * unsupported head_dim is rejected on the host with a message.
 *
 * Exit status 0 when every check passes; prints one line per check.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "oracle.h"
#include "paged_attn.h"

enum { B = 3, H = 2, D = 64, BS = 16, MAXB = 3, NBLK = 8, MSL = MAXB * BS };

static uint32_t lcg_state = 12345u;
static float lcg_uniform(void) {   /* in [-1, 1) */
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return (float)(lcg_state >> 8) / 8388608.0f - 1.0f;
}

#define HIP_OK(call)                                                   \
  do {                                                                 \
    hipError_t e_ = (call);                                            \
    if (e_ != hipSuccess) {                                            \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_)); \
      return 2;                                                        \
    }                                                                  \
  } while (0)

int main(void) {
  const int32_t lens[B] = {1, 17, 40};
  /* sequence b owns the listed physical blocks; block 1 is never owned */
  const int32_t owned[B][MAXB] = {{5, 1, 1}, {2, 7, 1}, {0, 3, 6}};
  const size_t kv_elems = (size_t)NBLK * H * BS * D;
  float* k = malloc(kv_elems * sizeof(float));
  float* v = malloc(kv_elems * sizeof(float));
  float* q = malloc((size_t)B * H * D * sizeof(float));
  float* bias = malloc((size_t)B * H * MSL * sizeof(float));
  float* out = malloc((size_t)B * H * D * sizeof(float));
  double* ref = malloc((size_t)B * H * D * sizeof(double));
  if (!k || !v || !q || !bias || !out || !ref) return 2;
  for (size_t i = 0; i < kv_elems; ++i) {
    const int blk = (int)(i / ((size_t)H * BS * D));
    k[i] = blk == 1 ? NAN : lcg_uniform();
    v[i] = blk == 1 ? NAN : lcg_uniform();
  }
  for (int i = 0; i < B * H * D; ++i) q[i] = lcg_uniform();
  for (int i = 0; i < B * H * MSL; ++i) bias[i] = lcg_uniform();

  void *dk, *dv, *dq, *dout;
  float* dbias;
  int32_t *dtable, *dlens;
  HIP_OK(hipMalloc(&dk, kv_elems * sizeof(float)));
  HIP_OK(hipMalloc(&dv, kv_elems * sizeof(float)));
  HIP_OK(hipMalloc(&dq, (size_t)B * H * D * sizeof(float)));
  HIP_OK(hipMalloc(&dout, (size_t)B * H * D * sizeof(float)));
  HIP_OK(hipMalloc((void**)&dbias, (size_t)B * H * MSL * sizeof(float)));
  HIP_OK(hipMalloc((void**)&dtable, sizeof(owned)));
  HIP_OK(hipMalloc((void**)&dlens, sizeof(lens)));
  HIP_OK(hipMemcpy(dk, k, kv_elems * sizeof(float), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, v, kv_elems * sizeof(float), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dq, q, (size_t)B * H * D * sizeof(float), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dbias, bias, (size_t)B * H * MSL * sizeof(float), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dtable, owned, sizeof(owned), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dlens, lens, sizeof(lens), hipMemcpyHostToDevice));

  printf("abi version %d\n", pa_abi_version());
  int failures = 0;
  const int32_t windows[2] = {-1, 5};
  for (int w = 0; w < 2; ++w) {
    const int32_t window = windows[w];
    const size_t ws_bytes = pa_decode_workspace_bytes(B, H, D, MSL, window, 0, PA_DTYPE_F32);
    void* ws = NULL;
    if (ws_bytes > 0) HIP_OK(hipMalloc(&ws, ws_bytes));
    const pa_status_t st =
        paged_attn_decode(dout, dq, dk, dv, dtable, dlens, dbias, window, 0.125f, B, H, H, D,
                          BS, MAXB, MSL, NBLK, PA_DTYPE_F32, 0, ws, ws_bytes, NULL);
    if (st != PA_OK) {
      printf("decode W=%d: status %d (%s)\n", window, (int)st, pa_last_error());
      return 1;
    }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(out, dout, (size_t)B * H * D * sizeof(float), hipMemcpyDeviceToHost));
    if (ws) HIP_OK(hipFree(ws));
    if (oracle_decode_f64(ref, q, k, v, &owned[0][0], lens, bias, window, 0.125, B, H, D, BS,
                          MAXB, MSL, 0) != 0) {
      printf("oracle rejected the case\n");
      return 1;
    }
    double err = 0.0;
    for (int i = 0; i < B * H * D; ++i) {
      const double d = fabs((double)out[i] - ref[i]);
      err = (d > err || isnan(d)) ? d : err;
    }
    const int ok = err <= 1e-5;
    printf("decode W=%d: max |gpu - oracle| = %.3e %s\n", window, err, ok ? "ok" : "FAIL");
    failures += !ok;
  }

  /* head_dim 96 is not supported: rejected on the host, before any HIP call */
  const pa_status_t bad =
      paged_attn_decode(dout, dq, dk, dv, dtable, dlens, dbias, -1, 0.125f, B, H, H, 96, BS,
                        MAXB, MSL, NBLK, PA_DTYPE_F32, 0, NULL, 0, NULL);
  const int bad_ok = bad == PA_ERR_UNSUPPORTED && strlen(pa_last_error()) > 0;
  printf("head_dim 96: status %d, message \"%s\" %s\n", (int)bad, pa_last_error(),
         bad_ok ? "ok" : "FAIL");
  failures += !bad_ok;

  hipFree(dk);
  hipFree(dv);
  hipFree(dq);
  hipFree(dout);
  hipFree(dbias);
  hipFree(dtable);
  hipFree(dlens);
  free(k);
  free(v);
  free(q);
  free(bias);
  free(out);
  free(ref);
  return failures == 0 ? 0 : 1;
}
