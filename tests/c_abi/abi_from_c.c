/* A C caller of the library: include/drgrpo.h compiled as C, linked against
 * libdrgrpo.so, driving the loss with nothing but the HIP runtime API.  Built
 * as a shared object (gcc -std=c11 -pedantic) by tests/test_c_abi.py and
 * called through ctypes. */
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "drgrpo.h"

/* CPU side: workspace sizes, status strings and rejections before a launch.
 * out[0..1]: workspace bytes for (N, C, V, G) and for an overflowing shape;
 * out[2..6]: the status of a NULL logits pointer, an unknown element type,
 * N % G != 0, a negative eps and a too small workspace. */
int c_abi_host_checks(int64_t N, int64_t C, int64_t V, int64_t G, int64_t* out,
                      char* status_text, size_t text_len) {
  /* host memory standing in for device buffers: nothing is launched */
  static _Alignas(256) unsigned char fake[1 << 16];
  void* p = fake;
  float* f = (float*)(void*)fake;
  out[0] = (int64_t)drgrpo_workspace_bytes(N, C, V, G);
  out[1] = (int64_t)drgrpo_workspace_bytes((int64_t)1 << 40, (int64_t)1 << 30, V, G);
  out[2] = drgrpo_loss_fwd_bwd(NULL, (const int64_t*)p, 0, f, f, NULL, G, 0.2f, 0.0f, 1.0f, f, p,
                               N, C, V, DRGRPO_BF16, p, (size_t)1 << 40, NULL);
  out[3] = drgrpo_loss_fwd_bwd(p, (const int64_t*)p, 0, f, f, NULL, G, 0.2f, 0.0f, 1.0f, f, p, N,
                               C, V, (drgrpo_dtype_t)7, p, (size_t)1 << 40, NULL);
  out[4] = drgrpo_loss_fwd_bwd(p, (const int64_t*)p, 0, f, f, NULL, G, 0.2f, 0.0f, 1.0f, f, p,
                               N + 1, C, V, DRGRPO_BF16, p, (size_t)1 << 40, NULL);
  out[5] = drgrpo_loss_fwd_bwd(p, (const int64_t*)p, 0, f, f, NULL, G, -0.2f, 0.0f, 1.0f, f, p,
                               N, C, V, DRGRPO_BF16, p, (size_t)1 << 40, NULL);
  out[6] = drgrpo_loss_fwd_bwd(p, (const int64_t*)p, 0, f, f, NULL, G, 0.2f, 0.0f, 1.0f, f, p, N,
                               C, V, DRGRPO_BF16, p, 16, NULL);
  strncpy(status_text, drgrpo_status_string((int)out[3]), text_len - 1);
  status_text[text_len - 1] = '\0';
  return 0;
}

/* GPU side: the whole loss from host arrays.  logits and dlogits are
 * bfloat16 bits [N, C, V]; returns the library's status, or 1000 + the HIP
 * error of the runtime call that failed. */
int c_abi_loss(const uint16_t* logits, const int64_t* tokens, int64_t eos_id, const float* rewards,
               const float* logp_old, int64_t N, int64_t C, int64_t V, int64_t G, float eps,
               float norm_const, float* loss, uint16_t* dlogits) {
  const size_t nl = (size_t)(N * C * V) * sizeof(uint16_t);
  const size_t nt = (size_t)(N * C);
  const size_t nws = drgrpo_workspace_bytes(N, C, V, G);
  void *d_logits = NULL, *d_dl = NULL, *d_ws = NULL;
  int64_t* d_tok = NULL;
  float *d_rew = NULL, *d_old = NULL, *d_loss = NULL;
  hipStream_t st = NULL;
  int rc = 0;
  hipError_t e;
#define HIP_OK(call)                  \
  do {                                \
    e = (call);                       \
    if (e != hipSuccess) {            \
      rc = 1000 + (int)e;             \
      goto done;                      \
    }                                 \
  } while (0)
  HIP_OK(hipStreamCreate(&st));
  HIP_OK(hipMalloc(&d_logits, nl));
  HIP_OK(hipMalloc(&d_dl, nl));
  HIP_OK(hipMalloc((void**)&d_tok, nt * sizeof(int64_t)));
  HIP_OK(hipMalloc((void**)&d_rew, (size_t)N * sizeof(float)));
  HIP_OK(hipMalloc((void**)&d_old, nt * sizeof(float)));
  HIP_OK(hipMalloc((void**)&d_loss, sizeof(float)));
  HIP_OK(hipMalloc(&d_ws, nws));
  HIP_OK(hipMemcpy(d_logits, logits, nl, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_tok, tokens, nt * sizeof(int64_t), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_rew, rewards, (size_t)N * sizeof(float), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_old, logp_old, nt * sizeof(float), hipMemcpyHostToDevice));
  rc = drgrpo_loss_fwd_bwd(d_logits, d_tok, eos_id, d_rew, d_old, NULL, G, eps, 0.0f, norm_const,
                           d_loss, d_dl, N, C, V, DRGRPO_BF16, d_ws, nws, (void*)st);
  if (rc != DRGRPO_OK) goto done;
  HIP_OK(hipStreamSynchronize(st));
  rc = drgrpo_device_status(d_ws, (void*)st);
  if (rc != DRGRPO_OK) goto done;
  HIP_OK(hipMemcpy(loss, d_loss, sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dlogits, d_dl, nl, hipMemcpyDeviceToHost));
done:
  hipFree(d_logits);
  hipFree(d_dl);
  hipFree(d_tok);
  hipFree(d_rew);
  hipFree(d_old);
  hipFree(d_loss);
  hipFree(d_ws);
  if (st) hipStreamDestroy(st);
  return rc;
#undef HIP_OK
}
