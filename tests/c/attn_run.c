/* The fused attention through the C ABI from plain C99 (no Python, no
   torch): reads a problem from a file, runs bs_layout_build and
   bs_attention_fwd on device buffers from the HIP runtime, writes O and the
   row log-sum-exp. The test that runs it compares them with the oracle.
   File (little endian): int32 Z, H, N, d, block, causal; float32 scale;
   uint8 layout[H][N/block][N/block]; float32 Q, K, V [Z][H][N][d].
   Output: float32 O [Z][H][N][d], then float32 lse [Z][H][N]. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "bsattn.h"

#define HIP_OK(call)                                                      \
  do {                                                                    \
    hipError_t e_ = (call);                                               \
    if (e_ != hipSuccess) {                                               \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));          \
      return 2;                                                           \
    }                                                                     \
  } while (0)

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n ? 0 : 1; }

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: attn_run IN OUT\n");
    return 2;
  }
  FILE* f = fopen(argv[1], "rb");
  if (!f) return 2;
  int32_t hdr[6];
  float scale;
  if (read_all(f, hdr, sizeof hdr) || read_all(f, &scale, sizeof scale)) return 2;
  const int Z = hdr[0], H = hdr[1], N = hdr[2], d = hdr[3], b = hdr[4], causal = hdr[5];
  const int nb = N / b;
  const size_t lay_n = (size_t)H * nb * nb, t_n = (size_t)Z * H * N * d, l_n = (size_t)Z * H * N;
  uint8_t* lay = (uint8_t*)malloc(lay_n);
  float* host = (float*)malloc(3 * t_n * sizeof(float));
  float* out = (float*)malloc((t_n + l_n) * sizeof(float));
  if (!lay || !host || !out) return 2;
  if (read_all(f, lay, lay_n) || read_all(f, host, 3 * t_n * sizeof(float))) return 2;
  fclose(f);

  uint8_t* d_lay;
  float *d_q, *d_k, *d_v, *d_o, *d_lse;
  HIP_OK(hipMalloc((void**)&d_lay, lay_n));
  HIP_OK(hipMalloc((void**)&d_q, t_n * sizeof(float)));
  HIP_OK(hipMalloc((void**)&d_k, t_n * sizeof(float)));
  HIP_OK(hipMalloc((void**)&d_v, t_n * sizeof(float)));
  HIP_OK(hipMalloc((void**)&d_o, t_n * sizeof(float)));
  HIP_OK(hipMalloc((void**)&d_lse, l_n * sizeof(float)));
  HIP_OK(hipMemcpy(d_lay, lay, lay_n, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_q, host, t_n * sizeof(float), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_k, host + t_n, t_n * sizeof(float), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_v, host + 2 * t_n, t_n * sizeof(float), hipMemcpyHostToDevice));

  bs_layout_t L = NULL;
  int rc = bs_layout_build(d_lay, H, nb, nb, b, NULL, &L);
  if (rc != BS_OK) {
    fprintf(stderr, "bs_layout_build: %d %s\n", rc, bs_last_error());
    return 1;
  }
  int64_t nnz = 0;
  if (bs_layout_nnz(L, &nnz) != BS_OK) return 1;
  rc = bs_attention_fwd(L, d_q, d_k, d_v, d_o, d_lse, Z, d, scale, causal ? BS_CAUSAL : 0, NULL, NULL, BS_F32,
                        NULL);
  if (rc != BS_OK) {
    fprintf(stderr, "bs_attention_fwd: %d %s\n", rc, bs_last_error());
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(out, d_o, t_n * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out + t_n, d_lse, l_n * sizeof(float), hipMemcpyDeviceToHost));
  bs_layout_free(L);
  HIP_OK(hipFree(d_lay));
  HIP_OK(hipFree(d_q));
  HIP_OK(hipFree(d_k));
  HIP_OK(hipFree(d_v));
  HIP_OK(hipFree(d_o));
  HIP_OK(hipFree(d_lse));

  FILE* g = fopen(argv[2], "wb");
  if (!g || fwrite(out, sizeof(float), t_n + l_n, g) != t_n + l_n) return 2;
  fclose(g);
  printf("attn_run ok: nnz %lld\n", (long long)nnz);
  free(lay);
  free(host);
  free(out);
  return 0;
}
