/*
 * A plain C client of the library: device memory and copies through the HIP
 * runtime's C API, one fa_fwd and one fa_fwd_ex call, results checked against
 * the CPU oracle (liboracle.so, test infrastructure).  No C++, no torch.
 * Prints "ABI_DEMO OK max_abs=..." and returns 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fa_fwd.h"

int oracle_attention_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t B, int64_t H,
                          int64_t N, int64_t d, double scale, int causal, const int64_t *rows, int64_t nrows,
                          double *out, double *lse);

static uint16_t to_bf16(double x) { /* round to nearest even from fp32 */
  float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fff + ((u >> 16) & 1);
  return (uint16_t)(u >> 16);
}
static double from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

#define CHECK(x)                                                    \
  do {                                                              \
    hipError_t e_ = (x);                                            \
    if (e_ != hipSuccess) {                                         \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_)); \
      return 2;                                                     \
    }                                                               \
  } while (0)

int main(void) {
  const int B = 2, H = 3, N = 333, d = 64;
  const size_t n = (size_t)B * H * N * d;
  uint16_t *hq = malloc(n * 2), *hk = malloc(n * 2), *hv = malloc(n * 2), *ho = malloc(n * 2);
  float *hl = malloc((size_t)B * H * N * 4);
  uint64_t st = 0x9E3779B97F4A7C15ull;
  for (size_t i = 0; i < n; ++i) { /* xorshift64 -> uniform(-1, 1) */
    st ^= st << 13, st ^= st >> 7, st ^= st << 17;
    hq[i] = to_bf16((double)(st >> 11) / 9007199254740992.0 * 2 - 1);
    st ^= st << 13, st ^= st >> 7, st ^= st << 17;
    hk[i] = to_bf16((double)(st >> 11) / 9007199254740992.0 * 2 - 1);
    st ^= st << 13, st ^= st >> 7, st ^= st << 17;
    hv[i] = to_bf16((double)(st >> 11) / 9007199254740992.0 * 2 - 1);
  }
  void *q, *k, *v, *o;
  float *l;
  CHECK(hipMalloc(&q, n * 2));
  CHECK(hipMalloc(&k, n * 2));
  CHECK(hipMalloc(&v, n * 2));
  CHECK(hipMalloc(&o, n * 2));
  CHECK(hipMalloc((void **)&l, (size_t)B * H * N * 4));
  CHECK(hipMemcpy(q, hq, n * 2, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(k, hk, n * 2, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(v, hv, n * 2, hipMemcpyHostToDevice));

  /* argument errors come back as codes, before any launch */
  if (fa_fwd(q, k, v, o, l, B, H, N, 96, 0.125f, 0, NULL) != FA_ERR_HEAD_DIM) return 3;
  if (fa_fwd(q, k, v, q, l, B, H, N, d, 0.125f, 0, NULL) != FA_ERR_ALIAS) return 3;

  const float scale = 0.125f;
  double worst = 0.0;
  int64_t *rows = malloc(sizeof(int64_t) * (size_t)B * H * N);
  double *ro = malloc(sizeof(double) * n), *rl = malloc(sizeof(double) * (size_t)B * H * N);
  for (int64_t r = 0; r < (int64_t)B * H * N; ++r) rows[r] = r;
  for (int call = 0; call < 2; ++call) {
    const int causal = call;
    int status;
    if (call == 0) {
      status = fa_fwd(q, k, v, o, l, B, H, N, d, scale, causal, NULL);
    } else { /* the same tensors through the descriptor entry point */
      fa_fwd_desc a;
      memset(&a, 0, sizeof a);
      a.q = q, a.k = k, a.v = v, a.out = o, a.lse = l;
      a.B = B, a.H = H, a.Nq = N, a.Nk = N, a.d = d;
      const long long s3[3] = {(long long)H * N * d, (long long)N * d, d};
      memcpy(a.q_stride, s3, sizeof s3), memcpy(a.k_stride, s3, sizeof s3);
      memcpy(a.v_stride, s3, sizeof s3), memcpy(a.o_stride, s3, sizeof s3);
      a.lse_stride[0] = (long long)H * N, a.lse_stride[1] = N;
      a.scale = scale, a.causal = causal, a.stream = NULL, a.dtype = FA_DTYPE_BF16;
      status = fa_fwd_ex(&a);
    }
    if (status != FA_OK) {
      fprintf(stderr, "call %d: %s\n", call, fa_strerror(status));
      return 4;
    }
    CHECK(hipDeviceSynchronize());
    CHECK(hipMemcpy(ho, o, n * 2, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(hl, l, (size_t)B * H * N * 4, hipMemcpyDeviceToHost));
    if (oracle_attention_rows(hq, hk, hv, B, H, N, d, scale, causal, rows, (int64_t)B * H * N, ro, rl) != 0) return 5;
    double sum = 0.0;
    for (size_t i = 0; i < n; ++i) {
      const double e = fabs(from_bf16(ho[i]) - ro[i]);
      if (!(e <= 2e-2)) return 6;
      if (e > worst) worst = e;
      sum += e;
    }
    if (!(sum / (double)n <= 2e-3)) return 8;  /* mean absolute error bound */
    for (int64_t r = 0; r < (int64_t)B * H * N; ++r)
      if (!(fabs(hl[r] - rl[r]) <= 1e-4 * fmax(1.0, fabs(rl[r])))) return 7;
  }
  printf("ABI_DEMO OK max_abs=%.3e version=%d\n", worst, fa_version());
  hipFree(q), hipFree(k), hipFree(v), hipFree(o), hipFree(l);
  free(hq), free(hk), free(hv), free(ho), free(hl), free(rows), free(ro), free(rl);
  return 0;
}
