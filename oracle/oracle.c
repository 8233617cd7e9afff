/*
 * Attention oracle: TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation of exact attention in
 * fp64.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * may load it; the GPU library never does, and the two share no code.
 *
 * What it computes (for every requested query row i of head (b, h)):
 *
 *   s_j   = scale * sum_c q[i][c] * k[j][c]          for every permitted key j
 *   m     = max_j s_j
 *   l     = sum_j exp(s_j - m)
 *   P_j   = exp(s_j - m) / l
 *   O[c]  = sum_j P_j * v[j][c]
 *   LSE   = m + ln(l)
 *
 * which is the attention rule softmax(Q K^T / sqrt(d)) V of "4 Triton and
 * Custom Kernels" (aisyseng.dev), section 4.7, equation 4.1, with the scale
 * passed in explicitly, evaluated with the "safe softmax" of the page
 * "FlashAttention and kernels" (gtadkapally.com), section "Softmax, the safe way" (subtract the row
 * maximum, then exponentiate, sum and divide).  The log-sum-exp side output is
 * the natural log of the softmax denominator of the scaled scores, L = m + log(l)
 * (same page, section "FlashAttention's forward pass", step 4).
 *
 * Permitted keys: all j in [0, N), or j <= i when causal (a token may attend to
 * itself and earlier tokens only; same page, its glossary entry "causal mask").
 *
 * The score row of each query is materialised in full before the softmax, as in
 * the naive three-step attention that "FlashAttention and kernels" contrasts with
 * FlashAttention (section "What naive attention actually does").  Sums run over ascending indices.
 * Inputs are 16-bit patterns of bfloat16 or of IEEE binary16 (fp16); widening
 * either to fp64 is exact.  Built without -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bfloat16 is the upper half of an IEEE binary32 value. */
static double oracle_bf16_to_f64(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent 0 holds zero and the subnormals f * 2^-24; exponent 31 holds the
 * infinities (f = 0) and NaNs; otherwise (1024 + f) * 2^(e - 25). */
static double oracle_f16_to_f64(uint16_t bits) {
  const int sign = bits >> 15, e = (bits >> 10) & 31, f = bits & 1023;
  double x;
  if (e == 0)
    x = ldexp((double)f, -24);
  else if (e == 31)
    x = f ? NAN : INFINITY;
  else
    x = ldexp((double)(1024 + f), e - 25);
  return sign ? -x : x;
}

/* dtype 0: bfloat16, 1: fp16. */
static double oracle_to_f64(uint16_t bits, int dtype) {
  return dtype ? oracle_f16_to_f64(bits) : oracle_bf16_to_f64(bits);
}

/* The element decoder on its own, so that tests can pin it. */
double oracle_element_to_f64(uint16_t bits, int dtype) { return oracle_to_f64(bits, dtype); }

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Nq query rows over Nk key rows per head (q [B, H, Nq, d], k and v [B, H, Nk, d]).
 * Permitted keys of query i: all j < Nk, or when causal j <= i as well (the
 * top-left alignment of the causal mask when Nq != Nk, the convention the
 * non-square causal check of "How to profile and optimise kernels" (dev.to,
 * Round 4, causal tile-skipping) compares against; every row keeps key 0).
 * rows: flat query row ids r = (b * H + h) * Nq + i, any order, each in
 * [0, B*H*Nq).  out: nrows * d doubles (row-major), lse: nrows doubles.
 * dtype: 0 = bfloat16 inputs, 1 = fp16 inputs.
 * Returns 0 on success, 1 on a bad argument, 2 if scratch memory is exhausted.
 */
int oracle_attention_rows_dt(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, double scale,
                             int causal, const int64_t *rows, int64_t nrows,
                             double *out, double *lse, int dtype) {
  if (!q || !k || !v || !rows || !out || !lse) return 1;
  if (dtype != 0 && dtype != 1) return 1;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0 || nrows < 0) return 1;
  const int64_t total_rows = B * H * Nq;
  for (int64_t t = 0; t < nrows; ++t)
    if (rows[t] < 0 || rows[t] >= total_rows) return 1;

  int failed = 0;
#pragma omp parallel
  {
    double *s = (double *)malloc((size_t)Nk * sizeof(double));
    double *qi = (double *)malloc((size_t)d * sizeof(double));
    if (!s || !qi) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t t = 0; t < nrows; ++t) {
        const int64_t r = rows[t];
        const int64_t head = r / Nq;     /* b * H + h */
        const int64_t i = r % Nq;        /* query position */
        const uint16_t *kh = k + head * Nk * d;
        const uint16_t *vh = v + head * Nk * d;
        /* keys 0 .. nkeys-1 */
        const int64_t nkeys = (causal && i + 1 < Nk) ? i + 1 : Nk;

        for (int64_t c = 0; c < d; ++c) qi[c] = oracle_to_f64(q[r * d + c], dtype);

        /* 1. scores of the permitted keys */
        for (int64_t j = 0; j < nkeys; ++j) {
          double acc = 0.0;
          for (int64_t c = 0; c < d; ++c) acc += qi[c] * oracle_to_f64(kh[j * d + c], dtype);
          s[j] = scale * acc;
        }
        /* 2. row maximum */
        double m = s[0];
        for (int64_t j = 1; j < nkeys; ++j)
          if (s[j] > m) m = s[j];
        /* 3. denominator */
        double l = 0.0;
        for (int64_t j = 0; j < nkeys; ++j) l += exp(s[j] - m);
        /* 4. probabilities, 5. weighted sum of the value rows */
        double *o = out + t * d;
        for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
        for (int64_t j = 0; j < nkeys; ++j) {
          const double p = exp(s[j] - m) / l;
          for (int64_t c = 0; c < d; ++c) o[c] += p * oracle_to_f64(vh[j * d + c], dtype);
        }
        /* 6. log-sum-exp of the scaled scores, natural log */
        lse[t] = m + log(l);
      }
    }
    free(s);
    free(qi);
  }
  return failed ? 2 : 0;
}

/*
 * The same definition for fp32 inputs (q [B, H, Nq, d], k and v [B, H, Nk, d]
 * as IEEE binary32 values; widening to fp64 is exact).  Arguments and return
 * codes as oracle_attention_rows_dt.
 */
int oracle_attention_rows_f32(const float *q, const float *k, const float *v,
                              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, double scale,
                              int causal, const int64_t *rows, int64_t nrows,
                              double *out, double *lse) {
  if (!q || !k || !v || !rows || !out || !lse) return 1;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0 || nrows < 0) return 1;
  const int64_t total_rows = B * H * Nq;
  for (int64_t t = 0; t < nrows; ++t)
    if (rows[t] < 0 || rows[t] >= total_rows) return 1;
  int failed = 0;
#pragma omp parallel
  {
    double *s = (double *)malloc((size_t)Nk * sizeof(double));
    if (!s) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t t = 0; t < nrows; ++t) {
        const int64_t r = rows[t], head = r / Nq, i = r % Nq;
        const float *qi = q + r * d, *kh = k + head * Nk * d, *vh = v + head * Nk * d;
        const int64_t nkeys = (causal && i + 1 < Nk) ? i + 1 : Nk;
        for (int64_t j = 0; j < nkeys; ++j) {
          double acc = 0.0;
          for (int64_t c = 0; c < d; ++c) acc += (double)qi[c] * (double)kh[j * d + c];
          s[j] = scale * acc;
        }
        double m = s[0];
        for (int64_t j = 1; j < nkeys; ++j)
          if (s[j] > m) m = s[j];
        double l = 0.0;
        for (int64_t j = 0; j < nkeys; ++j) l += exp(s[j] - m);
        double *o = out + t * d;
        for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
        for (int64_t j = 0; j < nkeys; ++j) {
          const double p = exp(s[j] - m) / l;
          for (int64_t c = 0; c < d; ++c) o[c] += p * (double)vh[j * d + c];
        }
        lse[t] = m + log(l);
      }
    }
    free(s);
  }
  return failed ? 2 : 0;
}

/* bfloat16 inputs. */
int oracle_attention_rows_qk(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, double scale,
                             int causal, const int64_t *rows, int64_t nrows,
                             double *out, double *lse) {
  return oracle_attention_rows_dt(q, k, v, B, H, Nq, Nk, d, scale, causal, rows, nrows, out, lse, 0);
}

/* The square case, N queries over N keys: rows r = (b * H + h) * N + i. */
int oracle_attention_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          int64_t B, int64_t H, int64_t N, int64_t d, double scale,
                          int causal, const int64_t *rows, int64_t nrows,
                          double *out, double *lse) {
  return oracle_attention_rows_qk(q, k, v, B, H, N, N, d, scale, causal, rows, nrows, out, lse);
}

/*
 * Gradients of the attention rule with respect to q, k and v, for an upstream
 * gradient dout of the output: the derivative of sum(dout . out) written out
 * through the chain rule (the backward pass FlashAttention recomputes from the
 * saved log-sum-exp: "FlashAttention and kernels" (gtadkapally.com), section
 * "FlashAttention-2, -3, and what came after", and "Kernels and FlashAttention"
 * (prathameshsaraf.com), on keeping L for the backward pass):
 *
 *   P_ij  = softmax_j(scale q_i . k_j)  over the permitted keys (causal: j <= i)
 *   dV_j  = sum_i P_ij dout_i
 *   dP_ij = dout_i . v_j
 *   D_i   = sum_j P_ij dP_ij
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale sum_j dS_ij k_j,    dK_j = scale sum_i dS_ij q_i
 *
 * Nq query rows over Nk key rows: q, dout (and dq) contiguous [B, H, Nq, d],
 * k, v (and dk, dv) contiguous [B, H, Nk, d], of bfloat16 (dtype 0) or fp16
 * (dtype 1); dq, dk, dv are doubles.  The permitted keys are those of the
 * forward oracle: all of them, or when causal j <= i (top-left alignment, so
 * with Nq < Nk the keys j >= Nq are never permitted and their gradients are 0).
 * One score row at a time (no Nq x Nk buffer): the dQ row is finished per
 * query, dK and dV accumulate over queries; each head is one OpenMP task, so
 * accumulation order is fixed.  Returns 0, 1 on a bad argument, 2 if scratch
 * memory is exhausted.
 */
int oracle_attention_bwd_qk(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                            int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, double scale, int causal,
                            double *dq, double *dk, double *dv, int dtype) {
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return 1;
  if (dtype != 0 && dtype != 1) return 1;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return 1;
  int failed = 0;
#pragma omp parallel
  {
    double *p = (double *)malloc((size_t)Nk * sizeof(double));
    double *dp = (double *)malloc((size_t)Nk * sizeof(double));
    double *qi = (double *)malloc((size_t)d * sizeof(double));
    double *gi = (double *)malloc((size_t)d * sizeof(double));
    if (!p || !dp || !qi || !gi) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t head = 0; head < B * H; ++head) {
        const uint16_t *qh = q + head * Nq * d, *kh = k + head * Nk * d;
        const uint16_t *vh = v + head * Nk * d, *gh = dout + head * Nq * d;
        double *dqh = dq + head * Nq * d, *dkh = dk + head * Nk * d, *dvh = dv + head * Nk * d;
        for (int64_t x = 0; x < Nk * d; ++x) dkh[x] = dvh[x] = 0.0;
        for (int64_t i = 0; i < Nq; ++i) {
          const int64_t nkeys = (causal && i + 1 < Nk) ? i + 1 : Nk;
          for (int64_t c = 0; c < d; ++c) {
            qi[c] = oracle_to_f64(qh[i * d + c], dtype);
            gi[c] = oracle_to_f64(gh[i * d + c], dtype);
          }
          /* probabilities of row i (the forward's definition) */
          double m = -INFINITY;
          for (int64_t j = 0; j < nkeys; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < d; ++c) acc += qi[c] * oracle_to_f64(kh[j * d + c], dtype);
            p[j] = scale * acc;
            if (p[j] > m) m = p[j];
          }
          double l = 0.0;
          for (int64_t j = 0; j < nkeys; ++j) l += exp(p[j] - m);
          for (int64_t j = 0; j < nkeys; ++j) p[j] = exp(p[j] - m) / l;
          /* dP_ij = dout_i . v_j and D_i = sum_j P_ij dP_ij */
          double D = 0.0;
          for (int64_t j = 0; j < nkeys; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < d; ++c) acc += gi[c] * oracle_to_f64(vh[j * d + c], dtype);
            dp[j] = acc;
            D += p[j] * acc;
          }
          for (int64_t c = 0; c < d; ++c) dqh[i * d + c] = 0.0;
          for (int64_t j = 0; j < nkeys; ++j) {
            const double ds = p[j] * (dp[j] - D);
            for (int64_t c = 0; c < d; ++c) {
              dvh[j * d + c] += p[j] * gi[c];
              dqh[i * d + c] += scale * ds * oracle_to_f64(kh[j * d + c], dtype);
              dkh[j * d + c] += scale * ds * qi[c];
            }
          }
        }
      }
    }
    free(p);
    free(dp);
    free(qi);
    free(gi);
  }
  return failed ? 2 : 0;
}

/* Square heads, N queries over N keys. */
int oracle_attention_bwd_dt(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                            int64_t B, int64_t H, int64_t N, int64_t d, double scale, int causal,
                            double *dq, double *dk, double *dv, int dtype) {
  return oracle_attention_bwd_qk(q, k, v, dout, B, H, N, N, d, scale, causal, dq, dk, dv, dtype);
}

/* bfloat16 inputs. */
int oracle_attention_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                         int64_t B, int64_t H, int64_t N, int64_t d, double scale, int causal,
                         double *dq, double *dk, double *dv) {
  return oracle_attention_bwd_dt(q, k, v, dout, B, H, N, d, scale, causal, dq, dk, dv, 0);
}
