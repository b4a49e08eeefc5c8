/*
 * oracle.c - plain fp64 CPU reference for the decode-phase linear layer
 *            y[M x N] = x[M x K] . W^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the GPU path links, loads or calls
 * this file; only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * What it follows:
 *   - The linear layer y = x W, one row of x per token, written out as a
 *     matrix product ("Multi-GPU Inference and Serving at Scale", Example 2,
 *     a column split).  Weights here are stored one row per output
 *     (N x K), so the product is x . W^T.
 *   - Weight-only FP8 with 128x128 block scales and 16-bit activations:
 *     every weight is dequantized with the scale of the 128x128 block it
 *     falls in, activations are never quantized ("9% faster GLM-5.3-Flash
 *     prefill with GPU-to-GPU IPC (and why TileLang didn't help)", section
 *     "TileLang: twice as fast, and no faster"; "Developing a custom Qwen2.5
 *     72B inference engine from scratch", section 6.2).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - W is row-major N x K (K contiguous); x is M x K; y is M x N.
 *   - The scale of weight (n, k) is S[n / 128][k / 128], S row-major with
 *     ceil(K / 128) columns; edge blocks are partial and use their own scale.
 *   - FP8 is OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no
 *     infinities, S.1111.111 is NaN, largest finite value 448.
 *   - bf16 is the upper half of an IEEE binary32 pattern.
 *
 * Arithmetic: every input value is exact in fp64; each product x*w is exact
 * in fp64 (8 + 4 + 24 significant bits); the K-term sum is a left-to-right
 * fp64 sum.  Alongside y the oracle returns A[m][n] = sum_k |x[m][k] w[n][k]|,
 * the scale of the tolerance bound |y - y_ref| <= 2e-3 A + 1e-6.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Value of a bf16 code: the code is the upper 16 bits of a binary32. */
double oracle_bf16_value(uint16_t code) {
  uint32_t bits = (uint32_t)code << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Value of an OCP E4M3FN code, from the format definition. */
double oracle_e4m3_value(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  if (e == 0xF && m == 0x7) return NAN;
  double mag = (e == 0) ? ldexp((double)m / 8.0, -6)          /* subnormal */
                        : ldexp(1.0 + (double)m / 8.0, e - 7);  /* normal    */
  return sign ? -mag : mag;
}

typedef struct {
  int dtype;            /* 0 = bf16 weights, 1 = e4m3 weights + block scales */
  const uint16_t* x;    /* [M][K] bf16 codes */
  const void* w;        /* [N][K] bf16 codes or e4m3 codes */
  const float* scale;   /* [ceil(N/128)][ceil(K/128)] (fp8 only) */
  int64_t M, N, K;
  double* y;            /* [M][N] */
  double* absum;        /* [M][N] or NULL */
  int64_t n_begin, n_end;
  const double* xv;     /* x decoded to fp64, [M][K] */
} job_t;

static void* run_rows(void* arg) {
  job_t* j = (job_t*)arg;
  const int64_t K = j->K, M = j->M, N = j->N;
  const int64_t kblocks = (K + 127) / 128;
  double* wrow = (double*)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
  if (!wrow) return (void*)1;
  for (int64_t n = j->n_begin; n < j->n_end; ++n) {
    /* Weight row n as exact fp64 values. */
    for (int64_t k = 0; k < K; ++k) {
      if (j->dtype == 0) {
        wrow[k] = oracle_bf16_value(((const uint16_t*)j->w)[n * K + k]);
      } else {
        double s = (double)j->scale[(n / 128) * kblocks + (k / 128)];
        wrow[k] = oracle_e4m3_value(((const uint8_t*)j->w)[n * K + k]) * s;
      }
    }
    for (int64_t m = 0; m < M; ++m) {
      const double* xr = j->xv + m * K;
      double acc = 0.0, mag = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double p = xr[k] * wrow[k];
        acc += p;
        mag += fabs(p);
      }
      j->y[m * N + n] = acc;
      if (j->absum) j->absum[m * N + n] = mag;
    }
  }
  free(wrow);
  return NULL;
}

/* Common driver: decodes x, splits output rows over `threads` threads.
 * Returns the number of threads used, or -1 on bad arguments / allocation. */
static int linear_f64(int dtype, const uint16_t* x, const void* w, const float* scale,
                      int64_t M, int64_t N, int64_t K, double* y, double* absum,
                      int threads) {
  if (M < 0 || N < 0 || K < 0 || !y || (M * K > 0 && !x) || (N * K > 0 && !w)) return -1;
  if (dtype == 1 && N * K > 0 && !scale) return -1;
  if (threads < 1) threads = 1;
  if (threads > N) threads = N > 0 ? (int)N : 1;
  double* xv = (double*)malloc((size_t)(M * K > 0 ? M * K : 1) * sizeof(double));
  if (!xv) return -1;
  for (int64_t i = 0; i < M * K; ++i) xv[i] = oracle_bf16_value(x[i]);

  job_t* jobs = (job_t*)calloc((size_t)threads, sizeof(job_t));
  pthread_t* tids = (pthread_t*)calloc((size_t)threads, sizeof(pthread_t));
  if (!jobs || !tids) { free(xv); free(jobs); free(tids); return -1; }
  int failed = 0;
  for (int t = 0; t < threads; ++t) {
    job_t* j = &jobs[t];
    j->dtype = dtype; j->x = x; j->w = w; j->scale = scale;
    j->M = M; j->N = N; j->K = K; j->y = y; j->absum = absum; j->xv = xv;
    j->n_begin = N * t / threads;
    j->n_end = N * (t + 1) / threads;
  }
  /* Threads 1..T-1 run beside this one; thread 0's share runs here.
   * A thread that cannot be created has its share run here as well. */
  char* live = (char*)calloc((size_t)threads, 1);
  if (!live) { free(xv); free(jobs); free(tids); return -1; }
  for (int t = 1; t < threads; ++t)
    live[t] = pthread_create(&tids[t], NULL, run_rows, &jobs[t]) == 0;
  if (run_rows(&jobs[0]) != NULL) failed = 1;
  for (int t = 1; t < threads; ++t) {
    if (live[t]) {
      void* r = NULL;
      pthread_join(tids[t], &r);
      if (r != NULL) failed = 1;
    } else if (run_rows(&jobs[t]) != NULL) {
      failed = 1;
    }
  }
  free(live);
  free(xv); free(jobs); free(tids);
  return failed ? -1 : threads;
}

/* y[m][n] = sum_k x[m][k] * w[n][k], bf16 x and bf16 W, in fp64. */
int oracle_linear_bf16(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N,
                       int64_t K, double* y, double* absum, int threads) {
  return linear_f64(0, x, w, NULL, M, N, K, y, absum, threads);
}

/* y[m][n] = sum_k x[m][k] * e4m3(q[n][k]) * S[n/128][k/128], in fp64. */
int oracle_linear_fp8_bs128(const uint16_t* x, const uint8_t* q, const float* scale,
                            int64_t M, int64_t N, int64_t K, double* y, double* absum,
                            int threads) {
  return linear_f64(1, x, q, scale, M, N, K, y, absum, threads);
}
