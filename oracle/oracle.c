/*
 * CPU oracle for the NVFP4 Mixture-of-Experts hot path.  TEST INFRASTRUCTURE
 * ONLY: loaded by the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark, never by the product path.  See oracle.h for the definitions
 * and their sources.  Plain loops, no blocking; OpenMP only splits independent
 * outer iterations.  Build with -ffp-contract=off so that every binary32 step of
 * the quantiser is a single correctly rounded operation.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- element formats (OCP OFP8 rev 1.0; OCP MX v1.0 "Element data types") ---- */

double orc_e2m1_value(int code) {
  /* E2M1: exponent bias 1; exponent 0 is the subnormal range 0.5 * m. */
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

double orc_e4m3_value(int code) {
  /* E4M3FN: exponent bias 7, exponent 0 subnormal, S.1111.111 is NaN, no inf. */
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* Magnitude tables, filled from the decode functions above when the library
 * is loaded. */
static double e4m3_mag[127], e2m1_mag[8];
static double e4m3_all[256];   /* value of every E4M3 code */
static int e2m1_twice_all[16]; /* twice the value of every E2M1 code: an integer */

__attribute__((constructor)) static void fill_tables(void) {
  for (int c = 0; c < 127; c++) e4m3_mag[c] = orc_e4m3_value(c);
  for (int c = 0; c < 8; c++) e2m1_mag[c] = orc_e2m1_value(c);
  for (int c = 0; c < 256; c++) e4m3_all[c] = orc_e4m3_value(c);
  for (int c = 0; c < 16; c++) e2m1_twice_all[c] = (int)(2.0 * orc_e2m1_value(c));
}

/* Nearest of the increasing magnitudes mag[0..n-1] to x >= 0, ties to the even
 * code; x above the largest magnitude maps to the largest code. */
static int nearest_even(double x, const double *mag, int n) {
  int lo = 0, hi = n - 1;            /* invariant: mag[lo] <= x, or lo == 0 */
  if (x >= mag[hi]) return hi;
  while (hi - lo > 1) {              /* find lo with mag[lo] <= x < mag[lo+1] */
    int mid = (lo + hi) / 2;
    if (mag[mid] <= x) lo = mid; else hi = mid;
  }
  double dl = x - mag[lo], du = mag[lo + 1] - x;
  if (dl < du) return lo;
  if (du < dl) return lo + 1;
  return (lo % 2 == 0) ? lo : lo + 1;
}

int orc_e4m3_round(float t) {
  return nearest_even((double)t, e4m3_mag, 127);
}
int orc_e2m1_round(float u) {
  return nearest_even((double)u, e2m1_mag, 8);
}

uint16_t orc_bf16_round(double x) {
  /* bf16 keeps 8 significant bits and binary32's exponent range. */
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isnan(x)) return 0x7FC0;
  int ex;
  frexp(a, &ex);                 /* a = f * 2^ex, f in [0.5, 1) */
  int ulp_exp = ex - 8;          /* 8 significant bits */
  if (ulp_exp < -133) ulp_exp = -133; /* bf16 subnormal spacing 2^-133 */
  double q = ldexp(a, -ulp_exp); /* exact */
  double r = nearbyint(q);       /* default rounding mode: nearest, ties to even */
  double v = ldexp(r, ulp_exp);
  float f = (float)v;            /* exact: v is a bf16 value (or overflows to inf) */
  uint32_t bits;
  memcpy(&bits, &f, 4);
  return (uint16_t)(sign | ((bits >> 16) & 0x7FFF));
}

double orc_bf16_value(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

/* ---- NVFP4 quantisation ---- */

void orc_quantize_nvfp4(const float *x, int64_t rows, int64_t C, int dynamic,
                        float g_in, uint8_t *q, uint8_t *sf, float *g_out) {
  float g = g_in;
  if (dynamic) {
    float amax = 0.0f;
    for (int64_t i = 0; i < rows * C; i++) {
      float a = fabsf(x[i]);
      if (a > amax) amax = a;
    }
    g = (amax > 0.0f) ? amax / 2688.0f : 1.0f;   /* 2688 = 6 * 448 */
    if (g_out) *g_out = g;
  }
  const float six_g = 6.0f * g;
  const int64_t nblk = C / 16;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    for (int64_t b = 0; b < nblk; b++) {
      const float *xb = x + r * C + b * 16;
      float amax_b = 0.0f;
      for (int i = 0; i < 16; i++) {
        float a = fabsf(xb[i]);
        if (a > amax_b) amax_b = a;
      }
      /* a zero block has scale 0 even when 6 g is 0 (an underflowed g): 0 / 0
       * counts as 0, not NaN */
      float t = (amax_b > 0.0f) ? amax_b / six_g : 0.0f;
      if (t > 448.0f) t = 448.0f;
      int s = orc_e4m3_round(t);
      sf[r * nblk + b] = (uint8_t)s;
      float s_val = (float)orc_e4m3_value(s);
      float sg = s_val * g;
      for (int i = 0; i < 16; i += 2) {
        int code[2];
        for (int h = 0; h < 2; h++) {
          float v = xb[i + h];
          int sign = signbit(v) ? 8 : 0;
          int mag = 0;
          /* a zero element has code 0 even when s * g underflows to 0 (0 / 0
           * counts as 0); a non-zero element over a zero s * g saturates at 6 */
          if (s_val != 0.0f && fabsf(v) > 0.0f) {
            float u = fabsf(v) / sg;
            if (u > 6.0f) u = 6.0f;
            mag = orc_e2m1_round(u);
          }
          code[h] = sign | mag;
        }
        q[r * (C / 2) + b * 8 + i / 2] = (uint8_t)(code[0] | (code[1] << 4));
      }
    }
  }
}

/* ---- routing ---- */

void orc_route(const float *logits, int T, int E, int k, int32_t *topk_ids,
               double *topk_w) {
#pragma omp parallel
  {
    char *taken = (char *)malloc((size_t)E);
#pragma omp for schedule(static)
    for (int t = 0; t < T; t++) {
      const float *L = logits + (int64_t)t * E;
      memset(taken, 0, (size_t)E);
      for (int j = 0; j < k; j++) {
        int best = -1;
        for (int e = 0; e < E; e++) {
          if (taken[e]) continue;
          /* scanning ids upward, a strictly larger logit is needed to replace
           * the current best: equal logits keep the lower id */
          if (best < 0 || L[e] > L[best]) best = e;
        }
        taken[best] = 1;
        topk_ids[(int64_t)t * k + j] = best;
      }
      double l0 = (double)L[topk_ids[(int64_t)t * k]];
      double denom = 0.0;
      for (int j = 0; j < k; j++) denom += exp((double)L[topk_ids[(int64_t)t * k + j]] - l0);
      for (int j = 0; j < k; j++)
        topk_w[(int64_t)t * k + j] = exp((double)L[topk_ids[(int64_t)t * k + j]] - l0) / denom;
    }
    free(taken);
  }
}

void orc_permute(const int32_t *topk_ids, int T, int E, int k,
                 int32_t *expert_offsets, int32_t *row_src,
                 int32_t *token_slot_row) {
  int64_t n = (int64_t)T * k;
  int64_t *next = (int64_t *)calloc((size_t)E + 1, sizeof(int64_t));
  for (int64_t i = 0; i < n; i++) next[topk_ids[i] + 1]++;
  for (int e = 0; e < E; e++) next[e + 1] += next[e];
  for (int e = 0; e <= E; e++) expert_offsets[e] = (int32_t)next[e];
  for (int64_t i = 0; i < n; i++) {
    int64_t p = next[topk_ids[i]]++;
    row_src[p] = (int32_t)(i / k);
    token_slot_row[i] = (int32_t)p;
  }
  free(next);
}

/* ---- grouped GEMM ---- */

/* Sum over one 16-element block of the products of doubled E2M1 values: an exact
 * integer, |P| <= 16 * 12 * 12 = 2304. */
static inline int block_dot(const int16_t *a, const int16_t *b) {
  int P = 0;
  for (int i = 0; i < 16; i++) P += a[i] * b[i];
  return P;
}

/* Decode one NVFP4 row of K elements into doubled integer values and FP64 block scales. */
static void decode_row(const uint8_t *q, const uint8_t *sf, int K, int16_t *v2, double *s) {
  for (int c = 0; c < K; c++) {
    uint8_t byte = q[c / 2];
    v2[c] = (int16_t)e2m1_twice_all[(c & 1) ? (byte >> 4) : (byte & 15)];
  }
  for (int b = 0; b < K / 16; b++) s[b] = e4m3_all[sf[b]];
}

void orc_grouped_gemm_rows(const uint8_t *A, const uint8_t *A_sf, float gA,
                           const int32_t *A_rows, const uint8_t *B,
                           const uint8_t *B_sf, const float *gB,
                           const int32_t *expert_offsets, int E, int N, int K,
                           const int32_t *rows, int64_t nrows, double *y) {
  const int nkb = K / 16;
  int64_t *mine = (int64_t *)malloc((size_t)(nrows > 0 ? nrows : 1) * sizeof(int64_t));
  int16_t *av = (int16_t *)malloc((size_t)(nrows > 0 ? nrows : 1) * K * sizeof(int16_t));
  double *as = (double *)malloc((size_t)(nrows > 0 ? nrows : 1) * nkb * sizeof(double));
  for (int e = 0; e < E; e++) {
    /* the requested rows that belong to expert e, decoded once */
    int64_t cnt = 0;
    for (int64_t i = 0; i < nrows; i++)
      if (rows[i] >= expert_offsets[e] && rows[i] < expert_offsets[e + 1]) mine[cnt++] = i;
    if (cnt == 0) continue;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < cnt; i++) {
      int64_t p = rows[mine[i]];
      int64_t r = A_rows ? A_rows[p] : p;
      decode_row(A + r * (K / 2), A_sf + r * nkb, K, av + i * K, as + i * nkb);
    }
    const uint8_t *Be = B + (int64_t)e * N * (K / 2);
    const uint8_t *Bse = B_sf + (int64_t)e * N * nkb;
    const double gscale = (double)gA * (double)gB[e];
    /* every output y[p, n] is computed by the same sequence of operations; the loops
     * only choose the order in which independent outputs are produced */
#pragma omp parallel
    {
      int16_t *bv = (int16_t *)malloc((size_t)K * sizeof(int16_t));
      double *bs = (double *)malloc((size_t)nkb * sizeof(double));
#pragma omp for schedule(static)
      for (int n = 0; n < N; n++) {
        decode_row(Be + (int64_t)n * (K / 2), Bse + (int64_t)n * nkb, K, bv, bs);
        for (int64_t i = 0; i < cnt; i++) {
          const int16_t *a = av + i * K;
          const double *sa = as + i * nkb;
          double acc = 0.0;
          for (int kb = 0; kb < nkb; kb++) {
            int P = block_dot(a + kb * 16, bv + kb * 16);
            acc += (double)P * sa[kb] * bs[kb] * 0.25;
          }
          y[mine[i] * (int64_t)N + n] = acc * gscale;
        }
      }
      free(bv);
      free(bs);
    }
  }
  free(mine);
  free(av);
  free(as);
}

/* ---- SwiGLU and FINALIZE ---- */

void orc_swiglu(const double *y1, int64_t R, int I, uint16_t *act) {
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < R; p++) {
    for (int i = 0; i < I; i++) {
      double gate = orc_bf16_value(orc_bf16_round(y1[p * 2 * I + i]));
      double up = orc_bf16_value(orc_bf16_round(y1[p * 2 * I + I + i]));
      double silu = gate / (1.0 + exp(-gate));
      act[p * I + i] = orc_bf16_round(silu * up);
    }
  }
}

void orc_finalize(const double *y2, const double *topk_w,
                  const int32_t *token_slot_row, int T, int k, int H,
                  double *out_f64, uint16_t *out_bf16) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; t++) {
    for (int h = 0; h < H; h++) {
      double acc = 0.0;
      for (int j = 0; j < k; j++) {
        int64_t p = token_slot_row[(int64_t)t * k + j];
        acc += topk_w[(int64_t)t * k + j] * y2[p * H + h];
      }
      if (out_f64) out_f64[(int64_t)t * H + h] = acc;
      if (out_bf16) out_bf16[(int64_t)t * H + h] = orc_bf16_round(acc);
    }
  }
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Thread count for the following calls (timing on one thread versus all cores). */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
