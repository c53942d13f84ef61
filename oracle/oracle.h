/*
 * CPU oracle for the NVFP4 Mixture-of-Experts hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the HIP library
 * against a plain, slow, obviously correct restatement of what the path
 * computes.  Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load it; the product path never does.  It shares no code,
 * header, table or helper with the HIP library.
 *
 * Arithmetic: exact decode of e2m1 / e4m3 codes, exact integer 16-element
 * block dot products, FP64 accumulation of the block terms, FP64 router
 * softmax, SwiGLU and FINALIZE.  The quantiser takes its rounding decisions in
 * IEEE binary32, the precision the quantised codes are defined in.
 *
 * Sources of each definition (web pages are cited by title and section):
 *  - FP4 E2M1 and FP8 E4M3 element encodings: OCP 8-bit Floating Point
 *    Specification (OFP8) rev 1.0 and OCP Microscaling Formats (MX) v1.0,
 *    section "Element data types".
 *  - Packed FP4 operands with one FP8 scale per 16 elements along K, for both
 *    operands: "Cracking the SM120 Shared Memory Ceiling", section "The Shared
 *    Memory Calculation" (the A/B tile and A/B scale terms).
 *  - One small GEMM per expert, grouped into one launch over a per-expert
 *    problem-size array: "Tracing the Failure: Debugging CUTLASS FP4 Tile
 *    Configurations on Blackwell SM120", section "Input Knowledge Required".
 *  - 256 experts, 8 active per token, ~32 rows per expert at decode: same page,
 *    section "The Broader Context".
 *  - NONE and FINALIZE epilogues, BF16 output: "The Epilogue That Broke the
 *    Kernel", section "The Insight: FINALIZE vs NONE".
 * Steps the pages leave open (routing softmax, the global scale, SwiGLU, the
 * requantisation and FINALIZE arithmetic) follow the readings recorded in the
 * design notes; each function below states the reading it implements.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Value of a 4-bit E2M1 code (bit 3 sign, bits 2:1 exponent, bit 0 mantissa). */
double orc_e2m1_value(int code);
/* Value of an 8-bit E4M3FN code (bias 7, no infinities); NaN codes give NaN. */
double orc_e4m3_value(int code);
/* Nearest E4M3FN code to t (0 <= t <= 448), ties to the even code. */
int orc_e4m3_round(float t);
/* Nearest E2M1 magnitude code (0..7) to u (0 <= u <= 6), ties to the even code. */
int orc_e2m1_round(float u);
/* bf16 bit pattern nearest to x (round to nearest, ties to even). */
uint16_t orc_bf16_round(double x);
/* Value of a bf16 bit pattern. */
double orc_bf16_value(uint16_t b);

/*
 * NVFP4 quantisation of x[rows, C] (C % 16 == 0), blocks of 16 along C.
 * dynamic != 0: g = amax(|x|) / 2688 (binary32), or 1 if amax is 0; *g_out = g.
 * dynamic == 0: g = g_in.
 * Per block: t = amax_b / (6 g); s = e4m3(min(t, 448)); u = |x| / (s g);
 * code = sign(x) | e2m1(min(u, 6)); blocks with s == 0 hold signed zeros.
 * Zero stays zero where g or s * g has underflowed to 0: a block whose maximum
 * is 0 gets s = 0 and a zero element gets magnitude code 0 (0 / 0 counts as 0);
 * a non-zero element over s * g == 0 saturates at 6.
 * q[rows, C/2]: element 2i in the low nibble of byte i.  sf[rows, C/16].
 */
void orc_quantize_nvfp4(const float *x, int64_t rows, int64_t C, int dynamic,
                        float g_in, uint8_t *q, uint8_t *sf, float *g_out);

/*
 * Top-k routing of logits[T, E]: the k largest logits of each token in
 * descending order, equal logits going to the lower expert id; weights are the
 * softmax over the k chosen logits (FP64).
 */
void orc_route(const float *logits, int T, int E, int k, int32_t *topk_ids,
               double *topk_w);

/*
 * Stable permutation of the T*k (token, slot) pairs into per-expert groups:
 * expert_offsets[E+1] is the exclusive prefix sum of the group sizes; within a
 * group the pairs keep their order t*k+j; row_src[p] is the token of permuted
 * row p and token_slot_row[t*k+j] the permuted row of pair (t, j).
 */
void orc_permute(const int32_t *topk_ids, int T, int E, int k,
                 int32_t *expert_offsets, int32_t *row_src,
                 int32_t *token_slot_row);

/*
 * Grouped NVFP4 GEMM, unrounded FP64 result for a list of permuted rows.
 * For permuted row p of expert e (offsets[e] <= p < offsets[e+1]) and column n:
 *   y = gA * gB[e] * sum_kb sA[r,kb] * sB[e,n,kb] * sum_{i<16} a[r,16kb+i] * b[e,n,16kb+i]
 * with r = A_rows ? A_rows[p] : p.  A is [*, K] NVFP4, B is [E, N, K] NVFP4.
 * rows[nrows] lists the permuted rows wanted; y is [nrows, N].
 */
void orc_grouped_gemm_rows(const uint8_t *A, const uint8_t *A_sf, float gA,
                           const int32_t *A_rows, const uint8_t *B,
                           const uint8_t *B_sf, const float *gB,
                           const int32_t *expert_offsets, int E, int N, int K,
                           const int32_t *rows, int64_t nrows, double *y);

/*
 * SwiGLU on y1[R, 2I] (gate = columns [0, I), up = columns [I, 2I)):
 * act = bf16(silu(bf16(gate)) * bf16(up)), silu(x) = x / (1 + exp(-x)) in FP64.
 */
void orc_swiglu(const double *y1, int64_t R, int I, uint16_t *act);

/*
 * FINALIZE: out[t, h] = sum_{j<k} w[t, j] * y2[token_slot_row[t*k+j], h],
 * summed in FP64 in slot order; out_f64 unrounded, out_bf16 rounded.
 */
void orc_finalize(const double *y2, const double *topk_w,
                  const int32_t *token_slot_row, int T, int k, int H,
                  double *out_f64, uint16_t *out_bf16);

/* Number of OpenMP threads the oracle runs on. */
int orc_num_threads(void);
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
