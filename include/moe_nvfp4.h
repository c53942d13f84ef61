/*
 * moe_nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 Mixture-of-Experts hot path.
 *
 * The path, for one MoE layer of T tokens, E experts, top-k routing, hidden H and
 * expert intermediate I:
 *   1. moe_route_permute   top-k routing of the router logits and the stable
 *                          permutation of the T*k (token, slot) pairs into
 *                          per-expert groups;
 *   2. moe_quantize_nvfp4  NVFP4 quantisation of the bf16 token activations;
 *   3. moe_grouped_gemm_nvfp4 (MOE_EPI_SWIGLU)  gate/up GEMM over the groups,
 *                          gathering token rows, with SwiGLU in the epilogue;
 *   4. moe_quantize_nvfp4  requantisation of the SwiGLU output;
 *   5. moe_grouped_gemm_nvfp4 (MOE_EPI_NONE)  down GEMM into a bf16 workspace;
 *   6. moe_finalize        router-weighted gather-reduce of each token's k rows
 *                          into the bf16 output.
 *
 * Sources (web pages cited by title and section):
 *  - Operands are FP4 E2M1 with one FP8 scale per 16 elements along the
 *    contraction dimension for both operands, BF16 output: "Cracking the SM120
 *    Shared Memory Ceiling", section "The Shared Memory Calculation"; the FP4 x
 *    FP4 -> BF16 kernel instantiation quoted in "The CUTLASS Tile That Wouldn't
 *    Fit: Debugging EP8 on Blackwell SM120", section "The Crash: A Deep-Dive into CUTLASS Tile Geometry".
 *  - Many small per-expert GEMMs in one launch driven by a per-expert
 *    problem-size array: "Tracing the Failure: Debugging CUTLASS FP4 Tile
 *    Configurations on Blackwell SM120", section "Input Knowledge Required".
 *  - 256 experts, 8 active per token, about 32 rows per expert at decode, GEMMs
 *    of about 32 x 2048 x 6144: same page, section "The Broader Context".
 *  - NONE (pass-through) and FINALIZE epilogues: "The Epilogue That Broke the
 *    Kernel", section "The Insight: FINALIZE vs NONE".
 *  - A truthful can-implement check, a workspace query and no exception across
 *    the interface: the failure traced in "Cracking the SM120 Shared Memory
 *    Ceiling", section "Tracing the Failure" (the check passed, initialisation
 *    then failed) and the warmup exception in "The CUTLASS Tile That Wouldn't
 *    Fit: Debugging EP8 on Blackwell SM120", section "The Crash: A Deep-Dive into CUTLASS Tile Geometry".
 *  - E2M1 / E4M3 encodings: OCP OFP8 rev 1.0 and OCP MX v1.0.
 *
 * Conventions for every entry point:
 *  - Every data pointer is a DEVICE pointer on the current HIP device, owned by
 *    the caller; the library allocates no device memory, keeps no pointer after
 *    it returns and holds no global state apart from a thread-local last HIP
 *    error code and the static scratch array of moe_grouped_gemm_nvfp4_noalloc
 *    (section 3a).  Tensor base pointers are 16-byte aligned (as every device
 *    allocation is) and tensors are dense, row-major.
 *  - Work is enqueued asynchronously on `stream` (0 = the null stream); no call
 *    synchronises with the device or copies device data to the host.
 *  - Arguments are validated on the host before any HIP call; failures return a
 *    status and enqueue nothing.  Nothing throws or aborts across the ABI.
 *  - Device-data invariants (expert ids in range, monotone offsets, finite
 *    values) are the caller's contract; indices read from device memory are
 *    clamped so that bad values cannot make a kernel access memory out of
 *    bounds.
 *  - Results are deterministic: no floating-point atomics; repeated calls on the
 *    same inputs produce identical bytes.
 *  - Element layout of NVFP4 tensors [rows, C]: codes [rows, C/2] bytes, element
 *    2i in the low nibble of byte i and 2i+1 in the high nibble; scales
 *    [rows, C/16] E4M3FN bytes (bias 7, max 448); one FP32 global scale g; the
 *    value of an element is e2m1(code) * e4m3(scale) * g.
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,       /* a size is negative, inconsistent or out of range */
  MOE_ERR_UNSUPPORTED = 3, /* valid but not supported by the kernels (e.g. K % 256) */
  MOE_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than the query returned */
  MOE_ERR_HIP = 5          /* a HIP launch failed; see moe_last_hip_error() */
} moe_status;

/* Static description of a status; never NULL. */
const char *moe_status_string(moe_status s);
/* hipError_t of the last MOE_ERR_HIP returned on the calling thread (0 if none). */
int moe_last_hip_error(void);

/* ---------------------------------------------------------------------------
 * 1. Routing and permutation.
 *
 * Defined by: the layer the pages measure routes every token to 8 of 256 experts, so
 * that at 1024 concurrent requests each expert sees about 32 rows ("Tracing the
 * Failure: Debugging CUTLASS FP4 Tile Configurations on Blackwell SM120", section "The
 * Broader Context"; "Peering into the Kernel", section "Input Knowledge Required"); the
 * grouped GEMM then runs one small GEMM per expert over a per-expert size array (same
 * first page, section "Input Knowledge Required").  The pages fix neither the router
 * arithmetic nor the row order, so this call takes the plainest readings: softmax over
 * the chosen logits, ties to the lower id, rows of a group in token order.
 * logits [T, E] f32 row-major.  For each token the k largest logits are taken in
 * descending order, equal logits going to the lower expert id:
 *   topk_ids [T, k] i32, topk_w [T, k] f32 = softmax over the k chosen logits
 *   (the renormalised top-k of the full softmax).
 * The T*k pairs (t, j), in the order t*k + j, are then grouped by expert, stably:
 *   expert_offsets [E+1] i32  exclusive prefix sum of the group sizes
 *                             (expert_offsets[E] = T*k);
 *   row_src [T*k] i32         token of permuted row p;
 *   token_slot_row [T*k] i32  permuted row of pair (t, j).
 * Limits: 0 <= T, 1 <= E <= 1024, 1 <= k <= min(E, 32), T*k < 2^31.
 * ws: at least moe_route_permute_workspace(T, E, k) bytes of device memory
 * (contents on entry irrelevant).
 * ------------------------------------------------------------------------- */
size_t moe_route_permute_workspace(int T, int E, int k);
moe_status moe_route_permute(const float *logits, int T, int E, int k, int32_t *topk_ids,
                             float *topk_w, int32_t *expert_offsets, int32_t *row_src,
                             int32_t *token_slot_row, void *ws, size_t ws_bytes,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------
 * 2. NVFP4 quantisation of x [rows, C] (C % 16 == 0), blocks of 16 along C.
 *
 * Defined by: the operand format the pages budget shared memory for -- packed 4-bit
 * elements and one 8-bit FP8 scale per 16 elements along K, for both operands
 * ("Cracking the SM120 Shared Memory Ceiling", sections "The Shared Memory
 * Calculation" and "Input Knowledge Required").  The pages give no quantisation
 * recipe; the global scale, the rounding of the block scale and of the elements below
 * are this library's readings (round to nearest even, saturating).
 * x_dtype: MOE_DTYPE_BF16 (x is uint16 bf16 bit patterns) or MOE_DTYPE_F32.
 * gs_mode MOE_GS_DYNAMIC: g = amax / 2688 in binary32 (1 if amax is 0), written
 *   to *gs; amax is max|x| over the whole tensor, or, when amax_in is not NULL,
 *   the maximum of |amax_in[i]| over its n_amax_in entries (e.g. the partial maxima
 *   a SwiGLU GEMM wrote; 0 entries give amax 0).
 * gs_mode MOE_GS_STATIC: g is read from *gs.
 * Then per block b: t = amax_b / (6 g), s = e4m3(min(t, 448)) (round to nearest
 * even), and per element u = |x| / (s g), code = sign(x) | e2m1(min(u, 6))
 * (round to nearest even); a block with s = 0 holds signed zeros.  Zero stays zero
 * where g or s g has underflowed to 0: 0 / 0 counts as 0 (a zero block gets s = 0, a zero
 * element magnitude code 0), a non-zero element over s g = 0 saturates at 6.  Every step
 * is a correctly rounded binary32 operation, so the output is bit-exact.
 * q [rows, C/2] u8, sf [rows, C/16] u8, gs: one f32.
 * Limits: rows >= 0, C >= 16, rows*C < 2^40.  ws: moe_quantize_nvfp4_workspace().
 * ------------------------------------------------------------------------- */
enum { MOE_DTYPE_BF16 = 0, MOE_DTYPE_F32 = 1 };
enum { MOE_GS_STATIC = 0, MOE_GS_DYNAMIC = 1 };
size_t moe_quantize_nvfp4_workspace(int64_t rows, int64_t C);
moe_status moe_quantize_nvfp4(const void *x, int x_dtype, int64_t rows, int64_t C, uint8_t *q,
                              uint8_t *sf, float *gs, int gs_mode, const float *amax_in,
                              int64_t n_amax_in, void *ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * 3. Grouped NVFP4 GEMM.
 *
 * Defined by: FP4 x FP4 -> BF16 block-scaled GEMMs, one per expert, in one grouped
 * launch over a per-expert problem-size array ("Tracing the Failure: Debugging CUTLASS
 * FP4 Tile Configurations on Blackwell SM120", sections "The Broader Context" and "Input
 * Knowledge Required"; the kernel instantiation in "The CUTLASS Tile That Wouldn't Fit:
 * Debugging EP8 on Blackwell SM120", section "The Crash: A Deep-Dive into CUTLASS Tile
 * Geometry"), with the NONE pass-through epilogue ("The Epilogue That Broke the Kernel",
 * section "The Insight: FINALIZE vs NONE").  SwiGLU between the two projections is this
 * library's reading of the expert MLP (gate columns first).  The can-implement check is
 * exact, unlike the one traced in "Cracking the SM120 Shared Memory Ceiling", section
 * "Tracing the Failure", which passed a configuration that then failed to initialise.
 * For expert e and permuted row p in [expert_offsets[e], expert_offsets[e+1]):
 *   y[p, n] = gA * gB[e] * sum_kb sA[r, kb] sB[e, n, kb] sum_{i<16} a[r, 16kb+i] b[e, n, 16kb+i]
 * with r = A_rows ? A_rows[p] : p.  Products are exact (fp16 MFMA on operands
 * dequantised exactly), sums are binary32.
 *   A [rows_A, K] NVFP4 (A, A_sf, *A_gs), B [E, N, K] NVFP4 (B, B_sf, B_gs[E]),
 *   expert_offsets [E+1] i32 on the device (group sizes are never read on the
 *   host), R = the number of permuted rows (the row capacity of D).
 * Epilogues:
 *   MOE_EPI_NONE    D bf16 [R, N]: D[p, n] = bf16(y[p, n]).
 *   MOE_EPI_SWIGLU  N = 2I; columns [0, I) are gate, [I, 2I) are up;
 *                   D bf16 [R, I]: D[p, i] = bf16(silu(bf16(y[p, i])) * bf16(y[p, I+i]))
 *                   with silu(x) = x / (1 + exp(-x)) in binary32 (hardware exp2 and
 *                   reciprocal: a few ulp of binary32), and
 *                   amax_out[moe_grouped_gemm_nvfp4_amax_slots(args)] f32 receives
 *                   partial maxima of |D| (their maximum is max|D|; unused slots 0),
 *                   for moe_quantize_nvfp4(..., amax_in = amax_out, ...).
 *   MOE_EPI_SWIGLU_NVFP4  the SwiGLU epilogue fused with NVFP4 quantisation of its bf16
 *                   result under a static, caller-calibrated global scale g2 = *D_gs
 *                   (device f32): D u8 [R, I/2] codes, D_sf u8 [R, I/16] E4M3 scales, with
 *                   exactly the steps of moe_quantize_nvfp4 in MOE_GS_STATIC mode (the
 *                   output equals SWIGLU followed by that call byte for byte).  A fused
 *                   gate/up epilogue that requantises in one pass is the "next" step after
 *                   the pages' FINALIZE/NONE epilogue modes ("The Epilogue That Broke the
 *                   Kernel", "The Insight: FINALIZE vs NONE"); the static scale replaces the
 *                   dynamic per-tensor amax, which needs a pass over all rows.  Packed
 *                   weights only; amax_out is not used.
 * Rows p >= expert_offsets[E] of D are not written.
 * B_layout MOE_LAYOUT_ROWMAJOR: B / B_sf as above.  MOE_LAYOUT_PACKED: B is the output of
 * moe_pack_weights_nvfp4 for the E*N weight rows (B_sf is ignored and may be NULL); this is
 * the layout the decode kernels stream with fully coalesced loads.
 * Supported: K % 256 == 0, N % 256 == 0, 1 <= E <= 65536, 0 <= R < 2^31; with the packed
 * layout also rows_A * K / 2 <= 2^31 - 4096 and N * K * 9 / 16 <= 2^31 - 4096 (one expert's
 * packed weights), MOE_ERR_UNSUPPORTED otherwise.
 * moe_grouped_gemm_nvfp4_can_implement() returns MOE_OK exactly when the
 * launch is supported; a supported launch then cannot fail on its
 * configuration.  ws: moe_grouped_gemm_nvfp4_workspace(args) bytes.  The
 * workspace and amax-slot queries read the shapes, layout and epilogue only (the
 * pointers may still be NULL, so they can size buffers before allocation): they
 * return 0 exactly when can_implement fails for a reason other than a NULL pointer.
 * ------------------------------------------------------------------------- */
typedef enum moe_epilogue { MOE_EPI_NONE = 0, MOE_EPI_SWIGLU = 1, MOE_EPI_SWIGLU_NVFP4 = 2 } moe_epilogue;
typedef enum moe_layout { MOE_LAYOUT_ROWMAJOR = 0, MOE_LAYOUT_PACKED = 1 } moe_layout;

typedef struct moe_gemm_args {
  const uint8_t *A;               /* [rows_A, K/2] */
  const uint8_t *A_sf;            /* [rows_A, K/16] */
  const float *A_gs;              /* one f32 */
  const int32_t *A_rows;          /* [R] gather map, or NULL for the identity */
  int64_t rows_A;                 /* rows of A */
  const uint8_t *B;               /* [E, N, K/2] */
  const uint8_t *B_sf;            /* [E, N, K/16] */
  const float *B_gs;              /* [E] */
  const int32_t *expert_offsets;  /* [E+1] */
  int32_t E, N, K;
  int64_t R;
  int32_t epilogue;               /* moe_epilogue */
  void *D;                        /* bf16 [R, N] (NONE), bf16 [R, N/2] (SWIGLU),
                                     u8 codes [R, N/4] (SWIGLU_NVFP4) */
  float *amax_out;                /* SWIGLU only */
  int32_t B_layout;               /* moe_layout */
  uint8_t *D_sf;                  /* SWIGLU_NVFP4 only: u8 scales [R, N/32] */
  const float *D_gs;              /* SWIGLU_NVFP4 only: static global scale g2 (one f32) */
} moe_gemm_args;

size_t moe_grouped_gemm_nvfp4_workspace(const moe_gemm_args *args);
int64_t moe_grouped_gemm_nvfp4_amax_slots(const moe_gemm_args *args);
moe_status moe_grouped_gemm_nvfp4_can_implement(const moe_gemm_args *args);
moe_status moe_grouped_gemm_nvfp4(const moe_gemm_args *args, void *ws, size_t ws_bytes,
                                  hipStream_t stream);

/* ---------------------------------------------------------------------------
 * 3a. The grouped GEMM without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops or harnesses that forbid
 * allocation).  Same arguments, validation, results and kernels as
 * moe_grouped_gemm_nvfp4; the workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES (1 MiB) inside the library instead, one per GPU, held until
 * the process ends.  Returns MOE_ERR_WORKSPACE when the launch needs more than that
 * (moe_grouped_gemm_nvfp4_workspace() > MOE_NOALLOC_SCRATCH_BYTES, about 65,000 work
 * items); calls nothing that allocates.  The first call on a device looks up that
 * device's copy of the array (a failure there returns MOE_ERR_HIP).  Every call on a GPU
 * shares that GPU's array: calls that may overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller.
 * ------------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES (1u << 20)
moe_status moe_grouped_gemm_nvfp4_noalloc(const moe_gemm_args *args, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * 3b. One-time weight preparation (this library's own layout; the pages load their tiles
 * with TMA instead, "Peering into the Kernel", section "Input Knowledge Required"):
 * regroup NVFP4 weights [rows, K] (codes B [rows, K/2],
 * scales B_sf [rows, K/16]; rows = E*N) into the packed layout the grouped GEMM streams:
 * per 16-row tile T and 256-wide K step s, a 2304-byte block at offset (T*K/256 + s)*2304
 * holding, in the order the 64 lanes of a wave load them (lane 16g + r, row 16T + r), two
 * 1 KB pieces q = 0..1 with each lane's code bytes [32g + 16q, +16) of the step, then 256
 * bytes with each lane's scale bytes [4g, 4g + 4) of the step.  A pure byte permutation (no
 * arithmetic): the packed buffer holds exactly rows*K*9/16 bytes.  Requires rows % 16 == 0,
 * K % 256 == 0.
 * ------------------------------------------------------------------------- */
size_t moe_pack_weights_nvfp4_bytes(int64_t rows, int K);
moe_status moe_pack_weights_nvfp4(const uint8_t *B, const uint8_t *B_sf, int64_t rows, int K,
                                  uint8_t *packed, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * 4. FINALIZE.  Defined by: the FINALIZE epilogue mode the pages contrast with NONE
 * ("The Epilogue That Broke the Kernel", section "The Insight: FINALIZE vs NONE"), whose
 * staging they price as an FP32 accumulator with a BF16 output ("Cracking the SM120
 * Shared Memory Ceiling", section "The Shared Memory Calculation"); its arithmetic is
 * read as the router-weighted sum of each token's k expert rows into BF16.
 * out[t, h] = bf16(sum_{j<k} topk_w[t, j] * Y[token_slot_row[t*k+j], h]),
 * summed in binary32 in slot order (a per-token gather-reduce: no atomics,
 * deterministic).  Y bf16 [R, H], topk_w f32 [T, k], token_slot_row i32 [T*k],
 * out bf16 [T, H].  Limits: T >= 0, 1 <= k <= 32, H % 8 == 0, H >= 8.
 * ------------------------------------------------------------------------- */
moe_status moe_finalize(const uint16_t *Y, int64_t R, const float *topk_w,
                        const int32_t *token_slot_row, int T, int k, int H, uint16_t *out,
                        hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_NVFP4_H */
