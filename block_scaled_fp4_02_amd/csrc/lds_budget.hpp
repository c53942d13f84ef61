// Compile-time LDS budget of the grouped NVFP4 GEMM tiles.
//
// The pages explain their tile failures with one shared-memory formula ("Cracking the SM120
// Shared Memory Ceiling", sections "The Shared Memory Calculation" and "Tracing the
// Failure"): a CUTLASS SM120 tile M x N x K with packed FP4 operands needs, per pipeline
// stage, M K / 2 bytes of A, K N / 2 of B and one FP8 scale byte per 16 elements along K
// for each (M K / 16 + K N / 16), and its epilogue stages the whole M x N output tile, 2
// bytes per element for the pass-through (NONE) epilogue and 4 for FINALIZE.  Against the
// 101,376 bytes a block may opt into on SM120 that rejects the FINALIZE variants of
// 128x128x256, 128x256x128 and 256x128x128: those configurations passed the can-implement
// check and then failed to initialise.
//
// This header holds that formula (a unit test reproduces the pages' table from it) and the
// same accounting for this library's own gfx950 tiles, whose LDS footprint each kernel
// checks with a static_assert against the 163,840 bytes of LDS of a CDNA4 compute unit,
// shared by the workgroups its launch bounds promise per CU.  A tile that does not fit is a
// compile error, never a launch that fails at run time.  Plain constexpr C++17 with no HIP
// dependency, so host code and tests can include it.
#pragma once

#include <stdint.h>

namespace moe {
namespace lds {

// Budgets.
constexpr int64_t kSm120OptInBlockBytes = 101376;   // SM120: opt-in maximum per block
constexpr int64_t kSm120BytesPerSm = 102400;        // SM120: shared memory per SM
constexpr int64_t kCdna4BytesPerCu = 163840;        // gfx950: LDS per compute unit (and per workgroup)

// ---- the pages' SM120 model ----------------------------------------------------------

// One mainloop stage of an M x N x K tile with packed FP4 operands and one FP8 scale per 16
// elements along K on both operands.
constexpr int64_t nvfp4_stage_bytes(int64_t M, int64_t N, int64_t K) {
  return M * K / 2 + K * N / 2 + M * (K / 16) + (K / 16) * N;
}

// Output staging of the epilogue: BF16 (NONE) or an FP32 accumulator with BF16 output
// (FINALIZE), priced by the pages at 2 and 4 bytes per output element.
constexpr int64_t epilogue_staging_bytes(int64_t M, int64_t N, bool finalize) {
  return M * N * (finalize ? 4 : 2);
}

constexpr int64_t sm120_tile_bytes(int64_t M, int64_t N, int64_t K, int64_t stages, bool finalize) {
  return stages * nvfp4_stage_bytes(M, N, K) + epilogue_staging_bytes(M, N, finalize);
}

// Stages an automatic carve-out could fit after the epilogue's staging (0: the tile cannot
// run at all).
constexpr int64_t stages_that_fit(int64_t M, int64_t N, int64_t K, bool finalize, int64_t budget) {
  const int64_t left = budget - epilogue_staging_bytes(M, N, finalize);
  return left <= 0 ? 0 : left / nvfp4_stage_bytes(M, N, K);
}

constexpr bool fits(int64_t bytes, int64_t budget) { return bytes <= budget; }

// ---- this library's gfx950 tiles --------------------------------------------------------
//
// Every packed-weight kernel streams its weights into registers; only the activation tile
// (and reduction or output staging) lives in LDS.  Sizes follow the shared-memory structs
// in gemm_lds.hip, gemm_ksplit.hip and gemm_rowmajor.hip exactly (each kernel asserts
// equality with its struct or array).

constexpr int64_t kKStepElems = 256;   // K elements per step of every kernel
constexpr int64_t kEpRowHalves = 72;   // NONE staging row: 64 bf16 columns + 8 of padding

// LDS kernels (gemm_lds_kernel, gemm_lds_wide_kernel): double-buffered fp16 activation
// fragments of up to `tiles` 16-row token tiles for one K step, in a union with the NONE
// epilogue's per-wave bf16 staging, plus one float per wave for the SwiGLU maxima.
constexpr int64_t lds_act_buffers_bytes(int64_t tiles) { return 2 * tiles * 16 * kKStepElems * 2; }
constexpr int64_t lds_none_staging_bytes(int64_t tiles, int64_t waves) {
  return waves * tiles * 16 * kEpRowHalves * 2;
}
constexpr int64_t lds_kernel_bytes(int64_t tiles, int64_t waves) {
  return (lds_act_buffers_bytes(tiles) > lds_none_staging_bytes(tiles, waves) ? lds_act_buffers_bytes(tiles)
                                                                              : lds_none_staging_bytes(tiles, waves)) +
         waves * 4;
}

// K-split kernel: every wave parks a partial tile of 4 weight tiles x `tiles` token tiles of
// 16 x 16 fp32 results, plus one float per wave for the SwiGLU maxima.
constexpr int64_t ksplit_kernel_bytes(int64_t tiles, int64_t waves) { return waves * (4 * tiles * 256 * 4 + 4); }

// Row-major kernel: with K split KS ways, KS - 1 of every KS waves park their partial tile
// (2 weight tiles x 2 token tiles of 32 x 32 fp32 results: 4096 floats) for the wave that
// adds them, plus the four SwiGLU maxima; without a split one placeholder float.
constexpr int64_t kRowMajorPartialFloats = 2 * 2 * 16 * 64;
constexpr int64_t rowmajor_kernel_bytes(int64_t ks) {
  return (ks > 1 ? (ks - 1) * (4 / ks) * kRowMajorPartialFloats * 4 : 4) + 4 * 4;
}

// Whether `per_workgroup` bytes allow `workgroups` resident workgroups on one CU.
constexpr bool fits_cu(int64_t per_workgroup, int64_t workgroups) {
  return per_workgroup * workgroups <= kCdna4BytesPerCu;
}

// The tile table the per-shape plan chooses from: output rows per work item (token rows),
// weight rows per work item, K per step, workgroups per CU, and LDS bytes per workgroup.
struct TileEntry {
  const char *name;
  int64_t token_rows, weight_rows, k_step, workgroups_per_cu, lds_bytes;
};

constexpr TileEntry kTileTable[] = {
    {"decode LDS kernel (4 waves)", 48, 256, kKStepElems, 3, lds_kernel_bytes(3, 4)},
    {"LDS kernel, 64-row chunks (4 waves)", 64, 256, kKStepElems, 2, lds_kernel_bytes(4, 4)},
    {"wide LDS kernel (8 waves)", 96, 512, kKStepElems, 1, lds_kernel_bytes(6, 8)},
    {"K split 2 ways (4 waves)", 32, 128, kKStepElems, 2, ksplit_kernel_bytes(2, 4)},
    {"K split 4 ways (4 waves)", 32, 64, kKStepElems, 2, ksplit_kernel_bytes(2, 4)},
    {"K split 8 ways (8 waves)", 32, 64, kKStepElems, 1, ksplit_kernel_bytes(2, 8)},
    {"row-major, K split 1 (4 waves)", 64, 256, kKStepElems, 2, rowmajor_kernel_bytes(1)},
    {"row-major, K split 2 (4 waves)", 64, 128, kKStepElems, 2, rowmajor_kernel_bytes(2)},
    {"row-major, K split 4 (4 waves)", 64, 64, kKStepElems, 2, rowmajor_kernel_bytes(4)},
};

constexpr bool table_fits() {
  for (const TileEntry &t : kTileTable)
    if (!fits_cu(t.lds_bytes, t.workgroups_per_cu)) return false;
  return true;
}
static_assert(table_fits(), "a tile of the plan exceeds the LDS of a CDNA4 compute unit");

}  // namespace lds
}  // namespace moe
