// Internal helpers shared by the gfx950 kernels of libmoe_nvfp4 (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_nvfp4.h"

namespace moe {

constexpr int kWave = 64;   // CDNA wavefront width
constexpr int kXcds = 8;    // MI355X: workgroups are dispatched round-robin over 8 XCDs

// Largest operand (packed weights of one expert, activation codes) that the packed-layout
// grouped GEMM addresses through one range-checked buffer descriptor.
constexpr int64_t kMaxPackedBufBytes = (int64_t(1) << 31) - 4096;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef float float4v __attribute__((ext_vector_type(4)));

// bf16 <-> f32 -------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (finite inputs; NaN stays NaN by the quiet bit).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// wave reductions ------------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Launch-error helper used by the host entry points.
moe_status launch_status(hipError_t e);

// Internal launchers (one per kernel family), defined next to their kernels. ----

hipError_t launch_route_permute(const float *logits, int T, int E, int k, int32_t *topk_ids,
                                float *topk_w, int32_t *expert_offsets, int32_t *row_src,
                                int32_t *token_slot_row, void *ws, hipStream_t stream);
size_t route_permute_ws_bytes(int T, int E, int k);

hipError_t launch_quantize(const void *x, int x_dtype, int64_t rows, int64_t C, uint8_t *q,
                           uint8_t *sf, float *gs, int gs_mode, const float *amax_in,
                           int64_t n_amax_in, void *ws, hipStream_t stream);
size_t quantize_ws_bytes(int64_t rows, int64_t C);

struct GemmPlan {
  int kernel;        // kernel family (gemm::Kernel)
  int chunk_rows;    // rows per work item
  int ks;            // K split across the waves of a workgroup: 1, 2 or 4
  int n_tile;        // weight rows (output columns of y) per workgroup
  int n_tiles;       // N / n_tile
  int64_t max_items; // upper bound on (expert, row chunk, n tile) work items
  int64_t grid;      // workgroups launched (max_items rounded up to the XCD count)
  bool inline_schedule;  // waves derive their items from the offsets (no schedule kernel)
  size_t ws_bytes;
};
GemmPlan plan_gemm(const moe_gemm_args &a);
hipError_t launch_grouped_gemm(const moe_gemm_args &a, const GemmPlan &plan, void *ws,
                               hipStream_t stream);

size_t packed_weights_bytes(int64_t rows, int K);
hipError_t launch_pack_weights(const uint8_t *B, const uint8_t *B_sf, int64_t rows, int K,
                               uint8_t *packed, hipStream_t stream);

hipError_t launch_finalize(const uint16_t *Y, int64_t R, const float *topk_w,
                           const int32_t *token_slot_row, int T, int k, int H, uint16_t *out,
                           hipStream_t stream);

}  // namespace moe
