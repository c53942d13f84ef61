// FINALIZE: the router-weighted combination of each token's k expert rows into its bf16
// output row.  The pages name FINALIZE as the epilogue mode that does more than the NONE
// pass-through and stage it as an FP32 accumulator plus a BF16 output ("The Epilogue That
// Broke the Kernel", section "The Insight: FINALIZE vs NONE"; "Cracking the SM120 Shared
// Memory Ceiling", section "The Shared Memory Calculation"); its arithmetic is the
// router-weighted scatter-add of the expert rows back to their tokens.
//
// Realised as a gather-reduce owned by the token: workgroup t reads the k rows
// Y[token_slot_row[t*k + j]] (j ascending) and accumulates w[t, j] * row in fp32, then
// rounds once to bf16.  No atomics, so the result is deterministic.  Memory-bound:
// k * H * 2 bytes read and H * 2 bytes written per token.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kMaxK = 32;

__device__ __forceinline__ void fma_bf16x2(float &a0, float &a1, float w, uint32_t v) {
  a0 = fmaf(w, __uint_as_float(v << 16), a0);
  a1 = fmaf(w, __uint_as_float(v & 0xffff0000u), a1);
}

__global__ __launch_bounds__(256) void finalize_kernel(const uint16_t *__restrict__ Y, int64_t R,
                                                       const float *__restrict__ topk_w,
                                                       const int32_t *__restrict__ token_slot_row,
                                                       int k, int H, uint16_t *__restrict__ out) {
  __shared__ int64_t row_off[kMaxK];
  __shared__ float wt[kMaxK];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < static_cast<unsigned>(k)) {
    int64_t p = token_slot_row[t * k + threadIdx.x];
    p = p < 0 ? 0 : (p >= R ? R - 1 : p);
    row_off[threadIdx.x] = p * H;
    wt[threadIdx.x] = topk_w[t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < H / 8; c += blockDim.x) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; j++) {
      const uint4 v = *reinterpret_cast<const uint4 *>(Y + row_off[j] + 8 * c);
      const float w = wt[j];
      fma_bf16x2(a[0], a[1], w, v.x);
      fma_bf16x2(a[2], a[3], w, v.y);
      fma_bf16x2(a[4], a[5], w, v.z);
      fma_bf16x2(a[6], a[7], w, v.w);
    }
    uint4 o;
    o.x = f32_to_bf16(a[0]) | (static_cast<uint32_t>(f32_to_bf16(a[1])) << 16);
    o.y = f32_to_bf16(a[2]) | (static_cast<uint32_t>(f32_to_bf16(a[3])) << 16);
    o.z = f32_to_bf16(a[4]) | (static_cast<uint32_t>(f32_to_bf16(a[5])) << 16);
    o.w = f32_to_bf16(a[6]) | (static_cast<uint32_t>(f32_to_bf16(a[7])) << 16);
    *reinterpret_cast<uint4 *>(out + t * H + 8 * c) = o;
  }
}

}  // namespace

hipError_t launch_finalize(const uint16_t *Y, int64_t R, const float *topk_w,
                           const int32_t *token_slot_row, int T, int k, int H, uint16_t *out,
                           hipStream_t stream) {
  if (T > 0) {
    const int threads = H / 8 >= 256 ? 256 : ((H / 8 + 63) / 64) * 64;
    hipLaunchKernelGGL(finalize_kernel, dim3(T), dim3(threads), 0, stream, Y, R, topk_w,
                       token_slot_row, k, H, out);
  }
  return hipGetLastError();
}

}  // namespace moe
