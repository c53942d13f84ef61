// MFMA throughput measurement kernels (libmoe_probes.so, used by the benchmark only; not part
// of the MoE ABI).  Every wave issues back-to-back matrix instructions on register operands,
// kChains independent accumulators deep so that no instruction waits for the result of the
// one before it, and touches memory once, to write its sums at the end.  Over a launch with
// several waves on every SIMD the rate is the dense MFMA ceiling at the clock the board holds
// under that load: the measured peak the benchmark reports beside the published one.
//
// Kinds: 0 = fp16 16x16x32 (the contraction the grouped GEMM kernels issue: the exact
// E2M1 x E4M3 products are formed in fp16), 1 = FP4 E2M1 16x16x128 with unit block scales
// (the matrix cores' own FP4 rate).  All operand elements are 1/8 (fp16) or 1/2 (E2M1) and
// chain j starts at j (distinct chains, which the compiler cannot merge), so every
// accumulator ends at an exact, known value the caller can check.  This file is built with
// the VGPR form of MFMA selected: with accumulation registers the compiler copied the
// accumulators around the loop on every trip.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef int int8v __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kChains = 8;
constexpr int kKinds = 2;
// flops of one instruction: 2 * 16 * 16 * K
constexpr double kFlopsPerMfma[kKinds] = {2.0 * 16 * 16 * 32, 2.0 * 16 * 16 * 128};

template <int KIND>
__global__ __launch_bounds__(kThreads) void mfma_peak_kernel(int iters, float *__restrict__ sink) {
  float4v acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; j++) acc[j] = float4v{1.f * j, 1.f * j, 1.f * j, 1.f * j};
  if constexpr (KIND == 0) {
    const _Float16 e = static_cast<_Float16>(0.125f);
    const half8 a = {e, e, e, e, e, e, e, e};
    for (int i = 0; i < iters; i++) {
#pragma unroll
      for (int j = 0; j < kChains; j++) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, a, acc[j], 0, 0, 0);
    }
  } else {
    // 0x11 per byte: two E2M1 codes 0b0001 = 0.5; the upper four dwords are not read for FP4
    const int w = 0x11111111;
    const int8v a = {w, w, w, w, 0, 0, 0, 0};
    for (int i = 0; i < iters; i++) {
#pragma unroll
      for (int j = 0; j < kChains; j++)   // formats 4 = E2M1 for both operands; scales 127 = 2^0 (E8M0)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, a, acc[j], 4, 4, 0, 127, 0, 127);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; j++) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = s;
}

}  // namespace

extern "C" {

int moe_probe_mfma_kinds(void) { return kKinds; }

// Flops one wave performs per loop trip of kind `kind` (kChains instructions), or 0.
double moe_probe_mfma_flops_per_wave_iter(int kind) {
  return (kind < 0 || kind >= kKinds) ? 0.0 : kChains * kFlopsPerMfma[kind];
}

// The value every wave writes to its sink entry after `iters` trips: lane 0's four
// accumulator elements of every chain, each j + iters * (K * a * a); integers below 2^24
// for iters <= 8192, so exact in fp32 whatever the order of the sum.
double moe_probe_mfma_expected_sink(int kind, int iters) {
  if (kind < 0 || kind >= kKinds) return 0.0;
  const double per_mfma = kind == 0 ? 32 * 0.125 * 0.125 : 128 * 0.5 * 0.5;
  double s = 0.0;
  for (int j = 0; j < kChains; j++) s += 4.0 * (j + per_mfma * iters);
  return s;
}

// Launches `groups` workgroups of 256 threads, each wave running `iters` trips; sink must hold
// groups * 4 floats.  Returns the hipError_t of the launch (or hipErrorInvalidValue).
int moe_probe_mfma_peak(int kind, int64_t groups, int iters, float *sink, hipStream_t stream) {
  if (!sink || kind < 0 || kind >= kKinds || groups < 1 || groups > (int64_t(1) << 20) || iters < 1 ||
      iters > 8192)
    return static_cast<int>(hipErrorInvalidValue);
  const dim3 grid(static_cast<uint32_t>(groups)), block(kThreads);
  if (kind == 0) hipLaunchKernelGGL(mfma_peak_kernel<0>, grid, block, 0, stream, iters, sink);
  else hipLaunchKernelGGL(mfma_peak_kernel<1>, grid, block, 0, stream, iters, sink);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
