// NVFP4 quantisation: FP4 E2M1 elements, one E4M3 scale per 16 consecutive elements of a
// row, one FP32 global scale per tensor.  The element and scale-block layout is the one
// the pages budget for ("Cracking the SM120 Shared Memory Ceiling", section "The Shared
// Memory Calculation": packed 4-bit elements, one 8-bit scale per 16 along K).
//
// Reading of the open steps: decode-direction global scale g = amax / (6 * 448) (1 for an
// all-zero tensor); block scale s = e4m3_rne(min(amax_b / (6 g), 448)); element code
// sign(x) | e2m1_rne(min(|x| / (s g), 6)), where 0 / 0 (a zero block or element over an
// underflowed g or s g) counts as 0.  Every step is one correctly rounded binary32
// operation in a fixed order, so the result is bit-exact against any implementation that
// takes the same steps.  Contraction is disabled in this file for that reason; the
// element quotients come from one reciprocal per block with an exact fma correction, which
// yields the correctly rounded quotient itself (block_quotient).
//
// Two kernels: amax_kernel writes up to kAmaxParts partial maxima into the workspace;
// quant_kernel (one thread per 16-element block) first reduces those partials itself
// (order-free, so every workgroup sees the same g) and then quantises.  Up to
// kDirectParts caller-provided maxima (e.g. a SwiGLU GEMM's partial maxima at a few hundred
// workgroups) are reduced by quant_kernel directly, without the amax_kernel launch: at those
// sizes the launch costs more than every workgroup reading the maxima.  Memory-bound:
// reads 2 (bf16) or 4 (f32) bytes and writes 0.5625 bytes per element.
#include "common.hpp"
#include "nvfp4_round.hpp"

#pragma clang fp contract(off)

namespace moe {
namespace {

constexpr int kAmaxParts = 256;
constexpr int kDirectParts = 1024;

__device__ __forceinline__ float load_abs_max8_bf16(const uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    m = fmaxf(m, fabsf(__uint_as_float(w[i] << 16)));
    m = fmaxf(m, fabsf(__uint_as_float(w[i] & 0xffff0000u)));
  }
  return m;
}

// Partial maxima, one per workgroup of kAmaxThreads.  Each thread takes kAmaxBatch grid-strided
// loads per round and issues them all before using any (a maximum does not mind an element
// read twice, so indices past the end are clamped to the last one instead of branched
// around): enough bytes in flight to stream HBM with at most kAmaxParts workgroups.
constexpr int kAmaxThreads = 1024;
constexpr int kAmaxBatch = 4;

__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(const void *__restrict__ x, int x_dtype, int64_t n,
                                                            const float *__restrict__ amax_in, int64_t n_in,
                                                            float *__restrict__ parts) {
  float m = 0.f;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (amax_in != nullptr) {
    for (int64_t i = tid; i < n_in; i += kAmaxBatch * stride) {
      float v[kAmaxBatch];
#pragma unroll
      for (int u = 0; u < kAmaxBatch; u++) v[u] = amax_in[min(i + u * stride, n_in - 1)];
#pragma unroll
      for (int u = 0; u < kAmaxBatch; u++) m = fmaxf(m, fabsf(v[u]));
    }
  } else if (x_dtype == MOE_DTYPE_BF16) {
    const uint4 *xv = static_cast<const uint4 *>(x);  // 8 bf16 per load; n % 16 == 0
    const int64_t nv = n / 8;
    for (int64_t i = tid; i < nv; i += kAmaxBatch * stride) {
      uint4 v[kAmaxBatch];
#pragma unroll
      for (int u = 0; u < kAmaxBatch; u++) v[u] = xv[min(i + u * stride, nv - 1)];
#pragma unroll
      for (int u = 0; u < kAmaxBatch; u++) m = fmaxf(m, load_abs_max8_bf16(v[u]));
    }
  } else {
    const float4 *xv = static_cast<const float4 *>(x);
    const int64_t nv = n / 4;
    for (int64_t i = tid; i < nv; i += kAmaxBatch * stride) {
      float4 v[kAmaxBatch];
#pragma unroll
      for (int u = 0; u < kAmaxBatch; u++) v[u] = xv[min(i + u * stride, nv - 1)];
#pragma unroll
      for (int u = 0; u < kAmaxBatch; u++)
        m = fmaxf(fmaxf(m, fmaxf(fabsf(v[u].x), fabsf(v[u].y))), fmaxf(fabsf(v[u].z), fabsf(v[u].w)));
    }
  }
  m = wave_max(m);
  __shared__ float wm[kAmaxThreads / 64];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = wm[0];
    for (int w = 1; w < kAmaxThreads / 64; w++) r = fmaxf(r, wm[w]);
    parts[blockIdx.x] = r;
  }
}

// PARTS: the most partial maxima the kernel reduces (64 lanes x PARTS / 64 loads each)
template <int PARTS>
__global__ __launch_bounds__(256) void quant_kernel(const void *__restrict__ x, int x_dtype,
                                                    int64_t nblk, uint8_t *__restrict__ q,
                                                    uint8_t *__restrict__ sf, float *__restrict__ gs,
                                                    int dynamic, const float *__restrict__ parts,
                                                    int nparts) {
  // the block's loads go out first, so their latency overlaps the global-scale reduction
  // and the barrier (a thread past the end loads the last block and drops it)
  const int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t bl = b < nblk ? b : nblk - 1;
  const bool bf16 = x_dtype == MOE_DTYPE_BF16;
  uint4 raw[4] = {};
  if (nblk > 0) {
    const uint4 *xv = static_cast<const uint4 *>(x) + (bf16 ? 2 : 4) * bl;
    raw[0] = xv[0];
    raw[1] = xv[1];
    if (!bf16) {
      raw[2] = xv[2];
      raw[3] = xv[3];
    }
  }
  __shared__ float sh_g;
  if (threadIdx.x < 64) {
    float g;
    if (dynamic) {
      // nparts <= PARTS: PARTS / 64 loads per lane, all in flight at once (indices clamped to
      // the last partial, which a maximum may read twice)
      constexpr int kPer = PARTS / 64;
      static_assert(PARTS % 64 == 0, "whole loads per lane");
      float v[kPer];
#pragma unroll
      for (int u = 0; u < kPer; u++) v[u] = parts[min(static_cast<int>(threadIdx.x) + 64 * u, nparts - 1)];
      float m = 0.f;
#pragma unroll
      for (int u = 0; u < kPer; u++) m = fmaxf(m, fabsf(v[u]));
      m = wave_max(m);
      g = (m > 0.f) ? m / 2688.0f : 1.0f;  // 2688 = 6 * 448
      if (blockIdx.x == 0 && threadIdx.x == 0) *gs = g;
    } else {
      g = *gs;
    }
    if (threadIdx.x == 0) sh_g = g;
  }
  __syncthreads();
  const float g = sh_g;
  if (b >= nblk) return;
  float v[16];
  if (bf16) {
    const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
    for (int i = 0; i < 8; i++) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[4 * i] = __uint_as_float(raw[i].x);
      v[4 * i + 1] = __uint_as_float(raw[i].y);
      v[4 * i + 2] = __uint_as_float(raw[i].z);
      v[4 * i + 3] = __uint_as_float(raw[i].w);
    }
  }
  float amax_b = 0.f;
#pragma unroll
  for (int i = 0; i < 16; i++) amax_b = fmaxf(amax_b, fabsf(v[i]));
  const float six_g = 6.0f * g;
  // zero stays zero where g has underflowed: a zero block gets scale 0 (not 0 / 0)
  const float t = amax_b > 0.f ? fminf(amax_b / six_g, 448.0f) : 0.f;
  const uint32_t s = e4m3_rne(t);
  const float sg = e4m3_value(s) * g;
  uint32_t packed[2] = {0u, 0u};
  const BlockDivisor d = block_divisor(sg, amax_b);
  if (d.fast) {
    // finite quotients: the hardware conversion saturates at 6 itself
#pragma unroll
    for (int h = 0; h < 2; h++) {
      float u[8];
#pragma unroll
      for (int i = 0; i < 8; i++) u[i] = block_quotient(fabsf(v[8 * h + i]), d);
      packed[h] = e2m1_pack8(u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      // a zero element gets code 0 even where s g has underflowed to 0 (0 / 0 counts as 0);
      // a non-zero one over s g = 0 saturates at 6
      const uint32_t mag = (s != 0u && fabsf(v[i]) > 0.f) ? e2m1_rne(fminf(fabsf(v[i]) / sg, 6.0f)) : 0u;
      packed[i >> 3] |= mag << (4 * (i & 7));
    }
  }
#pragma unroll
  for (int i = 0; i < 16; i++) packed[i >> 3] |= (__float_as_uint(v[i]) >> 31) << (4 * (i & 7) + 3);
  reinterpret_cast<uint2 *>(q)[b] = make_uint2(packed[0], packed[1]);
  sf[b] = static_cast<uint8_t>(s);
}

}  // namespace

size_t quantize_ws_bytes(int64_t, int64_t) { return kAmaxParts * sizeof(float); }

hipError_t launch_quantize(const void *x, int x_dtype, int64_t rows, int64_t C, uint8_t *q,
                           uint8_t *sf, float *gs, int gs_mode, const float *amax_in,
                           int64_t n_amax_in, void *ws, hipStream_t stream) {
  const int64_t n = rows * C;
  const int64_t nblk = n / 16;
  float *parts = static_cast<float *>(ws);
  const int dynamic = gs_mode == MOE_GS_DYNAMIC;
  int nparts = 0;
  // few caller-provided maxima: quant_kernel reduces them itself
  const bool direct = dynamic && amax_in != nullptr && n_amax_in >= 1 && n_amax_in <= kDirectParts;
  if (dynamic && !direct) {
    // partial maxima: ~4 per thread; tensor data: ~32 elements per thread
    const int64_t per_wg = kAmaxThreads * (amax_in ? 4 : 32);
    const int64_t g = ((amax_in ? n_amax_in : n) + per_wg - 1) / per_wg;
    nparts = static_cast<int>(g < 1 ? 1 : (g > kAmaxParts ? kAmaxParts : g));
    hipLaunchKernelGGL(amax_kernel, dim3(nparts), dim3(kAmaxThreads), 0, stream, x, x_dtype, n, amax_in,
                       n_amax_in, parts);
  }
  if (nblk > 0 || dynamic) {
    const int64_t grid = nblk > 0 ? (nblk + 255) / 256 : 1;  // one block still publishes g
    if (direct)
      hipLaunchKernelGGL(quant_kernel<kDirectParts>, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream, x,
                         x_dtype, nblk, q, sf, gs, dynamic, amax_in, static_cast<int>(n_amax_in));
    else
      hipLaunchKernelGGL(quant_kernel<kAmaxParts>, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream, x,
                         x_dtype, nblk, q, sf, gs, dynamic, parts, nparts);
  }
  return hipGetLastError();
}

}  // namespace moe
