// Streaming-read measurement kernel (libmoe_stream_probe.so, used by the benchmark only; not
// part of the MoE ABI).  It reads a device buffer once, 16 bytes per lane per load with every
// load of a round in flight together, and folds what it read into one word per wave so the
// loads cannot be dropped.  Its rate on a large buffer is the measured HBM read ceiling the
// benchmark reports beside the 8 TB/s spec figure; on one copy of a working set rotated over
// several copies (larger together than the on-die caches) it is the read rate at that size,
// launch start and drain included.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

// All loads are range-checked buffer loads (an offset at or past the range returns zeros and
// reads nothing), so a round issues its U loads unconditionally.  The grid strides over the
// buffer: with fewer workgroups than the buffer needs for one round, each loops.
template <int U, int POLICY>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint8_t *__restrict__ src, uint32_t bytes,
                                                               uint32_t *__restrict__ sink) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(src), 0,
                                                                      static_cast<int>(bytes), 0x00020000);
  const uint32_t stride = gridDim.x * kThreads * 16u;
  uint32_t acc = 0;
  for (uint64_t off = (static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x) * 16u; off < bytes;
       off += static_cast<uint64_t>(U) * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint64_t o = off + static_cast<uint64_t>(u) * stride;
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, o < bytes ? static_cast<uint32_t>(o) : 0x80000000u, 0,
                                                   POLICY);
    }
#pragma unroll
    for (int u = 0; u < U; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = acc;
}

// Variants: loads in flight per lane (4, 8, 16) x cache policy (default, non-temporal).
constexpr int kVariants = 6;
constexpr int variant_unroll(int v) { return v % 3 == 0 ? 4 : (v % 3 == 1 ? 8 : 16); }

}  // namespace

extern "C" {

int moe_probe_stream_read_variants(void) { return kVariants; }

// Loads in flight per lane (bits 0-7) and the non-temporal policy (bit 8) of variant v.
int moe_probe_stream_read_variant_info(int v) {
  if (v < 0 || v >= kVariants) return -1;
  return variant_unroll(v) | (v >= 3 ? 256 : 0);
}

// Workgroups of the launch for `bytes` with variant v: enough that one round covers the
// buffer, at most `max_groups` (fewer: each workgroup loops).
int64_t moe_probe_stream_read_groups(int64_t bytes, int variant, int64_t max_groups) {
  if (variant < 0 || variant >= kVariants) return 0;
  const int64_t per_group = static_cast<int64_t>(kThreads) * 16 * variant_unroll(variant);
  int64_t g = (bytes + per_group - 1) / per_group;
  if (g > max_groups) g = max_groups;
  return g < 1 ? 1 : g;
}

// Reads src[0, bytes) once (bytes % 16 == 0, bytes < 2^31) with variant v on `stream`; sink
// must hold groups * 4 words.  Returns the hipError_t of the launch (or hipErrorInvalidValue).
int moe_probe_stream_read(const void *src, int64_t bytes, int variant, int64_t groups, uint32_t *sink,
                          hipStream_t stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || bytes >= (int64_t(1) << 31) || groups < 1 ||
      groups > (int64_t(1) << 19) || variant < 0 || variant >= kVariants)   // the stride stays below 2^31
    return static_cast<int>(hipErrorInvalidValue);
  const dim3 grid(static_cast<uint32_t>(groups)), block(kThreads);
  const uint8_t *p = static_cast<const uint8_t *>(src);
  const uint32_t n = static_cast<uint32_t>(bytes);
  switch (variant) {
    case 0: hipLaunchKernelGGL((stream_read_kernel<4, 0>), grid, block, 0, stream, p, n, sink); break;
    case 1: hipLaunchKernelGGL((stream_read_kernel<8, 0>), grid, block, 0, stream, p, n, sink); break;
    case 2: hipLaunchKernelGGL((stream_read_kernel<16, 0>), grid, block, 0, stream, p, n, sink); break;
    case 3: hipLaunchKernelGGL((stream_read_kernel<4, 2>), grid, block, 0, stream, p, n, sink); break;
    case 4: hipLaunchKernelGGL((stream_read_kernel<8, 2>), grid, block, 0, stream, p, n, sink); break;
    default: hipLaunchKernelGGL((stream_read_kernel<16, 2>), grid, block, 0, stream, p, n, sink); break;
  }
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
