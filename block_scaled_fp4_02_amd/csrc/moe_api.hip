// Host side of the C ABI declared in moe_nvfp4.h: argument validation (before any HIP
// call), workspace queries, the truthful can-implement check and the launches on the
// caller's stream.  No entry point allocates, synchronises or throws.
#include "common.hpp"

#include <cstring>
#include <mutex>

namespace moe {
namespace {
thread_local int g_last_hip_error = 0;

// ---- scratch of the no-allocation grouped GEMM -------------------------------------------
//
// A static device array holds the grouped GEMM's workspace (the work-item list and its count)
// for moe_grouped_gemm_nvfp4_noalloc.  Every GPU the library runs on holds its own copy at
// its own address until the process ends.  On the host `scratch` is only a stand-in for the
// device variable: its device address is looked up once per device, with that device
// current, and only that address is ever passed to a kernel.
constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;
static_assert(kNoAllocScratchBytes == MOE_NOALLOC_SCRATCH_BYTES, "scratch size differs from the header");
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, null until looked up

hipError_t device_scratch(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

moe_status launch_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = static_cast<int>(e);
  return MOE_ERR_HIP;
}

namespace {

moe_status check_gemm(const moe_gemm_args *a, bool need_pointers) {
  if (a == nullptr) return MOE_ERR_NULL;
  if (a->E < 1 || a->E > 65536 || a->N < 1 || a->K < 1 || a->R < 0 || a->R >= (int64_t(1) << 31) ||
      a->rows_A < 0)
    return MOE_ERR_SHAPE;
  if (a->epilogue != MOE_EPI_NONE && a->epilogue != MOE_EPI_SWIGLU && a->epilogue != MOE_EPI_SWIGLU_NVFP4)
    return MOE_ERR_UNSUPPORTED;
  if (a->B_layout != MOE_LAYOUT_ROWMAJOR && a->B_layout != MOE_LAYOUT_PACKED) return MOE_ERR_UNSUPPORTED;
  if (a->epilogue == MOE_EPI_SWIGLU_NVFP4 && a->B_layout != MOE_LAYOUT_PACKED) return MOE_ERR_UNSUPPORTED;
  if (a->K % 16 != 0) return MOE_ERR_SHAPE;
  if (a->K % 256 != 0 || a->N % 256 != 0) return MOE_ERR_UNSUPPORTED;
  if (a->R > 0 && a->rows_A < 1) return MOE_ERR_SHAPE;
  // the packed kernel addresses the activation codes and each expert's packed weights
  // through 32-bit range-checked buffer descriptors (K >= 256 here; the bound on rows_A is
  // tested by division, so that no product can overflow)
  if (a->B_layout == MOE_LAYOUT_PACKED &&
      (a->rows_A > kMaxPackedBufBytes / (a->K / 2) || static_cast<int64_t>(a->N) * a->K / 16 * 9 > kMaxPackedBufBytes))
    return MOE_ERR_UNSUPPORTED;
  // item indices, row indices and workgroup counts stay in 32 bits
  const GemmPlan plan = plan_gemm(*a);
  if (plan.grid >= (int64_t(1) << 31) || static_cast<int64_t>(a->E) * a->N >= (int64_t(1) << 40))
    return MOE_ERR_UNSUPPORTED;
  if (need_pointers) {
    if (!a->B || !a->B_gs || !a->expert_offsets || !a->A_gs) return MOE_ERR_NULL;
    if (a->B_layout == MOE_LAYOUT_ROWMAJOR && !a->B_sf) return MOE_ERR_NULL;
    if (a->R > 0 && (!a->A || !a->A_sf || !a->D)) return MOE_ERR_NULL;
    if (a->epilogue == MOE_EPI_SWIGLU && !a->amax_out) return MOE_ERR_NULL;
    if (a->epilogue == MOE_EPI_SWIGLU_NVFP4 && (!a->D_gs || (a->R > 0 && !a->D_sf))) return MOE_ERR_NULL;
  }
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

const char *moe_status_string(moe_status s) {
  // a C caller may pass any int: read the bits rather than the enum value, which C++ only
  // defines within the enumerators' range
  int v = 0;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is negative, inconsistent or out of range";
    case MOE_ERR_UNSUPPORTED: return "configuration not supported by the gfx950 kernels";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "a HIP launch failed (see moe_last_hip_error)";
  }
  return "unknown status";
}

int moe_last_hip_error(void) { return g_last_hip_error; }

size_t moe_route_permute_workspace(int T, int E, int k) {
  if (T < 0 || E < 1 || E > 1024 || k < 1) return 0;
  return route_permute_ws_bytes(T, E, k);
}

moe_status moe_route_permute(const float *logits, int T, int E, int k, int32_t *topk_ids,
                             float *topk_w, int32_t *expert_offsets, int32_t *row_src,
                             int32_t *token_slot_row, void *ws, size_t ws_bytes,
                             hipStream_t stream) {
  if (T < 0 || E < 1 || E > 1024 || k < 1 || k > 32 || k > E ||
      static_cast<int64_t>(T) * k >= (int64_t(1) << 31))
    return MOE_ERR_SHAPE;
  if (!expert_offsets) return MOE_ERR_NULL;
  if (T > 0 && (!logits || !topk_ids || !topk_w || !row_src || !token_slot_row)) return MOE_ERR_NULL;
  if (!ws || ws_bytes < route_permute_ws_bytes(T, E, k)) return MOE_ERR_WORKSPACE;
  return launch_status(launch_route_permute(logits, T, E, k, topk_ids, topk_w, expert_offsets,
                                            row_src, token_slot_row, ws, stream));
}

size_t moe_quantize_nvfp4_workspace(int64_t rows, int64_t C) {
  if (rows < 0 || C < 16) return 0;
  return quantize_ws_bytes(rows, C);
}

moe_status moe_quantize_nvfp4(const void *x, int x_dtype, int64_t rows, int64_t C, uint8_t *q,
                              uint8_t *sf, float *gs, int gs_mode, const float *amax_in,
                              int64_t n_amax_in, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (rows < 0 || C < 16 || C % 16 != 0 || n_amax_in < 0) return MOE_ERR_SHAPE;
  if (rows > 0 && C > (int64_t(1) << 40) / rows) return MOE_ERR_SHAPE;
  if (x_dtype != MOE_DTYPE_BF16 && x_dtype != MOE_DTYPE_F32) return MOE_ERR_UNSUPPORTED;
  if (gs_mode != MOE_GS_STATIC && gs_mode != MOE_GS_DYNAMIC) return MOE_ERR_UNSUPPORTED;
  if (!gs) return MOE_ERR_NULL;
  if (rows > 0 && (!x || !q || !sf)) return MOE_ERR_NULL;
  if (gs_mode == MOE_GS_DYNAMIC && amax_in == nullptr && rows > 0 && !x) return MOE_ERR_NULL;
  if (!ws || ws_bytes < quantize_ws_bytes(rows, C)) return MOE_ERR_WORKSPACE;
  return launch_status(launch_quantize(x, x_dtype, rows, C, q, sf, gs, gs_mode, amax_in, n_amax_in,
                                       ws, stream));
}

size_t moe_grouped_gemm_nvfp4_workspace(const moe_gemm_args *args) {
  if (check_gemm(args, false) != MOE_OK) return 0;
  return plan_gemm(*args).ws_bytes;
}

int64_t moe_grouped_gemm_nvfp4_amax_slots(const moe_gemm_args *args) {
  if (check_gemm(args, false) != MOE_OK) return 0;
  return plan_gemm(*args).grid;
}

moe_status moe_grouped_gemm_nvfp4_can_implement(const moe_gemm_args *args) {
  return check_gemm(args, true);
}

moe_status moe_grouped_gemm_nvfp4(const moe_gemm_args *args, void *ws, size_t ws_bytes,
                                  hipStream_t stream) {
  const moe_status st = check_gemm(args, true);
  if (st != MOE_OK) return st;
  const GemmPlan plan = plan_gemm(*args);
  if (!ws || ws_bytes < plan.ws_bytes) return MOE_ERR_WORKSPACE;
  return launch_status(launch_grouped_gemm(*args, plan, ws, stream));
}

moe_status moe_grouped_gemm_nvfp4_noalloc(const moe_gemm_args *args, hipStream_t stream) {
  const moe_status st = check_gemm(args, true);
  if (st != MOE_OK) return st;
  const GemmPlan plan = plan_gemm(*args);
  if (plan.ws_bytes > kNoAllocScratchBytes) return MOE_ERR_WORKSPACE;
  void *ws = nullptr;
  const hipError_t e = device_scratch(&ws);
  if (e != hipSuccess) return launch_status(e);
  return launch_status(launch_grouped_gemm(*args, plan, ws, stream));
}

size_t moe_pack_weights_nvfp4_bytes(int64_t rows, int K) {
  if (rows < 0 || K < 256 || rows % 16 != 0 || K % 256 != 0) return 0;
  return packed_weights_bytes(rows, K);
}

moe_status moe_pack_weights_nvfp4(const uint8_t *B, const uint8_t *B_sf, int64_t rows, int K,
                                  uint8_t *packed, hipStream_t stream) {
  if (rows < 0 || K < 256 || rows >= (int64_t(1) << 40) / K) return MOE_ERR_SHAPE;
  if (rows % 16 != 0 || K % 256 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows / 16 * (K / 256) * 192 >= (int64_t(1) << 39)) return MOE_ERR_UNSUPPORTED;  // grid < 2^31
  if (rows > 0 && (!B || !B_sf || !packed)) return MOE_ERR_NULL;
  return launch_status(launch_pack_weights(B, B_sf, rows, K, packed, stream));
}

moe_status moe_finalize(const uint16_t *Y, int64_t R, const float *topk_w,
                        const int32_t *token_slot_row, int T, int k, int H, uint16_t *out,
                        hipStream_t stream) {
  if (T < 0 || k < 1 || k > 32 || H < 8 || R < 0) return MOE_ERR_SHAPE;
  if (H % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (T > 0 && R < 1) return MOE_ERR_SHAPE;
  if (T > 0 && (!Y || !topk_w || !token_slot_row || !out)) return MOE_ERR_NULL;
  return launch_status(launch_finalize(Y, R, topk_w, token_slot_row, T, k, H, out, stream));
}

}  // extern "C"
