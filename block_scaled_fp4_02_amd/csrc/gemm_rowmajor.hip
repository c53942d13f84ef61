// Grouped NVFP4 GEMM on row-major weights ([E, N, K/2] codes, [E, N, K/16] scales, as
// produced by moe_quantize_nvfp4): 32x32x16 fp16 MFMA, each wave owns two 32-row weight
// tiles (with the SwiGLU epilogue a (gate, up) pair) and the item's one or two 32-row token
// tiles, dequantising both operands into registers.  A lane of half h holds, in load q
// (0..3) of a K step, the 32 elements [128h + 32q, +32) of its row, so its eight scale
// blocks [8h, 8h + 8) are one contiguous 8-byte load.  KS: K split across the waves of a
// workgroup (1, 2, 4), partial tiles added in LDS in a fixed order.
#include "gemm_device.hpp"

namespace moe {
namespace gemm {
namespace {

template <int NM, int KS, int EPI>
__device__ __forceinline__ void rm_body(const Params &P, float *red, float *wmax, int b, int e,
                                        int row0, int nrows, int nt) {
  constexpr int TPW = 2;
  constexpr int NG = 4 / KS;
  constexpr int SPAN = NG * TPW * 32;                  // weight rows per workgroup
  constexpr int QS = 16;                               // code piece stride
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int ng = wv % NG;
  const int kq = wv / NG;
  const int r = lane & 31;    // row within a 32-row tile
  const int h = lane >> 5;    // lane half: which 128 of each 256 K elements
  const int I = P.N / 2;
  const int steps = P.K / kKStep;

  // first weight row of each of this wave's tiles
  int nrow[TPW];
#pragma unroll
  for (int j = 0; j < TPW; j++) {
    if (EPI == MOE_EPI_SWIGLU) {
      const int gate = nt * (SPAN / 2) + (ng * (TPW / 2) + j / 2) * 32;
      nrow[j] = (j & 1) ? I + gate : gate;
    } else {
      nrow[j] = nt * SPAN + (ng * TPW + j) * 32;
    }
  }
  const int64_t half_k = P.K / 2, k16 = P.K / 16;
  const uint8_t *bq[TPW];
  const uint8_t *bs[TPW];
#pragma unroll
  for (int j = 0; j < TPW; j++) {
    const int64_t row = static_cast<int64_t>(e) * P.N + nrow[j];
    bq[j] = P.B + (row + r) * half_k + 64 * h;
    bs[j] = P.B_sf + (row + r) * k16 + 8 * h;
  }
  // per-step advance of the weight pointers
  const int64_t b_code_step = kKStep / 2;
  const int64_t b_scale_step = kKStep / 16;

  // activation rows of the (one or two) 32-row tiles of the chunk
  constexpr int nm = NM;
  const uint8_t *aq[2];
  const uint8_t *as[2];
#pragma unroll
  for (int mt = 0; mt < 2; mt++) {
    const int m = mt * 32 + r;
    int64_t p = row0 + (m < nrows ? m : 0);
    int64_t src = P.A_rows ? static_cast<int64_t>(P.A_rows[p]) : p;
    src = src < 0 ? 0 : (src >= P.rows_A ? P.rows_A - 1 : src);
    aq[mt] = P.A + src * half_k + 64 * h;
    as[mt] = P.A_sf + src * k16 + 8 * h;
  }

  float16v acc[TPW][2];
#pragma unroll
  for (int j = 0; j < TPW; j++)
#pragma unroll
    for (int mt = 0; mt < 2; mt++) acc[j][mt] = float16v{};

  const int s_begin = kq * (steps / KS);
  const int iters = steps / KS;

  Frag fb[TPW], fa[2], nb[TPW], na[2];
#pragma unroll
  for (int j = 0; j < TPW; j++) load_frag(fb[j], bq[j] + s_begin * b_code_step, bs[j] + s_begin * b_scale_step, QS);
  load_frag(fa[0], aq[0] + s_begin * (kKStep / 2), as[0] + s_begin * (kKStep / 16), 16);
  if (nm == 2) load_frag(fa[1], aq[1] + s_begin * (kKStep / 2), as[1] + s_begin * (kKStep / 16), 16);

  for (int it = 0; it < iters; it++) {
    const int sn = s_begin + it + 1;
    const bool more = it + 1 < iters;
    if (more) {  // prefetch the next K step while this one computes
      load_frag(na[0], aq[0] + sn * (kKStep / 2), as[0] + sn * (kKStep / 16), 16);
      if (nm == 2) load_frag(na[1], aq[1] + sn * (kKStep / 2), as[1] + sn * (kKStep / 16), 16);
#pragma unroll
      for (int j = 0; j < TPW; j++) load_frag(nb[j], bq[j] + sn * b_code_step, bs[j] + sn * b_scale_step, QS);
    }
#pragma unroll
    for (int q = 0; q < 4; q++) {
#pragma unroll
      for (int d = 0; d < 4; d++) {
        // dword d of piece q: elements [128h + 32q + 8d, +8), scale block 8h + 2q + d/2,
        // i.e. byte 2(q % 2) + d/2 of scale word q/2
        const int sw = q >> 1, sb = 2 * (q & 1) + (d >> 1);
        const half8 af0 = dequant8(word(fa[0].q[q], d), e4m3_to_f16(sw ? fa[0].s.y : fa[0].s.x, sb));
        half8 af1;
        if (nm == 2) af1 = dequant8(word(fa[1].q[q], d), e4m3_to_f16(sw ? fa[1].s.y : fa[1].s.x, sb));
#pragma unroll
        for (int j = 0; j < TPW; j++) {
          const half8 bf = dequant8(word(fb[j].q[q], d), e4m3_to_f16(sw ? fb[j].s.y : fb[j].s.x, sb));
          acc[j][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf, af0, acc[j][0], 0, 0, 0);
          if (nm == 2) acc[j][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf, af1, acc[j][1], 0, 0, 0);
        }
      }
    }
    if (more) {
#pragma unroll
      for (int j = 0; j < TPW; j++) fb[j] = nb[j];
      fa[0] = na[0];
      if (nm == 2) fa[1] = na[1];
    }
  }

  // K split across waves: partial tiles added in LDS in a fixed order
  if constexpr (KS > 1) {
    constexpr int TILE = TPW * 2 * 16 * 64;
    float *mine = red + ((kq - 1) * NG + ng) * TILE;
    if (kq > 0) {
#pragma unroll
      for (int j = 0; j < TPW; j++)
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int i = 0; i < 16; i++) mine[((j * 2 + mt) * 16 + i) * 64 + lane] = acc[j][mt][i];
    }
    __syncthreads();
    if (kq == 0) {
#pragma unroll 1
      for (int o = 1; o < KS; o++) {
        const float *src = red + ((o - 1) * NG + ng) * TILE;
#pragma unroll
        for (int j = 0; j < TPW; j++)
#pragma unroll
          for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int i = 0; i < 16; i++) acc[j][mt][i] += src[((j * 2 + mt) * 16 + i) * 64 + lane];
      }
    }
  }

  // epilogue: D lane layout of the 32x32 tile -- weight row 8(i/4) + 4h + i%4, chunk row r
  const float gscale = (*P.A_gs) * P.B_gs[e];
  float amax = 0.f;
  if (kq == 0) {
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      const int m = mt * 32 + r;
      if (mt < nm && m < nrows) {
        const int64_t p = row0 + m;
        if (EPI == MOE_EPI_NONE) {
          uint16_t *drow = static_cast<uint16_t *>(P.D) + p * P.N;
#pragma unroll
          for (int j = 0; j < TPW; j++)
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++) {
              uint32_t lo = f32_to_bf16(acc[j][mt][4 * g4 + 0] * gscale) |
                            (static_cast<uint32_t>(f32_to_bf16(acc[j][mt][4 * g4 + 1] * gscale)) << 16);
              uint32_t hi = f32_to_bf16(acc[j][mt][4 * g4 + 2] * gscale) |
                            (static_cast<uint32_t>(f32_to_bf16(acc[j][mt][4 * g4 + 3] * gscale)) << 16);
              *reinterpret_cast<uint2 *>(drow + nrow[j] + 8 * g4 + 4 * h) = make_uint2(lo, hi);
            }
        } else {
          uint16_t *drow = static_cast<uint16_t *>(P.D) + p * I;
#pragma unroll
          for (int jp = 0; jp < TPW / 2; jp++)
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++) {
              uint16_t o[4];
#pragma unroll
              for (int c = 0; c < 4; c++) {
                o[c] = swiglu_bf16(acc[2 * jp][mt][4 * g4 + c] * gscale, acc[2 * jp + 1][mt][4 * g4 + c] * gscale);
                amax = fmaxf(amax, fabsf(bf16_to_f32(o[c])));
              }
              *reinterpret_cast<uint2 *>(drow + nrow[2 * jp] + 8 * g4 + 4 * h) =
                  make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16));
            }
        }
      }
    }
  }
  if (EPI == MOE_EPI_SWIGLU) {
    amax = wave_max(amax);
    if (lane == 0) wmax[wv] = amax;
    __syncthreads();
    if (threadIdx.x == 0) P.amax_out[b] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  }
}

constexpr int kRowMajorWgPerCu = 2;   // workgroups per CU the launch bounds promise

template <int KS, int EPI>
__global__ __launch_bounds__(256, kRowMajorWgPerCu) void gemm_rowmajor_kernel(Params P) {
  constexpr int TILE = 2 * 2 * 16 * 64;
  __shared__ float red[KS > 1 ? (KS - 1) * (4 / KS) * TILE : 1];
  __shared__ float wmax[4];
  static_assert(TILE == lds::kRowMajorPartialFloats && sizeof(red) + sizeof(wmax) == lds::rowmajor_kernel_bytes(KS),
                "LDS of the row-major kernel differs from its budget entry");
  static_assert(lds::fits_cu(lds::rowmajor_kernel_bytes(KS), kRowMajorWgPerCu), "row-major tile exceeds the CU's LDS");
  const int b = blockIdx.x;
  int4 item;
  if (!item_for_block(P, b, item)) {
    if (EPI == MOE_EPI_SWIGLU && threadIdx.x == 0) P.amax_out[b] = 0.f;
    return;
  }
  if (item.z > 32) rm_body<2, KS, EPI>(P, red, wmax, b, item.x, item.y, item.z, item.w);
  else rm_body<1, KS, EPI>(P, red, wmax, b, item.x, item.y, item.z, item.w);
}

}  // namespace

void launch_rowmajor(const Params &p, int epi, int ks, dim3 grid, hipStream_t stream) {
  const dim3 block(256);
  if (epi == MOE_EPI_SWIGLU) {
    if (ks == 1) hipLaunchKernelGGL((gemm_rowmajor_kernel<1, MOE_EPI_SWIGLU>), grid, block, 0, stream, p);
    else if (ks == 2) hipLaunchKernelGGL((gemm_rowmajor_kernel<2, MOE_EPI_SWIGLU>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((gemm_rowmajor_kernel<4, MOE_EPI_SWIGLU>), grid, block, 0, stream, p);
  } else {
    if (ks == 1) hipLaunchKernelGGL((gemm_rowmajor_kernel<1, MOE_EPI_NONE>), grid, block, 0, stream, p);
    else if (ks == 2) hipLaunchKernelGGL((gemm_rowmajor_kernel<2, MOE_EPI_NONE>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((gemm_rowmajor_kernel<4, MOE_EPI_NONE>), grid, block, 0, stream, p);
  }
}

}  // namespace gemm
}  // namespace moe
