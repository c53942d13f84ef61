// Grouped NVFP4 GEMM on packed weights for few groups (e.g. 8 experts x 32 rows): the four
// waves of a workgroup split K (2 or 4 ways) so that a grid of few (expert, n tile) items
// still has enough waves, and add their partial tiles in LDS in a fixed order
// (deterministic).  Each wave dequantises its own weight and activation fragments into
// registers (16x16x32 fp16 MFMA, fragment K order as in gemm_device.hpp); a workgroup covers
// (4 / KS) * 64 weight rows.
#include "gemm_device.hpp"

namespace moe {
namespace gemm {
namespace {

template <int NM, int KS, int EPI>
__device__ __forceinline__ void ks_body(const Params &P, float *red, float *wmax, int b, int e,
                                        int row0, int nrows, int nt) {
  constexpr int NG = 4 / KS;
  constexpr int SPAN = NG * 64;   // weight rows per workgroup
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int ng = wv % NG;
  const int kq = wv / NG;
  const int r = lane & 15;        // row within a 16-row tile
  const int g = lane >> 4;        // K group of the lane
  const int I = P.N / 2;
  const int steps = P.K / kKStep;

  // first weight row of the wave's four 16-row tiles (SwiGLU: gate, gate, up, up)
  int nrow[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    if (EPI == MOE_EPI_SWIGLU) {
      const int gate = nt * (SPAN / 2) + ng * 32 + (j & 1) * 16;
      nrow[j] = (j >= 2) ? I + gate : gate;
    } else {
      nrow[j] = nt * SPAN + ng * 64 + j * 16;
    }
  }
  // weight tiles: wave-uniform base pointers, per-lane 32-bit offsets
  const uint8_t *bbase[4];
#pragma unroll
  for (int j = 0; j < 4; j++)
    bbase[j] = P.B + (static_cast<int64_t>(e) * P.N + nrow[j]) / 16 * steps * kPackBlock;
  const uint32_t b_code_off = lane * 16, b_scale_off = 2048 + lane * 4;
  // token rows of the NM 16-row tiles of the chunk: 32-bit offsets into A
  // (rows_A * K / 2 < 2^32 is checked on the host)
  const uint32_t half_k = P.K / 2, k16 = P.K / 16;
  uint32_t aoff[NM];
#pragma unroll
  for (int mt = 0; mt < NM; mt++) {
    const int m = mt * 16 + r;
    int64_t p = row0 + (m < nrows ? m : 0);
    int64_t src = P.A_rows ? static_cast<int64_t>(P.A_rows[p]) : p;
    src = src < 0 ? 0 : (src >= P.rows_A ? P.rows_A - 1 : src);
    aoff[mt] = static_cast<uint32_t>(src);
  }

  float4v acc[4][NM];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int mt = 0; mt < NM; mt++) acc[j][mt] = float4v{};

  const int s_begin = kq * (steps / KS);
  const int iters = steps / KS;
  Frag16 fb[4], fa[NM], nb[4], na[NM];
  auto load_b = [&](Frag16 (&f)[4], int s) {
    const uint32_t so = static_cast<uint32_t>(s) * kPackBlock;
#pragma unroll
    for (int j = 0; j < 4; j++) load_frag16(f[j], bbase[j] + (so + b_code_off), bbase[j] + (so + b_scale_off), 1024);
  };
  auto load_a = [&](Frag16 (&f)[NM], int s) {
#pragma unroll
    for (int mt = 0; mt < NM; mt++)
        load_frag16(f[mt], P.A + (aoff[mt] * half_k + 32 * g + s * (kKStep / 2)),
                    P.A_sf + (aoff[mt] * k16 + 4 * g + s * (kKStep / 16)), 16);
  };
  load_a(fa, s_begin);
  load_b(fb, s_begin);

  for (int it = 0; it < iters; it++) {
    const bool more = it + 1 < iters;
    if (more) {
      load_a(na, s_begin + it + 1);
      load_b(nb, s_begin + it + 1);
    }
#pragma unroll
    for (int q = 0; q < 2; q++) {
      half2v bsc[4], asc[NM];
#pragma unroll
      for (int j = 0; j < 4; j++) bsc[j] = e4m3x2_to_f16(fb[j].s, q == 1);
#pragma unroll
      for (int mt = 0; mt < NM; mt++) asc[mt] = e4m3x2_to_f16(fa[mt].s, q == 1);
#pragma unroll
      for (int d = 0; d < 4; d++) {
        half8 af[NM];
#pragma unroll
        for (int mt = 0; mt < NM; mt++)
          af[mt] = dequant8(word(fa[mt].q[q], d), asc[mt][d >> 1]);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const half8 bf = dequant8(word(fb[j].q[q], d), bsc[j][d >> 1]);
#pragma unroll
          for (int mt = 0; mt < NM; mt++)
            acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf, af[mt], acc[j][mt], 0, 0, 0);
        }
      }
    }
    if (more) {
#pragma unroll
      for (int j = 0; j < 4; j++) fb[j] = nb[j];
#pragma unroll
      for (int mt = 0; mt < NM; mt++) fa[mt] = na[mt];
    }
  }

  if constexpr (KS > 1) {
    constexpr int TILE = 4 * kChunkTiles * 4 * 64;
    float *mine = red + ((kq - 1) * NG + ng) * TILE;
    if (kq > 0) {
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int mt = 0; mt < NM; mt++)
#pragma unroll
          for (int i = 0; i < 4; i++) mine[((j * kChunkTiles + mt) * 4 + i) * 64 + lane] = acc[j][mt][i];
    }
    __syncthreads();
    if (kq == 0) {
      for (int o = 1; o < KS; o++) {
        const float *src = red + ((o - 1) * NG + ng) * TILE;
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
          for (int mt = 0; mt < NM; mt++)
#pragma unroll
            for (int i = 0; i < 4; i++) acc[j][mt][i] += src[((j * kChunkTiles + mt) * 4 + i) * 64 + lane];
      }
    }
  }

  // epilogue: 16x16 D lane layout -- weight row 4g + i, token row r of the tile
  const float gscale = (*P.A_gs) * P.B_gs[e];
  float amax = 0.f;
  if (kq == 0) {
#pragma unroll
    for (int mt = 0; mt < NM; mt++) {
      const int m = mt * 16 + r;
      if (m < nrows) {
        const int64_t p = row0 + m;
        if (EPI == MOE_EPI_NONE) {
          uint16_t *drow = static_cast<uint16_t *>(P.D) + p * P.N;
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const uint32_t lo = f32_to_bf16(acc[j][mt][0] * gscale) |
                                (static_cast<uint32_t>(f32_to_bf16(acc[j][mt][1] * gscale)) << 16);
            const uint32_t hi = f32_to_bf16(acc[j][mt][2] * gscale) |
                                (static_cast<uint32_t>(f32_to_bf16(acc[j][mt][3] * gscale)) << 16);
            *reinterpret_cast<uint2 *>(drow + nrow[j] + 4 * g) = make_uint2(lo, hi);
          }
        } else {
          uint16_t *drow = static_cast<uint16_t *>(P.D) + p * I;
#pragma unroll
          for (int jp = 0; jp < 2; jp++) {
            uint16_t o[4];
#pragma unroll
            for (int c = 0; c < 4; c++) {
              o[c] = swiglu_bf16(acc[jp][mt][c] * gscale, acc[2 + jp][mt][c] * gscale);
              amax = fmaxf(amax, fabsf(bf16_to_f32(o[c])));
            }
            *reinterpret_cast<uint2 *>(drow + nrow[jp] + 4 * g) =
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

template <int KS, int EPI>
__global__ __launch_bounds__(256, 2) void gemm_ksplit_kernel(Params P) {
  constexpr int TILE = 4 * kChunkTiles * 4 * 64;
  __shared__ float red[KS > 1 ? (KS - 1) * (4 / KS) * TILE : 1];
  __shared__ float wmax[4];
  const int b = blockIdx.x;
  int4 item;
  if (!item_for_block(P, b, item)) {
    if (EPI == MOE_EPI_SWIGLU && threadIdx.x == 0) P.amax_out[b] = 0.f;
    return;
  }
  const int nm = (item.z + 15) / 16;   // workgroup-uniform
  if (nm <= 1) ks_body<1, KS, EPI>(P, red, wmax, b, item.x, item.y, item.z, item.w);
  else if (nm == 2) ks_body<2, KS, EPI>(P, red, wmax, b, item.x, item.y, item.z, item.w);
  else ks_body<3, KS, EPI>(P, red, wmax, b, item.x, item.y, item.z, item.w);
}

}  // namespace

void launch_ksplit(const Params &p, int epi, int ks, dim3 grid, hipStream_t stream) {
  const dim3 block(256);
  if (epi == MOE_EPI_SWIGLU) {
    if (ks == 2) hipLaunchKernelGGL((gemm_ksplit_kernel<2, MOE_EPI_SWIGLU>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((gemm_ksplit_kernel<4, MOE_EPI_SWIGLU>), grid, block, 0, stream, p);
  } else {
    if (ks == 2) hipLaunchKernelGGL((gemm_ksplit_kernel<2, MOE_EPI_NONE>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((gemm_ksplit_kernel<4, MOE_EPI_NONE>), grid, block, 0, stream, p);
  }
}

}  // namespace gemm
}  // namespace moe
