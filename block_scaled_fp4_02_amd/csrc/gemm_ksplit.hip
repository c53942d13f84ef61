// Grouped NVFP4 GEMM on packed weights for few work items (e.g. one 8-expert grouped GEMM of
// 32 rows each): the waves of a workgroup split K (KS = 2, 4 or 8 ways) so that a grid of
// few (expert, n tile) items still puts two waves on every SIMD, and add their partial tiles
// in LDS in a fixed order (deterministic).
//
// A workgroup has max(4, KS) waves: NG = waves / KS groups of 64 weight rows, each split
// over KS waves that take consecutive K ranges.  Chunks hold up to 32 rows (two 16-row
// token tiles).  Each wave dequantises its own weight and activation fragments into
// registers (16x16x32 fp16 MFMA, fragment K order as in gemm_device.hpp).  Weight and
// activation fragments rotate through three register sets, so the loads of step s + 2 are
// in flight while step s computes -- with few steps per wave (e.g. 3 at K = 6144, KS = 8)
// every load of the wave is issued before its first MFMA.  All loads are unconditional
// range-checked buffer loads (past the wave's K range they return zeros and read nothing),
// so the compiler counts the loads in flight exactly.
#include "gemm_device.hpp"

namespace moe {
namespace gemm {
namespace {

constexpr int kSplitTiles = 2;                       // token tiles per chunk
constexpr int kSplitTile = 4 * kSplitTiles * 4 * 64;  // floats of one wave's partial tile

template <int KS>
constexpr int split_waves() { return KS < 4 ? 4 : KS; }

template <int NM, int KS, int EPI>
__device__ __forceinline__ void ks_body(const Params &P, float *red, float *wmax, int b, int e,
                                        int row0, int nrows, int nt) {
  constexpr int WAVES = split_waves<KS>();
  constexpr int NG = WAVES / KS;
  constexpr int SPAN = NG * 64;   // weight rows per workgroup
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int ng = wv % NG;
  const int kq = wv / NG;
  const int r = lane & 15;        // row within a 16-row tile
  const int g = lane >> 4;        // K group of the lane
  const int I = P.N / 2;
  const int steps = P.K / kKStep;
  const int iters = steps / KS;
  const int s_begin = kq * iters;

  // first weight row of the wave's four 16-row tiles (SwiGLU: gate, gate, up, up)
  int nrow[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    if (EPI != MOE_EPI_NONE) {
      const int gate = nt * (SPAN / 2) + ng * 32 + (j & 1) * 16;
      nrow[j] = (j >= 2) ? I + gate : gate;
    } else {
      nrow[j] = nt * SPAN + ng * 64 + j * 16;
    }
  }
  const uint32_t expert_bytes = static_cast<uint32_t>(P.N / 16) * steps * kPackBlock;
  const BufRsrc rb = make_rsrc(P.B + static_cast<int64_t>(e) * expert_bytes, expert_bytes);
  uint32_t b_code[4], b_scale[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint32_t t = static_cast<uint32_t>(nrow[j] / 16) * steps * kPackBlock;
    b_code[j] = t + lane * 16;
    b_scale[j] = t + 2048 + lane * 4;
  }
  const uint32_t half_k = P.K / 2, k16 = P.K / 16;
  const BufRsrc ra_codes = make_rsrc(P.A, static_cast<uint32_t>(P.rows_A * half_k));
  const BufRsrc ra_scales = make_rsrc(P.A_sf, static_cast<uint32_t>(P.rows_A * k16));
  uint32_t a_code[NM], a_scale[NM];
#pragma unroll
  for (int mt = 0; mt < NM; mt++) {
    const int m = mt * 16 + r;
    int64_t p = row0 + (m < nrows ? m : 0);
    int64_t src = P.A_rows ? static_cast<int64_t>(P.A_rows[p]) : p;
    src = src < 0 ? 0 : (src >= P.rows_A ? P.rows_A - 1 : src);
    a_code[mt] = static_cast<uint32_t>(src) * half_k + 32 * g;
    a_scale[mt] = static_cast<uint32_t>(src) * k16 + 4 * g;
  }
  // it: step index within the wave's K range
  auto load_b = [&](Frag16 (&f)[4], int it) {
    const uint32_t so = it < iters ? static_cast<uint32_t>(s_begin + it) * kPackBlock : kOob;
#pragma unroll
    for (int j = 0; j < 4; j++) load_frag16_buf(f[j], rb, b_code[j] + so, 1024, rb, b_scale[j] + so);
  };
  auto load_a = [&](Frag16 (&f)[NM], int it) {
    const bool v = it < iters;
    const uint32_t s = static_cast<uint32_t>(s_begin + it);
#pragma unroll
    for (int mt = 0; mt < NM; mt++)
      load_frag16_buf(f[mt], ra_codes, v ? a_code[mt] + s * (kKStep / 2) : kOob, 16, ra_scales,
                      v ? a_scale[mt] + s * (kKStep / 16) : kOob);
  };

  float4v acc[4][NM];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int mt = 0; mt < NM; mt++) acc[j][mt] = float4v{};

  Frag16 b0[4], b1[4], b2[4], a0[NM], a1[NM], a2[NM];
  load_b(b0, 0);
  load_a(a0, 0);
  load_b(b1, 1);
  load_a(a1, 1);
  auto step = [&](const Frag16 (&fb)[4], const Frag16 (&fa)[NM], Frag16 (&bl)[4], Frag16 (&al)[NM], int it) {
    load_b(bl, it + 2);
    load_a(al, it + 2);
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
        for (int mt = 0; mt < NM; mt++) af[mt] = dequant8(word(fa[mt].q[q], d), asc[mt][d >> 1]);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const half8 bf = dequant8(word(fb[j].q[q], d), bsc[j][d >> 1]);
#pragma unroll
          for (int mt = 0; mt < NM; mt++)
            acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf, af[mt], acc[j][mt], 0, 0, 0);
        }
      }
    }
  };
  int it = 0;
  for (; it + 3 <= iters; it += 3) {
    step(b0, a0, b2, a2, it);
    step(b1, a1, b0, a0, it + 1);
    step(b2, a2, b1, a1, it + 2);
  }
  if (it < iters) step(b0, a0, b2, a2, it);
  if (it + 1 < iters) step(b1, a1, b0, a0, it + 1);

  // K parts 1..KS-1 leave their partial tiles in LDS; part 0 adds them in order 1, 2, ...
  if (kq > 0) {
    float *mine = red + ((kq - 1) * NG + ng) * kSplitTile;
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int mt = 0; mt < NM; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) mine[((j * kSplitTiles + mt) * 4 + i) * 64 + lane] = acc[j][mt][i];
  }
  __syncthreads();
  if (kq == 0) {
#pragma unroll 1
    for (int o = 1; o < KS; o++) {   // rolled: one partial tile's loads in flight at a time
      const float *src = red + ((o - 1) * NG + ng) * kSplitTile;
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int mt = 0; mt < NM; mt++)
#pragma unroll
          for (int i = 0; i < 4; i++) acc[j][mt][i] += src[((j * kSplitTiles + mt) * 4 + i) * 64 + lane];
    }
  }

  // epilogue: 16x16 D lane layout -- weight row 4g + i, token row r of the tile
  const float gscale = (*P.A_gs) * P.B_gs[e];
  if constexpr (EPI == MOE_EPI_SWIGLU_NVFP4) {
    if (kq == 0) {   // wave-uniform
      const float g2 = *P.D_gs;
#pragma unroll
      for (int mt = 0; mt < NM; mt++) {
        const int m = mt * 16 + r;
        const int64_t p = row0 + (m < nrows ? m : 0);
#pragma unroll
        for (int jp = 0; jp < 2; jp++) {
          const int blk = nrow[jp] / 16;
          swiglu_nvfp4_block(acc[jp][mt], acc[2 + jp][mt], gscale, g2, m < nrows,
                             static_cast<uint8_t *>(P.D) + p * (I / 2) + blk * 8, P.D_sf + p * (I / 16) + blk, g);
        }
      }
    }
    return;
  }
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
    if (threadIdx.x == 0) {
      float m = wmax[0];
      for (int w = 1; w < WAVES; w++) m = fmaxf(m, wmax[w]);
      P.amax_out[b] = m;
    }
  }
}

// Two waves per SIMD: 4-wave workgroups two per CU, 8-wave workgroups one per CU.
template <int KS, int EPI>
__global__ __launch_bounds__(64 * split_waves<KS>(), 8 / split_waves<KS>()) void gemm_ksplit_kernel(Params P) {
  constexpr int WAVES = split_waves<KS>();
  __shared__ float red[(KS - 1) * (WAVES / KS) * kSplitTile];
  __shared__ float wmax[WAVES];
  const int b = blockIdx.x;
  int4 item;
  if (!item_for_block(P, b, item)) {
    if (EPI == MOE_EPI_SWIGLU && threadIdx.x == 0) P.amax_out[b] = 0.f;
    return;
  }
  if (item.z <= 16) ks_body<1, KS, EPI>(P, red, wmax, b, item.x, item.y, item.z, item.w);
  else ks_body<2, KS, EPI>(P, red, wmax, b, item.x, item.y, item.z, item.w);
}

template <int EPI>
void launch_epi(const Params &p, int ks, dim3 grid, hipStream_t stream) {
  if (ks == 2) hipLaunchKernelGGL((gemm_ksplit_kernel<2, EPI>), grid, dim3(64 * split_waves<2>()), 0, stream, p);
  else if (ks == 4) hipLaunchKernelGGL((gemm_ksplit_kernel<4, EPI>), grid, dim3(64 * split_waves<4>()), 0, stream, p);
  else hipLaunchKernelGGL((gemm_ksplit_kernel<8, EPI>), grid, dim3(64 * split_waves<8>()), 0, stream, p);
}

}  // namespace

int ksplit_chunk_rows() { return kSplitTiles * 16; }
int ksplit_waves(int ks) { return ks < 4 ? 4 : ks; }

void launch_ksplit(const Params &p, int epi, int ks, dim3 grid, hipStream_t stream) {
  if (epi == MOE_EPI_SWIGLU) launch_epi<MOE_EPI_SWIGLU>(p, ks, grid, stream);
  else if (epi == MOE_EPI_SWIGLU_NVFP4) launch_epi<MOE_EPI_SWIGLU_NVFP4>(p, ks, grid, stream);
  else launch_epi<MOE_EPI_NONE>(p, ks, grid, stream);
}

}  // namespace gemm
}  // namespace moe
