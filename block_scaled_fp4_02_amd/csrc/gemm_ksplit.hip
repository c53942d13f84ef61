// Grouped NVFP4 GEMM on packed weights for few work items (e.g. one 8-expert grouped GEMM of
// 32 rows each): the waves of a workgroup split K (KS = 2, 4 or 8 ways) so that a grid of
// few (expert, n tile) items still puts two waves on every SIMD, and add their partial tiles
// in LDS in a fixed order (deterministic).
//
// A workgroup has max(4, KS) waves: NG = waves / KS groups of 64 weight rows, each split
// over KS waves that take consecutive K ranges (in the 8-wave workgroup the older wave on
// each SIMD takes one half step more than its partner: the SIMD issues from it first).
// Chunks hold up to 32 rows (two 16-row token tiles).  Each wave dequantises its own weight and activation fragments into
// registers (16x16x32 fp16 MFMA, fragment K order as in gemm_device.hpp).
//
// Streaming in half steps: a wave's K range is consumed 128 elements at a time (one of the
// two 32-element pieces of each lane's K group, with its two scale bytes), and only the
// next half step is in flight while one computes.  When every load of a wave is issued up
// front, the memory system returns the chip's requests in no particular order and a step is
// complete only once nearly all data has arrived, so no wave starts computing until late;
// with one half step of lead, data arrives roughly in the order it is used.  All loads are
// unconditional range-checked buffer loads (past the wave's K range they return zeros and
// read nothing), so the compiler counts the loads in flight exactly; the weight loads of an
// expert's last row chunk carry the non-temporal hint.
//
// After the K loop every wave parks its partial tile in LDS; then the waves of a row group
// share the reduction and the epilogue, each summing the KS partials of its own (weight
// tile, token tile) units in K-part order 0, 1, ... (the same sum in every run) and storing
// them.  The grid holds no more workgroups than fit on the chip at once; each loops over
// the items of virtual blocks blockIdx.x, + gridDim.x, ...
#include "gemm_device.hpp"

namespace moe {
namespace gemm {
namespace {

constexpr int kSplitTiles = 2;                       // token tiles per chunk
constexpr int kSplitTile = 4 * kSplitTiles * 4 * 64;  // floats of one wave's partial tile

template <int KS>
constexpr int split_waves() { return KS < 4 ? 4 : KS; }

// One lane's half of a K step for one 16-row tile: the 16 code bytes of piece q (elements
// [64g + 32q, +32) of the step) and the scale bytes 2q, 2q + 1 of its four blocks' word, in
// the low half of s.
struct Half16 {
  uint4 q;
  uint32_t s;
};

template <int POLICY = 0>
__device__ __forceinline__ void load_half16_buf(Half16 &f, BufRsrc rc, uint32_t code_off, BufRsrc rs,
                                                uint32_t scale_off) {
  const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rc, code_off, 0, POLICY);
  f.q = make_uint4(a.x, a.y, a.z, a.w);
  f.s = __builtin_amdgcn_raw_buffer_load_b16(rs, scale_off, 0, POLICY);
}

// First weight row of 16-row tile j (0..3) of row group ng in n tile nt.  SwiGLU tiles are
// gate, gate, up, up: up row I + r pairs with gate row r.
template <int KS, int EPI>
__device__ __forceinline__ int tile_row(const Params &P, int nt, int ng, int j) {
  constexpr int SPAN = (split_waves<KS>() / KS) * 64;   // weight rows per workgroup
  if (EPI != MOE_EPI_NONE) {
    const int gate = nt * (SPAN / 2) + ng * 32 + (j & 1) * 16;
    return j >= 2 ? P.N / 2 + gate : gate;
  }
  return nt * SPAN + ng * 64 + j * 16;
}

// Sum of the KS partial tiles of row group ng for weight tile j, token tile mt, in K-part
// order (lane layout of the 16x16 MFMA result).
template <int KS, int NG>
__device__ __forceinline__ float4v sum_partials(const float *red, int ng, int j, int mt, int lane) {
  float4v s;
#pragma unroll
  for (int i = 0; i < 4; i++) s[i] = red[(ng * kSplitTile) + ((j * kSplitTiles + mt) * 4 + i) * 64 + lane];
#pragma unroll
  for (int o = 1; o < KS; o++) {
    const float *src = red + (o * NG + ng) * kSplitTile;
#pragma unroll
    for (int i = 0; i < 4; i++) s[i] += src[((j * kSplitTiles + mt) * 4 + i) * 64 + lane];
  }
  return s;
}

// One work item (expert e, rows [row0, row0 + nrows), n tile nt); returns the wave's
// max |act| for the SWIGLU epilogue (0 otherwise).  NT: the expert's last row chunk, whose
// weight loads carry the non-temporal hint.
template <int NM, int KS, int EPI, bool NT>
__device__ __forceinline__ float ks_body(const Params &P, float *red, int e, int row0, int nrows, int nt) {
  constexpr int WAVES = split_waves<KS>();
  constexpr int NG = WAVES / KS;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int ng = wv % NG;
  const int kq = wv / NG;
  const int r = lane & 15;        // row within a 16-row tile
  const int g = lane >> 4;        // K group of the lane
  const int I = P.N / 2;
  const int steps = P.K / kKStep;
  // K range of this wave in half steps: 2 * steps / KS each, except that with one 8-wave
  // workgroup per CU the first wave on each SIMD (K parts 0-3: the older wave, which the SIMD
  // issues from first) takes one half step more and its partner one fewer
  const int base = 2 * steps / KS;
  const int delta = (KS == 8 && base >= 4) ? 1 : 0;
  const int halves = base + (kq < KS / 2 ? delta : -delta);
  const int h_begin = kq * base + (kq < KS / 2 ? kq : KS - kq) * delta;
  // global scales, loaded at the start: left in the epilogue the compiler issues these
  // loads after the last MFMA and waits a full memory round trip for them
  const float gscale = (*P.A_gs) * P.B_gs[e];

  const uint32_t expert_bytes = static_cast<uint32_t>(P.N / 16) * steps * kPackBlock;
  const BufRsrc rb = make_rsrc(P.B + static_cast<int64_t>(e) * expert_bytes, expert_bytes);
  uint32_t b_code[4], b_scale[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint32_t t = static_cast<uint32_t>(tile_row<KS, EPI>(P, nt, ng, j) / 16) * steps * kPackBlock;
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
  // Half h of the wave's K range is half h_begin + h of the row: piece q = that % 2 of step
  // that / 2.
  auto load_b = [&](Half16 (&f)[4], int h) {
    const int hg = h_begin + h;
    const uint32_t so = h < halves ? static_cast<uint32_t>(hg >> 1) * kPackBlock : kOob;
    const uint32_t q = static_cast<uint32_t>(hg & 1);
#pragma unroll
    for (int j = 0; j < 4; j++)
      load_half16_buf<NT ? kNonTemporal : 0>(f[j], rb, b_code[j] + so + q * 1024, rb, b_scale[j] + so + 2 * q);
  };
  auto load_a = [&](Half16 (&f)[NM], int h) {
    const bool v = h < halves;
    const int hg = h_begin + h;
    const uint32_t s = static_cast<uint32_t>(hg >> 1);
    const uint32_t q = static_cast<uint32_t>(hg & 1);
#pragma unroll
    for (int mt = 0; mt < NM; mt++)
      load_half16_buf(f[mt], ra_codes, v ? a_code[mt] + s * (kKStep / 2) + 16 * q : kOob, ra_scales,
                      v ? a_scale[mt] + s * (kKStep / 16) + 2 * q : kOob);
  };

  float4v acc[4][NM];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int mt = 0; mt < NM; mt++) acc[j][mt] = float4v{};

  // MFMA d of a half takes dword d of the piece, elements [64g + 32q + 8d, +8), whose scale
  // is byte d / 2 of the half's scale pair.
  auto compute = [&](const Half16 (&fb)[4], const Half16 (&fa)[NM]) {
    half2v bsc[4], asc[NM];
#pragma unroll
    for (int j = 0; j < 4; j++) bsc[j] = e4m3x2_to_f16(fb[j].s, false);
#pragma unroll
    for (int mt = 0; mt < NM; mt++) asc[mt] = e4m3x2_to_f16(fa[mt].s, false);
#pragma unroll
    for (int d = 0; d < 4; d++) {
      half8 af[NM];
#pragma unroll
      for (int mt = 0; mt < NM; mt++) af[mt] = dequant8(word(fa[mt].q, d), asc[mt][d >> 1]);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const half8 bf = dequant8(word(fb[j].q, d), bsc[j][d >> 1]);
#pragma unroll
        for (int mt = 0; mt < NM; mt++)
          acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf, af[mt], acc[j][mt], 0, 0, 0);
      }
    }
  };
  // two register sets: the loads of half h + 1 are issued as half h starts computing
  Half16 b0[4], b1[4], a0[NM], a1[NM];
  load_b(b0, 0);
  load_a(a0, 0);
  int h = 0;
  for (; h + 2 <= halves; h += 2) {
    load_b(b1, h + 1);
    load_a(a1, h + 1);
    compute(b0, a0);
    load_b(b0, h + 2);
    load_a(a0, h + 2);
    compute(b1, a1);
  }
  if (h < halves) compute(b0, a0);   // an odd count: b0 holds the last half

  // every wave parks its partial tile; the row group's KS waves then share the units
  float *mine = red + (kq * NG + ng) * kSplitTile;
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int mt = 0; mt < NM; mt++)
#pragma unroll
      for (int i = 0; i < 4; i++) mine[((j * kSplitTiles + mt) * 4 + i) * 64 + lane] = acc[j][mt][i];
  __syncthreads();

  // epilogue: 16x16 D lane layout -- weight row 4g + i of the tile, token row r
  float amax = 0.f;
  if constexpr (EPI == MOE_EPI_NONE) {
    for (int u = kq; u < 4 * NM; u += KS) {   // unit u = (weight tile u / NM, token tile u % NM)
      const int j = u / NM, mt = u % NM;
      const float4v s = sum_partials<KS, NG>(red, ng, j, mt, lane);
      const int m = mt * 16 + r;
      if (m < nrows) {
        uint16_t *drow = static_cast<uint16_t *>(P.D) + (row0 + m) * static_cast<int64_t>(P.N);
        const uint32_t lo = f32_to_bf16(s[0] * gscale) | (static_cast<uint32_t>(f32_to_bf16(s[1] * gscale)) << 16);
        const uint32_t hi = f32_to_bf16(s[2] * gscale) | (static_cast<uint32_t>(f32_to_bf16(s[3] * gscale)) << 16);
        *reinterpret_cast<uint2 *>(drow + tile_row<KS, EPI>(P, nt, ng, j) + 4 * g) = make_uint2(lo, hi);
      }
    }
  } else {
    for (int u = kq; u < 2 * NM; u += KS) {   // unit u = (gate tile u / NM, token tile u % NM)
      const int jp = u / NM, mt = u % NM;
      const float4v gate = sum_partials<KS, NG>(red, ng, jp, mt, lane);
      const float4v up = sum_partials<KS, NG>(red, ng, jp + 2, mt, lane);
      const int m = mt * 16 + r;
      const int col = tile_row<KS, EPI>(P, nt, ng, jp);   // act column of the gate tile
      if constexpr (EPI == MOE_EPI_SWIGLU_NVFP4) {
        // all lanes take part (the block maximum is exchanged between lanes of a row)
        const int64_t p = row0 + (m < nrows ? m : 0);
        const int blk = col / 16;
        swiglu_nvfp4_block(gate, up, gscale, *P.D_gs, m < nrows,
                           static_cast<uint8_t *>(P.D) + p * (I / 2) + blk * 8, P.D_sf + p * (I / 16) + blk, g);
      } else if (m < nrows) {
        uint16_t *drow = static_cast<uint16_t *>(P.D) + (row0 + m) * static_cast<int64_t>(I);
        uint16_t o[4];
#pragma unroll
        for (int c = 0; c < 4; c++) {
          o[c] = swiglu_bf16(gate[c] * gscale, up[c] * gscale);
          amax = fmaxf(amax, fabsf(bf16_to_f32(o[c])));
        }
        *reinterpret_cast<uint2 *>(drow + col + 4 * g) =
            make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16));
      }
    }
  }
  return amax;
}

// Two waves per SIMD: 4-wave workgroups two per CU, 8-wave workgroups one per CU.
template <int KS, int EPI>
__global__ __launch_bounds__(64 * split_waves<KS>(), 8 / split_waves<KS>()) void gemm_ksplit_kernel(Params P) {
  constexpr int WAVES = split_waves<KS>();
  __shared__ float red[WAVES * kSplitTile];
  __shared__ float wmax[WAVES];
  static_assert(sizeof(red) + sizeof(wmax) == lds::ksplit_kernel_bytes(kSplitTiles, WAVES),
                "LDS of the K-split kernel differs from its budget entry");
  static_assert(lds::fits_cu(lds::ksplit_kernel_bytes(kSplitTiles, WAVES), 8 / WAVES),
                "K-split tile exceeds the CU's LDS");
  float amax = 0.f;
  for (int vb = blockIdx.x;; vb += gridDim.x) {   // a multiple of 8 apart: the same XCD
    int4 item;
    bool last;
    if (!item_for_block<false>(P, vb, item, last)) break;
    float m;
    if (last) m = item.z <= 16 ? ks_body<1, KS, EPI, true>(P, red, item.x, item.y, item.z, item.w)
                               : ks_body<2, KS, EPI, true>(P, red, item.x, item.y, item.z, item.w);
    else m = item.z <= 16 ? ks_body<1, KS, EPI, false>(P, red, item.x, item.y, item.z, item.w)
                          : ks_body<2, KS, EPI, false>(P, red, item.x, item.y, item.z, item.w);
    amax = fmaxf(amax, m);
    __syncthreads();   // the next item rewrites the partial tiles
  }
  if (EPI == MOE_EPI_SWIGLU) {
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
    __syncthreads();
    if (threadIdx.x == 0) {
      float m = wmax[0];
      for (int w = 1; w < WAVES; w++) m = fmaxf(m, wmax[w]);
      P.amax_out[blockIdx.x] = m;
    }
  }
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
