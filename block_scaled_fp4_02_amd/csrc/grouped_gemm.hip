// Grouped NVFP4 GEMM for small per-expert row counts (decode), on CDNA4 MFMA.
//
// What it computes: one GEMM per expert over that expert's rows, all experts in one
// launch, with the group sizes read on the device -- the grouped launch with a
// per-expert problem-size array of "Tracing the Failure: Debugging CUTLASS FP4 Tile
// Configurations on Blackwell SM120" (section "Input Knowledge Required"), FP4 operands
// with one FP8 scale per 16 elements along K on both sides ("Cracking the SM120 Shared
// Memory Ceiling", section "The Shared Memory Calculation"), and the NONE pass-through
// epilogue of "The Epilogue That Broke the Kernel" (section "The Insight: FINALIZE vs
// NONE"), plus a SwiGLU epilogue for the gate/up projection.
//
// Design (not the pages' SM120 tile; this is for gfx950):
//  * At ~32 rows per expert the kernel is bound by streaming the packed weights from HBM
//    (about 110 FLOP per weight byte, far under the MFMA ridge).  Every weight byte is
//    read exactly once, straight into registers, by the one wave that uses it; no LDS
//    staging of B.  Each wave owns 2 x 32 weight rows and all (<= 64) rows of its chunk.
//  * Exactness: E2M1 x E4M3 has at most 6 significant bits and lies in [2^-10, 2688], so
//    each element times its block scale is exact in fp16.  Both operands are dequantised
//    that way (hardware FP4->fp16 conversion, then a packed fp16 multiply by the block
//    scale), so a plain fp16 MFMA with fp32 accumulation sums exact products; the two
//    global scales multiply the fp32 result.  (gfx950's block-scaled FP4 MFMA takes
//    power-of-two scales per 32 elements and cannot carry an E4M3 scale per 16.)
//  * K permutation: the contraction is order-free and every element carries its own
//    scale after dequantisation, so lane halves may take any K order as long as both
//    operands use the same one.  Here a lane of half h holds, in load q (0..3) of a
//    256-wide K step, the 32 elements [128h + 32q, +32) of its row, so its eight scale
//    blocks [8h, 8h + 8) are one contiguous 8-byte load; a row's 128 bytes per step are
//    covered by the lane pair over the four loads.
//  * Work list: a one-workgroup schedule kernel turns expert_offsets into items
//    (expert, row chunk of <= 64, n tile), ordered expert-major then n tile then chunk.
//    The grid is the host-side upper bound; workgroup b runs on XCD b % 8, so the items
//    are dealt to XCDs in contiguous ranges (neighbouring n tiles of one expert share
//    that XCD's L2 for the activation rows).  Items past the device-side count exit.
//  * Few experts (e.g. 8 groups): the four waves of a workgroup split K (2 or 4 ways)
//    and add their partial tiles in LDS in a fixed order -- deterministic.
#include "common.hpp"

#include <algorithm>

namespace moe {
namespace {

constexpr int kKStep = 256;   // K elements per wave iteration
constexpr int kChunkRows = 64;  // rows per work item (two 32-row MFMA tiles)

struct GemmParams {
  const uint8_t *A;
  const uint8_t *A_sf;
  const float *A_gs;
  const int32_t *A_rows;
  int64_t rows_A;
  const uint8_t *B;
  const uint8_t *B_sf;
  const float *B_gs;
  int E, N, K;
  void *D;
  float *amax_out;
  const int4 *items;
  const int *count;
};

// ---- work list ---------------------------------------------------------------

__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t *__restrict__ offsets, int E,
                                                        int64_t R, int n_tiles, int64_t max_items,
                                                        int4 *__restrict__ items,
                                                        int *__restrict__ count) {
  __shared__ int64_t scan[1024];
  int64_t carry = 0;
  for (int base = 0; base < E; base += 1024) {
    const int e = base + static_cast<int>(threadIdx.x);
    int64_t lo = 0, rows = 0;
    if (e < E) {
      lo = offsets[e];
      lo = lo < 0 ? 0 : (lo > R ? R : lo);
      int64_t hi = offsets[e + 1];
      hi = hi < lo ? lo : (hi > R ? R : hi);
      rows = hi - lo;
    }
    const int64_t chunks = (rows + kChunkRows - 1) / kChunkRows;
    const int64_t mine = chunks * n_tiles;
    scan[threadIdx.x] = mine;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int64_t add = threadIdx.x >= static_cast<unsigned>(o) ? scan[threadIdx.x - o] : 0;
      __syncthreads();
      scan[threadIdx.x] += add;
      __syncthreads();
    }
    const int64_t first = carry + scan[threadIdx.x] - mine;
    for (int64_t nt = 0; nt < n_tiles; nt++) {
      for (int64_t c = 0; c < chunks; c++) {
        const int64_t w = first + nt * chunks + c;
        if (w < max_items) {
          const int64_t r0 = lo + c * kChunkRows;
          const int64_t nr = rows - c * kChunkRows;
          items[w] = make_int4(e, static_cast<int>(r0), static_cast<int>(nr < kChunkRows ? nr : kChunkRows),
                               static_cast<int>(nt));
        }
      }
    }
    carry += scan[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) *count = static_cast<int>(carry < max_items ? carry : max_items);
}

// ---- operand dequantisation ----------------------------------------------------

// 8 E2M1 codes (one dword, element 2i in the low nibble of byte i) times scale s -> 8 fp16.
__device__ __forceinline__ half8 dequant8(uint32_t codes, _Float16 s) {
  const half2v sc = {s, s};
  const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * sc;
  const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * sc;
  const half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * sc;
  const half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * sc;
  return half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// E4M3FN byte `sel` (0..3) of a dword -> fp16 (exact: every E4M3 value is an fp16 value).
// `sel` is a constant once the caller's loops are unrolled.
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t w, int sel) {
  const float f = sel == 0 ? __builtin_amdgcn_cvt_f32_fp8(w, 0)
                : sel == 1 ? __builtin_amdgcn_cvt_f32_fp8(w, 1)
                : sel == 2 ? __builtin_amdgcn_cvt_f32_fp8(w, 2)
                           : __builtin_amdgcn_cvt_f32_fp8(w, 3);
  return static_cast<_Float16>(f);
}

struct Frag {       // one lane's share of a 32-row operand tile for one 256-wide K step
  uint4 q[4];       // 4 x 16 bytes of codes: elements [128h + 32q, +32)
  uint2 s;          // the 8 scale bytes of blocks [8h, 8h + 8) of the step
};

// codes / scales point at the lane's row, already offset by the lane half.
__device__ __forceinline__ void load_frag(Frag &f, const uint8_t *codes, const uint8_t *scales) {
#pragma unroll
  for (int q = 0; q < 4; q++) f.q[q] = *reinterpret_cast<const uint4 *>(codes + 16 * q);
  f.s = *reinterpret_cast<const uint2 *>(scales);
}

__device__ __forceinline__ uint32_t word(const uint4 &v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// ---- the kernel ----------------------------------------------------------------

template <int KS, int EPI>
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(GemmParams P) {
  constexpr int NG = 4 / KS;  // groups of 64 weight rows per workgroup
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int ng = wv % NG;
  const int kq = wv / NG;
  const int r = lane & 31;    // row within a 32-row tile
  const int h = lane >> 5;    // lane half: which 32 of each 64 K elements

  // work item for this workgroup (contiguous ranges per XCD)
  const int b = blockIdx.x;
  const int count = *P.count;
  const int per_xcd = (count + kXcds - 1) / kXcds;
  const int jx = b / kXcds;
  const int w = (b % kXcds) * per_xcd + jx;
  if (jx >= per_xcd || w >= count) {
    if (EPI == MOE_EPI_SWIGLU && threadIdx.x == 0) P.amax_out[b] = 0.f;
    return;
  }
  const int4 item = P.items[w];
  const int e = item.x, row0 = item.y, nrows = item.z, nt = item.w;
  const int I = P.N / 2;

  // weight rows of this wave's two 32-row tiles
  int nrow[2];
  if (EPI == MOE_EPI_SWIGLU) {
    nrow[0] = nt * (NG * 32) + ng * 32;  // gate
    nrow[1] = I + nrow[0];               // matching up rows
  } else {
    nrow[0] = nt * (NG * 64) + ng * 64;
    nrow[1] = nrow[0] + 32;
  }
  const int64_t half_k = P.K / 2, k16 = P.K / 16;
  const uint8_t *bq[2];
  const uint8_t *bs[2];
#pragma unroll
  for (int s = 0; s < 2; s++) {
    const int64_t row = static_cast<int64_t>(e) * P.N + nrow[s] + r;
    bq[s] = P.B + row * half_k + 64 * h;
    bs[s] = P.B_sf + row * k16 + 8 * h;
  }
  // activation rows of the (one or two) 32-row tiles of the chunk
  const int nm = nrows > 32 ? 2 : 1;
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

  float16v acc[2][2];
#pragma unroll
  for (int s = 0; s < 2; s++)
#pragma unroll
    for (int mt = 0; mt < 2; mt++) acc[s][mt] = float16v{};

  const int k_len = P.K / KS;
  const int k_begin = kq * k_len;
  const int iters = k_len / kKStep;

  Frag fb[2], fa[2], nb[2], na[2];
#pragma unroll
  for (int s = 0; s < 2; s++) load_frag(fb[s], bq[s] + k_begin / 2, bs[s] + k_begin / 16);
  load_frag(fa[0], aq[0] + k_begin / 2, as[0] + k_begin / 16);
  if (nm == 2) load_frag(fa[1], aq[1] + k_begin / 2, as[1] + k_begin / 16);

  for (int it = 0; it < iters; it++) {
    const int kn = k_begin + (it + 1) * kKStep;
    const bool more = it + 1 < iters;
    if (more) {  // prefetch the next K step while this one computes
#pragma unroll
      for (int s = 0; s < 2; s++) load_frag(nb[s], bq[s] + kn / 2, bs[s] + kn / 16);
      load_frag(na[0], aq[0] + kn / 2, as[0] + kn / 16);
      if (nm == 2) load_frag(na[1], aq[1] + kn / 2, as[1] + kn / 16);
    }
#pragma unroll
    for (int q = 0; q < 4; q++) {
#pragma unroll
      for (int d = 0; d < 4; d++) {
        // dword d of load q: elements [128h + 32q + 8d, +8), scale block 8h + 2q + d/2,
        // i.e. byte 2(q % 2) + d/2 of scale word q/2
        const int sw = q >> 1, sb = 2 * (q & 1) + (d >> 1);
        half8 bf[2];
#pragma unroll
        for (int s = 0; s < 2; s++)
          bf[s] = dequant8(word(fb[s].q[q], d), e4m3_to_f16(sw ? fb[s].s.y : fb[s].s.x, sb));
        const half8 af0 = dequant8(word(fa[0].q[q], d), e4m3_to_f16(sw ? fa[0].s.y : fa[0].s.x, sb));
#pragma unroll
        for (int s = 0; s < 2; s++)
          acc[s][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[s], af0, acc[s][0], 0, 0, 0);
        if (nm == 2) {
          const half8 af1 = dequant8(word(fa[1].q[q], d), e4m3_to_f16(sw ? fa[1].s.y : fa[1].s.x, sb));
#pragma unroll
          for (int s = 0; s < 2; s++)
            acc[s][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[s], af1, acc[s][1], 0, 0, 0);
        }
      }
    }
    if (more) {
#pragma unroll
      for (int s = 0; s < 2; s++) fb[s] = nb[s];
      fa[0] = na[0];
      if (nm == 2) fa[1] = na[1];
    }
  }

  // K split across waves: partial tiles added in LDS in a fixed order
  if constexpr (KS > 1) {
    __shared__ float red[(KS - 1) * NG * 2 * 2 * 16 * 64];
    float *mine = red + ((kq - 1) * NG + ng) * (2 * 2 * 16 * 64);
    if (kq > 0) {
#pragma unroll
      for (int s = 0; s < 2; s++)
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int i = 0; i < 16; i++) mine[((s * 2 + mt) * 16 + i) * 64 + lane] = acc[s][mt][i];
    }
    __syncthreads();
    if (kq == 0) {
      for (int o = 1; o < KS; o++) {
        const float *src = red + ((o - 1) * NG + ng) * (2 * 2 * 16 * 64);
#pragma unroll
        for (int s = 0; s < 2; s++)
#pragma unroll
          for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int i = 0; i < 16; i++) acc[s][mt][i] += src[((s * 2 + mt) * 16 + i) * 64 + lane];
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
          for (int s = 0; s < 2; s++)
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++) {
              uint32_t lo = f32_to_bf16(acc[s][mt][4 * g4 + 0] * gscale) |
                            (static_cast<uint32_t>(f32_to_bf16(acc[s][mt][4 * g4 + 1] * gscale)) << 16);
              uint32_t hi = f32_to_bf16(acc[s][mt][4 * g4 + 2] * gscale) |
                            (static_cast<uint32_t>(f32_to_bf16(acc[s][mt][4 * g4 + 3] * gscale)) << 16);
              *reinterpret_cast<uint2 *>(drow + nrow[s] + 8 * g4 + 4 * h) = make_uint2(lo, hi);
            }
        } else {
          uint16_t *drow = static_cast<uint16_t *>(P.D) + p * I;
#pragma unroll
          for (int g4 = 0; g4 < 4; g4++) {
            uint16_t o[4];
#pragma unroll
            for (int c = 0; c < 4; c++) {
              const float gate = round_bf16(acc[0][mt][4 * g4 + c] * gscale);
              const float up = round_bf16(acc[1][mt][4 * g4 + c] * gscale);
              const float silu = gate / (1.0f + expf(-gate));
              o[c] = f32_to_bf16(silu * up);
              amax = fmaxf(amax, fabsf(bf16_to_f32(o[c])));
            }
            *reinterpret_cast<uint2 *>(drow + nrow[0] + 8 * g4 + 4 * h) =
                make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16));
          }
        }
      }
    }
  }
  if (EPI == MOE_EPI_SWIGLU) {
    __shared__ float wmax[4];
    amax = wave_max(amax);
    if (lane == 0) wmax[wv] = amax;
    __syncthreads();
    if (threadIdx.x == 0) P.amax_out[b] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  }
}

template <int KS, int EPI>
void launch_ks(const GemmParams &p, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((grouped_gemm_kernel<KS, EPI>), dim3(static_cast<uint32_t>(grid)), dim3(256), 0,
                     stream, p);
}

}  // namespace

GemmPlan plan_gemm(const moe_gemm_args &a) {
  GemmPlan p{};
  const int64_t chunk_bound = (a.R + kChunkRows - 1) / kChunkRows + a.E;
  const int64_t chunk_est = std::max<int64_t>(a.E, (a.R + kChunkRows - 1) / kChunkRows);
  p.ks = 1;
  for (int cand = 1; cand <= 4; cand *= 2) {
    if (a.K % (kKStep * cand) != 0) break;
    p.ks = cand;
    if (chunk_est * (a.N / (256 / cand)) >= 2 * 256) break;  // at least ~2 workgroups per CU
  }
  p.n_tile = 256 / p.ks;
  p.n_tiles = a.N / p.n_tile;
  p.max_items = static_cast<int64_t>(p.n_tiles) * chunk_bound;
  p.grid = (p.max_items + kXcds - 1) / kXcds * kXcds;
  p.ws_bytes = 16 + static_cast<size_t>(p.max_items) * sizeof(int4);
  return p;
}

hipError_t launch_grouped_gemm(const moe_gemm_args &a, const GemmPlan &plan, void *ws,
                               hipStream_t stream) {
  int *count = static_cast<int *>(ws);
  int4 *items = reinterpret_cast<int4 *>(static_cast<char *>(ws) + 16);
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, stream, a.expert_offsets, a.E, a.R,
                     plan.n_tiles, plan.max_items, items, count);
  GemmParams p{a.A, a.A_sf, a.A_gs, a.A_rows, a.rows_A, a.B, a.B_sf, a.B_gs, a.E, a.N, a.K,
               a.D, a.amax_out, items, count};
  const bool swiglu = a.epilogue == MOE_EPI_SWIGLU;
  switch (plan.ks) {
    case 1: swiglu ? launch_ks<1, MOE_EPI_SWIGLU>(p, plan.grid, stream) : launch_ks<1, MOE_EPI_NONE>(p, plan.grid, stream); break;
    case 2: swiglu ? launch_ks<2, MOE_EPI_SWIGLU>(p, plan.grid, stream) : launch_ks<2, MOE_EPI_NONE>(p, plan.grid, stream); break;
    default: swiglu ? launch_ks<4, MOE_EPI_SWIGLU>(p, plan.grid, stream) : launch_ks<4, MOE_EPI_NONE>(p, plan.grid, stream); break;
  }
  return hipGetLastError();
}

}  // namespace moe
