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
constexpr int kChunkRows = 64;    // rows per work item, row-major kernel (two 32-row MFMA tiles)
constexpr int kChunkRows16 = 48;  // rows per work item, packed kernel (three 16-row MFMA tiles)
constexpr int kTok16 = kChunkRows16 / 16;

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
                                                        int64_t R, int chunk_rows, int n_tiles, int64_t max_items,
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
    const int64_t chunks = (rows + chunk_rows - 1) / chunk_rows;
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
          const int64_t r0 = lo + c * chunk_rows;
          const int64_t nr = rows - c * chunk_rows;
          items[w] = make_int4(e, static_cast<int>(r0), static_cast<int>(nr < chunk_rows ? nr : chunk_rows),
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

// E4M3FN bytes (2*hi, 2*hi + 1) of a dword -> two fp16 (exact: every E4M3 value is an fp16
// value; the converter's scale operand is 1.0, a power of two, which it applies exactly).
__device__ __forceinline__ half2v e4m3x2_to_f16(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
            : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
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

// codes / scales point at the lane's data for the step; qs = distance between the four
// 16-byte code pieces (16 in the row-major layout, 1024 in the packed layout).
__device__ __forceinline__ void load_frag(Frag &f, const uint8_t *codes, const uint8_t *scales, int qs) {
#pragma unroll
  for (int q = 0; q < 4; q++) f.q[q] = *reinterpret_cast<const uint4 *>(codes + qs * q);
  f.s = *reinterpret_cast<const uint2 *>(scales);
}

__device__ __forceinline__ uint32_t word(const uint4 &v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// ---- the packed weight layout ---------------------------------------------------
//
// Weights [rows, K] (rows = E * N, rows % 16 == 0, K % 256 == 0) are regrouped into
// blocks of 2304 bytes, one per (16-row tile T, 256-wide K step s), at byte offset
// (T * K/256 + s) * 2304, holding exactly what one wave loads for that tile and step, in
// lane order (lane l = 16g + r, g = 0..3, r = 0..15): two 1 KB pieces q = 0..1 where lane l
// has the 16 code bytes [32g + 16q, +16) of the step for row 16T + r, then 256 bytes where
// lane l has the 4 scale bytes [4g, 4g + 4) of the step for row 16T + r.  Every weight load
// of the packed kernel is one contiguous 1 KB (or 256 B) wave access with the scales in the
// same stream.

constexpr int kPackBlock = 2304;

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t *__restrict__ B,
                                                   const uint8_t *__restrict__ B_sf, int64_t rows,
                                                   int K, uint8_t *__restrict__ out) {
  const int steps = K / kKStep;
  const int64_t nblocks = rows / 16 * steps;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  // per block: 128 code pieces of 16 bytes, then 64 scale pieces of 4 bytes
  const int64_t blk = i / 192;
  const int piece = static_cast<int>(i % 192);
  if (blk >= nblocks) return;
  const int64_t T = blk / steps;
  const int s = static_cast<int>(blk % steps);
  uint8_t *dst = out + blk * kPackBlock;
  if (piece < 128) {
    const int q = piece >> 6, l = piece & 63, r = l & 15, g = l >> 4;
    const uint8_t *src = B + (T * 16 + r) * (K / 2) + s * 128 + 32 * g + 16 * q;
    *reinterpret_cast<uint4 *>(dst + q * 1024 + l * 16) = *reinterpret_cast<const uint4 *>(src);
  } else {
    const int l = piece - 128, r = l & 15, g = l >> 4;
    const uint8_t *src = B_sf + (T * 16 + r) * (K / 16) + s * 16 + 4 * g;
    *reinterpret_cast<uint32_t *>(dst + 2048 + l * 4) = *reinterpret_cast<const uint32_t *>(src);
  }
}

// ---- packed-weight kernel: 16x16x32 fp16 MFMA ---------------------------------------
//
// A wave owns four 16-row weight tiles (64 rows) and all 16-row token tiles of its chunk
// (up to four), so padding is at most 15 token rows.  Per 256-wide K step and 16-row tile
// a lane of group g holds the 64 elements [64g, 64g + 64) of its row: MFMA j = 4q + d (q =
// 0..1, d = 0..3) takes dword d of piece q, elements [64g + 32q + 8d, +8), whose scale is
// byte 2q + d/2 of the lane's scale word.  Token tiles use the same K order.

struct Frag16 {   // one lane's share of a 16-row tile for one 256-wide K step
  uint4 q[2];     // code pieces: elements [64g + 32q, +32)
  uint32_t s;     // scale bytes of blocks [4g, 4g + 4)
};

__device__ __forceinline__ void load_frag16(Frag16 &f, const uint8_t *codes, const uint8_t *scales, int qs) {
  f.q[0] = *reinterpret_cast<const uint4 *>(codes);
  f.q[1] = *reinterpret_cast<const uint4 *>(codes + qs);
  f.s = *reinterpret_cast<const uint32_t *>(scales);
}

// Buffer resources (raw, byte-addressed) with hardware range checking: an access at an
// offset at or past `bytes` returns zeros and reads no memory.  Ranges stay below kOob, so
// kOob plus any in-range offset is out of range without wrapping.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kOob = 0x80000000u;
static_assert(kMaxPackedBufBytes + 4096 <= kOob, "buffer ranges must stay below the out-of-range offset");

__device__ __forceinline__ BufRsrc make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ void load_frag16_buf(Frag16 &f, BufRsrc rc, uint32_t code_off, uint32_t qs, BufRsrc rs,
                                                uint32_t scale_off) {
  const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rc, code_off, 0, 0);
  const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rc, code_off + qs, 0, 0);
  f.q[0] = make_uint4(a.x, a.y, a.z, a.w);
  f.q[1] = make_uint4(b.x, b.y, b.z, b.w);
  f.s = __builtin_amdgcn_raw_buffer_load_b32(rs, scale_off, 0, 0);
}

template <int NM, int KS, int EPI>
__device__ __forceinline__ void ks_body(const GemmParams &P, float *red, float *wmax, int b, int e,
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
    constexpr int TILE = 4 * kTok16 * 4 * 64;
    float *mine = red + ((kq - 1) * NG + ng) * TILE;
    if (kq > 0) {
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int mt = 0; mt < NM; mt++)
#pragma unroll
          for (int i = 0; i < 4; i++) mine[((j * kTok16 + mt) * 4 + i) * 64 + lane] = acc[j][mt][i];
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
            for (int i = 0; i < 4; i++) acc[j][mt][i] += src[((j * kTok16 + mt) * 4 + i) * 64 + lane];
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
              const float gate = round_bf16(acc[jp][mt][c] * gscale);
              const float up = round_bf16(acc[2 + jp][mt][c] * gscale);
              const float silu = gate / (1.0f + expf(-gate));
              o[c] = f32_to_bf16(silu * up);
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
__global__ __launch_bounds__(256, 2) void grouped_gemm16_kernel(GemmParams P) {
  constexpr int TILE = 4 * kTok16 * 4 * 64;
  __shared__ float red[KS > 1 ? (KS - 1) * (4 / KS) * TILE : 1];
  __shared__ float wmax[4];
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
  const int nm = (item.z + 15) / 16;   // workgroup-uniform
  if (nm <= 1) ks_body<1, KS, EPI>(P, red, wmax, b, item.x, item.y, item.z, item.w);
  else if (nm == 2) ks_body<2, KS, EPI>(P, red, wmax, b, item.x, item.y, item.z, item.w);
  else ks_body<3, KS, EPI>(P, red, wmax, b, item.x, item.y, item.z, item.w);
}

// Packed weights, activation tile shared through LDS (K split 1 only).  The four waves
// of a workgroup use the same activation rows, so each K step's activation tile is
// dequantised once per workgroup: wave w < NM turns 16-row token tile w into eight fp16
// MFMA operand fragments per lane in LDS (double-buffered, one barrier per step), and
// every wave reads them back with 16-byte LDS loads.  Weights stream into registers as in
// grouped_gemm16_kernel.  NM (token tiles of the chunk) is a template parameter so that the
// K loop is straight-line code the compiler can schedule (one dispatch per workgroup).
struct LdsShared {
  uint4 a[2][kTok16][8][64];   // [buffer][token tile][MFMA of step][lane]
  float wmax[4];
};

template <int NM, int EPI>
__device__ __forceinline__ void lds_body(const GemmParams &P, LdsShared &sh, int b, int e, int row0,
                                         int nrows, int nt) {
  constexpr int SPAN = 256;       // weight rows per workgroup (4 waves x 64)
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int I = P.N / 2;
  const int steps = P.K / kKStep;

  int nrow[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    if (EPI == MOE_EPI_SWIGLU) {
      const int gate = nt * (SPAN / 2) + wv * 32 + (j & 1) * 16;
      nrow[j] = (j >= 2) ? I + gate : gate;
    } else {
      nrow[j] = nt * SPAN + wv * 64 + j * 16;
    }
  }
  // All operand loads are buffer loads through range-checked descriptors (one over this
  // expert's packed weights, two over the activation codes and scales).  A load past the
  // last K step, or by a wave that produces no activation tile, gets an offset beyond the
  // range: it returns zeros without touching memory.  So every step issues the same loads
  // unconditionally, and the compiler can count the loads still in flight exactly (a load
  // behind a branch makes it wait for all of them).
  const uint32_t expert_bytes = static_cast<uint32_t>(P.N / 16) * steps * kPackBlock;
  const BufRsrc rb = make_rsrc(P.B + static_cast<int64_t>(e) * expert_bytes, expert_bytes);
  uint32_t b_code[4], b_scale[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    b_code[j] = static_cast<uint32_t>(nrow[j] / 16) * steps * kPackBlock + lane * 16;
    b_scale[j] = static_cast<uint32_t>(nrow[j] / 16) * steps * kPackBlock + 2048 + lane * 4;
  }

  const bool a_writer = wv < NM;   // wave-uniform: this wave produces token tile wv
  const uint32_t half_k = P.K / 2, k16 = P.K / 16;
  const BufRsrc ra_codes = make_rsrc(P.A, static_cast<uint32_t>(P.rows_A * half_k));
  const BufRsrc ra_scales = make_rsrc(P.A_sf, static_cast<uint32_t>(P.rows_A * k16));
  uint32_t a_code = 0, a_scale = 0;
  if (a_writer) {
    const int m = wv * 16 + r;
    int64_t p = row0 + (m < nrows ? m : 0);
    int64_t src = P.A_rows ? static_cast<int64_t>(P.A_rows[p]) : p;
    src = src < 0 ? 0 : (src >= P.rows_A ? P.rows_A - 1 : src);
    a_code = static_cast<uint32_t>(src) * half_k + 32 * g;
    a_scale = static_cast<uint32_t>(src) * k16 + 4 * g;
  }
  auto load_a = [&](Frag16 &f, int s) {
    const bool v = a_writer && s < steps;
    load_frag16_buf(f, ra_codes, v ? a_code + s * (kKStep / 2) : kOob, 16, ra_scales,
                    v ? a_scale + s * (kKStep / 16) : kOob);
  };
  auto store_a = [&](const Frag16 &f, int buf) {
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const half2v sc = e4m3x2_to_f16(f.s, q == 1);
#pragma unroll
      for (int d = 0; d < 4; d++) {
        const half8 v = dequant8(word(f.q[q], d), sc[d >> 1]);
        sh.a[buf][wv][4 * q + d][lane] = __builtin_bit_cast(uint4, v);
      }
    }
  };
  auto load_b = [&](Frag16 (&f)[4], int s) {
    const uint32_t so = s < steps ? static_cast<uint32_t>(s) * kPackBlock : kOob;
#pragma unroll
    for (int j = 0; j < 4; j++) load_frag16_buf(f[j], rb, b_code[j] + so, 1024, rb, b_scale[j] + so);
  };

  float4v acc[4][NM];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int mt = 0; mt < NM; mt++) acc[j][mt] = float4v{};

  // Weight fragments rotate through three register sets: the loads of step s + 2 are in
  // flight while step s computes.  Loads are issued in the same order in the prologue as in
  // every step (weights of a step, then its activation tile).
  Frag16 f0[4], f1[4], f2[4], ra, ra0;
  load_b(f0, 0);
  load_a(ra0, 0);
  load_b(f1, 1);
  load_a(ra, 1);
  if (a_writer) store_a(ra0, 0);
  __syncthreads();

  auto step = [&](const Frag16 (&fb)[4], Frag16 (&fl)[4], int s) {
    const int buf = s & 1;
    load_b(fl, s + 2);
#pragma unroll
    for (int q = 0; q < 2; q++) {
      half2v bsc[4];   // scales of blocks 2q, 2q + 1 of each tile
#pragma unroll
      for (int j = 0; j < 4; j++) bsc[j] = e4m3x2_to_f16(fb[j].s, q == 1);
#pragma unroll
      for (int d = 0; d < 4; d++) {
        half8 af[NM];
#pragma unroll
        for (int mt = 0; mt < NM; mt++) af[mt] = __builtin_bit_cast(half8, sh.a[buf][mt][4 * q + d][lane]);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const half8 bf = dequant8(word(fb[j].q[q], d), bsc[j][d >> 1]);
#pragma unroll
          for (int mt = 0; mt < NM; mt++)
            acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf, af[mt], acc[j][mt], 0, 0, 0);
        }
      }
    }
    if (a_writer && s + 1 < steps) store_a(ra, buf ^ 1);   // activation tile of step s + 1
    load_a(ra, s + 2);
    __syncthreads();
  };
  int s = 0;
  for (; s + 3 <= steps; s += 3) {
    step(f0, f2, s);
    step(f1, f0, s + 1);
    step(f2, f1, s + 2);
  }
  if (s < steps) step(f0, f2, s);
  if (s + 1 < steps) step(f1, f0, s + 1);

  const float gscale = (*P.A_gs) * P.B_gs[e];
  float amax = 0.f;
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
            const float gate = round_bf16(acc[jp][mt][c] * gscale);
            const float up = round_bf16(acc[2 + jp][mt][c] * gscale);
            const float silu = gate / (1.0f + expf(-gate));
            o[c] = f32_to_bf16(silu * up);
            amax = fmaxf(amax, fabsf(bf16_to_f32(o[c])));
          }
          *reinterpret_cast<uint2 *>(drow + nrow[jp] + 4 * g) =
              make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16));
        }
      }
    }
  }
  if (EPI == MOE_EPI_SWIGLU) {
    amax = wave_max(amax);
    if (lane == 0) sh.wmax[wv] = amax;
    __syncthreads();
    if (threadIdx.x == 0) P.amax_out[b] = fmaxf(fmaxf(sh.wmax[0], sh.wmax[1]), fmaxf(sh.wmax[2], sh.wmax[3]));
  }
}

template <int EPI>
__global__ __launch_bounds__(256, 2) void grouped_gemm16_lds_kernel(GemmParams P) {
  __shared__ LdsShared sh;
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
  const int nm = (item.z + 15) / 16;   // workgroup-uniform
  if (nm <= 1) lds_body<1, EPI>(P, sh, b, item.x, item.y, item.z, item.w);
  else if (nm == 2) lds_body<2, EPI>(P, sh, b, item.x, item.y, item.z, item.w);
  else lds_body<3, EPI>(P, sh, b, item.x, item.y, item.z, item.w);
}

// ---- the kernel ----------------------------------------------------------------
//
// Row-major weights, 32x32x16 fp16 MFMA.  KS: K split across the waves of a workgroup
// (1, 2, 4); NG = 4 / KS wave groups along N; each wave owns two 32-row weight tiles (with
// the SwiGLU epilogue a (gate, up) pair), so a workgroup covers NG * 64 weight rows.
template <int NM, int KS, int EPI>
__device__ __forceinline__ void rm_body(const GemmParams &P, float *red, float *wmax, int b, int e,
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
                const float gate = round_bf16(acc[2 * jp][mt][4 * g4 + c] * gscale);
                const float up = round_bf16(acc[2 * jp + 1][mt][4 * g4 + c] * gscale);
                const float silu = gate / (1.0f + expf(-gate));
                o[c] = f32_to_bf16(silu * up);
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

template <int KS, int EPI>
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(GemmParams P) {
  constexpr int TILE = 2 * 2 * 16 * 64;
  __shared__ float red[KS > 1 ? (KS - 1) * (4 / KS) * TILE : 1];
  __shared__ float wmax[4];
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
  if (item.z > 32) rm_body<2, KS, EPI>(P, red, wmax, b, item.x, item.y, item.z, item.w);
  else rm_body<1, KS, EPI>(P, red, wmax, b, item.x, item.y, item.z, item.w);
}

template <int EPI>
void launch_epi(const GemmParams &p, const GemmPlan &plan, bool packed, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(plan.grid)), block(256);
  if (packed) {
    if (plan.ks == 1) hipLaunchKernelGGL((grouped_gemm16_lds_kernel<EPI>), grid, block, 0, stream, p);
    else if (plan.ks == 2) hipLaunchKernelGGL((grouped_gemm16_kernel<2, EPI>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((grouped_gemm16_kernel<4, EPI>), grid, block, 0, stream, p);
  } else {
    if (plan.ks == 1) hipLaunchKernelGGL((grouped_gemm_kernel<1, EPI>), grid, block, 0, stream, p);
    else if (plan.ks == 2) hipLaunchKernelGGL((grouped_gemm_kernel<2, EPI>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((grouped_gemm_kernel<4, EPI>), grid, block, 0, stream, p);
  }
}

}  // namespace

GemmPlan plan_gemm(const moe_gemm_args &a) {
  GemmPlan p{};
  const int chunk = a.B_layout == MOE_LAYOUT_PACKED ? kChunkRows16 : kChunkRows;
  p.chunk_rows = chunk;
  const int64_t chunk_bound = (a.R + chunk - 1) / chunk + a.E;
  const int64_t chunk_est = std::max<int64_t>(a.E, (a.R + chunk - 1) / chunk);
  // A workgroup covers 256 weight rows (four waves x 64); for few groups the waves split K
  // (2 or 4 ways) so that there are at least ~2 workgroups per CU.
  p.ks = 1;
  for (int cand = 1; cand <= 4; cand *= 2) {
    if (a.K % (kKStep * cand) != 0) break;
    p.ks = cand;
    if (chunk_est * (a.N / (256 / cand)) >= 2 * 256) break;
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
                     plan.chunk_rows, plan.n_tiles, plan.max_items, items, count);
  GemmParams p{a.A, a.A_sf, a.A_gs, a.A_rows, a.rows_A, a.B, a.B_sf, a.B_gs, a.E, a.N, a.K,
               a.D, a.amax_out, items, count};
  const bool packed = a.B_layout == MOE_LAYOUT_PACKED;
  if (a.epilogue == MOE_EPI_SWIGLU) launch_epi<MOE_EPI_SWIGLU>(p, plan, packed, stream);
  else launch_epi<MOE_EPI_NONE>(p, plan, packed, stream);
  return hipGetLastError();
}

size_t packed_weights_bytes(int64_t rows, int K) { return static_cast<size_t>(rows) * K / 16 * 9; }

hipError_t launch_pack_weights(const uint8_t *B, const uint8_t *B_sf, int64_t rows, int K,
                               uint8_t *packed, hipStream_t stream) {
  const int64_t nblocks = rows / 16 * (K / kKStep);
  const int64_t threads = nblocks * 192;
  if (threads > 0)
    hipLaunchKernelGGL(pack_kernel, dim3(static_cast<uint32_t>((threads + 255) / 256)), dim3(256), 0,
                       stream, B, B_sf, rows, K, packed);
  return hipGetLastError();
}

}  // namespace moe
