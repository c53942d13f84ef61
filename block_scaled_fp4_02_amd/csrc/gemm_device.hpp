// Device-side pieces shared by the grouped NVFP4 GEMM kernels (gemm_*.hip): kernel
// parameters, the work-item mapping, operand fragments and their loads, and the exact
// NVFP4 -> fp16 dequantisation.  Not part of the ABI.
//
// Exactness: an E2M1 element times its E4M3 block scale has at most 6 significant bits and
// lies in [2^-10, 2688], so it is exact in fp16.  Both operands are dequantised that way
// (hardware FP4 -> fp16 conversion, then a packed fp16 multiply by the block scale), so a
// plain fp16 MFMA with fp32 accumulation sums exact products; the two global scales
// multiply the fp32 result in the epilogue.  (gfx950's block-scaled FP4 MFMA takes
// power-of-two scales per 32 elements and cannot carry an E4M3 scale per 16.)
#pragma once

#include "common.hpp"
#include "lds_budget.hpp"
#include "nvfp4_round.hpp"

namespace moe {
namespace gemm {

constexpr int kKStep = 256;       // K elements per step of every kernel
constexpr int kPackBlock = 2304;  // bytes of one (16-row tile, K step) block of packed weights

struct Params {
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
  // Work items (expert, first row, rows, n tile), ordered expert-major, then n tile, then
  // row chunk.  With items == nullptr every wave derives its own from the offsets.
  const int4 *items;   // from the schedule kernel, or nullptr
  const int *count;    // number of valid items (with items)
  const int32_t *offsets;
  int64_t R;
  int chunk_rows, n_tiles;
  uint8_t *D_sf;        // SwiGLU + NVFP4 epilogue: scales of D, and the static global scale
  const float *D_gs;
  int nt_per_item;      // 256-row n tiles per work item (four-wave LDS kernel, one K step)
};

// Largest expert count for which waves derive their work item from the offsets themselves
// (one wave-wide pass, an expert per lane); above it, for short items, repeating the pass in
// thousands of workgroups costs more than one schedule kernel that writes the item list.
constexpr int kMaxInlineScheduleExperts = 64;
// Up to this many experts launches whose items span at least kInlineScheduleMinK of K (long
// items) also look up their items in the kernel, four experts per lane.
constexpr int kMaxInlineScheduleExpertsLongK = 4 * 64;
constexpr int kInlineScheduleMinK = 1024;

// Rows of expert e (offsets clamped to [0, R] and made monotone) and its first row.
__device__ __forceinline__ int expert_rows(const Params &P, int e, int64_t &lo) {
  lo = P.offsets[e];
  lo = lo < 0 ? 0 : (lo > P.R ? P.R : lo);
  int64_t hi = P.offsets[e + 1];
  hi = hi < lo ? lo : (hi > P.R ? P.R : hi);
  return static_cast<int>(hi - lo);
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

// The schedule kernel stores an item's n tile with this bit set when the item is the last
// row chunk of its expert: the launch's final read of that n tile's weights, which the
// packed-weight kernels then load with the non-temporal hint (earlier chunks re-read the
// same weights from L2, so they keep the default policy).
constexpr int kLastChunkFlag = 1 << 30;

// The in-kernel lookup below for up to 4 * 64 experts (launches with long work items, where
// one round trip per workgroup costs less than a schedule launch): lane l covers experts
// 4l .. 4l + 3, whose five offsets it loads together (indices clamped to E: the array has
// E + 1 entries); then the same wave-wide scan and owner lane as for one expert per lane.
__device__ __forceinline__ bool item_for_block_4(const Params &P, int b, int4 &item, bool &last) {
  const int jx = b / kXcds;
  const int lane = threadIdx.x & 63;
  const int cr = P.chunk_rows;
  int32_t o[5];
#pragma unroll
  for (int q = 0; q < 5; q++) o[q] = P.offsets[min(4 * lane + q, P.E)];
  int rows[4], lo[4], chunks[4];
  int mine = 0;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    int64_t l = o[q];
    l = l < 0 ? 0 : (l > P.R ? P.R : l);
    int64_t h = o[q + 1];
    h = h < l ? l : (h > P.R ? P.R : h);
    const bool valid = 4 * lane + q < P.E;
    rows[q] = valid ? static_cast<int>(h - l) : 0;
    lo[q] = static_cast<int>(l);
    chunks[q] = (rows[q] + cr - 1) / cr;
    mine += chunks[q] * P.n_tiles;
  }
  const int incl = wave_inclusive_scan(mine);
  const int count = __builtin_amdgcn_readlane(incl, kWave - 1);
  const int per_xcd = (count + kXcds - 1) / kXcds;
  const int w = (b % kXcds) * per_xcd + jx;
  if (jx >= per_xcd || w >= count) return false;
  const int local = w - (incl - mine);
  const uint64_t owner = __ballot(mine > 0 && local >= 0 && local < mine);
  const int src = __builtin_ctzll(owner);
  int l_src = __builtin_amdgcn_readlane(local, src);
  // which of the owner's four experts (scalar: everything derived from the item stays uniform)
  int e = 4 * src, c_src = 0, rows_src = 0, lo_src = 0;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const int cq = __builtin_amdgcn_readlane(chunks[q], src);
    const int rq = __builtin_amdgcn_readlane(rows[q], src);
    const int lq = __builtin_amdgcn_readlane(lo[q], src);
    const int items_q = cq * P.n_tiles;
    if (c_src == 0) {
      if (l_src < items_q) {
        e = 4 * src + q;
        c_src = cq;
        rows_src = rq;
        lo_src = lq;
      } else {
        l_src -= items_q;
      }
    }
  }
  const int nt = l_src / c_src, c = l_src % c_src;
  const int nr = rows_src - c * cr;
  item = make_int4(e, lo_src + c * cr, nr < cr ? nr : cr, nt);
  last = c == c_src - 1;
  return true;
}

// Work item of workgroup b, or false if it has none; `last` is true for the last row chunk
// of the item's expert.  Workgroup b runs on XCD b % 8, so
// the items are dealt to XCDs in contiguous ranges: neighbouring items (the n tiles and row
// chunks of one expert) share that XCD's L2.  The result is wave-uniform.  Without an item
// list (at most kMaxInlineScheduleExperts = 64 experts) lane e reads the offsets of expert e
// once and the wave derives the count and the item from them in one pass; up to
// kMaxInlineScheduleExpertsLongK experts each lane takes four (item_for_block_4), in kernels
// built with kFourPerLane (the K-split kernel is not: it looks up an item per loop trip, and
// the larger lookup there costs it registers and time).
static_assert(kMaxInlineScheduleExperts <= kWave, "inline scheduling keeps one expert per lane");
static_assert(kMaxInlineScheduleExpertsLongK <= 4 * kWave, "the long-K lookup keeps four experts per lane");
template <bool kFourPerLane = true>
__device__ __forceinline__ bool item_for_block(const Params &P, int b, int4 &item, bool &last) {
  const int jx = b / kXcds;
  if (P.items) {
    const int count = *P.count;
    const int per_xcd = (count + kXcds - 1) / kXcds;
    const int w = (b % kXcds) * per_xcd + jx;
    if (jx >= per_xcd || w >= count) return false;
    item = P.items[w];
    last = (item.w & kLastChunkFlag) != 0;
    item.w &= ~kLastChunkFlag;
    return true;
  }
  const int lane = threadIdx.x & 63;
  const int cr = P.chunk_rows;
  if (kFourPerLane && P.E > kWave) return item_for_block_4(P, b, item, last);
  int64_t lo = 0;
  int rows = 0, chunks = 0;
  if (lane < P.E) {
    rows = expert_rows(P, lane, lo);
    chunks = (rows + cr - 1) / cr;
  }
  const int mine = chunks * P.n_tiles;
  const int incl = wave_inclusive_scan(mine);
  // uniform: keep the count, and everything derived from it, in SGPRs
  const int count = __builtin_amdgcn_readlane(incl, kWave - 1);
  const int per_xcd = (count + kXcds - 1) / kXcds;
  const int w = (b % kXcds) * per_xcd + jx;
  if (jx >= per_xcd || w >= count) return false;
  const int local = w - (incl - mine);   // index of w among expert `lane`'s items
  const uint64_t owner = __ballot(mine > 0 && local >= 0 && local < mine);
  // the owner lane's values, read as scalars so that everything the kernel derives from the
  // item stays in SGPRs (w < count, so exactly one lane owns it)
  const int src = __builtin_ctzll(owner);
  const int c_src = __builtin_amdgcn_readlane(chunks, src);
  const int l_src = __builtin_amdgcn_readlane(local, src);
  const int rows_src = __builtin_amdgcn_readlane(rows, src);
  const int lo_src = __builtin_amdgcn_readlane(static_cast<int>(lo), src);
  const int nt = l_src / c_src, c = l_src % c_src;
  const int nr = rows_src - c * cr;
  item = make_int4(src, lo_src + c * cr, nr < cr ? nr : cr, nt);
  last = c == c_src - 1;
  return true;
}

__device__ __forceinline__ bool item_for_block(const Params &P, int b, int4 &item) {
  bool last;
  return item_for_block(P, b, item, last);
}

// ---- dequantisation ------------------------------------------------------------------

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

__device__ __forceinline__ uint32_t word(const uint4 &v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// ---- operand fragments ------------------------------------------------------------------

// Row-major layout, 32x32x16 MFMA: one lane's share of a 32-row tile for one K step.
struct Frag {
  uint4 q[4];       // 4 x 16 bytes of codes: elements [128h + 32q, +32)
  uint2 s;          // the 8 scale bytes of blocks [8h, 8h + 8) of the step
};

// codes / scales point at the lane's data for the step; qs = distance between the four
// 16-byte code pieces.
__device__ __forceinline__ void load_frag(Frag &f, const uint8_t *codes, const uint8_t *scales, int qs) {
#pragma unroll
  for (int q = 0; q < 4; q++) f.q[q] = *reinterpret_cast<const uint4 *>(codes + qs * q);
  f.s = *reinterpret_cast<const uint2 *>(scales);
}

// 16x16x32 MFMA: one lane's share of a 16-row tile for one K step.  A lane l = 16g + r holds
// row r, elements [64g, 64g + 64) of the step in two 32-element pieces; MFMA j = 4q + d
// (q = 0..1, d = 0..3) takes dword d of piece q, elements [64g + 32q + 8d, +8), whose scale
// is byte 2q + d/2 of the lane's scale word.  Both operands use this K order (the
// contraction is order-free and every element carries its own scale).
struct Frag16 {
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

// Cache-policy operand of a buffer load: 0 (default) or kNonTemporal (the gfx950 "nt" bit:
// the lines are streamed, not kept for reuse).
constexpr int kNonTemporal = 2;

template <int POLICY = 0>
__device__ __forceinline__ void load_frag16_buf(Frag16 &f, BufRsrc rc, uint32_t code_off, uint32_t qs, BufRsrc rs,
                                                uint32_t scale_off) {
  const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rc, code_off, 0, POLICY);
  const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rc, code_off + qs, 0, POLICY);
  f.q[0] = make_uint4(a.x, a.y, a.z, a.w);
  f.q[1] = make_uint4(b.x, b.y, b.z, b.w);
  f.s = __builtin_amdgcn_raw_buffer_load_b32(rs, scale_off, 0, POLICY);
}

// ---- epilogue ---------------------------------------------------------------------------

// SwiGLU of one (gate, up) pair of fp32 results already times the global scales: both are
// rounded to bf16 first, silu(x) = x / (1 + exp(-x)) in binary32 with the hardware exp2 and
// reciprocal (a few ulp of binary32, far below the bf16 rounding of the result; exp(-x)
// overflowing to +inf gives silu = -0), the product is rounded to bf16.
__device__ __forceinline__ uint16_t swiglu_bf16(float gate_acc, float up_acc) {
  const float gate = round_bf16(gate_acc);
  const float up = round_bf16(up_acc);
  const float silu = gate * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(gate * -1.4426950408889634f));
  return f32_to_bf16(silu * up);
}

// SwiGLU + NVFP4 epilogue for one token row and one 16-column block of act in the 16x16
// MFMA D layout, where lane group g holds the block's columns 4g .. 4g + 3 (gate and up
// accumulators of those columns, already summed).  The bf16 SwiGLU values are quantised
// with the static global scale g2 by exactly the steps of the quantiser (binary32, no
// contraction): the four lanes of the row exchange their block maxima, each packs its four
// codes into two bytes, lane group 0 writes the scale byte.  All lanes of the wave execute
// it (the shuffles pair lanes of the same row); `store` only predicates the writes.
__device__ __forceinline__ void swiglu_nvfp4_block(const float4v &gate, const float4v &up, float gscale, float g2,
                                                   bool store, uint8_t *codes, uint8_t *scale, int g) {
#pragma clang fp contract(off)
  float v[4];
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < 4; c++) {
    v[c] = bf16_to_f32(swiglu_bf16(gate[c] * gscale, up[c] * gscale));
    amax = fmaxf(amax, fabsf(v[c]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
  const float six_g = 6.0f * g2;
  const float t = amax > 0.f ? fminf(amax / six_g, 448.0f) : 0.f;   // 0 / 0 counts as 0
  const uint32_t s = e4m3_rne(t);
  const float sg = e4m3_value(s) * g2;
  uint32_t packed = 0u;
  const BlockDivisor d = block_divisor(sg, amax);
  if (d.fast) {
    float u[4];
#pragma unroll
    for (int c = 0; c < 4; c++) u[c] = block_quotient(fabsf(v[c]), d);
    packed = e2m1_pack4(u);
  } else {
#pragma unroll
    for (int c = 0; c < 4; c++)
      packed |= ((s != 0u && fabsf(v[c]) > 0.f) ? e2m1_rne(fminf(fabsf(v[c]) / sg, 6.0f)) : 0u) << (4 * c);
  }
#pragma unroll
  for (int c = 0; c < 4; c++) packed |= (__float_as_uint(v[c]) >> 31) << (4 * c + 3);
  if (store) {
    *reinterpret_cast<uint16_t *>(codes + 2 * g) = static_cast<uint16_t>(packed);
    if (g == 0) *scale = static_cast<uint8_t>(s);
  }
}

// ---- launchers (one per kernel family) -------------------------------------------------

enum Kernel { kLds = 0, kKSplit = 1, kRowMajor = 2, kLdsWide = 3, kLds64 = 4 };

// Token tiles (16 rows) per work item of the packed-weight kernels.
constexpr int kChunkTiles = 3;       // gemm_lds_kernel (4 waves, 256 weight rows)
constexpr int kChunkTiles64 = 4;     // gemm_lds64_kernel (4 waves, 256 weight rows, 2 per CU)
constexpr int kWideChunkTiles = 6;   // gemm_lds_wide_kernel (8 waves, 512 weight rows)

void launch_lds(const Params &p, int epi, dim3 grid, hipStream_t stream);
void launch_lds64(const Params &p, int epi, dim3 grid, hipStream_t stream);
void launch_lds_wide(const Params &p, int epi, dim3 grid, hipStream_t stream);
void launch_ksplit(const Params &p, int epi, int ks, dim3 grid, hipStream_t stream);
int ksplit_chunk_rows();      // rows per work item of the K-split kernel
int ksplit_waves(int ks);     // waves per workgroup of the K-split kernel
void launch_rowmajor(const Params &p, int epi, int ks, dim3 grid, hipStream_t stream);

}  // namespace gemm
}  // namespace moe
