// Grouped NVFP4 GEMM: work list, weight packing, per-shape plan and dispatch.
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
// Design (not the pages' SM120 tiles; this is for gfx950):
//  * Work list: items (expert, row chunk, n tile), ordered expert-major, then n tile, then
//    chunk; the last chunk of an expert is flagged (its weight loads are non-temporal).
//    Up to 64 experts (256 when K >= 1024, where items are long enough to absorb the
//    lookup, except in the K-split kernel) every wave derives its own item from
//    expert_offsets (a wave-wide sum and scan, no extra launch); above that a schedule
//    kernel writes the list first (each of its workgroups scans the offsets and writes a
//    slice of the items).  The grid is the host-side upper bound on the item count; items
//    past the device-side count exit.
//  * Per-shape plan (the counterpart of the pages' tile table, chosen from host-known sizes
//    only, so a supported launch cannot fail on its configuration):
//      packed weights, >= 96 rows per expert       -> wide LDS kernel, 96-row chunks, 512-row n tiles
//      packed weights, one item per (expert, n tile)
//        filling two workgroups per CU, <= 40 rows
//        per expert on average                     -> LDS kernel, 64-row chunks, 2 per CU
//      packed weights, enough items for the chip   -> LDS kernel, 48-row chunks
//      packed weights, few items (e.g. 8 groups)   -> K split 2/4/8 ways across a
//                                                     workgroup's waves, 32-row chunks
//      row-major weights                           -> 32x32 MFMA kernel, 64-row chunks
//    Kernel details are in gemm_lds.hip, gemm_ksplit.hip and gemm_rowmajor.hip.
#include "gemm_device.hpp"

#include <algorithm>

namespace moe {
namespace gemm {
namespace {

// ---- work list ---------------------------------------------------------------

// A grid of workgroups: each computes, per block of 1024 experts, the chunk counts and an
// inclusive scan of the item counts (wave scans plus a scan of the 16 wave totals), then
// writes its slice of the block's items, finding each item's expert by binary search over
// the scan.  Item counts stay below 2^31 (the grid bound is checked on the host).
__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t *__restrict__ offsets, int E,
                                                        int64_t R, int chunk_rows, int n_tiles, int64_t max_items,
                                                        int4 *__restrict__ items,
                                                        int *__restrict__ count) {
  __shared__ int incl[1024];     // inclusive scan of the block's per-expert item counts
  __shared__ int first_row[1024];
  __shared__ int n_rows[1024];
  __shared__ int n_chunks[1024];
  __shared__ int wave_total[16];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int G = static_cast<int>(gridDim.x), gi = static_cast<int>(blockIdx.x);
  int carry = 0;
  for (int base = 0; base < E; base += 1024) {
    const int e = base + t;
    int lo = 0, rows = 0;
    if (e < E) {
      int64_t l = offsets[e];
      l = l < 0 ? 0 : (l > R ? R : l);
      int64_t h = offsets[e + 1];
      h = h < l ? l : (h > R ? R : h);
      lo = static_cast<int>(l);
      rows = static_cast<int>(h - l);
    }
    const int chunks = (rows + chunk_rows - 1) / chunk_rows;
    int v = chunks * n_tiles;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(v, o, kWave);
      if (lane >= o) v += u;
    }
    if (lane == 63) wave_total[wv] = v;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wv; w++) before += wave_total[w];
    incl[t] = before + v;
    first_row[t] = lo;
    n_rows[t] = rows;
    n_chunks[t] = chunks;
    __syncthreads();
    const int block_items = incl[1023];
    const int per = (block_items + G - 1) / G;   // this workgroup's slice of the block
    const int w_end = block_items < (gi + 1) * per ? block_items : (gi + 1) * per;
    for (int w = gi * per + t; w < w_end && carry + w < max_items; w += 1024) {
      int a = 0, b = 1023;   // first expert slot with incl > w
      while (a < b) {
        const int m = (a + b) >> 1;
        if (incl[m] > w) b = m;
        else a = m + 1;
      }
      const int ch = n_chunks[a];
      const int local = w - (incl[a] - ch * n_tiles);
      const int nt = local / ch, c = local - nt * ch;
      const int nr = n_rows[a] - c * chunk_rows;
      items[carry + w] = make_int4(base + a, first_row[a] + c * chunk_rows, nr < chunk_rows ? nr : chunk_rows,
                                   nt | (c == ch - 1 ? kLastChunkFlag : 0));
    }
    carry += block_items;
    __syncthreads();
  }
  if (gi == 0 && t == 0) *count = static_cast<int>(carry < max_items ? carry : max_items);
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

}  // namespace
}  // namespace gemm

using namespace gemm;

// Work items and waves for `chunk` rows per item: every expert has at least one chunk in
// the estimate, an empty one none (the grid bound counts one extra chunk per expert).
static int64_t chunk_estimate(const moe_gemm_args &a, int chunk) {
  return std::max<int64_t>(a.E, (a.R + chunk - 1) / chunk);
}

GemmPlan plan_gemm(const moe_gemm_args &a) {
  GemmPlan p{};
  constexpr int64_t kFullChip = 2 * 4 * 256;   // two waves on every SIMD of the 256 CUs
  if (a.B_layout == MOE_LAYOUT_PACKED) {
    p.kernel = kLds;
    p.chunk_rows = kChunkTiles * 16;
    p.ks = 1;
    p.n_tile = 256;
    if (a.R / a.E >= 96 && a.N % 512 == 0) {
      // hundreds of rows per expert: the wide kernel (96-row chunks, 512 weight rows)
      p.kernel = kLdsWide;
      p.chunk_rows = kWideChunkTiles * 16;
      p.n_tile = 512;
    } else if (a.K > kKStep && static_cast<int64_t>(a.E) * (a.N / 256) > 256 &&
               static_cast<int64_t>(a.E) * (a.N / 256) <= 2 * 256 && a.R <= static_cast<int64_t>(a.E) * 40) {
      // tens of rows per expert and one item per (expert, n tile) fills two workgroups per
      // CU: 64-row chunks keep an expert of up to 64 rows in one item (two per CU)
      p.kernel = kLds64;
      p.chunk_rows = kChunkTiles64 * 16;
    } else if (a.K == kKStep && a.epilogue == MOE_EPI_NONE) {
      // one K step per item: several 256-row n tiles per item reuse the activation tile the
      // workgroup dequantised into LDS (the item's start-up -- lookup, row indices, activation
      // loads, barrier -- otherwise dominates); keep about three items per workgroup slot
      for (const int m : {4, 3, 2}) {
        if ((a.N / 256) % m == 0 && chunk_estimate(a, p.chunk_rows) * (a.N / 256 / m) >= 3 * 768) {
          p.n_tile = 256 * m;
          break;
        }
      }
    } else if (chunk_estimate(a, p.chunk_rows) * (a.N / 256) * 4 < kFullChip) {
      // few items: split K across the waves of a workgroup (2, 4 or 8 ways)
      const int chunk = ksplit_chunk_rows();
      for (int cand = 2; cand <= 8; cand *= 2) {
        if (a.K % (kKStep * cand) != 0) break;
        p.kernel = kKSplit;
        p.chunk_rows = chunk;
        p.ks = cand;
        p.n_tile = 64 * (ksplit_waves(cand) / cand);
        if (chunk_estimate(a, chunk) * (a.N / p.n_tile) * ksplit_waves(cand) >= kFullChip) break;
      }
    }
  } else {
    // row-major weights: four waves of two 32-row tiles, K split 1, 2 or 4 ways
    p.kernel = kRowMajor;
    p.chunk_rows = 64;
    p.ks = 1;
    for (int cand = 1; cand <= 4; cand *= 2) {
      if (a.K % (kKStep * cand) != 0) break;
      p.ks = cand;
      if (chunk_estimate(a, p.chunk_rows) * (a.N / (256 / cand)) >= 2 * 256) break;
    }
    p.n_tile = 256 / p.ks;
  }
  p.n_tiles = a.N / p.n_tile;
  const int64_t chunk_bound = (a.R + p.chunk_rows - 1) / p.chunk_rows + a.E;
  p.max_items = static_cast<int64_t>(p.n_tiles) * chunk_bound;
  p.grid = (p.max_items + kXcds - 1) / kXcds * kXcds;
  if (p.kernel == kKSplit) {
    // the K-split kernel loops over its items: launch no more workgroups than fit on the
    // chip at once (256 CUs; one 8-wave or two 4-wave workgroups per CU), so that no empty
    // workgroup waits for a CU at the end (a multiple of the 8 XCDs)
    const int64_t resident = static_cast<int64_t>(256) * (8 / ksplit_waves(p.ks));
    p.grid = std::min<int64_t>(p.grid, resident);
  }
  p.inline_schedule = a.E <= kMaxInlineScheduleExperts ||
                      (a.E <= kMaxInlineScheduleExpertsLongK && a.K >= kInlineScheduleMinK && p.kernel != kKSplit);
  p.ws_bytes = p.inline_schedule ? 16 : 16 + static_cast<size_t>(p.max_items) * sizeof(int4);
  return p;
}

hipError_t launch_grouped_gemm(const moe_gemm_args &a, const GemmPlan &plan, void *ws,
                               hipStream_t stream) {
  int *count = static_cast<int *>(ws);
  int4 *items = nullptr;
  if (!plan.inline_schedule) {
    items = reinterpret_cast<int4 *>(static_cast<char *>(ws) + 16);
    // about 2048 items per workgroup (each repeats the cheap scan), at most 128 workgroups
    const int64_t g = std::min<int64_t>(128, std::max<int64_t>(1, (plan.max_items + 2047) / 2048));
    hipLaunchKernelGGL(schedule_kernel, dim3(static_cast<uint32_t>(g)), dim3(1024), 0, stream, a.expert_offsets,
                       a.E, a.R, plan.chunk_rows, plan.n_tiles, plan.max_items, items, count);
  }
  const Params p{a.A, a.A_sf, a.A_gs, a.A_rows, a.rows_A, a.B, a.B_sf, a.B_gs, a.E, a.N, a.K,
                 a.D, a.amax_out, items, count, a.expert_offsets, a.R, plan.chunk_rows, plan.n_tiles,
                 a.D_sf, a.D_gs, plan.kernel == kLds ? plan.n_tile / 256 : 1};
  const dim3 grid(static_cast<uint32_t>(plan.grid));
  switch (plan.kernel) {
    case kLds: launch_lds(p, a.epilogue, grid, stream); break;
    case kLdsWide: launch_lds_wide(p, a.epilogue, grid, stream); break;
    case kLds64: launch_lds64(p, a.epilogue, grid, stream); break;
    case kKSplit: launch_ksplit(p, a.epilogue, plan.ks, grid, stream); break;
    default: launch_rowmajor(p, a.epilogue, plan.ks, grid, stream); break;
  }
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
