// Grouped NVFP4 GEMM on packed weights with the activation tile shared through LDS -- the
// kernels for per-expert row counts from a few rows (decode) to hundreds (prefill).
//
// A workgroup (four waves) computes one work item: 256 weight rows (each wave owns four
// 16-row tiles, 64 rows) times the item's chunk of up to MAXT 16-row token tiles, over all
// of K, with 16x16x32 fp16 MFMA.
//  * Weights: every weight byte is read once per item, straight into registers, by the one
//    wave that uses it (packed layout: each load is one contiguous 1 KB or 256 B wave
//    access), and dequantised there.  Weight fragments alternate between two register
//    sets: step s + 1 loads while step s computes.
//  * Activations: the token tiles are the same for the four waves, so each K step's tiles
//    are dequantised once per workgroup -- wave w turns tiles w, w + 4, ... into fp16 MFMA
//    operand fragments in LDS (double-buffered, one barrier per step) -- and every wave
//    reads them back with 16-byte LDS loads (lane-ordered, conflict-free).
//  * All operand loads are buffer loads through range-checked descriptors.  A load past the
//    last K step, or for a token tile the chunk does not have, gets an offset beyond the
//    range: it returns zeros without touching memory.  So every step issues the same loads
//    unconditionally, and the compiler can count the loads still in flight exactly (a load
//    behind a branch makes it wait for all of them).
//  * NM (token tiles of the item) is a template parameter, so the K loop is straight-line
//    code.
//  * In the four-wave kernel the expert's last row chunk loads its weights with the
//    non-temporal hint (no later item of the launch reads them again); earlier chunks keep
//    them in L2 for the next chunk.
// Chunks of up to 48 rows (three token tiles), 49,168 bytes of LDS and at most 168 VGPRs, so three
// workgroups share a CU and overlap one another's loads, dequantisation and MFMAs.  A second
// four-wave kernel takes 64-row chunks (four tiles, 65,552 bytes, two workgroups per CU) for
// launches of about two items per CU, where a 48-row chunk's remainder items would put a
// third workgroup on some CUs; an eight-wave kernel shares 96-row chunks at prefill sizes.  Per step
// and wave: 264 VALU (weight dequantisation) for 32*NM MFMAs.  At decode sizes the kernel
// streams weights (HBM-bound); at hundreds of rows per expert it runs the same tile over
// several chunks, whose repeated weight reads are adjacent items on one XCD and hit its L2.
// (A 128-row tile with one workgroup per CU measured slower: one wave per SIMD leaves no
// other wave to issue VALU while the MFMA pipe is busy.)
#include "gemm_device.hpp"

namespace moe {
namespace gemm {
namespace {

// Row of the NONE epilogue's staging area: a wave's 64 bf16 output columns of one token row
// (128 B) plus 16 B of padding, so that the 16 rows a store instruction of the MFMA layout
// touches fall in different LDS banks and every row starts 16-byte aligned.
constexpr int kEpRow = 72;
static_assert(kEpRow == lds::kEpRowHalves, "NONE staging row differs from the LDS budget");

template <int MAXT, int WAVES>
struct LdsShared {
  union {
    uint4 a[2][MAXT][8][64];                  // [buffer][token tile][MFMA of step][lane]
    uint16_t ep[WAVES][MAXT * 16][kEpRow];    // NONE epilogue: [wave][token row][column]
  };
  float wmax[WAVES];
};

template <int NM, int EPI, bool NT, int MAXT, int WAVES>
__device__ __forceinline__ void lds_body(const Params &P, LdsShared<MAXT, WAVES> &sh, int b, int e, int row0, int nrows,
                                         int nt) {
  constexpr int SPAN = 64 * WAVES;                  // weight rows per workgroup
  // Activation tiles are dequantised by the first AW waves only.  In the 8-wave kernel the
  // first wave on each SIMD (the older one, which the SIMD issues from first) otherwise
  // reaches every step's barrier well ahead of its partner (per-wave timestamps: 26-28 % of
  // its K loop spent waiting there, against 1-5 % for the second wave), so it takes the
  // activation work.
  constexpr int AW = WAVES == 8 ? 4 : WAVES;
  constexpr int TPW = (MAXT + AW - 1) / AW;   // token tiles a dequantising wave handles per step
  static_assert(NM <= MAXT, "token tiles exceed the LDS buffer");
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int I = P.N / 2;
  const int steps = P.K / kKStep;

  int nrow[4];   // first weight row of the wave's four tiles (SwiGLU: gate, gate, up, up)
#pragma unroll
  for (int j = 0; j < 4; j++) {
    if (EPI != MOE_EPI_NONE) {
      const int gate = nt * (SPAN / 2) + wv * 32 + (j & 1) * 16;
      nrow[j] = (j >= 2) ? I + gate : gate;
    } else {
      nrow[j] = nt * SPAN + wv * 64 + j * 16;
    }
  }
  const uint32_t expert_bytes = static_cast<uint32_t>(P.N / 16) * steps * kPackBlock;
  const BufRsrc rb = make_rsrc(P.B + static_cast<int64_t>(e) * expert_bytes, expert_bytes);
  uint32_t b_code[4], b_scale[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    b_code[j] = static_cast<uint32_t>(nrow[j] / 16) * steps * kPackBlock + lane * 16;
    b_scale[j] = static_cast<uint32_t>(nrow[j] / 16) * steps * kPackBlock + 2048 + lane * 4;
  }

  // token tiles wv + AW * i this wave dequantises (wave-uniform validity)
  const uint32_t half_k = P.K / 2, k16 = P.K / 16;
  const BufRsrc ra_codes = make_rsrc(P.A, static_cast<uint32_t>(P.rows_A * half_k));
  const BufRsrc ra_scales = make_rsrc(P.A_sf, static_cast<uint32_t>(P.rows_A * k16));
  bool a_tile[TPW];
  uint32_t a_code[TPW], a_scale[TPW];
  // token rows: the row-index loads of all tiles are issued before any is used (each index
  // is a row of the item, so no branch is needed around them)
  int64_t src_row[TPW];
#pragma unroll
  for (int i = 0; i < TPW; i++) {
    const int t = wv + AW * i;
    a_tile[i] = wv < AW && t < NM;
    const int m = t * 16 + r;
    src_row[i] = row0 + (m < nrows ? m : 0);
  }
  if (P.A_rows) {
    int32_t idx[TPW];
#pragma unroll
    for (int i = 0; i < TPW; i++) idx[i] = P.A_rows[src_row[i]];
#pragma unroll
    for (int i = 0; i < TPW; i++) src_row[i] = idx[i];
  }
#pragma unroll
  for (int i = 0; i < TPW; i++) {
    int64_t src = src_row[i];
    src = src < 0 ? 0 : (src >= P.rows_A ? P.rows_A - 1 : src);
    a_code[i] = a_tile[i] ? static_cast<uint32_t>(src) * half_k + 32 * g : 0;
    a_scale[i] = a_tile[i] ? static_cast<uint32_t>(src) * k16 + 4 * g : 0;
  }
  auto load_a = [&](Frag16 (&f)[TPW], int s) {
#pragma unroll
    for (int i = 0; i < TPW; i++) {
      const bool v = a_tile[i] && s < steps;
      load_frag16_buf(f[i], ra_codes, v ? a_code[i] + s * (kKStep / 2) : kOob, 16, ra_scales,
                      v ? a_scale[i] + s * (kKStep / 16) : kOob);
    }
  };
  auto store_a = [&](const Frag16 (&f)[TPW], int buf) {
#pragma unroll
    for (int i = 0; i < TPW; i++) {
      if (!a_tile[i]) continue;
#pragma unroll
      for (int q = 0; q < 2; q++) {
        const half2v sc = e4m3x2_to_f16(f[i].s, q == 1);
#pragma unroll
        for (int d = 0; d < 4; d++) {
          const half8 v = dequant8(word(f[i].q[q], d), sc[d >> 1]);
          sh.a[buf][wv + AW * i][4 * q + d][lane] = __builtin_bit_cast(uint4, v);
        }
      }
    }
  };
  auto load_b = [&](Frag16 (&f)[4], int s) {
    const uint32_t so = s < steps ? static_cast<uint32_t>(s) * kPackBlock : kOob;
#pragma unroll
    for (int j = 0; j < 4; j++)
      load_frag16_buf<NT ? kNonTemporal : 0>(f[j], rb, b_code[j] + so, 1024, rb, b_scale[j] + so);
  };

  float4v acc[4][NM];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int mt = 0; mt < NM; mt++) acc[j][mt] = float4v{};

  // Each step first writes the activation tiles of the next step into the other LDS buffer
  // (every wave finished reading it before the last barrier), loads the tiles of the step
  // after that and the next step's weights, then runs its MFMAs: a writer wave whose weights
  // are still in flight spends the wait on activation work.  The prologue issues the same
  // loads in the same order.
  Frag16 f0[4], f1[4], ra[TPW], ra0[TPW];
  load_a(ra0, 0);
  // keep the first activation tiles' loads ahead of the weight loads, so that their
  // dequantisation below waits for them alone
  __builtin_amdgcn_sched_barrier(0);
  load_a(ra, 1);
  load_b(f0, 0);
  store_a(ra0, 0);
  __syncthreads();
  // global scales, loaded during the first step: left in the epilogue the compiler issues
  // these loads after the last MFMA and waits a full round trip for them; before the first
  // barrier they delay it
  const float gscale = (*P.A_gs) * P.B_gs[e];

  auto step = [&](const Frag16 (&fb)[4], Frag16 (&fl)[4], int s) {
    const int buf = s & 1;
    if (s + 1 < steps) store_a(ra, buf ^ 1);   // activation tiles of step s + 1
    load_a(ra, s + 2);
    load_b(fl, s + 1);
#pragma unroll
    for (int q = 0; q < 2; q++) {
      half2v bsc[4];   // scales of blocks 2q, 2q + 1 of each weight tile
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
    __syncthreads();
  };
  int s = 0;
  for (; s + 2 <= steps; s += 2) {
    step(f0, f1, s);
    step(f1, f0, s + 1);
  }
  if (s < steps) step(f0, f1, s);

  // epilogue: 16x16 D lane layout -- weight row 4g + i, token row r of the tile
  if constexpr (EPI == MOE_EPI_SWIGLU_NVFP4) {
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
    return;
  }
  if constexpr (EPI == MOE_EPI_NONE) {
    // Stage the wave's bf16 tile in LDS in row order, then store whole 128-byte row pieces:
    // in the MFMA layout a lane holds 4 consecutive columns of one row, so each store
    // instruction would write 16 separate 32-byte pieces of 16 rows.  (The last K step ended
    // with a barrier, so the activation buffers that share this space are free.)
    uint16_t(*ep)[kEpRow] = sh.ep[wv];
#pragma unroll
    for (int mt = 0; mt < NM; mt++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const uint32_t lo = f32_to_bf16(acc[j][mt][0] * gscale) |
                            (static_cast<uint32_t>(f32_to_bf16(acc[j][mt][1] * gscale)) << 16);
        const uint32_t hi = f32_to_bf16(acc[j][mt][2] * gscale) |
                            (static_cast<uint32_t>(f32_to_bf16(acc[j][mt][3] * gscale)) << 16);
        *reinterpret_cast<uint2 *>(&ep[mt * 16 + r][j * 16 + 4 * g]) = make_uint2(lo, hi);
      }
    __syncthreads();
    const int c = lane & 7;    // 16-byte piece of the row
    const int col = nrow[0] + 8 * c;   // the wave's 64 columns start at nrow[0]
#pragma unroll
    for (int k = 0; k < 2 * NM; k++) {
      const int m = 8 * k + (lane >> 3);
      const uint4 v = *reinterpret_cast<const uint4 *>(&ep[m][8 * c]);
      if (m < nrows)
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(P.D) + (row0 + m) * static_cast<int64_t>(P.N) + col) = v;
    }
    return;
  }
  // SWIGLU: act columns nrow[jp] + 4g .. + 3 of token row m
  float amax = 0.f;
#pragma unroll
  for (int mt = 0; mt < NM; mt++) {
    const int m = mt * 16 + r;
    if (m < nrows) {
      uint16_t *drow = static_cast<uint16_t *>(P.D) + (row0 + m) * static_cast<int64_t>(I);
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
  if (EPI == MOE_EPI_SWIGLU) {
    amax = wave_max(amax);
    if (lane == 0) sh.wmax[wv] = amax;
    __syncthreads();
    if (threadIdx.x == 0) {
      float m = sh.wmax[0];
      for (int w = 1; w < WAVES; w++) m = fmaxf(m, sh.wmax[w]);
      P.amax_out[b] = m;
    }
  }
}

// One K step (K = 256) and P.nt_per_item consecutive 256-row n tiles per item, NONE epilogue:
// the chunk's activation tiles are dequantised into LDS once and serve every n tile, and each
// n tile's weights load while the previous one computes.  With a single K step the start of
// an item (item lookup, row indices, activation loads and dequantisation, a barrier) costs
// about as much as its MFMAs, so it is paid once per several n tiles.
template <int NM, bool NT>
__device__ __forceinline__ void lds_k1_body(const Params &P, LdsShared<kChunkTiles, 4> &sh, int e, int row0,
                                            int nrows, int nt_item) {
  constexpr int WAVES = 4;
  constexpr int TPW = (kChunkTiles + WAVES - 1) / WAVES;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int ntpi = P.nt_per_item;
  const int col0 = nt_item * ntpi * 256 + wv * 64;   // first weight row of the wave in n tile 0
  const uint32_t expert_bytes = static_cast<uint32_t>(P.N / 16) * kPackBlock;   // one K step
  const BufRsrc rb = make_rsrc(P.B + static_cast<int64_t>(e) * expert_bytes, expert_bytes);

  const uint32_t half_k = P.K / 2, k16 = P.K / 16;
  const BufRsrc ra_codes = make_rsrc(P.A, static_cast<uint32_t>(P.rows_A * half_k));
  const BufRsrc ra_scales = make_rsrc(P.A_sf, static_cast<uint32_t>(P.rows_A * k16));
  Frag16 ra[TPW];
  bool a_tile[TPW];
#pragma unroll
  for (int i = 0; i < TPW; i++) {
    const int t = wv + WAVES * i;
    a_tile[i] = t < NM;
    uint32_t code = kOob, scale = kOob;
    if (a_tile[i]) {
      const int m = t * 16 + r;
      int64_t p = row0 + (m < nrows ? m : 0);
      int64_t src = P.A_rows ? static_cast<int64_t>(P.A_rows[p]) : p;
      src = src < 0 ? 0 : (src >= P.rows_A ? P.rows_A - 1 : src);
      code = static_cast<uint32_t>(src) * half_k + 32 * g;
      scale = static_cast<uint32_t>(src) * k16 + 4 * g;
    }
    load_frag16_buf(ra[i], ra_codes, code, 16, ra_scales, scale);
  }
  // weights of n tile t (past the item's last n tile: out of range, zeros)
  auto load_b = [&](Frag16 (&f)[4], int t) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint32_t blk = t < ntpi ? static_cast<uint32_t>((col0 + t * 256 + j * 16) / 16) * kPackBlock : kOob;
      load_frag16_buf<NT ? kNonTemporal : 0>(f[j], rb, blk + lane * 16, 1024, rb, blk + 2048 + lane * 4);
    }
  };
  Frag16 f0[4], f1[4];
  load_b(f0, 0);
#pragma unroll
  for (int i = 0; i < TPW; i++) {
    if (!a_tile[i]) continue;
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const half2v sc = e4m3x2_to_f16(ra[i].s, q == 1);
#pragma unroll
      for (int d = 0; d < 4; d++)
        sh.a[0][wv + WAVES * i][4 * q + d][lane] = __builtin_bit_cast(uint4, dequant8(word(ra[i].q[q], d), sc[d >> 1]));
    }
  }
  __syncthreads();
  const float gscale = (*P.A_gs) * P.B_gs[e];

  auto compute_store = [&](const Frag16 (&fb)[4], int t) {
    // the activation fragments read below are the same for every n tile: without this
    // compiler-only memory clobber their 8 * NM LDS reads are hoisted out of the loop and
    // held in registers (spills at 168 VGPRs); it emits no instruction
    asm volatile("" ::: "memory");
    float4v acc[4][NM];
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int mt = 0; mt < NM; mt++) acc[j][mt] = float4v{};
#pragma unroll
    for (int q = 0; q < 2; q++) {
      half2v bsc[4];
#pragma unroll
      for (int j = 0; j < 4; j++) bsc[j] = e4m3x2_to_f16(fb[j].s, q == 1);
#pragma unroll
      for (int d = 0; d < 4; d++) {
        half8 af[NM];
#pragma unroll
        for (int mt = 0; mt < NM; mt++) af[mt] = __builtin_bit_cast(half8, sh.a[0][mt][4 * q + d][lane]);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const half8 bf = dequant8(word(fb[j].q[q], d), bsc[j][d >> 1]);
#pragma unroll
          for (int mt = 0; mt < NM; mt++)
            acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf, af[mt], acc[j][mt], 0, 0, 0);
        }
      }
    }
    // 16x16 D lane layout: weight row 4g + i of tile j, token row r of tile mt.  A lane holds
    // 4 consecutive columns of one row, so storing from registers writes 16 separate 32-byte
    // pieces per instruction.  Instead each wave stages its 64 bf16 columns of every row in
    // the second activation buffer (unused with one K step): 128 B per row, its eight 16-byte
    // pieces XOR-swizzled by the row so that the 8-byte writes of the MFMA layout spread over
    // the banks; then each lane stores one 16-byte piece and 8 lanes write a whole 128-byte
    // row piece.  The area is private to the wave: 4 waves x 48 rows x 128 B = the buffer.
    uint4 *stage = &sh.a[1][0][0][0] + wv * (kChunkTiles * 16 * 8);
#pragma unroll
    for (int mt = 0; mt < NM; mt++) {
      const int m = mt * 16 + r;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const uint32_t lo = f32_to_bf16(acc[j][mt][0] * gscale) |
                            (static_cast<uint32_t>(f32_to_bf16(acc[j][mt][1] * gscale)) << 16);
        const uint32_t hi = f32_to_bf16(acc[j][mt][2] * gscale) |
                            (static_cast<uint32_t>(f32_to_bf16(acc[j][mt][3] * gscale)) << 16);
        const int piece = (2 * j + (g >> 1)) ^ (m & 7);   // columns 16j + 4g .. + 3
        reinterpret_cast<uint2 *>(stage + m * 8 + piece)[g & 1] = make_uint2(lo, hi);
      }
    }
    __syncthreads();
    // lane: row 8k + (lane >> 3) of round k, piece c = lane & 7; the row's swizzle
    // (lane >> 3) ^ c is the same in every round
    const int rl = lane >> 3, c = lane & 7;
    const uint4 *src = stage + rl * 8 + (c ^ rl);
    uint16_t *dst = static_cast<uint16_t *>(P.D) + (row0 + rl) * static_cast<int64_t>(P.N) + col0 + t * 256 + 8 * c;
    const int64_t dst_step = 8 * static_cast<int64_t>(P.N);
#pragma unroll
    for (int k = 0; k < 2 * NM; k++) {
      const uint4 v = src[64 * k];
      if (8 * k + rl < nrows) *reinterpret_cast<uint4 *>(dst + k * dst_step) = v;
    }
  };
#pragma unroll 1
  for (int t = 0; t < ntpi; t += 2) {
    load_b(f1, t + 1);
    compute_store(f0, t);
    load_b(f0, t + 2);
    if (t + 1 < ntpi) compute_store(f1, t + 1);
  }
}

// LDS budget (lds_budget.hpp): the shared struct is exactly the budget entry, and the
// workgroups the launch bounds promise per CU fit in its 160 KB.
constexpr int kLdsWgPerCu = 3;
constexpr int kLds64WgPerCu = 2;
constexpr int kWideWgPerCu = 1;
static_assert(sizeof(LdsShared<kChunkTiles, 4>) == lds::lds_kernel_bytes(kChunkTiles, 4),
              "LDS of the four-wave kernel differs from its budget entry");
static_assert(lds::fits_cu(sizeof(LdsShared<kChunkTiles, 4>), kLdsWgPerCu), "four-wave tile exceeds the CU's LDS");
static_assert(sizeof(LdsShared<kChunkTiles64, 4>) == lds::lds_kernel_bytes(kChunkTiles64, 4),
              "LDS of the 64-row four-wave kernel differs from its budget entry");
static_assert(lds::fits_cu(sizeof(LdsShared<kChunkTiles64, 4>), kLds64WgPerCu),
              "64-row four-wave tile exceeds the CU's LDS");
static_assert(sizeof(LdsShared<kWideChunkTiles, 8>) == lds::lds_kernel_bytes(kWideChunkTiles, 8),
              "LDS of the eight-wave kernel differs from its budget entry");
static_assert(lds::fits_cu(sizeof(LdsShared<kWideChunkTiles, 8>), kWideWgPerCu), "eight-wave tile exceeds the CU's LDS");

template <int EPI>
__global__ __launch_bounds__(256, kLdsWgPerCu) void gemm_lds_kernel(Params P) {
  __shared__ LdsShared<kChunkTiles, 4> sh;
  const int b = blockIdx.x;
  int4 item;
  bool last;
  if (!item_for_block(P, b, item, last)) {
    if (EPI == MOE_EPI_SWIGLU && threadIdx.x == 0) P.amax_out[b] = 0.f;
    return;
  }
  const int nm = (item.z + 15) / 16;   // workgroup-uniform
  if constexpr (EPI == MOE_EPI_NONE) {
    if (P.nt_per_item > 1) {   // one K step, several n tiles per item
      if (last) {
        if (nm <= 1) lds_k1_body<1, true>(P, sh, item.x, item.y, item.z, item.w);
        else if (nm == 2) lds_k1_body<2, true>(P, sh, item.x, item.y, item.z, item.w);
        else lds_k1_body<3, true>(P, sh, item.x, item.y, item.z, item.w);
      } else {
        if (nm <= 1) lds_k1_body<1, false>(P, sh, item.x, item.y, item.z, item.w);
        else if (nm == 2) lds_k1_body<2, false>(P, sh, item.x, item.y, item.z, item.w);
        else lds_k1_body<3, false>(P, sh, item.x, item.y, item.z, item.w);
      }
      return;
    }
  }
  if (last) {   // the expert's last chunk: no later item re-reads these weights
    if (nm <= 1) lds_body<1, EPI, true>(P, sh, b, item.x, item.y, item.z, item.w);
    else if (nm == 2) lds_body<2, EPI, true>(P, sh, b, item.x, item.y, item.z, item.w);
    else lds_body<3, EPI, true>(P, sh, b, item.x, item.y, item.z, item.w);
  } else {
    if (nm <= 1) lds_body<1, EPI, false>(P, sh, b, item.x, item.y, item.z, item.w);
    else if (nm == 2) lds_body<2, EPI, false>(P, sh, b, item.x, item.y, item.z, item.w);
    else lds_body<3, EPI, false>(P, sh, b, item.x, item.y, item.z, item.w);
  }
}

// About two work items per CU of tens of rows each (one 256-row n tile of each expert's
// gate/up or down projection, e.g. 256 experts x 2 n tiles or 32 experts x 16): 64-row
// chunks, so that every expert of up to 64 rows is a single item, and two workgroups per CU.
// With 48-row chunks the few experts above 48 rows added a third item on some CUs, and
// those CUs set the launch's duration.
template <int EPI>
__global__ __launch_bounds__(256, kLds64WgPerCu) void gemm_lds64_kernel(Params P) {
  __shared__ LdsShared<kChunkTiles64, 4> sh;
  const int b = blockIdx.x;
  int4 item;
  bool last;
  if (!item_for_block(P, b, item, last)) {
    if (EPI == MOE_EPI_SWIGLU && threadIdx.x == 0) P.amax_out[b] = 0.f;
    return;
  }
  const int nm = (item.z + 15) / 16;   // workgroup-uniform
  if (last) {
    if (nm <= 1) lds_body<1, EPI, true>(P, sh, b, item.x, item.y, item.z, item.w);
    else if (nm == 2) lds_body<2, EPI, true>(P, sh, b, item.x, item.y, item.z, item.w);
    else if (nm == 3) lds_body<3, EPI, true>(P, sh, b, item.x, item.y, item.z, item.w);
    else lds_body<4, EPI, true>(P, sh, b, item.x, item.y, item.z, item.w);
  } else {
    if (nm <= 1) lds_body<1, EPI, false>(P, sh, b, item.x, item.y, item.z, item.w);
    else if (nm == 2) lds_body<2, EPI, false>(P, sh, b, item.x, item.y, item.z, item.w);
    else if (nm == 3) lds_body<3, EPI, false>(P, sh, b, item.x, item.y, item.z, item.w);
    else lds_body<4, EPI, false>(P, sh, b, item.x, item.y, item.z, item.w);
  }
}

// Hundreds of rows per expert: eight waves share one activation tile of up to six token
// tiles (96 rows), so each dequantised weight element serves twice as many tokens as in
// gemm_lds_kernel, while two waves per SIMD (one workgroup of 512 threads per CU, 110,624
// bytes of LDS: the 96 KB activation buffers share a union with the 108 KB NONE staging
// area) keep VALU and MFMA issuing side by side.  Token tiles rounded up to an even count.
template <int EPI>
__global__ __launch_bounds__(512, kWideWgPerCu) void gemm_lds_wide_kernel(Params P) {
  __shared__ LdsShared<kWideChunkTiles, 8> sh;
  const int b = blockIdx.x;
  int4 item;
  if (!item_for_block(P, b, item)) {
    if (EPI == MOE_EPI_SWIGLU && threadIdx.x == 0) P.amax_out[b] = 0.f;
    return;
  }
  // default cache policy throughout: an expert's ~6 chunks run side by side on one XCD, and
  // non-temporal loads in its last chunk evicted lines its siblings were still reading
  // (prefill GEMMs +3 %)
  const int nm = (item.z + 15) / 16;   // workgroup-uniform
  if (nm <= 2) lds_body<2, EPI, false>(P, sh, b, item.x, item.y, item.z, item.w);
  else if (nm <= 4) lds_body<4, EPI, false>(P, sh, b, item.x, item.y, item.z, item.w);
  else lds_body<6, EPI, false>(P, sh, b, item.x, item.y, item.z, item.w);
}

}  // namespace

void launch_lds(const Params &p, int epi, dim3 grid, hipStream_t stream) {
  const dim3 block(256);
  if (epi == MOE_EPI_SWIGLU) hipLaunchKernelGGL(gemm_lds_kernel<MOE_EPI_SWIGLU>, grid, block, 0, stream, p);
  else if (epi == MOE_EPI_SWIGLU_NVFP4)
    hipLaunchKernelGGL(gemm_lds_kernel<MOE_EPI_SWIGLU_NVFP4>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(gemm_lds_kernel<MOE_EPI_NONE>, grid, block, 0, stream, p);
}

void launch_lds64(const Params &p, int epi, dim3 grid, hipStream_t stream) {
  const dim3 block(256);
  if (epi == MOE_EPI_SWIGLU) hipLaunchKernelGGL(gemm_lds64_kernel<MOE_EPI_SWIGLU>, grid, block, 0, stream, p);
  else if (epi == MOE_EPI_SWIGLU_NVFP4)
    hipLaunchKernelGGL(gemm_lds64_kernel<MOE_EPI_SWIGLU_NVFP4>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(gemm_lds64_kernel<MOE_EPI_NONE>, grid, block, 0, stream, p);
}

void launch_lds_wide(const Params &p, int epi, dim3 grid, hipStream_t stream) {
  const dim3 block(512);
  if (epi == MOE_EPI_SWIGLU) hipLaunchKernelGGL(gemm_lds_wide_kernel<MOE_EPI_SWIGLU>, grid, block, 0, stream, p);
  else if (epi == MOE_EPI_SWIGLU_NVFP4)
    hipLaunchKernelGGL(gemm_lds_wide_kernel<MOE_EPI_SWIGLU_NVFP4>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(gemm_lds_wide_kernel<MOE_EPI_NONE>, grid, block, 0, stream, p);
}

}  // namespace gemm
}  // namespace moe
