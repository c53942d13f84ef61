// Top-k routing and the stable permutation of (token, slot) pairs into per-expert groups.
//
// The pages give 256 experts with 8 active per token and one small GEMM per expert
// driven by a per-expert problem-size array ("Tracing the Failure: Debugging CUTLASS
// FP4 Tile Configurations on Blackwell SM120", sections "The Broader Context" and
// "Input Knowledge Required").  Routing is the renormalised top-k softmax; the group
// sizes stay on the device as an exclusive prefix sum.
//
// Kernels (all integer work is exact, so the outputs are bit-identical run to run):
//   topk_kernel        one wavefront per token: k rounds of a wave arg-max over the
//                      token's logits (ties -> lower id; 64-bit keys reduced with DPP lane
//                      moves), then the softmax of the k winners in slot order.  Sized by
//                      the expert count (1..16 logits per lane).
//   chunk_count_kernel one workgroup per chunk of 256 tokens: a 256-bit token bitmap
//                      per expert in LDS (order-free OR), popcounts -> counts[chunk][e].
//   scatter_kernel     one workgroup per chunk: from the chunk counts, the start of each
//                      expert's rows in this chunk (column prefix over earlier chunks plus
//                      an exclusive scan over experts; chunk 0 also writes expert_offsets);
//                      then rebuild the bitmaps; the rank of token t
//                      in expert e's group within the chunk is the popcount of the bits
//                      below t, which is the stable order t*k + j because a token names
//                      each expert at most once.
//   count_scatter_kernel  up to kFusedMaxTokens tokens: the scatter without the count
//                      launch -- each workgroup histograms all T*k ids in LDS (all rows, and
//                      the rows of earlier chunks) and takes its bases from that.
#include "common.hpp"


namespace moe {
namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxPerLane = kMaxE / kWave;  // logits held per lane
constexpr int kChunk = 256;                 // tokens per permutation chunk
constexpr int kWords = kChunk / 64;         // 64-bit bitmap words per expert

// A candidate (logit v, expert id) as one 64-bit key whose unsigned order is the selection
// order: larger logit first, then lower id.  High word: the float's bits made monotone
// (negative values inverted, positive ones with the sign bit set); low word: ~id.  Key 0
// marks "no candidate" (every real key has a high word >= 0x007fffff).
__device__ __forceinline__ uint64_t cand_key(float v, int id) {
  const uint32_t b = __float_as_uint(v + 0.0f);   // -0 -> +0: equal logits must tie on the id
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(id));
}

__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t ord = static_cast<uint32_t>(key >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}

__device__ __forceinline__ int key_id(uint64_t key) { return static_cast<int>(~static_cast<uint32_t>(key)); }

// One DPP step of a wave max over 64-bit keys: take the partner lane's key (selected by
// the DPP control; rows outside row_mask keep their own) if it is larger.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t k) {
  const int lo = static_cast<int>(static_cast<uint32_t>(k));
  const int hi = static_cast<int>(k >> 32);
  const uint32_t plo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xf, false));
  const uint32_t phi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xf, false));
  const uint64_t p = (static_cast<uint64_t>(phi) << 32) | plo;
  return p > k ? p : k;
}

// Maximum key over the wave, read from lane 63 (wave-uniform): pairs within quads, then
// the two halves of each 8-lane group, the two halves of each 16-lane row, then the rows
// through the row broadcasts of lanes 15 and 31.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  k = dpp_max_step<0xb1, 0xf>(k);    // quad_perm [1, 0, 3, 2]
  k = dpp_max_step<0x4e, 0xf>(k);    // quad_perm [2, 3, 0, 1]
  k = dpp_max_step<0x141, 0xf>(k);   // row_half_mirror
  k = dpp_max_step<0x140, 0xf>(k);   // row_mirror
  k = dpp_max_step<0x142, 0xa>(k);   // row_bcast15 into rows 1 and 3
  k = dpp_max_step<0x143, 0xc>(k);   // row_bcast31 into rows 2 and 3
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(k)), 63));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(k >> 32), 63));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// PER = logits per lane (E <= 64 PER).  All of a lane's logit loads are issued before any is
// used (an out-of-range lane reads the token's last logit and discards it), so they share one
// memory latency instead of waiting in turn behind a branch each.
template <int PER>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T, int E,
                                                   int k, int32_t *__restrict__ topk_ids,
                                                   float *__restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float *L = logits + static_cast<int64_t>(t) * E;
  float lv[PER];
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int e = lane + kWave * i;
    lv[i] = L[e < E ? e : E - 1];
  }
  uint64_t key[PER];   // this lane's candidates: experts lane + 64 i (0: none / taken)
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int e = lane + kWave * i;
    key[i] = e < E ? cand_key(lv[i], e) : 0ull;
  }
  float my_v = 0.f;
  int my_id = 0;
  for (int j = 0; j < k; j++) {
    uint64_t best = 0ull;
#pragma unroll
    for (int i = 0; i < PER; i++) best = key[i] > best ? key[i] : best;
    const uint64_t win = wave_max_key(best);
    const int id = key_id(win);
    if ((id & 63) == lane) {
#pragma unroll
      for (int i = 0; i < PER; i++)
        if (i == (id >> 6)) key[i] = 0ull;
    }
    if (lane == j) {
      my_v = key_value(win);
      my_id = id;
    }
  }
  const float v0 = __shfl(my_v, 0, kWave);
  const float ex = (lane < k) ? expf(my_v - v0) : 0.f;
  float denom = 0.f;
  for (int i = 0; i < k; i++) denom += __shfl(ex, i, kWave);  // slot order, same in every lane
  if (lane < k) {
    topk_ids[static_cast<int64_t>(t) * k + lane] = my_id;
    topk_w[static_cast<int64_t>(t) * k + lane] = ex / denom;
  }
}

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// A token's k expert ids are read kIdBatch at a time, every load of a batch issued before any
// is used (indices past the token's last id re-read that id and are discarded): in a loop over
// a run-time k each load would otherwise wait for the one before it.
constexpr int kIdBatch = 8;

__device__ __forceinline__ void load_id_batch(const int32_t *__restrict__ tok_ids, int k, int j0,
                                              int32_t (&v)[kIdBatch]) {
#pragma unroll
  for (int u = 0; u < kIdBatch; u++) v[u] = tok_ids[min(j0 + u, k - 1)];
}

// Fill the chunk's per-expert token bitmaps (bm[e * kWords + w]).
__device__ __forceinline__ void build_bitmaps(unsigned long long *bm, const int32_t *__restrict__ ids, int T,
                                              int E, int k, int chunk) {
  for (int i = threadIdx.x; i < E * kWords; i += blockDim.x) bm[i] = 0ull;
  __syncthreads();
  const int t = chunk * kChunk + threadIdx.x;
  if (t < T) {
    const unsigned long long bit = 1ull << (threadIdx.x & 63);
    const int32_t *tok_ids = ids + static_cast<int64_t>(t) * k;
    for (int j0 = 0; j0 < k; j0 += kIdBatch) {
      int32_t v[kIdBatch];
      load_id_batch(tok_ids, k, j0, v);
#pragma unroll
      for (int u = 0; u < kIdBatch; u++)
        if (j0 + u < k) atomicOr(&bm[clamp_expert(v[u], E) * kWords + (threadIdx.x >> 6)], bit);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kChunk) void chunk_count_kernel(const int32_t *__restrict__ ids, int T,
                                                             int E, int k,
                                                             int32_t *__restrict__ counts) {
  __shared__ unsigned long long bm[kMaxE * kWords];
  build_bitmaps(bm, ids, T, E, k, blockIdx.x);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kWords; w++) c += __popcll(bm[e * kWords + w]);
    counts[static_cast<int64_t>(blockIdx.x) * E + e] = c;
  }
}

constexpr int kPer = kMaxE / kChunk;   // experts per thread in the scans below

// base[e] = expert_offsets[e] + before[e] from each expert's total rows and rows in earlier
// chunks (thread t holds experts t * kPer .. + kPer): an exclusive scan of the totals over
// experts.  Workgroup 0 also writes expert_offsets.
__device__ __forceinline__ void bases_from_totals(int (&total)[kPer], int (&before)[kPer], int E, int chunk,
                                                  int32_t *base, int32_t *wave_total,
                                                  int32_t *__restrict__ offsets) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; i++) {
    if (t * kPer + i >= E) total[i] = before[i] = 0;
    mine += total[i];
  }
  int v = mine;   // inclusive scan of per-thread totals: wave scan, then the 4 wave totals
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  if (lane == 63) wave_total[wv] = v;
  __syncthreads();
  int excl = v - mine;
  for (int w = 0; w < wv; w++) excl += wave_total[w];
#pragma unroll
  for (int i = 0; i < kPer; i++) {
    const int e = t * kPer + i;
    if (e < E) {
      base[e] = excl + before[i];
      if (chunk == 0) offsets[e] = excl;
      if (chunk == 0 && e == E - 1) offsets[E] = excl + total[i];
    }
    excl += total[i];
  }
  __syncthreads();
}

// Per workgroup (chunk c): base[e] = expert_offsets[e] + (rows of expert e in chunks < c),
// from the read-only chunk counts -- a column sum per expert, then the scan above.
__device__ __forceinline__ void chunk_bases(const int32_t *__restrict__ counts, int nchunks, int E, int chunk,
                                            int32_t *base, int32_t *wave_total,
                                            int32_t *__restrict__ offsets) {
  const int t = threadIdx.x;
  constexpr int kBatch = 8;              // chunks whose counts are loaded together
  int total[kPer], before[kPer];
#pragma unroll
  for (int i = 0; i < kPer; i++) total[i] = before[i] = 0;
  // consecutive experts per thread keep the scan simple; every load of a batch is issued
  // before any is summed (indices clamped into the table, out-of-range terms dropped)
  for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
    int n[kPer][kBatch];
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      const int e = min(t * kPer + i, E - 1);
#pragma unroll
      for (int u = 0; u < kBatch; u++)
        n[i][u] = counts[static_cast<int64_t>(min(c0 + u, nchunks - 1)) * E + e];
    }
#pragma unroll
    for (int i = 0; i < kPer; i++)
#pragma unroll
      for (int u = 0; u < kBatch; u++) {
        const int c = c0 + u;
        total[i] += c < nchunks ? n[i][u] : 0;
        before[i] += c < chunk ? n[i][u] : 0;
      }
  }
  bases_from_totals(total, before, E, chunk, base, wave_total, offsets);
}

// Rows of this chunk's tokens: the rank of token t in expert e's rows within the chunk is the
// popcount of the chunk bitmap's bits below t.
__device__ __forceinline__ void scatter_chunk(const int32_t *__restrict__ ids, int T, int E, int k,
                                              const unsigned long long *bm, const int32_t *base,
                                              int32_t *__restrict__ row_src,
                                              int32_t *__restrict__ token_slot_row) {
  const int t = blockIdx.x * kChunk + threadIdx.x;
  if (t >= T) return;
  const int word = threadIdx.x >> 6;
  const unsigned long long below = (1ull << (threadIdx.x & 63)) - 1ull;
  const int64_t n = static_cast<int64_t>(T) * k;
  const int32_t *tok_ids = ids + static_cast<int64_t>(t) * k;
  for (int j0 = 0; j0 < k; j0 += kIdBatch) {
    int32_t v[kIdBatch];
    load_id_batch(tok_ids, k, j0, v);
#pragma unroll
    for (int u = 0; u < kIdBatch; u++) {
      if (j0 + u >= k) break;
      const int e = clamp_expert(v[u], E);
      int rank = __popcll(bm[e * kWords + word] & below);
      for (int w = 0; w < word; w++) rank += __popcll(bm[e * kWords + w]);
      int64_t p = static_cast<int64_t>(base[e]) + rank;
      p = p < 0 ? 0 : (p >= n ? n - 1 : p);
      row_src[p] = t;
      token_slot_row[static_cast<int64_t>(t) * k + j0 + u] = static_cast<int32_t>(p);
    }
  }
}

__global__ __launch_bounds__(kChunk) void scatter_kernel(const int32_t *__restrict__ ids, int T, int E,
                                                         int k, const int32_t *__restrict__ counts, int nchunks,
                                                         int32_t *__restrict__ offsets,
                                                         int32_t *__restrict__ row_src,
                                                         int32_t *__restrict__ token_slot_row) {
  __shared__ unsigned long long bm[kMaxE * kWords];
  __shared__ int32_t base[kMaxE];
  __shared__ int32_t wave_total[kChunk / 64];
  chunk_bases(counts, nchunks, E, blockIdx.x, base, wave_total, offsets);
  build_bitmaps(bm, ids, T, E, k, blockIdx.x);
  scatter_chunk(ids, T, E, k, bm, base, row_src, token_slot_row);
}

// Up to this many tokens the count launch is folded into the scatter: every workgroup reads
// all T * k ids (at most 128 K ids, from L2) instead of a count table.
constexpr int kFusedMaxTokens = 4096;

__global__ __launch_bounds__(kChunk) void count_scatter_kernel(const int32_t *__restrict__ ids, int T, int E,
                                                               int k, int32_t *__restrict__ offsets,
                                                               int32_t *__restrict__ row_src,
                                                               int32_t *__restrict__ token_slot_row) {
  __shared__ unsigned long long bm[kMaxE * kWords];
  __shared__ int32_t base[kMaxE];
  __shared__ int32_t hist_all[kMaxE];
  __shared__ int32_t hist_before[kMaxE];
  __shared__ int32_t wave_total[kChunk / 64];
  const int t = threadIdx.x;
  for (int e = t; e < E; e += kChunk) hist_all[e] = hist_before[e] = 0;
  __syncthreads();
  // rows per expert over all tokens, and over the tokens of earlier chunks (ids before
  // index `cut`); integer counts, so the order of the LDS additions does not matter
  const int64_t n = static_cast<int64_t>(T) * k;
  const int64_t cut = static_cast<int64_t>(blockIdx.x) * kChunk * k;
  constexpr int kBatch = 8;   // id loads issued together per thread
  for (int64_t i0 = 0; i0 < n; i0 += kBatch * kChunk) {
    int32_t v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; u++) {
      const int64_t i = i0 + u * kChunk + t;
      v[u] = ids[i < n ? i : n - 1];
    }
#pragma unroll
    for (int u = 0; u < kBatch; u++) {
      const int64_t i = i0 + u * kChunk + t;
      if (i < n) {
        const int e = clamp_expert(v[u], E);
        atomicAdd(&hist_all[e], 1);
        if (i < cut) atomicAdd(&hist_before[e], 1);
      }
    }
  }
  __syncthreads();
  int total[kPer], before[kPer];
#pragma unroll
  for (int i = 0; i < kPer; i++) {
    const int e = min(t * kPer + i, E - 1);
    total[i] = hist_all[e];
    before[i] = hist_before[e];
  }
  bases_from_totals(total, before, E, blockIdx.x, base, wave_total, offsets);
  build_bitmaps(bm, ids, T, E, k, blockIdx.x);
  scatter_chunk(ids, T, E, k, bm, base, row_src, token_slot_row);
}

// No tokens: every group is empty.
__global__ __launch_bounds__(kMaxE) void zero_offsets_kernel(int E, int32_t *__restrict__ offsets) {
  for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = 0;
}

}  // namespace

size_t route_permute_ws_bytes(int T, int E, int /*k*/) {
  const int64_t nchunks = (static_cast<int64_t>(T) + kChunk - 1) / kChunk;
  return static_cast<size_t>((nchunks > 0 ? nchunks : 1) * E * sizeof(int32_t));
}

hipError_t launch_route_permute(const float *logits, int T, int E, int k, int32_t *topk_ids,
                                float *topk_w, int32_t *expert_offsets, int32_t *row_src,
                                int32_t *token_slot_row, void *ws, hipStream_t stream) {
  int32_t *counts = static_cast<int32_t *>(ws);
  const int nchunks = (T + kChunk - 1) / kChunk;
  if (T > 0) {
    const dim3 tg((T + 3) / 4), tb(256);
    if (E <= 64) hipLaunchKernelGGL(topk_kernel<1>, tg, tb, 0, stream, logits, T, E, k, topk_ids, topk_w);
    else if (E <= 128) hipLaunchKernelGGL(topk_kernel<2>, tg, tb, 0, stream, logits, T, E, k, topk_ids, topk_w);
    else if (E <= 256) hipLaunchKernelGGL(topk_kernel<4>, tg, tb, 0, stream, logits, T, E, k, topk_ids, topk_w);
    else if (E <= 512) hipLaunchKernelGGL(topk_kernel<8>, tg, tb, 0, stream, logits, T, E, k, topk_ids, topk_w);
    else hipLaunchKernelGGL(topk_kernel<kMaxPerLane>, tg, tb, 0, stream, logits, T, E, k, topk_ids, topk_w);
    if (T <= kFusedMaxTokens) {
      hipLaunchKernelGGL(count_scatter_kernel, dim3(nchunks), dim3(kChunk), 0, stream, topk_ids, T, E, k,
                         expert_offsets, row_src, token_slot_row);
    } else {
      hipLaunchKernelGGL(chunk_count_kernel, dim3(nchunks), dim3(kChunk), 0, stream, topk_ids, T, E,
                         k, counts);
      hipLaunchKernelGGL(scatter_kernel, dim3(nchunks), dim3(kChunk), 0, stream, topk_ids, T, E, k,
                         counts, nchunks, expert_offsets, row_src, token_slot_row);
    }
  } else {
    hipLaunchKernelGGL(zero_offsets_kernel, dim3(1), dim3(kMaxE), 0, stream, E, expert_offsets);
  }
  return hipGetLastError();
}

}  // namespace moe
