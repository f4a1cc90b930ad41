// Dispatch of (token, k) pairs to contiguous per-expert segments: a counting
// sort keyed by expert, stable in the pair id q = t*K + k.  The per-block
// expert histograms come from the router kernel; here they are summed and
// scanned into segment offsets and per-block bases, and each block then
// scatters its pairs in order.  All integer work: the result is bit-exact.
//
// The pages say only that the router picks which experts receive a token
// ("One Token Through Qwen3.6", section "The Router"; "Qwen3.6-35B-A3B —
// Architecture Overview", section "MoE FFN: 256 Experts": only 8 of 256 fire
// per token); grouping the pairs by expert is how this implementation lets
// each expert run once as a dense GEMM over its rows.
#include "kernels.hpp"
#include "group_dispatch.hpp"

namespace moe {

namespace {

// Pairs per expert, from the count kernel to the place kernel: the first E
// words of h, which the gate_up GEMM writes only later (this path serves
// batches of more than 2048 tokens, whose h holds far more than E words).
__device__ __forceinline__ int32_t* expert_counts(const Work& w) { return reinterpret_cast<int32_t*>(w.h); }

// Inclusive prefix sum over the 256 threads of a block (4 wavefronts).
__device__ int block_inclusive_scan(int v, int* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  int add = 0;
  for (int i = 0; i < wave; ++i) add += wave_tot[i];
  __syncthreads();
  return v + add;
}

// One workgroup per expert: exclusive prefix of the expert's count over the
// router blocks (written back in place as each block's base inside the
// expert's segment) and the expert's total (expert_counts).
__global__ __launch_bounds__(256) void dispatch_count_kernel(LayerArgs L, int T, Work w) {
  __shared__ int wave_tot[4];
  const int e = blockIdx.x, E = L.E;
  const int nblk = router_blocks(T);
  const int per = (nblk + 255) / 256;            // blocks per thread, contiguous
  const int b0 = threadIdx.x * per, b1 = min(nblk, b0 + per);
  int run = 0;
  for (int b = b0; b < b1; ++b) run += w.blk_counts[(size_t)b * E + e];
  const int incl = block_inclusive_scan(run, wave_tot);
  int base = incl - run;
  for (int b = b0; b < b1; ++b) {
    const int c = w.blk_counts[(size_t)b * E + e];
    w.blk_counts[(size_t)b * E + e] = base;
    base += c;
  }
  if (threadIdx.x == 255) expert_counts(w)[e] = incl;
}

// Segment offsets from the expert totals and the tile prefix sums of both
// grouped GEMMs (group E is the shared expert, T rows), into LDS.  Every
// workgroup of the place kernel computes them itself from the 256 totals,
// which saves a single-workgroup launch between the count and the place
// kernels (MI355X, dispatch phase over three alternating repeats: 18.4-18.7
// -> 16.9-17.1 us at 4096 tokens, 20.4-20.7 -> 19.8-20.2 us at 16384).
__device__ void dispatch_scan(LayerArgs L, int T, const Work& w, int* wave_tot, int* s_off, int* s_tgu, int* s_tdn) {
  const int e = threadIdx.x;
  const int E = L.E, K = L.K;
  const int bmg = gemm_bm(T, K, E, true), bng = gemm_bn(T, K, E, true);
  const int bmd = gemm_bm(T, K, E, false), bnd = gemm_bn(T, K, E, false);
  const int cnt = e < E ? expert_counts(w)[e] : 0;
  const int incl = block_inclusive_scan(cnt, wave_tot);
  if (e < E) s_off[e] = incl - cnt;
  if (e == 0) s_off[E] = T * K;

  // Tiles per group: ceil(rows / bm) row tiles x (weight rows / bn) column
  // tiles, each GEMM with its own tile shape (gemm_bm, gemm_bn).
  int gu = 0, dn = 0;
  if (e < E) {
    gu = ((cnt + bmg - 1) / bmg) * ((2 * L.I + bng - 1) / bng);
    dn = ((cnt + bmd - 1) / bmd) * (L.H / bnd);
  }
  const int gu_incl = block_inclusive_scan(gu, wave_tot);
  const int dn_incl = block_inclusive_scan(dn, wave_tot);
  if (e < E) {
    s_tgu[e] = gu_incl - gu;
    s_tdn[e] = dn_incl - dn;
  }
  if (e == E - 1) {
    s_tgu[E] = gu_incl;
    s_tdn[E] = dn_incl;
    s_tgu[E + 1] = gu_incl + ((T + bmg - 1) / bmg) * ((2 * L.Is + bng - 1) / bng);
    s_tdn[E + 1] = dn_incl + ((T + bmd - 1) / bmd) * (L.H / bnd);
  }
  __syncthreads();
}

// Workgroup g of the group tiles (E: the shared expert): the descriptors of
// its tiles in both grouped GEMMs, in gemm_tile_order.
__device__ void dispatch_tiles(LayerArgs L, int T, const Work& w, int g, const int* s_off, const int* s_tgu,
                               const int* s_tdn) {
  const int E = L.E;
  const int bmg = gemm_bm(T, L.K, E, true), bng = gemm_bn(T, L.K, E, true);
  const int bmd = gemm_bm(T, L.K, E, false), bnd = gemm_bn(T, L.K, E, false);
  const bool shared = g == E;
  const int seg0 = shared ? 0 : s_off[g];
  const int nrows = shared ? T : s_off[g + 1] - seg0;
  const int mtg = (nrows + bmg - 1) / bmg, mtd = (nrows + bmd - 1) / bmd;
  const int ngu = (2 * (shared ? L.Is : L.I) + bng - 1) / bng, ndn = L.H / bnd;
  const int bgu = s_tgu[g], bdn = s_tdn[g];
  const int rbg = gemm_row_block(T, L.K, E, true), rbd = gemm_row_block(T, L.K, E, false);
  for (int i = threadIdx.x; i < mtg * ngu; i += 256) {
    int mi, nt;
    gemm_tile_order(i, mtg, ngu, rbg, mi, nt);
    w.tdesc_gu[bgu + i] = make_int4(g, seg0, nrows, mi | (nt << 16));
  }
  for (int i = threadIdx.x; i < mtd * ndn; i += 256) {
    int mi, nt;
    gemm_tile_order(i, mtd, ndn, rbd, mi, nt);
    w.tdesc_dn[bdn + i] = make_int4(g, seg0, nrows, mi | (nt << 16));
  }
}

// Stable scatter of router block blk's pairs (at most 32*K <= 256).  A
// token's K experts are distinct, so a pair's rank among the block's pairs of
// its expert is the number of the block's earlier tokens that chose that
// expert: the population of the expert's token mask below its token.
__device__ void dispatch_scatter(LayerArgs L, int T, const Work& w, int blk, const int* s_off) {
  static_assert(kRouterTokens == 32, "one 32-bit token mask per expert");
  __shared__ uint32_t mask[256];
  const int E = L.E, K = L.K;
  const int j = threadIdx.x;
  const int q0 = blk * kRouterTokens * K;
  const int n = min(kRouterTokens * K, T * K - q0);
  const int key = j < n ? min(max(w.topk_idx[q0 + j], 0), E - 1) : 0;
  const int tl = j / K;
  mask[j] = 0u;   // E <= 256 = the block size
  __syncthreads();
  if (j < n) atomicOr(&mask[key], 1u << tl);
  __syncthreads();
  if (j < n) {
    const int rank = __popc(mask[key] & ((1u << tl) - 1u));
    const int slot = s_off[key] + w.blk_counts[(size_t)blk * E + key] + rank;
    w.perm[slot] = q0 + j;
    w.slot_of[q0 + j] = slot;
    w.slot_tok[slot] = (q0 + j) / K;
  }
}

// Tile descriptors and the scatter depend only on the offsets, tile prefix
// sums and block bases, so they share one launch: workgroups 0 .. E write the
// groups' tile descriptors, the rest scatter one router block each.
// Workgroup 0 also publishes the offsets and tile prefix sums for the GEMMs
// and zeroes the persistent GEMMs' claim counters.
__global__ __launch_bounds__(256) void dispatch_place_kernel(LayerArgs L, int T, Work w) {
  __shared__ int wave_tot[4];
  __shared__ int s_off[257], s_tgu[258], s_tdn[258];
  dispatch_scan(L, T, w, wave_tot, s_off, s_tgu, s_tdn);
  const int b = blockIdx.x, E = L.E;
  if (b == 0) {
    for (int e = threadIdx.x; e <= E; e += 256) w.offsets[e] = s_off[e];
    for (int g = threadIdx.x; g <= E + 1; g += 256) {
      w.tiles_gu[g] = s_tgu[g];
      w.tiles_dn[g] = s_tdn[g];
    }
    if (threadIdx.x < 16) w.claims[32 * threadIdx.x] = 0;
  }
  if (b <= E) dispatch_tiles(L, T, w, b, s_off, s_tgu, s_tdn);
  else dispatch_scatter(L, T, w, b - (E + 1), s_off);
}

// Batches of at most kSmallBlocks router blocks: the whole dispatch in one
// workgroup.  Token masks per (block, expert) are built in LDS; an expert's
// count in a block is its mask's population, the pair's rank among the
// block's pairs of that expert is the population of the mask below its
// token (tokens of a block are distinct per expert, and pair ids grow with
// the token), so the slots equal those of the multi-kernel path.
constexpr int kSmallBlocks = kDispatchSmallBlocks;
constexpr int kSmallThreads = 1024;

__global__ __launch_bounds__(kSmallThreads) void dispatch_small_kernel(LayerArgs L, int T, Work w) {
  __shared__ uint32_t s_mask[kSmallBlocks * 256];
  __shared__ int s_base[kSmallBlocks * 256];
  __shared__ int s_cnt[256], s_off[257], s_tgu[258], s_tdn[258];
  __shared__ int wave_tot[kSmallThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = L.E, K = L.K, TK = T * K;
  const int bmg = gemm_bm(T, K, E, true), bng = gemm_bn(T, K, E, true);
  const int bmd = gemm_bm(T, K, E, false), bnd = gemm_bn(T, K, E, false);
  const int nblk = router_blocks(T);
  for (int i = tid; i < nblk * E; i += kSmallThreads) s_mask[i] = 0u;
  __syncthreads();
  for (int q = tid; q < TK; q += kSmallThreads) {
    const int t = q / K, b = t / kRouterTokens;
    atomicOr(&s_mask[b * E + w.topk_idx[q]], 1u << (t - b * kRouterTokens));
  }
  __syncthreads();
  // Per expert: exclusive prefix of its counts over the blocks.
  if (tid < E) {
    int run = 0;
    for (int b = 0; b < nblk; ++b) {
      s_base[b * E + tid] = run;
      run += __popc(s_mask[b * E + tid]);
    }
    s_cnt[tid] = run;
  }
  __syncthreads();
  // Segment offsets and tile prefix sums (one wave per quantity, 256 experts
  // as four per lane; group E is the shared expert with T rows).
  if (wave < 3) {
    int v[4], run = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      const int cnt = e < E ? s_cnt[e] : 0;
      v[j] = wave == 0 ? cnt
                       : (wave == 1 ? ((cnt + bmg - 1) / bmg) * ((2 * L.I + bng - 1) / bng)
                                    : ((cnt + bmd - 1) / bmd) * (L.H / bnd));
      run += v[j];
    }
    int incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(incl, o, 64);
      if (lane >= o) incl += n;
    }
    int ex = incl - run;
    int* dst = wave == 0 ? s_off : (wave == 1 ? s_tgu : s_tdn);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      if (e < E) dst[e] = ex;
      ex += v[j];
    }
    if (lane == 63) {
      dst[E] = incl;
      if (wave == 1) dst[E + 1] = incl + ((T + bmg - 1) / bmg) * ((2 * L.Is + bng - 1) / bng);
      if (wave == 2) dst[E + 1] = incl + ((T + bmd - 1) / bmd) * (L.H / bnd);
    }
  }
  __syncthreads();
  for (int e = tid; e <= E; e += kSmallThreads) w.offsets[e] = s_off[e];
  for (int g = tid; g <= E + 1; g += kSmallThreads) {
    w.tiles_gu[g] = s_tgu[g];
    w.tiles_dn[g] = s_tdn[g];
  }
  if (tid < 16) w.claims[32 * tid] = 0;   // claim counters of the persistent GEMMs
  // Tile descriptors in gemm_tile_order, one item per (group, column tile)
  // of either GEMM, waves over column tiles and lanes over groups.  Item
  // (g, nt) writes column tile nt of every row block of group g: a block of
  // `rows` row tiles starts at b0 * ncol and holds that column tile at
  // nt * rows + row.  (Small batches give the shared group many row tiles,
  // so one thread per group would be a long serial path.)
  {
    const int ngu_r = (2 * L.I + bng - 1) / bng, ngu_s = (2 * L.Is + bng - 1) / bng;
    const int ndn = L.H / bnd, gumax = max(ngu_r, ngu_s), ncols = gumax + ndn;
    const int rbg = gemm_row_block(T, L.K, E, true), rbd = gemm_row_block(T, L.K, E, false);
    for (int c = wave; c < ncols; c += kSmallThreads / 64) {
      for (int g = lane; g <= E; g += 64) {
        const bool shared = g == E, gu = c < gumax;
        const int ncol = gu ? (shared ? ngu_s : ngu_r) : ndn, nt = gu ? c : c - gumax;
        if (nt >= ncol) continue;
        const int seg0 = shared ? 0 : s_off[g];
        const int nrows = shared ? T : s_cnt[g];
        const int bm = gu ? bmg : bmd, mt = (nrows + bm - 1) / bm, rb = gu ? rbg : rbd;
        int4* base = gu ? w.tdesc_gu + s_tgu[g] : w.tdesc_dn + s_tdn[g];
        for (int b0 = 0; b0 < mt; b0 += rb) {
          const int rows = min(rb, mt - b0);
          int4* d = base + b0 * ncol + nt * rows;
          for (int r = 0; r < rows; ++r) d[r] = make_int4(g, seg0, nrows, (b0 + r) | (nt << 16));
        }
      }
    }
  }
  // Scatter.
  for (int q = tid; q < TK; q += kSmallThreads) {
    const int t = q / K, b = t / kRouterTokens, e = w.topk_idx[q];
    const uint32_t below = s_mask[b * E + e] & ((1u << (t - b * kRouterTokens)) - 1u);
    const int slot = s_off[e] + s_base[b * E + e] + __popc(below);
    w.perm[slot] = q;
    w.slot_of[q] = slot;
    w.slot_tok[slot] = t;
  }
}

// Batches of at most kGroupPairs (token, expert) pairs: one workgroup per
// group, so that the descriptors and slots are written by the whole grid
// instead of one workgroup (MI355X, 64 tokens: dispatch phase 10.7 -> 7.8 us,
// step 255.6 -> 252.5 us over three alternating repeats); see
// group_dispatch.hpp.
constexpr int kGroupPairs = 2048;

__global__ __launch_bounds__(kGroupThreads) void dispatch_group_kernel(LayerArgs L, int T, Work w) {
  constexpr int kPer = kGroupPairs / kGroupThreads;
  const int TK = T * L.K;
  int idx[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int q = threadIdx.x + j * kGroupThreads;
    idx[j] = q < TK ? w.topk_idx[q] : -1;
  }
  dispatch_group<kPer>(L, T, w, blockIdx.x, idx);
}

}  // namespace

hipError_t launch_dispatch(const LayerArgs& L, int T, const Work& w, hipStream_t s) {
  if ((int64_t)T * L.K <= kGroupPairs && T <= kGroupTokens) {   // (E <= 256 is checked at the boundary)
    hipLaunchKernelGGL(dispatch_group_kernel, dim3(L.E + 1), dim3(kGroupThreads), 0, s, L, T, w);
    return hipGetLastError();
  }
  if (dispatch_single_block(T)) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(kSmallThreads), 0, s, L, T, w);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(L.E), dim3(256), 0, s, L, T, w);
  hipLaunchKernelGGL(dispatch_place_kernel, dim3(L.E + 1 + router_blocks(T)), dim3(256), 0, s, L, T, w);
  return hipGetLastError();
}

}  // namespace moe
