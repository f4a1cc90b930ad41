// Launchers of the gfx950 MoE kernels (host side), implemented in the .hip files.
#pragma once

#include <hip/hip_runtime.h>
#include "common.hpp"

namespace moe {

// Router tile: tokens per router workgroup (also the dispatch block size).
constexpr int kRouterTokens = 32;
// Grouped-GEMM tile: rows (slots) per tile, weight rows per tile.  Batches
// of at most 8 slots per expert on average (T K <= 8 E) use 32-row tiles:
// their groups are a few rows each, and the smaller tile leaves LDS for four
// workgroups per CU instead of two, which hides the start of the short down
// tiles (MI355X: 64 tokens 257 -> 252 us, 128 tokens 285 -> 281 us; at 384
// and 512 tokens the shared expert's 12-16 row tiles, each re-reading its
// weights, cost more than that saves: 313 -> 320 and 326 -> 330 us).
constexpr int kGemmBM = 160;
constexpr int kGemmBMSmall = 32;
constexpr int kGemmBNW = 128;   // weight rows per tile: gate_up 64 gate + 64 up; down 128 H cols
// Large batches: gate_up in 192-row tiles of 256 weight rows (eight waves
// per workgroup); the down projection keeps 160 x 128.
constexpr int kGemmBMWide = 192;
constexpr int kGemmBNWide = 256;
__host__ __device__ inline bool gemm_small_rows(int64_t T, int K, int E) { return T * K <= 8 * (int64_t)E; }
// From two 160-row tiles per expert on average.
__host__ __device__ inline bool gemm_wide(int64_t T, int K, int E) { return T * K >= 2 * (int64_t)E * kGemmBM; }
// Rows and weight rows per tile of either GEMM.
__host__ __device__ inline int gemm_bm(int64_t T, int K, int E, bool gate_up) {
  return gemm_small_rows(T, K, E) ? kGemmBMSmall : (gate_up && gemm_wide(T, K, E) ? kGemmBMWide : kGemmBM);
}
__host__ __device__ inline int gemm_bn(int64_t T, int K, int E, bool gate_up) {
  return gate_up && gemm_wide(T, K, E) ? kGemmBNWide : kGemmBNW;
}
// Upper bound of the tiles of one grouped GEMM (workspace and grid size):
// every group adds at most one partial row tile.  Counted with 160 x 128
// tiles, it also bounds the fewer 192 x 256 tiles of large batches.  Past the switch to 160-row
// tiles the bound keeps the 32-row bound of the largest small batch, so it
// never decreases as T grows (a workspace sized for T serves smaller batches).
__host__ __device__ inline int64_t gemm_tile_bound_bm(int64_t T, int K, int E, int wrows, int wrows_shared, int bm) {
  const int64_t nt = (wrows + kGemmBNW - 1) / kGemmBNW, nts = (wrows_shared + kGemmBNW - 1) / kGemmBNW;
  return ((T * K + bm - 1) / bm + E) * nt + ((T + bm - 1) / bm) * nts;
}
__host__ __device__ inline int64_t gemm_tile_bound(int64_t T, int K, int E, int wrows, int wrows_shared) {
  if (gemm_small_rows(T, K, E)) return gemm_tile_bound_bm(T, K, E, wrows, wrows_shared, kGemmBMSmall);
  const int64_t small_max = 8 * (int64_t)E / K;   // largest batch with 32-row tiles
  const int64_t a = gemm_tile_bound_bm(small_max, K, E, wrows, wrows_shared, kGemmBMSmall);
  const int64_t b = gemm_tile_bound_bm(T, K, E, wrows, wrows_shared, kGemmBM);
  return a > b ? a : b;
}

// Order of a group's mt x nct tiles in the dispatch list: blocks of rb row
// tiles, within a block column tile major and row tile minor (rb = 1: row
// tile major).  Consecutive tiles run side by side on one XCD, so a block's
// activation rows are fetched once for all its column tiles and its weight
// columns once for all its row tiles (through that XCD's L2); a group of at
// most rb row tiles is simply column tile major.  The down projection and the
// large-batch gate_up take blocks of eight row tiles.  The other gate_up
// tiles go row tile major: the shared expert's gate/up weights (2 MB) stay
// in L2 across all its row tiles anyway, and its x rows are then shared by
// consecutive tiles (MI355X, 4096 tokens, gate_up over three alternating
// repeats: 240-244 -> 234-240 us).  Row tile major measured slower for the
// down projection (Zipf(1.1) over 16384 tokens: 410-414 -> 429-430 us) and
// for the large-batch gate_up (617-620 -> 624-630 us).
constexpr int kGemmRowBlock = 8;
__host__ __device__ inline int gemm_row_block(int64_t T, int K, int E, bool gate_up) {
  return gate_up && !gemm_wide(T, K, E) ? 1 : kGemmRowBlock;
}
__host__ __device__ inline void gemm_tile_order(int i, int mt, int nct, int rb, int& mi, int& nt) {
  const int full = (mt / rb) * rb * nct;   // tiles of the full row blocks
  int b, rows, j;
  if (i < full) {
    b = i / (rb * nct);
    rows = rb;
    j = i - b * rb * nct;
  } else {
    b = mt / rb;
    rows = mt - b * rb;
    j = i - full;
  }
  nt = j / rows;
  mi = b * rb + (j - nt * rows);
}

__host__ __device__ inline int router_blocks(int64_t T) { return (int)((T + kRouterTokens - 1) / kRouterTokens); }
// Batches of at most this many router blocks are dispatched by one workgroup,
// which builds its own token masks (no per-block histograms needed).
constexpr int kDispatchSmallBlocks = 64;
__host__ __device__ inline bool dispatch_single_block(int64_t T) { return router_blocks(T) <= kDispatchSmallBlocks; }
// Columns of a row of router partial sums: E logits, the shared gate, padding
// to a multiple of 4.
__host__ __device__ inline int router_cols(int E) { return (E + 1 + 3) & ~3; }
// Slices of H the router's logits GEMM is split into for T tokens.
int router_ksplit(int T, int H);
// Upper bound of ksplit(T') * T' over T' <= T (rows of router partial sums).
int64_t router_partial_rows(int64_t T, int H);

// Fused decode path (T <= kDecodeMaxT, H <= 2048, I <= 512, Is <= 512, and the
// per-workgroup row shares of decode_fits).
constexpr int kDecodeMaxT = 16;

// Control block at the start of every workspace (uint32 words), shared by
// both paths and written by nothing else, so its words keep their meaning
// across calls of either path.  Tags are call-unique and never 0; a
// zero-filled block holds no call's tag.
constexpr int kCtlError = 0;   // tag of the latest call one of whose waits timed out
constexpr int kCtlLast = 1;    // tag of the latest call that used the workspace
constexpr int kCtlTimeouts = 2;  // calls one of whose waits timed out, since the block was zeroed
constexpr int kCtlFlags = 32;  // fused path: + x * kDecodeFlagStride, copy x of the arrival flags
// 100 MHz wall-clock ticks a fused-path wait may take before it gives up (0.25 s).
constexpr unsigned long long kDefaultWaitTicks = 25000000ull;

struct DecodeArgs {
  LayerArgs L;
  const bf16_t* x;      // [T, H]
  int T;
  int route_only;       // 1: stop after routing and write offsets/perm
  bf16_t* out;          // [T, H]
  uint32_t* ctl;        // control block: error word, arrival flags (kDecodeReplicas copies)
  uint64_t* logits_t;   // kDecodeReplicas copies of [T, 256] tagged logits (fp32 bits in the high
                        // word, the call tag in the low word), copy stride decode_logit_stride(T)
  float* logits_out;    // optional [T, E] fp32 logits (route)
  int32_t* topk_idx;    // [T, K]
  float* topk_w;        // [T, K]
  float* gate_s;        // [T] shared-expert gate sigma(x . w_g)
  bf16_t* h;            // [T*K, I] per (token, k) pair, routing weight applied
  bf16_t* h_sh;         // [T, Is]
  int32_t* offsets_out; // route-only: [E + 1]
  int32_t* perm_out;    // route-only: [T*K]
  unsigned long long epoch;   // call-unique; its low 32 bits (never 0) tag this call's logits
  unsigned long long wait_ticks;   // budget of each bounded wait (100 MHz ticks); 0: give up at the first miss
  const bf16_t* norm_w; // optional [H]: x is RMSNorm(x) with this weight (the sub-block form)
  float eps;            // RMSNorm epsilon
  const bf16_t* residual;  // optional [T, H]: out = bf16(residual + layer output)
};
// Cross-workgroup data of the decode path is published in one copy per XCD
// (readers poll the copy of their own XCD).
constexpr int kDecodeReplicas = 8;
constexpr int kDecodeMaxGrid = 256;
constexpr int kDecodeFlagStride = kDecodeMaxGrid + 32;   // words between flag copies
constexpr int kDecodeCtlWords = 32 + kDecodeReplicas * kDecodeFlagStride;
// Elements (uint64) between logit copies: T rows of 256, plus a 512-byte skew.
__host__ __device__ inline int decode_logit_stride(int T) { return T * 256 + 64; }

hipError_t launch_decode(const DecodeArgs& a, int grid, hipStream_t s);
int decode_max_grid(int num_cus);
// True when a grid of `grid` workgroups can hold the layer's per-workgroup
// shares of router rows, the shared gate row, shared gate/up rows and output
// rows (16-row tiles).
bool decode_fits(int H, int E, int Is, int grid);

// psum_out (optional): per router block, the sum over its tokens of every
// expert's full-softmax probability (the load-balance statistic's input).
hipError_t launch_router(const LayerArgs& L, const bf16_t* x, int T, const Work& w,
                         float* logits_out, hipStream_t s, float* psum_out = nullptr);
// Load-balance statistic from the block probability sums and the dispatch
// offsets: lb [1], mean_prob [E] (optional), counts [E] (optional).
// Stable ranks of the scores [R, E] (fp32 if dtype == 0, else bf16), E <= 256.
hipError_t launch_ranks(const void* logits, int dtype, int R, int E, int32_t* ranks, hipStream_t s);
hipError_t launch_load_balance(const LayerArgs& L, int T, const Work& w, float* lb, float* mean_prob,
                               int32_t* counts, hipStream_t s);
hipError_t launch_dispatch(const LayerArgs& L, int T, const Work& w, hipStream_t s);
// Fused small-batch route (T <= kRouteMaxT, H <= 2048): router logits, top-K
// selection and the per-group dispatch in one launch whose workgroups hand
// data to each other through the workspace's tagged exchange region (w.lt)
// with bounded waits; the same outputs as launch_router + launch_dispatch
// (block histograms and probability sums aside, which it does not form).
constexpr int kRouteMaxT = 64;
constexpr int kRouteSelStride = kRouteMaxT * 8;   // words between the copies of the published selections
__host__ __device__ inline bool route_fused_fits(int64_t T, int H, int K) {
  return T >= 1 && T <= kRouteMaxT && H <= 2048 && H % 128 == 0 && K <= 8;
}
hipError_t launch_route_fused(const LayerArgs& L, const bf16_t* x, int T, const Work& w, float* logits_out,
                              unsigned long long wait_ticks, hipStream_t s);
// window (optional): int4 {first routed tile, count, first shared tile, count}
// selecting part of the dispatch tile list; slot_map (optional): expert ->
// weight block index (cache slot) for the routed groups.
hipError_t launch_gate_up(const LayerArgs& L, const bf16_t* x, int T, const Work& w,
                          int num_cus, hipStream_t s, const int* window = nullptr, const int* slot_map = nullptr);
hipError_t launch_down(const LayerArgs& L, int T, const Work& w, int num_cus, hipStream_t s,
                       const int* window = nullptr, const int* slot_map = nullptr);
// [E, R, Kd] row-major bf16 -> the MFMA-tile layout (R % 16 == 0, Kd % 64 == 0).
hipError_t launch_pack_tiles(const bf16_t* src, bf16_t* dst, int E, int R, int Kd, hipStream_t s);
// Streamed experts: plan the rounds after dispatch (C slots, R rounds), then
// per round copy its experts from host memory into the slots.
hipError_t launch_stream_plan(const LayerArgs& L, const Work& w, int C, int R, hipStream_t s);
hipError_t launch_stream_copy(const LayerArgs& L, const void* host_gu, const void* host_dn, void* slot_gu,
                              void* slot_dn, const Work& w, int C, int r, hipStream_t s);
// residual (optional): out = bf16(residual + combined sum), one rounding.
hipError_t launch_combine(const LayerArgs& L, int T, const Work& w, bf16_t* out, hipStream_t s,
                          const bf16_t* residual = nullptr);
// x = bf16(h / sqrt(mean(h^2) + eps) * w), one wave per token.
hipError_t launch_rmsnorm(const bf16_t* h, const bf16_t* w, float eps, int T, int H, bf16_t* x, hipStream_t s);

}  // namespace moe
