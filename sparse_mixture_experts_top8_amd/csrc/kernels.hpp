// Launchers of the gfx950 MoE kernels (host side), implemented in the .hip files.
#pragma once

#include <hip/hip_runtime.h>
#include "common.hpp"

namespace moe {

// Router tile: tokens per router workgroup (also the dispatch block size).
constexpr int kRouterTokens = 32;
// Grouped-GEMM tile: rows (slots) per tile, weight rows per tile.
constexpr int kGemmBM = 64;
constexpr int kGemmBNW = 128;   // weight rows per tile: gate_up 64 gate + 64 up; down 128 H cols

__host__ __device__ inline int router_blocks(int64_t T) { return (int)((T + kRouterTokens - 1) / kRouterTokens); }

hipError_t launch_router(const LayerArgs& L, const bf16_t* x, int T, const Work& w,
                         float* logits_out, hipStream_t s);
hipError_t launch_dispatch(const LayerArgs& L, int T, const Work& w, hipStream_t s);
hipError_t launch_gate_up(const LayerArgs& L, const bf16_t* x, int T, const Work& w,
                          int num_cus, hipStream_t s);
hipError_t launch_down(const LayerArgs& L, int T, const Work& w, int num_cus, hipStream_t s);
hipError_t launch_combine(const LayerArgs& L, int T, const Work& w, bf16_t* out, hipStream_t s);

}  // namespace moe
