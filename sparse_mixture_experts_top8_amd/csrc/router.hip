// Router of the MoE layer on gfx950: logits = x W_r^T with bf16 MFMA, then per
// token a wavefront-level top-K (descending logit, ties to the lower expert
// index), the softmax renormalised over the selected experts, the shared-expert
// gate scalar sigmoid(x . w_sg), and a per-block expert histogram that the
// dispatch step turns into segment offsets.
//
// Definition: "Qwen3.6-35B-A3B — Architecture Overview", section "MoE FFN: 256
// Experts" (router Linear 2048 -> 256, softmax, top-8, renormalise to sum 1;
// shared expert scaled by sigmoid(Linear(x, 1))); Linnet model page, Blocks:
// SparseMoe (gate: Linear<H, Experts>, shared_expert_gate: Linear<H, 1>, ranks).
//
// Softmax over all experts followed by renormalisation over the K selected is
// the same quantity as a softmax over the K selected logits alone (the full
// denominator cancels); the kernel computes the latter.
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kTok = kRouterTokens;      // 32 tokens per workgroup
constexpr int kLdsStride = 256 + 4;      // padded logits row (E <= 256)

// Logits accumulate in fp32 MFMA accumulators; every 256 elements of H the
// partial sums are folded into a second fp32 total, which keeps the rounding
// error of the long dot product near that of a pairwise sum.
__global__ __launch_bounds__(256) void router_topk_kernel(LayerArgs L, const bf16_t* __restrict__ x,
                                                         int T, Work w, float* __restrict__ logits_out) {
  __shared__ float lg[kTok * kLdsStride];
  __shared__ int hist[256];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.x * kTok;
  const int H = L.H, E = L.E, K = L.K;
  hist[tid] = 0;

  // ---- logits tile [32 tokens x E] with v_mfma_f32_16x16x32_bf16 ----
  // Lane l supplies row (l % 16) and k-group 8*(l / 16) of both operands;
  // the result lands as D[4*(l/16) + r][l % 16].
  const int nsub_e = (E + 15) >> 4;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const bf16_t* arow[2];
  bool aval[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int t = t0 + 16 * i + r16;
    aval[i] = t < T;
    arow[i] = x + (size_t)(aval[i] ? t : 0) * H + kq;
  }
  const bf16_t* brow[4];
  bool bval[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    int j = wave + 4 * jj;
    int e = 16 * j + r16;
    bval[jj] = (j < nsub_e) && (e < E);
    brow[jj] = L.router_w + (size_t)(bval[jj] ? e : 0) * H + kq;
  }
  f32x4 acc[2][4], tot[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
      tot[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  for (int k0 = 0; k0 < H; k0 += 32) {
    u32x4 a[2], b[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = aval[i] ? ld16(arow[i] + k0) : zero4;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) b[jj] = bval[jj] ? ld16(brow[jj] + k0) : zero4;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      if (wave + 4 * jj < nsub_e) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[i]), as_bf16x8(b[jj]),
                                                               acc[i][jj], 0, 0, 0);
      }
    }
    if (((k0 + 32) & 255) == 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          tot[i][jj] += acc[i][jj];
          acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
  }
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    int j = wave + 4 * jj;
    int e = 16 * j + r16;
    if (j < nsub_e && e < E) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) lg[(16 * i + 4 * (lane >> 4) + r) * kLdsStride + e] = tot[i][jj][r];
    }
  }
  __syncthreads();

  // ---- per token: top-K, renormalised weights, shared gate, histogram ----
  for (int tl = wave; tl < kTok; tl += 4) {
    const int t = t0 + tl;
    if (t >= T) break;
    float v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      int e = lane + 64 * c;
      v[c] = e < E ? lg[tl * kLdsStride + e] : -INFINITY;
      if (v[c] != v[c]) v[c] = -INFINITY;  // NaN never outranks a number
    }
    if (logits_out) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        int e = lane + 64 * c;
        if (e < E) logits_out[(size_t)t * E + e] = lg[tl * kLdsStride + e];
      }
    }
    float sel_v[8];
    int sel_i[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sel_v[k] = 0.f;
      sel_i[k] = 0;
      if (k < K) {
        // Best candidate of this lane: lowest column wins ties (strict >).
        // Padding columns (e >= E) hold -inf and lose every tie to a real
        // expert, so the selected index is always below E.
        float bv = v[0];
        int bi = lane;
#pragma unroll
        for (int c = 1; c < 4; ++c)
          if (v[c] > bv) { bv = v[c]; bi = lane + 64 * c; }
        // Wavefront arg-max under the order (higher value, then lower index).
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          float ov = __shfl_xor(bv, o, kWave);
          int oi = __shfl_xor(bi, o, kWave);
          if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
        }
        sel_v[k] = bv;
        sel_i[k] = bi;
        if ((bi & 63) == lane) {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if ((bi >> 6) == c) v[c] = -INFINITY;
        }
      }
    }
    // Renormalised softmax over the selected logits (sel_v[0] is the maximum).
    float den = 0.f, mine_w = 0.f;
    int mine_i = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < K) {
        float p = __expf(sel_v[k] - sel_v[0]);
        den += p;
        if (lane == k) { mine_w = p; mine_i = sel_i[k]; }
      }
    }
    if (lane < K) {
      w.topk_idx[(size_t)t * K + lane] = mine_i;
      w.topk_w[(size_t)t * K + lane] = mine_w / den;
      atomicAdd(&hist[mine_i], 1);
    }
    // Shared-expert gate: sigmoid(x[t] . w_sg), four elements per lane per step.
    float part = 0.f;
    const bf16_t* xr = x + (size_t)t * H;
    for (int h0 = 4 * lane; h0 < H; h0 += 256) {
      uint2 xv = *reinterpret_cast<const uint2*>(xr + h0);
      uint2 gv = *reinterpret_cast<const uint2*>(L.sh_expert_gate + h0);
      part += bf16_to_f32(xv.x & 0xFFFFu) * bf16_to_f32(gv.x & 0xFFFFu);
      part += bf16_to_f32(xv.x >> 16) * bf16_to_f32(gv.x >> 16);
      part += bf16_to_f32(xv.y & 0xFFFFu) * bf16_to_f32(gv.y & 0xFFFFu);
      part += bf16_to_f32(xv.y >> 16) * bf16_to_f32(gv.y >> 16);
    }
    part = wave_sum(part);
    if (lane == 0) w.gate_s[t] = sigmoidf_(part);
  }
  __syncthreads();
  if (tid < E) w.blk_counts[(size_t)blockIdx.x * E + tid] = hist[tid];
}

}  // namespace

hipError_t launch_router(const LayerArgs& L, const bf16_t* x, int T, const Work& w,
                         float* logits_out, hipStream_t s) {
  const int nblk = router_blocks(T);
  hipLaunchKernelGGL(router_topk_kernel, dim3(nblk), dim3(256), 0, s, L, x, T, w, logits_out);
  return hipGetLastError();
}

}  // namespace moe
