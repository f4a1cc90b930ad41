// RMSNorm of the MoE sub-block's input on gfx950: x[t] = bf16( h[t] /
// sqrt(mean_j h[t, j]^2 + eps) * w ).
//
// Definition: "Qwen3.6-35B-A3B — Architecture Overview", Stage 2: Transform
// Blocks (RMSNorm -> MoE FFN -> +residual); Linnet model page, AttentionLayer /
// DeltaLayer (post_attention_layernorm: RmsNorm<H, T>) and RmsNorm (param
// weight [H]).  The pages give no formula: the textbook RMSNorm, the weight
// multiplying directly, eps from the caller.
//
// One wave per token: lane l takes the 8-element chunks l, l + 64, ... of the
// row; the sum of squares is taken per lane in chunk order, then over the wave
// in a fixed tree, so the result is reproducible; the row is read again (from
// cache) to scale it.  1 / sqrt in fp32 (IEEE sqrt and divide).
#include "kernels.hpp"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void rmsnorm_kernel(const bf16_t* __restrict__ h, const bf16_t* __restrict__ w,
                                                      float eps, int T, int H, bf16_t* __restrict__ x) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const bf16_t* row = h + (size_t)t * H;
  const int nch = H / 8;   // 16-byte chunks per row
  float ss = 0.f;
  for (int c = lane; c < nch; c += 64) {
    const u32x4 v = ld16(row + 8 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_to_f32(v[j] & 0xFFFFu), b = bf16_to_f32(v[j] >> 16);
      ss += a * a;
      ss += b * b;
    }
  }
  const float r = 1.0f / sqrtf(wave_sum_f32(ss) / (float)H + eps);
  for (int c = lane; c < nch; c += 64) {
    const u32x4 v = ld16(row + 8 * c), wv = ld16(w + 8 * c);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = pack_bf16x2(bf16_to_f32(v[j] & 0xFFFFu) * r * bf16_to_f32(wv[j] & 0xFFFFu),
                         bf16_to_f32(v[j] >> 16) * r * bf16_to_f32(wv[j] >> 16));
    st16(x + (size_t)t * H + 8 * c, o);
  }
}

}  // namespace

hipError_t launch_rmsnorm(const bf16_t* h, const bf16_t* w, float eps, int T, int H, bf16_t* x, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((T + 3) / 4), dim3(256), 0, s, h, w, eps, T, H, x);
  return hipGetLastError();
}

}  // namespace moe
