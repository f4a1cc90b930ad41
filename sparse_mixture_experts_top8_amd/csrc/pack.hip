// Routed expert weights in the MFMA-tile layout the grouped GEMMs stream
// best: for each expert, each block of 16 consecutive rows and each 64-wide
// k-step, 2 KB holding half h (0, 1) then lane l (0..63) then 8 elements, lane
// l carrying row 16 * block + l % 16 and elements 16 (l / 16) + 8 h .. + 7 of
// the k-step (the fragment that lane feeds to v_mfma_f32_16x16x32_bf16).  A
// wave's load instruction then reads 1 KB of consecutive bytes, and a wave
// walks its block's k-steps through consecutive memory.  Values are the same,
// only their places change, so results are bit-identical to the row-major
// layout.
#include "kernels.hpp"

namespace moe {

namespace {

// One thread per 16-byte chunk of the tiled output of a [E, R, Kd] tensor.
__global__ __launch_bounds__(256) void pack_tiles_kernel(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst,
                                                         int R, int Kd, size_t nchunks) {
  const size_t c = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nchunks) return;
  const int lane = (int)(c & 63), h = (int)((c >> 6) & 1);
  const size_t unit = c >> 7;                    // (expert, block, k-step)
  const int nk = Kd / 64, nb = R / 16;
  const int ks = (int)(unit % nk);
  const size_t eb = unit / nk;
  const int blk = (int)(eb % nb);
  const size_t e = eb / nb;
  const int row = 16 * blk + (lane & 15);
  const int k = 64 * ks + 16 * (lane >> 4) + 8 * h;
  st16(dst + 8 * c, ld16(src + (e * R + row) * (size_t)Kd + k));
}

}  // namespace

hipError_t launch_pack_tiles(const bf16_t* src, bf16_t* dst, int E, int R, int Kd, hipStream_t s) {
  const size_t n = (size_t)E * R * Kd / 8;
  hipLaunchKernelGGL(pack_tiles_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, dst, R, Kd, n);
  return hipGetLastError();
}

}  // namespace moe
