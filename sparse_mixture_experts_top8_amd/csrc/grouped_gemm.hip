// Grouped expert GEMMs on gfx950 MFMA (v_mfma_f32_32x32x16_bf16), one group
// per routed expert plus one for the shared expert (group E, all T tokens).
//
//  gate_up:  for the rows of group g (gathered x rows of its tokens)
//            G = A Wg^T, U = A Wu^T,  h = SiLU(G) * U  -> bf16
//  down:     Y = h Wd^T, scaled in the epilogue by the routing weight of the
//            row (shared rows: by sigmoid(x . w_sg)) -> bf16 per row
//
// Definition: "Qwen3.6-35B-A3B — Architecture Overview", section "MoE FFN: 256
// Experts" (expert_e(x) = SiLU(x W_gate_e) * (x W_up_e) W_down_e, gate and up
// merged as [256, 1024, 2048]; shared expert of the same form, scaled by
// sigmoid(Linear(x, 1))); Linnet model page, Blocks: SparseMoe
// (gate_up_proj [E, 2I, H], down_proj [E, H, I]) and SwiGlu.
//
// Both operands are K-contiguous (activation rows, and weights stored
// [Out, In]), so every 16-byte load feeds eight MFMA k-elements directly.
// Tiles: 64 rows x 128 weight rows (gate_up: 64 gate + 64 up columns of the
// same inner range; down: 128 output columns), 64-deep k steps staged
// through LDS with the next step prefetched into registers.
//
// Scheduling: a persistent grid whose size is a multiple of 8.  Workgroups are
// handed to the eight XCDs round-robin, so workgroup i runs on XCD i % 8; the
// tile list is cut into eight contiguous ranges and XCD x walks range x.
// Neighbouring tiles share a weight slab (row tiles of one column tile) or an
// activation block (column tiles of one row tile), and these then meet in the
// same 4 MB L2.
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int BM = kGemmBM;     // 64 rows
constexpr int BNW = kGemmBNW;   // 128 weight rows
constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements; +16 B breaks the 128 B row period

__device__ __forceinline__ int find_group(const int* __restrict__ prefix, int E, int t) {
  // Largest g in [0, E] with prefix[g] <= t (prefix is non-decreasing, prefix[0] = 0).
  int lo = 0, hi = E;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <bool GATE_UP>
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(LayerArgs L, const bf16_t* __restrict__ x,
                                                             int T, Work w) {
  __shared__ __attribute__((aligned(16))) bf16_t As[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[BNW * LDS_STRIDE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int E = L.E, K = L.K, H = L.H;
  const int* __restrict__ prefix = GATE_UP ? w.tiles_gu : w.tiles_dn;
  const int ntiles = prefix[E + 1];

  const int per_xcd = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, slot_in_xcd = blockIdx.x >> 3;
  const int chunk = (ntiles + 7) >> 3;
  const int t_end = min(ntiles, (xcd + 1) * chunk);

  for (int tile = xcd * chunk + slot_in_xcd; tile < t_end; tile += per_xcd) {
    const int g = find_group(prefix, E, tile);
    const bool shared = (g == E);
    const int seg0 = shared ? 0 : w.offsets[g];
    const int nrows = shared ? T : (w.offsets[g + 1] - seg0);
    const int mt = (nrows + BM - 1) / BM;
    const int local = tile - prefix[g];
    const int m0 = (local % mt) * BM;
    const int nt = local / mt;
    const int inner = shared ? L.Is : L.I;
    const int kdim = GATE_UP ? H : inner;

    // ---- per-thread source rows: 2 A chunks and 4 B chunks of 16 B per k step ----
    const bf16_t* a_src[2];
    bool a_ok[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 3, col = (c & 7) * 8;
      const int row = m0 + r;
      a_ok[i] = row < nrows;
      const int rr = a_ok[i] ? row : 0;
      if (GATE_UP) {
        const int tok = shared ? rr : (w.perm[seg0 + rr] / K);
        a_src[i] = x + (size_t)tok * H + col;
      } else {
        a_src[i] = shared ? (w.h_sh + (size_t)rr * L.Is + col) : (w.h + (size_t)(seg0 + rr) * L.I + col);
      }
    }
    const bf16_t* b_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 3, col = (c & 7) * 8;
      if (GATE_UP) {
        // r < 64: gate row nt*64 + r; r >= 64: up row nt*64 + r - 64.
        const int inner_row = nt * 64 + (r & 63);
        if (shared)
          b_src[i] = (r < 64 ? L.sh_gate_w : L.sh_up_w) + (size_t)inner_row * H + col;
        else
          b_src[i] = L.gate_up_w + ((size_t)g * 2 * L.I + (r < 64 ? 0 : L.I) + inner_row) * H + col;
      } else {
        const int n = nt * BNW + r;
        b_src[i] = shared ? (L.sh_down_w + (size_t)n * L.Is + col)
                          : (L.down_w + ((size_t)g * H + n) * L.I + col);
      }
    }

    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    u32x4 ra[2], rb[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) ra[i] = a_ok[i] ? ld16(a_src[i]) : zero4;
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[i] = ld16(b_src[i]);

    f32x16 acc0, acc1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { acc0[r] = 0.f; acc1[r] = 0.f; }

    // MFMA operand rows of this wave inside the tile.
    const int a_row = 32 * wm + (lane & 31);
    const int b_row0 = GATE_UP ? (32 * wn + (lane & 31)) : (64 * wn + (lane & 31));
    const int b_row1 = GATE_UP ? (64 + 32 * wn + (lane & 31)) : (64 * wn + 32 + (lane & 31));
    const int kofs = 8 * (lane >> 5);

    for (int k0 = 0; k0 < kdim; k0 += BK) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i;
        *reinterpret_cast<u32x4*>(&As[(c >> 3) * LDS_STRIDE + (c & 7) * 8]) = ra[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i;
        *reinterpret_cast<u32x4*>(&Bs[(c >> 3) * LDS_STRIDE + (c & 7) * 8]) = rb[i];
      }
      __syncthreads();
      if (k0 + BK < kdim) {
#pragma unroll
        for (int i = 0; i < 2; ++i) ra[i] = a_ok[i] ? ld16(a_src[i] + k0 + BK) : zero4;
#pragma unroll
        for (int i = 0; i < 4; ++i) rb[i] = ld16(b_src[i] + k0 + BK);
      }
#pragma unroll
      for (int kk = 0; kk < BK; kk += 16) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(&As[a_row * LDS_STRIDE + kk + kofs]));
        const bf16x8 b0 = as_bf16x8(*reinterpret_cast<const u32x4*>(&Bs[b_row0 * LDS_STRIDE + kk + kofs]));
        const bf16x8 b1 = as_bf16x8(*reinterpret_cast<const u32x4*>(&Bs[b_row1 * LDS_STRIDE + kk + kofs]));
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc1, 0, 0, 0);
      }
      __syncthreads();
    }

    // ---- epilogue: D[8*(r/4) + 4*(lane/32) + r%4][lane%32] ----
    const int col = lane & 31;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + 32 * wm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= nrows) continue;
      if (GATE_UP) {
        const float hv = siluf_(acc0[r]) * acc1[r];
        const int icol = nt * 64 + 32 * wn + col;
        bf16_t* dst = shared ? (w.h_sh + (size_t)row * L.Is) : (w.h + (size_t)(seg0 + row) * L.I);
        dst[icol] = (bf16_t)f32_to_bf16(hv);
      } else {
        float scale;
        size_t yrow;
        if (shared) {
          scale = w.gate_s[row];
          yrow = (size_t)T * K + row;
        } else {
          scale = w.topk_w[w.perm[seg0 + row]];
          yrow = (size_t)(seg0 + row);
        }
        bf16_t* dst = w.y + yrow * H + nt * BNW + 64 * wn + col;
        dst[0] = (bf16_t)f32_to_bf16(scale * acc0[r]);
        dst[32] = (bf16_t)f32_to_bf16(scale * acc1[r]);
      }
    }
  }
}

// out[t] = bf16( sum_k y[slot_of(t, k)] + y[T*K + t] ), k in order, fp32 sum.
__global__ __launch_bounds__(256) void combine_kernel(int T, int H, int K, Work w, bf16_t* __restrict__ out) {
  const int per_tok = H >> 3;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)T * per_tok) return;
  const int t = (int)(idx / per_tok), c = (int)(idx % per_tok) * 8;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (int k = 0; k <= K; ++k) {
    const size_t row = k < K ? (size_t)w.slot_of[(size_t)t * K + k] : (size_t)T * K + t;
    const u32x4 v = ld16(w.y + row * H + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += bf16_to_f32(v[j] & 0xFFFFu);
      acc[2 * j + 1] += bf16_to_f32(v[j] >> 16);
    }
  }
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
  st16(out + (size_t)t * H + c, o);
}

int persistent_grid(int num_cus) {
  int g = num_cus * 2;
  return ((g + 7) / 8) * 8;
}

}  // namespace

hipError_t launch_gate_up(const LayerArgs& L, const bf16_t* x, int T, const Work& w, int num_cus,
                          hipStream_t s) {
  hipLaunchKernelGGL(grouped_gemm_kernel<true>, dim3(persistent_grid(num_cus)), dim3(256), 0, s, L, x, T, w);
  return hipGetLastError();
}

hipError_t launch_down(const LayerArgs& L, int T, const Work& w, int num_cus, hipStream_t s) {
  hipLaunchKernelGGL(grouped_gemm_kernel<false>, dim3(persistent_grid(num_cus)), dim3(256), 0, s, L,
                     (const bf16_t*)nullptr, T, w);
  return hipGetLastError();
}

hipError_t launch_combine(const LayerArgs& L, int T, const Work& w, bf16_t* out, hipStream_t s) {
  const size_t n = (size_t)T * (L.H / 8);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, T, L.H, L.K, w, out);
  return hipGetLastError();
}

}  // namespace moe
