// Router of the MoE layer on gfx950 (grouped path): logits = x W_r^T with bf16
// MFMA, then per token the top-K (descending logit, ties to the lower expert
// index), the softmax renormalised over the selected experts, the
// shared-expert gate scalar sigmoid(x . w_sg), and a per-block expert
// histogram that the dispatch step turns into segment offsets.
//
// Definition: "Qwen3.6-35B-A3B — Architecture Overview", section "MoE FFN: 256
// Experts" (router Linear 2048 -> 256, softmax, top-8, renormalise to sum 1;
// shared expert scaled by sigmoid(Linear(x, 1))); Linnet model page, Blocks:
// SparseMoe (gate: Linear<H, Experts>, shared_expert_gate: Linear<H, 1>, ranks).
//
// Softmax over all experts followed by renormalisation over the K selected is
// the same quantity as a softmax over the K selected logits alone (the full
// denominator cancels); the kernel computes the latter.
//
// Logits: one workgroup per (64-token tile, or 16- or 32-token tile for small
// batches and 128-token tile for large ones, slice of H); the shared gate row
// rides along as column E, so the E + 1 columns are 17 MFMA column blocks of
// 16.  Wave w of n owns column blocks w, w + n, ... (n = 4, or 8 for the
// LDS-staged kernel's 64- and 128-token tiles) and streams their router rows
// through registers in 64-wide k-steps (each row's whole 128-byte line per
// step), writing fp32 partial sums (one fp32 accumulator chain of at most
// H / 32 MFMAs per slice).  The tile's x rows go to LDS once per k-step and
// every wave reads them there (router_logits_lds_kernel, tiles of 32 tokens
// and more); 16-token tiles load them per wave (router_logits_kernel).  For
// large batches the router is read once per 64 or 128 tokens through L2.
// Small batches split H into up to H/64 slices so that the launch still spans
// the chip.
//
// Selection, two kernels.
// router_select_kernel (for the load-balance statistic, which needs its
// per-block probability sums): one workgroup of 16 waves per 32 tokens sums
// the slices in a fixed order and selects, two tokens per wave, and writes
// the block histograms of the multi-launch dispatch;
// everything else uses router_select_tok_kernel (one wave per token; block
// histograms by integer atomics where the dispatch needs them).
#include "kernels.hpp"
#include "lds_pipe.hpp"

namespace moe {

namespace {

constexpr int kTok = kRouterTokens;      // 32 tokens per select block
constexpr int kSmallT = 256;             // up to this many tokens: 32-token logits tiles, else 64
                                         // (up to 64 tokens: 16-token tiles, twice the workgroups on
                                         // the launch's short path; decode64 router 14.45 -> 14.1 us)
constexpr int kLargeT = 8192;            // from this many tokens: 128-token logits tiles (the router is
                                         // read half as often; zipf16384 router 90 -> 80 us, while at
                                         // 4096 tokens the extra H slices cost more than that saves)
constexpr int kColBlocks = 5;            // column blocks per wave of four (17 for E = 256, plus the gate column)
constexpr int kMaxSub = 17;              // column blocks of 16 for E <= 256 plus the gate column
constexpr int kDepth = 2;                // 64-wide k-steps in flight per wave (router_logits_kernel)
constexpr int kMaxRouterCols = 260;      // router_cols(256)

// kTB 16-token blocks per workgroup.
template <int kTB>
__global__ __launch_bounds__(256) void router_logits_kernel(LayerArgs L, const bf16_t* __restrict__ x, int T,
                                                            int ksplit, float* __restrict__ part,
                                                            int* __restrict__ hist_zero, int hist_n,
                                                            uint32_t* __restrict__ ctl, uint32_t tag) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // The call's tag goes into the workspace's latest-call word (this path has
  // no waits, so the call never matches the error word).
  if (ctl && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) ctl[kCtlLast] = tag;
  // The selection adds its pairs to these block histograms (integer atomics):
  // they start at zero.
  if (hist_zero) {
    const int nwg = gridDim.x * gridDim.y, wg = blockIdx.y * gridDim.x + blockIdx.x;
    for (int i = wg * 256 + tid; i < hist_n; i += nwg * 256) hist_zero[i] = 0;
  }
  const int t0 = blockIdx.x * 16 * kTB, s = blockIdx.y;
  const int H = L.H, E = L.E, Ep = router_cols(E);
  const int nsub = (E + 1 + 15) >> 4;               // column blocks incl. the gate column
  // k advances 64 at a time; lane quarter q (lane / 16) covers elements
  // 16 q .. 16 q + 15 of the step with two consecutive 16-byte loads (MFMA
  // halves 0 and 1), the same order for both operands, so each row's whole
  // 128-byte line is requested at once.
  const int r16 = lane & 15, kq = (lane >> 4) * 16;
  const int klen = H / ksplit, kbeg = s * klen, nk = klen / 64;

  // Operand rows of this lane: x rows of the 16-token blocks, weight rows of
  // the wave's column blocks (rows past T or E + 1 repeat a valid row and
  // their outputs are dropped).
  const bf16_t* arow[kTB];
#pragma unroll
  for (int i = 0; i < kTB; ++i) arow[i] = x + (size_t)min(t0 + 16 * i + r16, T - 1) * H + kbeg + kq;
  const bf16_t* brow[kColBlocks];
#pragma unroll
  for (int jj = 0; jj < kColBlocks; ++jj) {
    const int e = min(16 * (wave + 4 * jj) + r16, E);
    brow[jj] = (e < E ? L.router_w + (size_t)e * H : L.sh_expert_gate) + kbeg + kq;
  }
  f32x4 acc[kTB][kColBlocks];
#pragma unroll
  for (int i = 0; i < kTB; ++i)
#pragma unroll
    for (int jj = 0; jj < kColBlocks; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Ring of kDepth 64-wide k-steps; loads of k-steps past the slice repeat
  // its last step (always in bounds) and are not used.
  u32x4 ra[kDepth][kTB][2], rb[kDepth][kColBlocks][2];
  auto issue = [&](int st, int ks) {
    const int k = 64 * min(ks, nk - 1);
#pragma unroll
    for (int i = 0; i < kTB; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) ra[st][i][h] = ld16(arow[i] + k + 8 * h);
#pragma unroll
    for (int jj = 0; jj < kColBlocks; ++jj)
#pragma unroll
      for (int h = 0; h < 2; ++h) rb[st][jj][h] = ld16(brow[jj] + k + 8 * h);
  };
#pragma unroll
  for (int st = 0; st < kDepth; ++st) issue(st, st);
  for (int k0 = 0; k0 < nk; k0 += kDepth) {
#pragma unroll
    for (int st = 0; st < kDepth; ++st) {
      const int ks = k0 + st;
      if (ks < nk) {
#pragma unroll
        for (int jj = 0; jj < kColBlocks; ++jj) {
          if (wave + 4 * jj < nsub) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int i = 0; i < kTB; ++i)
                acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ra[st][i][h]),
                                                                     as_bf16x8(rb[st][jj][h]), acc[i][jj], 0, 0, 0);
          }
        }
      }
      issue(st, ks + kDepth);
    }
  }
  // D[4 (lane / 16) + r][lane % 16] of each 16 x 16 block.
  float* out = part + (size_t)s * T * Ep;
#pragma unroll
  for (int jj = 0; jj < kColBlocks; ++jj) {
    const int e = 16 * (wave + 4 * jj) + r16;
    if (wave + 4 * jj < nsub && e <= E) {
#pragma unroll
      for (int i = 0; i < kTB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + 16 * i + 4 * (lane >> 4) + r;
          if (t < T) out[(size_t)t * Ep + e] = acc[i][jj][r];
        }
    }
  }
}

// The same logits for tiles of 32, 64 or 128 tokens, with the tile's x rows
// staged in LDS: each 64-wide k-step of them goes to LDS once by direct-to-LDS
// loads (a four-stage ring, three steps in flight, the row swizzle of the
// grouped GEMMs) and every wave reads its MFMA operands from there, while its
// router rows stream through registers.  Where each wave loaded the x rows
// itself, the four waves' copies met only in the 32 KB L1 (a deeper register
// ring was slower: zipf16384 router 78 -> 87 us).  Per accumulator the MFMAs
// run in the same k order, so the sums are the same.
//
// Waves per workgroup of the LDS-staged logits kernel: eight for 64- and
// 128-token tiles (two per SIMD, each with at most three column blocks;
// 200 registers instead of 304 at 64 tokens, prefill4096 router phase
// 28.0-28.4 -> 27.0-27.9 us; 252 instead of 420 at 128 tokens, with one
// operand array for both k halves, zipf16384 58.1-59.0 -> 52.9-54.0 us),
// four for 32-token tiles (which give eight waves no whole direct-to-LDS
// load per step).
constexpr int router_lds_waves(int tb) { return tb >= 4 ? 8 : 4; }

template <int kTB, int kNW = router_lds_waves(kTB)>
__global__ __launch_bounds__(64 * kNW, 1) void router_logits_lds_kernel(LayerArgs L, const bf16_t* __restrict__ x, int T,
                                                                  int ksplit, float* __restrict__ part,
                                                                  int* __restrict__ hist_zero, int hist_n,
                                                                  uint32_t* __restrict__ ctl, uint32_t tag) {
  using namespace pipe;
  constexpr int NS = 4;
  constexpr int kRows = 16 * kTB, kStage = kRows * 128;
  constexpr int kCB = (kMaxSub + kNW - 1) / kNW;     // column blocks per wave
  constexpr int kDma = kRows * 8 / (64 * kNW);       // direct-to-LDS instructions per wave per step
  constexpr int kVm = kDma + 2 * kCB;                // loads per wave per step
  static_assert(kDma >= 1 && 3 * kVm <= 63, "x rows and router rows per step");
  __shared__ __attribute__((aligned(1024))) char lds[NS * kStage];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (ctl && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) ctl[kCtlLast] = tag;
  if (hist_zero) {
    const int nwg = gridDim.x * gridDim.y, wg = blockIdx.y * gridDim.x + blockIdx.x;
    for (int i = wg * (64 * kNW) + tid; i < hist_n; i += nwg * (64 * kNW)) hist_zero[i] = 0;
  }
  const int t0 = blockIdx.x * kRows, s = blockIdx.y;
  const int H = L.H, E = L.E, Ep = router_cols(E);
  const int nsub = (E + 1 + 15) >> 4;
  const int wv = uni(wave);
  const int r16 = lane & 15, q = lane >> 4;
  const int klen = H / ksplit, kbeg = s * klen, nk = klen / 64;
  const int nsteps = ((nk + NS - 1) / NS) * NS;     // padded to the ring; padding steps add nothing
  const uint32_t lds_base = (uint32_t)(size_t)(lds_ptr_t)lds;

  // x rows: instruction j of wave w writes row 8 (kNW j + w) + lane / 8 of a
  // stage, stored chunk lane % 8 holding chunk (lane % 8) ^ swz(row); rows
  // past T repeat row T - 1 (their outputs are dropped).
  const bf16_t* a_src[kDma];
#pragma unroll
  for (int j = 0; j < kDma; ++j) {
    const int r = 8 * (kNW * j + wv) + (lane >> 3);
    a_src[j] = x + (size_t)min(t0 + r, T - 1) * H + kbeg + ((lane & 7) ^ lds_swizzle(r)) * 8;
  }
  // Router rows of the wave's column blocks wave + kNW jj (rows past E + 1
  // repeat row E; blocks past the last are loaded, not used, so every wave
  // issues the same loads); lane quarter q reads elements 16 q .. 16 q + 15.
  const bf16_t* brow[kCB];
#pragma unroll
  for (int jj = 0; jj < kCB; ++jj) {
    const int e = min(16 * (wv + kNW * jj) + r16, E);
    brow[jj] = (e < E ? L.router_w + (size_t)e * H : L.sh_expert_gate) + kbeg + 16 * q;
  }
  u32x4 wb[NS][kCB][2];
  auto issue = [&](u32x4 (&wbs)[kCB][2], int st, int ks) {
    const int kv = min(ks, nk - 1);
#pragma unroll
    for (int j = 0; j < kDma; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(a_src[j] + 64 * kv), (lds_ptr_t)(lds + st * kStage + 1024 * (kNW * j + wv)),
                                       16, 0, 0);
#pragma unroll
    for (int jj = 0; jj < kCB; ++jj)
#pragma unroll
      for (int h = 0; h < 2; ++h) wbs[jj][h] = ld16(brow[jj] + 64 * kv + 8 * h);
  };
  f32x4 acc[kTB][kCB];
#pragma unroll
  for (int i = 0; i < kTB; ++i)
#pragma unroll
    for (int jj = 0; jj < kCB; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(wb[0], 0, 0);
  issue(wb[1], 1, 1);
  issue(wb[2], 2, 2);
  // One k-step (YOUNGER: steps already requested after this one; ISSUE:
  // whether it requests step ks + 3), as in grouped_gemm_kernel.
  auto step = [&](auto younger_c, auto issue_c, u32x4 (&wcur)[kCB][2], u32x4 (&wnext)[kCB][2], int st,
                  int ks) {
    wait_vm<decltype(younger_c)::value * kVm>();
    barrier();
    if constexpr (decltype(issue_c)::value) issue(wnext, (st + 3) % NS, ks + 3);
    if (ks < nk) {
      const uint32_t sa0 = lds_base + st * kStage + r16 * 128 + (((2 * q) ^ lds_swizzle(r16)) << 4);
      const uint32_t sa1 = lds_base + st * kStage + r16 * 128 + (((2 * q + 1) ^ lds_swizzle(r16)) << 4);
      if constexpr (kNW == 8 && kTB == 8) {
        // One operand array for both k halves (two waves per SIMD cover the
        // reads' latency; a second array would not fit in 256 registers).
        u32x4 X[kTB];
        lds_read_group<0>(X, sa0, std::make_integer_sequence<int, kTB>{});
        wait_lds_keep<0>(X);
#pragma unroll
        for (int jj = 0; jj < kCB; ++jj)
          if (wv + kNW * jj < nsub)
#pragma unroll
            for (int i = 0; i < kTB; ++i) acc[i][jj] = mfma16(X[i], wcur[jj][0], acc[i][jj]);
        lds_read_group<0>(X, sa1, std::make_integer_sequence<int, kTB>{});
        wait_lds_keep<0>(X);
#pragma unroll
        for (int jj = 0; jj < kCB; ++jj)
          if (wv + kNW * jj < nsub)
#pragma unroll
            for (int i = 0; i < kTB; ++i) acc[i][jj] = mfma16(X[i], wcur[jj][1], acc[i][jj]);
      } else {
        u32x4 X[kTB], Y[kTB];
        lds_read_group<0>(X, sa0, std::make_integer_sequence<int, kTB>{});
        lds_read_group<0>(Y, sa1, std::make_integer_sequence<int, kTB>{});
        wait_lds_keep<kTB>(X);
#pragma unroll
        for (int jj = 0; jj < kCB; ++jj)
          if (wv + kNW * jj < nsub)
#pragma unroll
            for (int i = 0; i < kTB; ++i) acc[i][jj] = mfma16(X[i], wcur[jj][0], acc[i][jj]);
        wait_lds_keep<0>(Y);
#pragma unroll
        for (int jj = 0; jj < kCB; ++jj)
          if (wv + kNW * jj < nsub)
#pragma unroll
            for (int i = 0; i < kTB; ++i) acc[i][jj] = mfma16(Y[i], wcur[jj][1], acc[i][jj]);
      }
    }
  };
  using c0 = std::integral_constant<int, 0>;
  using c1 = std::integral_constant<int, 1>;
  using c2 = std::integral_constant<int, 2>;
  using yes = std::true_type;
  using no = std::false_type;
  int k4 = 0;
  for (; k4 + NS < nsteps; k4 += NS) {
    step(c2{}, yes{}, wb[0], wb[3], 0, k4);
    step(c2{}, yes{}, wb[1], wb[0], 1, k4 + 1);
    step(c2{}, yes{}, wb[2], wb[1], 2, k4 + 2);
    step(c2{}, yes{}, wb[3], wb[2], 3, k4 + 3);
  }
  step(c2{}, yes{}, wb[0], wb[3], 0, k4);
  step(c2{}, no{}, wb[1], wb[0], 1, k4 + 1);
  step(c1{}, no{}, wb[2], wb[1], 2, k4 + 2);
  step(c0{}, no{}, wb[3], wb[2], 3, k4 + 3);

  // D[4 (lane / 16) + r][lane % 16] of each 16 x 16 block.
  float* out = part + (size_t)s * T * Ep;
#pragma unroll
  for (int jj = 0; jj < kCB; ++jj) {
    const int e = 16 * (wv + kNW * jj) + r16;
    if (wv + kNW * jj < nsub && e <= E) {
#pragma unroll
      for (int i = 0; i < kTB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + 16 * i + 4 * q + r;
          if (t < T) out[(size_t)t * Ep + e] = acc[i][jj][r];
        }
    }
  }
}

// One workgroup of 16 waves per 32 tokens.  First all threads sum the slices
// of the tile's partial rows in a fixed order (every slice of an item in
// flight at once) into LDS; then each wave selects for two tokens: top-K,
// weights, gate, block histogram.
constexpr int kSelWaves = 16;
constexpr int kMaxSlices = 16;
static_assert(kSelWaves * 2 == kTok, "two tokens per wave");

__global__ __launch_bounds__(kSelWaves * 64) void router_select_kernel(LayerArgs L, int T, int ksplit,
                                                                      const float* __restrict__ part, Work w,
                                                                      float* __restrict__ logits_out,
                                                                      float* __restrict__ psum_out) {
  __shared__ __attribute__((aligned(16))) float s_lg[kTok][kMaxRouterCols];
  __shared__ int hist[256];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int E = L.E, K = L.K, Ep = router_cols(E), c4n = Ep / 4;
  const int t0 = blockIdx.x * kTok;
  if (tid < 256) hist[tid] = 0;
  for (int idx = tid; idx < kTok * c4n; idx += kSelWaves * 64) {
    const int tl = idx / c4n, c4 = idx - tl * c4n;
    const float* src = part + (size_t)min(t0 + tl, T - 1) * Ep + 4 * c4;
    u32x4 q[kMaxSlices];
#pragma unroll
    for (int i = 0; i < kMaxSlices; ++i)
      if (i < ksplit) q[i] = ld16(src + (size_t)i * T * Ep);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kMaxSlices; ++i)
      if (i < ksplit)
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] += __uint_as_float(q[i][c]);
    *reinterpret_cast<f32x4*>(&s_lg[tl][4 * c4]) = v;
  }
  __syncthreads();
  float lv[2][4];
  int tt[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tl = 2 * wave + j;
    tt[j] = t0 + tl;
    // Columns 4 lane .. 4 lane + 3; past E they are outside the top-K's valid
    // range (reads stay inside the padded row).
#pragma unroll
    for (int c = 0; c < 4; ++c) lv[j][c] = s_lg[tl][min(4 * lane + c, kMaxRouterCols - 1)];
    float zg = s_lg[tl][E];
    if (L.logits_bf16) {
      // Scores typed bf16: everything below (ranking, softmax, the gate, the
      // logits written out) sees the rounded values.
#pragma unroll
      for (int c = 0; c < 4; ++c) lv[j][c] = round_bf16(lv[j][c]);
      zg = round_bf16(zg);
    }
    if (tt[j] < T && lane == 0) w.gate_s[tt[j]] = sigmoidf_(zg);
    if (logits_out && tt[j] < T) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (4 * lane + c < E) logits_out[(size_t)tt[j] * E + 4 * lane + c] = lv[j][c];
    }
  }
  int ix[2];
  float wv[2];
  topk_select<2>(lv, E, K, lane, ix, wv);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (tt[j] < T && lane < K) {
      w.topk_idx[(size_t)tt[j] * K + lane] = ix[j];
      w.topk_w[(size_t)tt[j] * K + lane] = wv[j];
      atomicAdd(&hist[ix[j]], 1);
    }
  }
  if (psum_out) {
    // Load-balance input: each token's full softmax over the E experts
    // (written over its logits in LDS), then per expert the sum over the
    // block's tokens in token order.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t mk = 0u;
#pragma unroll
      for (int c = 0; c < 4; ++c) mk = max(mk, 4 * lane + c < E ? logit_key(lv[j][c]) : 0u);
      const float mx = key_logit(wave_max_u32(mk));
      float z[4], zs = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        z[c] = 4 * lane + c < E ? __expf(lv[j][c] - mx) : 0.f;
        zs += z[c];
      }
      const float inv = 1.0f / wave_sum_f32(zs);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (4 * lane + c < E) s_lg[2 * wave + j][4 * lane + c] = z[c] * inv;
    }
  }
  __syncthreads();
  if (tid < E) w.blk_counts[(size_t)blockIdx.x * E + tid] = hist[tid];
  if (psum_out && tid < E) {
    float acc = 0.f;
    const int nt = min(kTok, T - t0);
    for (int tl = 0; tl < nt; ++tl) acc += s_lg[tl][tid];
    psum_out[(size_t)blockIdx.x * E + tid] = acc;
  }
}

// The selection spread over the chip: one wave per token, four tokens per
// workgroup.  Lane l holds columns 4 l .. 4 l + 3 (the top-K's layout),
// summed over the slices in the same order as router_select_kernel, so the
// results are the same bit for bit.  For the multi-launch dispatch
// (block_hist) each selected pair is counted into its router block's
// histogram, which the logits kernel zeroed.
// kS: an upper bound of ksplit (the slice registers are sized by it).
template <int kS>
__global__ __launch_bounds__(256) void router_select_tok_kernel(LayerArgs L, int T, int ksplit,
                                                                const float* __restrict__ part, Work w,
                                                                float* __restrict__ logits_out, int block_hist) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;   // the whole wave; no barrier below
  const int E = L.E, K = L.K, Ep = router_cols(E);
  const float* src = part + (size_t)t * Ep;
  const size_t sstride = (size_t)T * Ep;
  const bool have = 4 * lane < Ep;
  u32x4 q[kS];
  float g[kS];
#pragma unroll
  for (int i = 0; i < kS; ++i)
    if (i < ksplit) {
      q[i] = have ? ld16(src + i * sstride + 4 * lane) : u32x4{0u, 0u, 0u, 0u};
      g[i] = src[i * sstride + E];
    }
  float lv[1][4] = {{0.f, 0.f, 0.f, 0.f}};
  float zg = 0.f;
#pragma unroll
  for (int i = 0; i < kS; ++i)
    if (i < ksplit) {
#pragma unroll
      for (int c = 0; c < 4; ++c) lv[0][c] += __uint_as_float(q[i][c]);
      zg += g[i];
    }
  if (L.logits_bf16) {
#pragma unroll
    for (int c = 0; c < 4; ++c) lv[0][c] = round_bf16(lv[0][c]);
    zg = round_bf16(zg);
  }
  if (lane == 0) w.gate_s[t] = sigmoidf_(zg);
  if (logits_out) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (4 * lane + c < E) logits_out[(size_t)t * E + 4 * lane + c] = lv[0][c];
  }
  int ix[1];
  float wv[1];
  topk_select<1>(lv, E, K, lane, ix, wv);
  if (lane < K) {
    w.topk_idx[(size_t)t * K + lane] = ix[0];
    w.topk_w[(size_t)t * K + lane] = wv[0];
    // The multi-launch dispatch takes per-block expert histograms; integer
    // sums do not depend on the order of the additions.
    if (block_hist) atomicAdd(&w.blk_counts[(size_t)(t / kTok) * E + ix[0]], 1);
  }
}

// Full stable ranking of each row's scores: rank[e] = the number of experts
// that score higher, plus those that score the same with a lower index.  One
// wave per row.  Each expert gets the 64-bit key (order-preserving score key,
// then the complement of its index), so "ahead of e" is one unsigned compare;
// the row's keys go to LDS (padded to a multiple of 2 with key 0, which no
// score maps to: NaN takes -inf's key), and each lane counts, for its experts
// e = lane + 64 i, the keys above theirs (every lane reads the same words at
// a time: broadcasts).  E^2 compares per row: the kernel is ALU-bound.
constexpr int kRankRows = 4;

__global__ __launch_bounds__(64 * kRankRows) void ranks_kernel(const void* __restrict__ logits, int dtype, int R,
                                                              int E, int32_t* __restrict__ ranks) {
  __shared__ __attribute__((aligned(16))) uint64_t s_key[kRankRows][256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * kRankRows + wave;
  const bool row_ok = r < R;
  uint64_t mine[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    uint64_t k = 0u;
    if (row_ok && e < E) {
      const size_t o = (size_t)r * E + e;
      const float v = dtype ? bf16_to_f32(static_cast<const bf16_t*>(logits)[o])
                            : static_cast<const float*>(logits)[o];
      k = ((uint64_t)logit_key(v) << 32) | (uint32_t)(0xFFFFu - e);
    }
    s_key[wave][e] = k;   // e < 256: the whole padded row is written
    mine[i] = k;
  }
  __syncthreads();
  if (!row_ok) return;
  int cnt[4] = {0, 0, 0, 0};
  const int E2 = (E + 1) & ~1;
#pragma unroll 4
  for (int j0 = 0; j0 < E2; j0 += 2) {
    const uint64_t k0 = s_key[wave][j0], k1 = s_key[wave][j0 + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) cnt[i] += (int)(k0 > mine[i]) + (int)(k1 > mine[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (lane + 64 * i < E) ranks[(size_t)r * E + lane + 64 * i] = cnt[i];
}

// Load-balance statistic, one workgroup of 1024 threads: per expert, four
// threads sum the block probability sums of four contiguous block ranges
// (eight loads in flight each), the ranges are added in order, the pair count
// comes from the segment offsets; lb = E * sum_e (count_e / (T K)) *
// (psum_e / T), summed in double over the experts in a fixed tree order.
__global__ __launch_bounds__(1024) void load_balance_kernel(LayerArgs L, int T, Work w, float* __restrict__ lb,
                                                            float* __restrict__ mean_prob,
                                                            int32_t* __restrict__ counts) {
  __shared__ float s_part[4][256];
  __shared__ double s_term[256];
  const int tid = threadIdx.x, e = tid & 255, part = tid >> 8, E = L.E, K = L.K;
  const int nblk = router_blocks(T);
  const int per = (nblk + 3) >> 2, b0 = part * per, b1 = min(nblk, b0 + per);
  float ps = 0.f;
  if (e < E) {
    for (int b = b0; b < b1; b += 8) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = b + i < b1 ? w.psum[(size_t)(b + i) * E + e] : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ps += v[i];
    }
  }
  s_part[part][e] = ps;
  __syncthreads();
  if (tid < 256) {
    double term = 0.0;
    if (e < E) {
      const float tot = (s_part[0][e] + s_part[1][e]) + (s_part[2][e] + s_part[3][e]);
      const int cnt = w.offsets[e + 1] - w.offsets[e];
      if (mean_prob) mean_prob[e] = tot / (float)T;
      if (counts) counts[e] = cnt;
      term = (double)cnt * (double)tot;
    }
    s_term[e] = term;
  }
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) s_term[tid] += s_term[tid + o];
    __syncthreads();
  }
  if (tid == 0) *lb = (float)(s_term[0] * (double)E / ((double)T * K * (double)T));
}

}  // namespace

static int logits_tile(int T) { return T <= 64 ? 16 : (T <= kSmallT ? 32 : (T >= kLargeT ? 128 : 64)); }

int router_ksplit(int T, int H) {
  const int ntiles = (T + logits_tile(T) - 1) / logits_tile(T);
  int s = 1;
  while (2 * s <= H / 64 && 2 * s <= 16 && ntiles * s < 256) s *= 2;
  return s;
}

// Rows of partial sums the logits kernel writes is ksplit(T) * T.  Upper
// bound over every batch of at most T tokens (workspace sizing, which must
// not shrink as T grows): ksplit <= min(16, H / 64), and when ksplit >= 2 it
// was doubled from a value whose product with the tile count was below 256,
// so ksplit * T < 512 * tile(T); every term is non-decreasing in T.
int64_t router_partial_rows(int64_t T, int H) {
  const int64_t cap = std::min(16, H / 64);
  return std::max<int64_t>(T, std::min<int64_t>(cap * T, 512 * (int64_t)logits_tile((int)T)));
}

hipError_t launch_router(const LayerArgs& L, const bf16_t* x, int T, const Work& w,
                         float* logits_out, hipStream_t s, float* psum_out) {
  const int ks = router_ksplit(T, L.H), tile = logits_tile(T);
  const dim3 grid((T + tile - 1) / tile, ks);
  // Per-token selection unless the load-balance statistic's block sums are
  // wanted; its block histograms (multi-launch dispatch only) start at zero.
  const bool per_token = psum_out == nullptr;
  const bool block_hist = per_token && !dispatch_single_block(T);
  int* hz = block_hist ? w.blk_counts : nullptr;
  const int hn = router_blocks(T) * L.E;
  if (tile == 16)
    hipLaunchKernelGGL(router_logits_kernel<1>, grid, dim3(256), 0, s, L, x, T, ks, w.rlog, hz, hn, w.ctl,
                       w.call_tag);
  else if (tile == 32)
    hipLaunchKernelGGL(router_logits_lds_kernel<2>, grid, dim3(64 * router_lds_waves(2)), 0, s, L, x, T, ks, w.rlog, hz, hn, w.ctl,
                       w.call_tag);
  else if (tile == 64)
    hipLaunchKernelGGL(router_logits_lds_kernel<4>, grid, dim3(64 * router_lds_waves(4)), 0, s, L, x, T, ks, w.rlog, hz, hn, w.ctl,
                       w.call_tag);
  else
    hipLaunchKernelGGL(router_logits_lds_kernel<8>, grid, dim3(64 * router_lds_waves(8)), 0, s, L, x, T, ks, w.rlog, hz, hn, w.ctl,
                       w.call_tag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (per_token) {
    // The slice registers sized for the split in use: fewer registers, more
    // waves per SIMD (two slices: 18 VGPRs instead of 90, zipf16384 router
    // phase 52.7-54.0 -> 50.9-52.2 us; four: 60).
    auto k = ks <= 2 ? router_select_tok_kernel<2> : ks <= 4 ? router_select_tok_kernel<4> : router_select_tok_kernel<kMaxSlices>;
    hipLaunchKernelGGL(k, dim3((T + 3) / 4), dim3(256), 0, s, L, T, ks, (const float*)w.rlog, w, logits_out,
                       block_hist ? 1 : 0);
  }
  else
    hipLaunchKernelGGL(router_select_kernel, dim3(router_blocks(T)), dim3(kSelWaves * 64), 0, s, L, T, ks,
                       (const float*)w.rlog, w, logits_out, psum_out);
  return hipGetLastError();
}

hipError_t launch_ranks(const void* logits, int dtype, int R, int E, int32_t* ranks, hipStream_t s) {
  hipLaunchKernelGGL(ranks_kernel, dim3((R + kRankRows - 1) / kRankRows), dim3(64 * kRankRows), 0, s, logits, dtype,
                     R, E, ranks);
  return hipGetLastError();
}

hipError_t launch_load_balance(const LayerArgs& L, int T, const Work& w, float* lb, float* mean_prob,
                               int32_t* counts, hipStream_t s) {
  hipLaunchKernelGGL(load_balance_kernel, dim3(1), dim3(1024), 0, s, L, T, w, lb, mean_prob, counts);
  return hipGetLastError();
}

}  // namespace moe
