// Fused route of the MoE layer for small grouped batches (T <= kRouteMaxT
// tokens) on gfx950: router logits, top-K selection and dispatch in one
// launch.  Separately they are three short launches (logits over H slices,
// selection, per-group dispatch), each mostly latency at these sizes.
//
// Definition: "Qwen3.6-35B-A3B — Architecture Overview", section "MoE FFN: 256
// Experts" (router Linear 2048 -> 256, softmax, top-8 renormalised; shared
// expert scaled by sigmoid(Linear(x, 1))); "One Token Through Qwen3.6",
// section "The Router" (the router decides which experts a token needs).
//
// Phases, by workgroup index (a workgroup takes every role its index has):
//   A  (wg < column blocks x token blocks) the 16 x 16 tile of logits of
//      tokens 16 tb .. 16 tb + 15 and router rows 16 cb .. 16 cb + 15 (row E:
//      the shared gate), with the arithmetic of the separate router kernels:
//      one MFMA chain per slice of H, in the same k order and operand roles
//      (x rows A, router rows B), the slices' tiles summed from zero in slice
//      order as the selection kernel sums the partial rows, so routing is
//      bitwise the same on both paths.  Wave w takes slices w, w + 4, ...
//      Logits are published as 64-bit (value, tag) words, the data being its
//      own flag; the gate row goes to gate_s as sigmoid.
//   K  (wg < T / 4) one wave per token polls its E tagged logits, selects
//      (topk_select: descending logit, ties to the lower index, softmax over
//      the selected), writes topk_idx / topk_w and publishes the selections,
//      one copy per XCD.
//   D  (wg <= E) every group's workgroup polls its XCD's copy of all T K
//      selections and runs the per-group dispatch (group_dispatch.hpp).  A
//      per-token flag set once the selection stores had completed, polled by
//      one wave, measured slower (kernel 14.2 -> 15.8 us at 64 tokens): the
//      extra store round trip costs more than the polling traffic it saves.
// No phase waits on a later one, so the grid drains if every workgroup is
// resident; every wait is bounded (handoff.hpp), indices read from published
// words are clamped, and a timed-out call is flagged in the control block.
// The call tag is unique per call, so words left by earlier calls never match
// and the region needs no clearing.
#include "kernels.hpp"
#include "handoff.hpp"
#include "group_dispatch.hpp"
#include "lds_pipe.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxSlices = 16;            // H slices (router_ksplit <= 16)
constexpr int kMaxWaveSteps = 8;          // 64-wide k-steps per wave over its slices: H / 256 (H <= 2048)
constexpr int kSelPer = kRouteMaxT * 8 / kThreads;   // selections per thread in phase D
static_assert(kSelPer * kThreads == kRouteMaxT * 8, "phase D covers T K <= kRouteMaxT * 8 pairs");

__global__ __launch_bounds__(kThreads) void route_fused_kernel(LayerArgs L, const bf16_t* __restrict__ x, int T,
                                                               int ksplit, Work w, float* __restrict__ logits_out,
                                                               unsigned long long wait_ticks) {
  using pipe::kOutside;
  using pipe::make_rsrc;
  using pipe::rsrc_t;
  const int E = L.E, K = L.K, H = L.H, TK = T * K;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wg = blockIdx.x;
  const uint32_t tag = w.call_tag;
  uint32_t* ctl = w.ctl;
  uint64_t* lt = w.lt;                                  // [kRouteMaxT][256] tagged logits
  uint64_t* sel = w.lt + (size_t)kRouteMaxT * 256;      // kDecodeReplicas copies of [T K] tagged selections
  const int xcc = (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 7);   // HW_REG_XCC_ID[3:0]
  const int ncb = (E + 1 + 15) >> 4, ntb = (T + 15) >> 4;

  __shared__ f32x4 s_part[kMaxSlices][kWave];   // each slice's 16 x 16 tile
  if (wg == 0 && tid == 0) st_dev(ctl + kCtlLast, tag);

  // ---------------- phase A: a 16 x 16 tile of logits ----------------
  if (wg < ncb * ntb) {
    const int cb = wg % ncb, tb = wg / ncb;
    const int r16 = lane & 15, kq = (lane >> 4) * 16;
    const int klen = H / ksplit, nk = klen / 64, nf = H / 256;   // nf: this wave's slices x their k-steps
    // Rows past T or E + 1 repeat a valid row; their outputs are dropped.
    const bf16_t* arow = x + (size_t)min(16 * tb + r16, T - 1) * H + kq;
    const int eb = min(16 * cb + r16, E);
    const bf16_t* brow = (eb < E ? L.router_w + (size_t)eb * H : L.sh_expert_gate) + kq;
    // Step f of the wave: k-step f % nk of its slice f / nk (slice wave + 4 (f / nk)).
    u32x4 ra[kMaxWaveSteps][2], rb[kMaxWaveSteps][2];
#pragma unroll
    for (int f = 0; f < kMaxWaveSteps; ++f)
      if (f < nf) {
        const int j = f / nk, k = (wave + kWaves * j) * klen + 64 * (f - j * nk);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          ra[f][h] = ld16(arow + k + 8 * h);
          rb[f][h] = ld16(brow + k + 8 * h);
        }
      }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int f = 0; f < kMaxWaveSteps; ++f)
      if (f < nf) {
        const int j = f / nk, ks = f - j * nk;
        if (ks == 0) acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ra[f][h]), as_bf16x8(rb[f][h]), acc, 0, 0, 0);
        if (ks == nk - 1) s_part[wave + kWaves * j][lane] = acc;
      }
    __syncthreads();
    // Thread (token tt, router row ee) of the tile: D[4 (l / 16) + i][l % 16]
    // (token 4 (l / 16) + i, row l % 16) is component i of lane l.
    const int tt = tid >> 4, ee = tid & 15;
    const int ll = (tt >> 2) * 16 + ee, ii = tt & 3;
    float v = 0.f;
    for (int sl = 0; sl < ksplit; ++sl) v += s_part[sl][ll][ii];
    const int er = 16 * cb + ee, t = 16 * tb + tt;
    if (t < T && er <= E) {
      // Scores typed bf16 (the layer's option) are rounded after the sum, as
      // the selection kernel rounds them.
      if (L.logits_bf16) v = round_bf16(v);
      if (er < E) {
        // Slot 64 (e % 4) + e / 4 of the token's row: the reader lane that owns
        // experts 4 l .. 4 l + 3 finds them 512 bytes apart.
        st_dev(lt + (size_t)t * 256 + 64 * (er & 3) + (er >> 2), ((uint64_t)__float_as_uint(v) << 32) | tag);
        if (logits_out) logits_out[(size_t)t * E + er] = v;
      } else {
        w.gate_s[t] = sigmoidf_(v);
      }
    }
  }

  // ---------------- phase K: one wave per token selects ----------------
  {
    const int t = 4 * wg + wave;
    if (t < T) {
      const rsrc_t r_lt = make_rsrc(lt + (size_t)t * 256, 256u * 8u);
      float lv[1][4];
      auto ready = [&] {
        bool ok = true;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int ex = 4 * lane + c;
          const bool in = ex < E;
          // One 64-bit device-scope load: value and tag come from the same store.
          const auto w2 = __builtin_amdgcn_raw_buffer_load_b64(r_lt, in ? 8u * (uint32_t)(64 * c + lane) : kOutside,
                                                               0, 16);
          ok = ok && (!in || w2[0] == tag);
          lv[0][c] = __uint_as_float(w2[1]);
        }
        return __ballot(!ok) == 0ull;
      };
      wait_until(ready, ctl, tag, wait_ticks);
      int ix[1];
      float wv[1];
      topk_select<1>(lv, E, K, lane, ix, wv);
      if (lane < K) {
        w.topk_idx[(size_t)t * K + lane] = ix[0];
        w.topk_w[(size_t)t * K + lane] = wv[0];
        const uint64_t sv = ((uint64_t)(uint32_t)ix[0] << 32) | tag;
#pragma unroll
        for (int r = 0; r < kDecodeReplicas; ++r) st_dev(sel + (size_t)r * kRouteSelStride + t * K + lane, sv);
      }
    }
  }

  // ---------------- phase D: the per-group dispatch ----------------
  if (wg <= E) {
    const rsrc_t r_sel = make_rsrc(sel + (size_t)xcc * kRouteSelStride, (uint32_t)TK * 8u);
    int idx[kSelPer];
    auto ready = [&] {
      bool ok = true;
#pragma unroll
      for (int j = 0; j < kSelPer; ++j) {
        const int q = tid + j * kThreads;
        const bool in = q < TK;
        const auto w2 = __builtin_amdgcn_raw_buffer_load_b64(r_sel, in ? 8u * (uint32_t)q : kOutside, 0, 16);
        ok = ok && (!in || w2[0] == tag);
        // Clamped: after a timed-out wait the word may be stale.
        idx[j] = in ? min(max((int)w2[1], 0), E - 1) : -1;
      }
      return __ballot(!ok) == 0ull;
    };
    wait_until(ready, ctl, tag, wait_ticks);
    dispatch_group<kSelPer>(L, T, w, wg, idx);
  }
}

}  // namespace

hipError_t launch_route_fused(const LayerArgs& L, const bf16_t* x, int T, const Work& w, float* logits_out,
                              unsigned long long wait_ticks, hipStream_t s) {
  if (!route_fused_fits(T, L.H, L.K)) return hipErrorInvalidValue;
  const int ncb = (L.E + 1 + 15) / 16, ntb = (T + 15) / 16;
  const int grid = std::max(std::max(ncb * ntb, L.E + 1), (T + 3) / 4);
  const int ks = router_ksplit(T, L.H);   // the slices the separate router kernels would use
  if (ks % kWaves != 0 || ks > kMaxSlices || (L.H / ks) % 64 != 0 || L.H / 256 > kMaxWaveSteps)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(route_fused_kernel, dim3(grid), dim3(kThreads), 0, s, L, x, T, ks, w, logits_out, wait_ticks);
  return hipGetLastError();
}

}  // namespace moe
