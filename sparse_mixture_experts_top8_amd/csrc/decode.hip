// Fused decode path of the MoE layer for small batches (T <= 64 tokens) on
// gfx950: one persistent, co-resident launch that streams only the weights
// of the experts the tokens select.
//
// Definition of the layer: "Qwen3.6-35B-A3B — Architecture Overview", section
// "MoE FFN: 256 Experts" (router Linear, softmax, top-8 renormalised; SwiGLU
// experts; sigmoid-gated shared expert); Linnet model page, Blocks: SparseMoe.
// "One Token Through Qwen3.6", sections "The Router" and "One Complete Decode
// Step": the router decides which expert weights a token needs at all, so a
// decode step only has to read those.
//
// Phases, chained through device-scope counters in the workspace (no host
// round trip, no second launch):
//   A  router: tasks of 4 router rows (the last one also the shared-expert
//      gate row) x all tokens; shared expert gate/up: tasks of 16 inner rows.
//      Router tasks publish fp32 logits (and the shared gate scalar).
//   K  top-K per token: for T <= kLocalTopkT every workgroup selects all
//      tokens' experts itself from the published logits (one hand-off less);
//      otherwise workgroup t selects token t's and publishes them.
//   L  each workgroup builds, in LDS, the list of touched experts and each
//      expert's (token, k) pairs in pair-id order (the same stable grouping
//      as the counting sort).
//   B  routed gate/up: tasks of (touched expert, 16 inner rows) applied to the
//      tokens routed to that expert; h = w * SiLU(x.Wg) * (x.Wu) is published
//      in bf16 per (token, k) pair, already scaled by the routing weight.
//   C  down + combine: each workgroup owns 8 output rows; its waves split the
//      experts (touched ones, then the shared expert), each accumulating
//      W_down[rows] . h into a tile with the tokens as columns, so the
//      weighted sum over experts happens inside the MFMA accumulators; the
//      four wave tiles are added in LDS in a fixed order (no float atomics,
//      bitwise reproducible).
//
// Every task is a 16-row x 16-column tile on v_mfma_f32_16x16x32_bf16 (rows:
// weight rows, columns: tokens), with the hidden dimension split across the
// four waves and their partial tiles summed in LDS; no cross-lane
// reductions and no unrolled straight-line code beyond one task's loads
// (the whole kernel stays far below the instruction-cache size).
//
// Cross-workgroup data on MI355X: each XCD has its own write-back L2, and the
// agent-scope release/acquire fences that keep plain stores coherent across
// XCDs are L2 write-backs and invalidates, far too costly to issue per task.
// Instead every value one workgroup hands to another is written and read with
// agent-scope atomic accesses (write-through to, and read from, the device
// coherence point); a wave publishes by waiting for its stores to complete
// (s_waitcnt) and then bumping a counter, and readers poll counters with
// agent-scope loads.  Weights and x are never written and use plain loads.
//
// Start protocol: the host passes a call-unique 64-bit epoch.  Workgroup 0
// zeroes the counters and then publishes the epoch; every other workgroup
// sees the epoch before it touches a counter, so stale values from an earlier
// call are never read.  Every wait is bounded in time (see wait_until), so
// the grid always drains.
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxKSteps = 16;       // 32-wide k-steps in one wave's quarter of H (H <= 2048)
constexpr int kDownRows = 8;         // output rows of one down tile
constexpr int kDownGroups = 8;       // experts per down batch
constexpr int kDownKSteps = 4;       // 32-wide k-steps of the inner dimension per wave (inner <= 512)
constexpr int kLocalTopkT = 16;      // up to this many tokens every workgroup runs the top-K itself
constexpr unsigned long long kWaitTicks = 25000000ull;  // 0.25 s of the 100 MHz clock

// Control block layout (uint32 words); every counter has its own 128-byte
// line so that pollers of one counter do not queue behind another's.
constexpr int kLine = 32;                  // words per 128-byte line
constexpr int kCtlEpoch = 0;               // 64-bit epoch in words 0-1
constexpr int kCtlError = 1 * kLine;       // nonzero after a timed-out wait
constexpr int kCtlLogits = 2 * kLine;      // router rows published
constexpr int kCtlTopk = 3 * kLine;        // tokens whose top-K is published
constexpr int kCtlH = 4 * kLine;           // + kLine * g: inner rows of h finished for group g (E = shared)
static_assert(kDecodeCtlWords >= kCtlH + kLine * 257, "control block too small");

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// Weights are read once per call: non-temporal loads keep them from evicting
// the kernel's code and the small hot data (x, h, counters) from the caches.
__device__ __forceinline__ u32x4 ldw(const bf16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---- device-coherent accesses ----
__device__ __forceinline__ uint32_t ld_cnt(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Published data (written by other workgroups with write-through stores) is
// read with device-scope buffer loads (sc1): they bypass any XCD-local cached
// copy, so no L2 invalidate is needed after a hand-off.  Buffer loads past the
// resource's size return zero, which masks fragments without a branch.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutside = 0x80000000u;   // out of range even after adding a k offset
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 ld_pub16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16);
}
__device__ __forceinline__ float ld_pub_f(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 16));
}
__device__ __forceinline__ int ld_pub_i(rsrc_t r, uint32_t off) {
  return (int)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 16);
}

// All of this wave's earlier memory operations have completed (stores at the
// coherence point).
__device__ __forceinline__ void stores_complete() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Bounded wait: gives up after kWaitTicks (or at once once any wave gave up),
// records `code` in the error word and returns; indices read from shared state
// are clamped by their users, so a timed-out wait yields wrong numbers, never
// an out-of-bounds access.
template <typename Ready>
__device__ __forceinline__ void wait_until(Ready ready, uint32_t* err, uint32_t code) {
  if (!ready()) {
    const unsigned long long t0 = wall_clock64();
    uint32_t n = 0;
    while (!ready()) {
      __builtin_amdgcn_s_sleep(2);
      if ((++n & 31u) == 0u && (ld_cnt(err) != 0u || wall_clock64() - t0 > kWaitTicks)) {
        __hip_atomic_fetch_or(err, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Top-K of one token's published logits by one wave: descending logit, ties to
// the lower expert index; lane k < K receives the k-th index and its weight,
// the softmax over the selected logits (equal to the full softmax renormalised).
__device__ __noinline__ void topk_token(rsrc_t logits, int t, int E, int K, int lane, int* idx_out, float* w_out) {
  float v[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    v[c] = ld_pub_f(logits, 4u * (uint32_t)(t * E + min(e, E - 1)));
  }
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (lane + 64 * c >= E || v[c] != v[c]) v[c] = -INFINITY;
  float vmax = 0.f, den = 0.f, mine_v = 0.f;
  int mine_i = 0;
  for (int k = 0; k < K; ++k) {
    // Lane-local best (strict > keeps the lower column on ties); padding
    // columns hold -inf and lose every tie to a real expert.
    float bv = v[0];
    int bi = lane;
#pragma unroll
    for (int c = 1; c < 4; ++c)
      if (v[c] > bv) { bv = v[c]; bi = lane + 64 * c; }
    float wv;
    int wi;
    wave_argmax(bv, bi, &wv, &wi);
    if ((wi & 63) == lane) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((wi >> 6) == c) v[c] = -INFINITY;
    }
    if (k == 0) vmax = wv;
    den += __expf(wv - vmax);
    if (lane == k) { mine_v = wv; mine_i = wi; }
  }
  *idx_out = clamp_expert(mine_i, E);
  *w_out = __expf(mine_v - vmax) / den;
}

__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  const LayerArgs& L = a.L;
  const int H = L.H, E = L.E, K = L.K, I = L.I, Is = L.Is, T = a.T;
  const int TK = T * K;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int G = gridDim.x;
  const int m = lane & 15;            // A-operand row / B-operand column of this lane
  const int kq = (lane >> 4) * 8;     // this lane's 8 elements inside a 32-wide k-step
  const int nks = H / 128;            // k-steps in this wave's quarter of H
  const int kbeg = wave * (H / 4);
  uint32_t* ctl = a.ctl;
  uint32_t* err = ctl + kCtlError;
  unsigned long long* epoch_p = reinterpret_cast<unsigned long long*>(ctl + kCtlEpoch);
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const f32x4 zf4 = {0.f, 0.f, 0.f, 0.f};
  const rsrc_t r_logits = make_rsrc(a.logits, (size_t)T * E * 4);

  __shared__ int s_cnt[257];
  __shared__ int s_off[258];
  __shared__ int s_cur[257];
  __shared__ int s_list[kDecodeMaxT * 8];
  __shared__ int s_tidx[kDecodeMaxT * 8];
  __shared__ float s_tw[kDecodeMaxT * 8];
  __shared__ int s_touched[257];
  __shared__ int s_ntouched;
  __shared__ float s_red[kWaves][4][256];   // per wave: up to four 16x16 partial tiles

  // ---------------- start: counters zeroed, then the epoch published ----------------
  // Workgroup 0's threads zero one counter word each, then thread 0 publishes
  // the epoch once every store has completed.
  if (blockIdx.x == 0) {
    for (int i = tid; i < 3 + E + 1; i += kThreads)
      __hip_atomic_store(ctl + kCtlError + kLine * i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    stores_complete();
    __syncthreads();
    if (tid == 0) __hip_atomic_store(epoch_p, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  bool epoch_seen = false;
  auto see_epoch = [&]() {
    if (!epoch_seen) {
      wait_until([&] { return __hip_atomic_load(epoch_p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch; },
                 err, 2u);
      epoch_seen = true;
    }
  };
  // Every wave's stores are complete, then thread 0 counts n arrivals.
  auto publish = [&](uint32_t* cnt, uint32_t n) {
    stores_complete();
    __syncthreads();
    if (wave == 0) {
      see_epoch();
      if (lane == 0) __hip_atomic_fetch_add(cnt, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  // Gate/up task: rows [inner0, inner0 + R) of group g's gate and up
  // projections (g == E: the shared expert) against the tokens of the group,
  // h = SiLU(gate) * up, scaled by the routing weight for routed experts,
  // stored as bf16 pairs.  R is even and at most 16.
  auto gate_up_task = [&](int g, int inner0, int R) {
    // Loads are unconditional: tile rows >= R repeat row R - 1 and columns
    // beyond the group's tokens repeat its first token; those outputs are
    // never used.  k-steps beyond H / 128 repeat the last one and are skipped.
    const bool sh = g == E;
    const int mr = min(m, R - 1);
    const size_t grow = sh ? (size_t)(inner0 + mr) * H : ((size_t)g * 2 * I + inner0 + mr) * H;
    const size_t urow = sh ? (size_t)(inner0 + mr) * H : ((size_t)g * 2 * I + I + inner0 + mr) * H;
    const bf16_t* gp = (sh ? L.sh_gate_w : L.gate_up_w) + grow + kbeg + kq;
    const bf16_t* up = (sh ? L.sh_up_w : L.gate_up_w) + urow + kbeg + kq;
    u32x4 ag[kMaxKSteps], au[kMaxKSteps];
#pragma unroll
    for (int ks = 0; ks < kMaxKSteps; ++ks) {
      const int kk = 32 * min(ks, nks - 1);
      ag[ks] = ldw(gp + kk);
      au[ks] = ldw(up + kk);
    }
    const int p0 = sh ? 0 : s_off[g];
    const int ncol = sh ? T : s_off[g + 1] - p0;
    for (int cb = 0; cb < ncol; cb += 16) {
      const int c = min(cb + m, ncol - 1);
      const int tok = sh ? c : s_list[p0 + c] / K;
      const bf16_t* xp = a.x + (size_t)tok * H + kbeg + kq;
      u32x4 xf[kMaxKSteps];
#pragma unroll
      for (int ks = 0; ks < kMaxKSteps; ++ks) xf[ks] = ld16(xp + 32 * min(ks, nks - 1));
      f32x4 dg = zf4, du = zf4;
#pragma unroll
      for (int ks = 0; ks < kMaxKSteps; ++ks) {
        if (ks < nks) {
          dg = mfma16(ag[ks], xf[ks], dg);
          du = mfma16(au[ks], xf[ks], du);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s_red[wave][0][(4 * (lane >> 4) + r) * 16 + m] = dg[r];
        s_red[wave][1][(4 * (lane >> 4) + r) * 16 + m] = du[r];
      }
      __syncthreads();
      // Thread: inner rows i0, i0 + 1 of column cc.
      if (tid < 128) {
        const int i0 = 2 * (tid >> 4), cl = tid & 15, cc = cb + cl;
        if (i0 < R && cc < ncol) {
          float hv[2];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int idx = (i0 + j) * 16 + cl;
            const float gs = (s_red[0][0][idx] + s_red[1][0][idx]) + (s_red[2][0][idx] + s_red[3][0][idx]);
            const float us = (s_red[0][1][idx] + s_red[1][1][idx]) + (s_red[2][1][idx] + s_red[3][1][idx]);
            hv[j] = siluf_(gs) * us;
          }
          bf16_t* dst;
          if (sh) {
            dst = a.h_sh + (size_t)cc * Is + inner0 + i0;
          } else {
            const int q = s_list[p0 + cc];
            const float w = s_tw[q];
            hv[0] *= w;
            hv[1] *= w;
            dst = a.h + (size_t)q * I + inner0 + i0;
          }
          st_dev(reinterpret_cast<uint32_t*>(dst), pack_bf16x2(hv[0], hv[1]));
        }
      }
      __syncthreads();
    }
    publish(ctl + kCtlH + kLine * g, (uint32_t)R);
  };

  // ---------------- phase A: router rows and shared-expert gate/up rows ----------------
  const int nR = (E + 1 + 3) / 4;
  int SR = 2;                                   // shared rows per task: power of two >= Is / G
  while (SR < 16 && SR * G < Is) SR <<= 1;
  const int nS = a.route_only ? 0 : Is / SR;
  for (int task = blockIdx.x; task < nR + nS; task += G) {
    if (task < nR) {
      // Router rows 4*task + m (m < 4); row E is the shared-expert gate row.
      // Tile rows >= 4 (and rows past E) repeat a valid row; ignored below.
      const int e_row = min(4 * task + min(m, 3), E);
      const bf16_t* rp = (e_row < E ? L.router_w + (size_t)e_row * H : L.sh_expert_gate) + kbeg + kq;
      u32x4 af[kMaxKSteps];
#pragma unroll
      for (int ks = 0; ks < kMaxKSteps; ++ks) af[ks] = ldw(rp + 32 * min(ks, nks - 1));
      for (int cb = 0; cb < T; cb += 16) {
        const int t = min(cb + m, T - 1);
        const bf16_t* xp = a.x + (size_t)t * H + kbeg + kq;
        u32x4 xf[kMaxKSteps];
#pragma unroll
        for (int ks = 0; ks < kMaxKSteps; ++ks) xf[ks] = ld16(xp + 32 * min(ks, nks - 1));
        f32x4 d = zf4;
#pragma unroll
        for (int ks = 0; ks < kMaxKSteps; ++ks)
          if (ks < nks) d = mfma16(af[ks], xf[ks], d);
#pragma unroll
        for (int r = 0; r < 4; ++r) s_red[wave][0][(4 * (lane >> 4) + r) * 16 + m] = d[r];
        __syncthreads();
        if (tid < 64) {
          const int i = tid >> 4, c = tid & 15;
          const int e = 4 * task + i, tt = cb + c;
          if (e <= E && tt < T) {
            const float v = (s_red[0][0][tid] + s_red[1][0][tid]) + (s_red[2][0][tid] + s_red[3][0][tid]);
            if (e < E) st_dev(a.logits + (size_t)tt * E + e, v);
            else st_dev(a.gate_s + tt, sigmoidf_(v));
          }
        }
        __syncthreads();
      }
      publish(ctl + kCtlLogits, (uint32_t)min(4, E + 1 - 4 * task));
    } else {
      gate_up_task(E, SR * (task - nR), SR);
    }
  }

  // ---------------- phase K: top-K selections into LDS ----------------
  if (T <= kLocalTopkT) {
    // Wave 0 polls; the barrier releases the others.
    if (wave == 0) {
      see_epoch();
      wait_until([&] { return ld_cnt(ctl + kCtlLogits) >= (uint32_t)(E + 1); }, err, 1u);
    }
    __syncthreads();
    if (wave < T) {
      for (int t = wave; t < T; t += kWaves) {
        int ix;
        float wv;
        topk_token(r_logits, t, E, K, lane, &ix, &wv);
        if (lane < K) { s_tidx[t * K + lane] = ix; s_tw[t * K + lane] = wv; }
      }
    }
  } else {
    if (wave == 0 && (int)blockIdx.x < T) {
      see_epoch();
      wait_until([&] { return ld_cnt(ctl + kCtlLogits) >= (uint32_t)(E + 1); }, err, 1u);
      const int t = blockIdx.x;
      int ix;
      float wv;
      topk_token(r_logits, t, E, K, lane, &ix, &wv);
      if (lane < K) {
        st_dev(a.topk_idx + (size_t)t * K + lane, ix);
        st_dev(a.topk_w + (size_t)t * K + lane, wv);
      }
      stores_complete();
      if (lane == 0) __hip_atomic_fetch_add(ctl + kCtlTopk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (wave == 0) {
      see_epoch();
      wait_until([&] { return ld_cnt(ctl + kCtlTopk) >= (uint32_t)T; }, err, 1u);
      const rsrc_t r_ti = make_rsrc(a.topk_idx, (size_t)TK * 4), r_tw = make_rsrc(a.topk_w, (size_t)TK * 4);
      for (int q = lane; q < TK; q += 64) {
        s_tidx[q] = clamp_expert(ld_pub_i(r_ti, 4u * q), E);
        s_tw[q] = ld_pub_f(r_tw, 4u * q);
      }
    }
  }
  __syncthreads();

  // ---------------- phase L: per-expert pair lists in LDS ----------------
  if (wave == 0) {
    for (int e = lane; e <= 256; e += 64) s_cnt[e] = 0;
    __builtin_amdgcn_wave_barrier();
    for (int q = lane; q < TK; q += 64) atomicAdd(&s_cnt[s_tidx[q]], 1);
    __builtin_amdgcn_wave_barrier();
    // Exclusive scan of the E counts (four per lane).
    int c4[4], run = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      c4[j] = e < E ? s_cnt[e] : 0;
      run += c4[j];
    }
    int incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += n;
    }
    int base = incl - run;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      if (e < E) { s_off[e] = base; s_cur[e] = base; }
      base += c4[j];
    }
    if (lane == 63) s_off[E] = incl;
    __builtin_amdgcn_wave_barrier();
    // Stable placement: a pair's slot is its expert's cursor plus the number
    // of earlier lanes in this 64-pair chunk with the same expert.
    const unsigned long long lt = (1ull << lane) - 1ull;
    for (int q0 = 0; q0 < TK; q0 += 64) {
      const int q = q0 + lane;
      const bool valid = q < TK;
      const int key = valid ? s_tidx[q] : 511;
      unsigned long long peers = __ballot(valid);
#pragma unroll
      for (int b = 0; b < 9; ++b) {
        const unsigned long long msk = __ballot((key >> b) & 1);
        peers &= ((key >> b) & 1) ? msk : ~msk;
      }
      const int rank = __popcll(peers & lt);
      const int cnt = __popcll(peers);
      if (valid) s_list[s_cur[key] + rank] = q;
      __builtin_amdgcn_wave_barrier();
      if (valid && rank == cnt - 1) s_cur[key] += cnt;
      __builtin_amdgcn_wave_barrier();
    }
    // Touched experts, ascending.
    int nt = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const bool hit = e < E && s_cnt[e] > 0;
      const unsigned long long msk = __ballot(hit);
      if (hit) s_touched[nt + __popcll(msk & lt)] = e;
      nt += __popcll(msk);
    }
    if (lane == 0) s_ntouched = nt;
  }
  __syncthreads();

  if (a.route_only) {
    if (blockIdx.x == 0) {
      for (int e = tid; e <= E; e += kThreads) a.offsets_out[e] = s_off[e];
      for (int q = tid; q < TK; q += kThreads) {
        a.perm_out[q] = s_list[q];
        a.topk_idx[q] = s_tidx[q];
        a.topk_w[q] = s_tw[q];
      }
    }
    return;
  }
  const int U = s_ntouched;
  const int ng = U + 1;   // touched experts, then the shared expert (group index U)

  // Down tiles of this workgroup: rows [8 * tile, 8 * tile + 8).  The inner
  // dimension is split over the waves (wave w takes the contiguous k-steps
  // [4w, 4w + 4)); routed experts are taken in batches of kDownGroups with
  // all of a batch's loads in flight together.  The shared expert's rows and
  // the first routed batch's rows are loaded now, before phase B, so that
  // their latency overlaps it (they do not depend on h).
  // Rows >= 8 of the tile repeat row 7, experts past the list repeat the last
  // one and k-steps past the inner size repeat the last one; those outputs
  // are ignored or their MFMAs skipped.
  const int ntiles = (H + kDownRows - 1) / kDownRows;
  auto koff = [&](int s4, int nk) { return 32 * min(kDownKSteps * wave + s4, nk - 1) + kq; };
  auto down_rows = [&](int tile, int gb, u32x4 (*ad)[kDownKSteps]) {
    const int r = min(kDownRows * tile + min(m, kDownRows - 1), H - 1);
#pragma unroll
    for (int j = 0; j < kDownGroups; ++j) {
      const bf16_t* rp = L.down_w + ((size_t)s_touched[min(gb + j, max(U - 1, 0))] * H + r) * I;
#pragma unroll
      for (int s4 = 0; s4 < kDownKSteps; ++s4) ad[j][s4] = ldw(rp + koff(s4, I / 32));
    }
  };
  u32x4 ad[kDownGroups][kDownKSteps];
  u32x4 ash[kDownKSteps];
  const bool has_tile = (int)blockIdx.x < ntiles;
  if (has_tile) {
    const int r = min(kDownRows * (int)blockIdx.x + min(m, kDownRows - 1), H - 1);
#pragma unroll
    for (int s4 = 0; s4 < kDownKSteps; ++s4) ash[s4] = ldw(L.sh_down_w + (size_t)r * Is + koff(s4, Is / 32));
    if (U > 0) down_rows(blockIdx.x, 0, ad);
  }

  // ---------------- phase B: routed gate/up tasks ----------------
  {
    const int nib = I / 16;
    for (int task = blockIdx.x; task < U * nib; task += G) gate_up_task(s_touched[task / nib], 16 * (task % nib), 16);
  }

  // ---------------- phase C: down projection and combine ----------------
  // acc[cb]: this wave's partial 16x16 tile (rows: the tile's output rows,
  // columns: tokens 16 cb .. 16 cb + 15), summed over experts in a fixed order.
  const int ncb = (T + 15) / 16;
  const rsrc_t r_h = make_rsrc(a.h, (size_t)TK * I * 2);
  const rsrc_t r_hsh = make_rsrc(a.h_sh, (size_t)T * Is * 2);
  const rsrc_t r_gs = make_rsrc(a.gate_s, (size_t)T * 4);
  for (int tile = blockIdx.x; tile < ntiles; tile += G) {
    const bool first_tile = tile == (int)blockIdx.x;
    f32x4 acc[4] = {zf4, zf4, zf4, zf4};
    // Shared expert first: its h was finished in phase A.
    if (wave == 0) {
      see_epoch();
      wait_until([&] { return ld_cnt(ctl + kCtlH + kLine * E) >= (uint32_t)Is; }, err, 1u);
    }
    __syncthreads();
    if (!first_tile) {
      const int r = min(kDownRows * tile + min(m, kDownRows - 1), H - 1);
#pragma unroll
      for (int s4 = 0; s4 < kDownKSteps; ++s4) ash[s4] = ldw(L.sh_down_w + (size_t)r * Is + koff(s4, Is / 32));
    }
    for (int cb = 0; cb < ncb; ++cb) {
      const int t = 16 * cb + m;
      const uint32_t row = t < T ? 2u * (uint32_t)(t * Is) : kOutside;
      u32x4 bf[kDownKSteps];
#pragma unroll
      for (int s4 = 0; s4 < kDownKSteps; ++s4) bf[s4] = ld_pub16(r_hsh, row + 2u * koff(s4, Is / 32));
      const float sgt = ld_pub_f(r_gs, t < T ? 4u * t : kOutside);
      f32x4 d = zf4;
#pragma unroll
      for (int s4 = 0; s4 < kDownKSteps; ++s4)
        if (kDownKSteps * wave + s4 < Is / 32) d = mfma16(ash[s4], bf[s4], d);
      d *= sgt;
#pragma unroll
      for (int c4i = 0; c4i < 4; ++c4i)
        if (c4i == cb) acc[c4i] += d;
    }
    // Routed experts: wave 0 waits until every touched expert's h is
    // complete (lanes poll different experts); the barrier releases the rest.
    if (wave == 0) {
      wait_until([&] {
        bool ok = true;
        for (int gi = lane; gi < U; gi += 64) ok = ok && ld_cnt(ctl + kCtlH + kLine * s_touched[gi]) >= (uint32_t)I;
        return __ballot(!ok) == 0ull;
      }, err, 1u);
    }
    __syncthreads();
    for (int gb = 0; gb < U; gb += kDownGroups) {
      if (gb > 0 || !first_tile) down_rows(tile, gb, ad);
      for (int cb = 0; cb < ncb; ++cb) {
        // This lane's column is token t.  Stage 1: the pair of (t, expert) for
        // every expert of the batch; stage 2: all h loads; stage 3: zero the
        // fragments of tokens without that expert; stage 4: MFMAs.
        const int t = 16 * cb + m, tc = min(t, T - 1);
        int hq[kDownGroups];
#pragma unroll
        for (int j = 0; j < kDownGroups; ++j) {
          const int g = s_touched[min(gb + j, U - 1)];
          int q = -1;
          for (int k = 0; k < K; ++k) q = s_tidx[tc * K + k] == g ? tc * K + k : q;
          hq[j] = (t < T && gb + j < U) ? q : -1;
        }
        u32x4 bf[kDownGroups][kDownKSteps];
#pragma unroll
        for (int j = 0; j < kDownGroups; ++j) {
          const uint32_t row = hq[j] >= 0 ? 2u * (uint32_t)(hq[j] * I) : kOutside;
#pragma unroll
          for (int s4 = 0; s4 < kDownKSteps; ++s4) bf[j][s4] = ld_pub16(r_h, row + 2u * koff(s4, I / 32));
        }
        f32x4 d = zf4;
#pragma unroll
        for (int j = 0; j < kDownGroups; ++j) {
          if (gb + j >= U) continue;
#pragma unroll
          for (int s4 = 0; s4 < kDownKSteps; ++s4)
            if (kDownKSteps * wave + s4 < I / 32) d = mfma16(ad[j][s4], bf[j][s4], d);
        }
#pragma unroll
        for (int c4i = 0; c4i < 4; ++c4i)
          if (c4i == cb) acc[c4i] += d;
      }
    }
    // Sum the four waves' tiles in a fixed order and write rows < 8 of each column.
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_red[wave][cb][(4 * (lane >> 4) + r) * 16 + m] = acc[cb][r];
    __syncthreads();
    for (int e = tid; e < ncb * 128; e += kThreads) {
      const int cb = e >> 7, i = (e >> 4) & 7, c = e & 15;
      const int idx = i * 16 + c;
      const int t = 16 * cb + c, r = kDownRows * tile + i;
      if (t < T && r < H) {
        const float v = (s_red[0][cb][idx] + s_red[1][cb][idx]) + (s_red[2][cb][idx] + s_red[3][cb][idx]);
        a.out[(size_t)t * H + r] = (bf16_t)f32_to_bf16(v);
      }
    }
    __syncthreads();
  }
}

}  // namespace

// Plain launch of at most one workgroup per CU: with the device otherwise idle
// every workgroup is resident at once.  Should some not be (other kernels
// occupying CUs), the bounded waits still let every wave finish, and the
// error word in the workspace reports it.
hipError_t launch_decode(const DecodeArgs& args, int grid, hipStream_t s) {
  hipLaunchKernelGGL(decode_kernel, dim3(grid), dim3(kThreads), 0, s, args);
  return hipGetLastError();
}

int decode_max_grid(int num_cus) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(decode_kernel), kThreads,
                                                   0) != hipSuccess)
    return 0;
  return per_cu * num_cus;
}

}  // namespace moe
