// Fused decode path of the MoE layer for small batches (1 <= T <= 16 tokens)
// on gfx950: one launch, one workgroup per CU, that streams only the weights of
// the experts the tokens select.
//
// Definition of the layer: "Qwen3.6-35B-A3B — Architecture Overview", section
// "MoE FFN: 256 Experts" (router Linear, softmax, top-8 renormalised; SwiGLU
// experts; sigmoid-gated shared expert); Linnet model page, Blocks: SparseMoe.
// "One Token Through Qwen3.6", sections "The Router" and "One Complete Decode
// Step": the router decides which expert weights a token needs at all, so a
// decode step only has to read those.
//
// Phases (no host round trip, no second launch):
//   A  every workgroup computes its share of the router rows (the shared-expert
//      gate row is router row E) and of the shared expert's gate/up rows for
//      all tokens; it publishes its logits tagged with the call's tag, and
//      h_sh = sigma(x . w_g) * SiLU(g) * u (it evaluates the gate row itself).
//   K  every workgroup polls the tagged logits until all carry this call's
//      tag (the data is its own completion flag) and selects every token's
//      top-K.
//   L  every workgroup builds, in LDS, the touched-expert list and each
//      expert's (token, k) pairs in pair-id order (the counting-sort order).
//   B  routed gate/up in blocks of (expert, 8 inner rows); h = w * SiLU(g) * u
//      is published in bf16 per pair, routing weight applied.   [grid hand-off]
//   C  down projection + combine, output-row stationary: each workgroup owns a
//      few output rows and adds W_down[e][rows] . h over the shared expert and
//      every touched expert, in a fixed order, then writes out.
//
// Weight streams are software pipelined: a wave keeps the loads of the next
// blocks (phase B) or stages (phase C) in flight while it computes the current
// one, and the down-projection weights of the first stages are requested during
// phase B, since they do not depend on h.  Every tile is a 16 x 16 tile of
// v_mfma_f32_16x16x32_bf16 whose columns are tokens (phases A and C) or one
// expert's pairs (phase B), with the contraction split over the four waves;
// partial tiles meet in LDS in a fixed order, so results are bitwise
// reproducible.
//
// Cross-workgroup data on MI355X: each XCD has its own write-back L2, and the
// agent-scope release/acquire fences that keep plain stores coherent across
// XCDs are L2 write-backs and invalidates, far too costly per hand-off.  Every
// value one workgroup hands to another is written with agent-scope
// (write-through) stores and read with device-scope buffer loads (sc1).
//
// Every poll of the whole grid on a few shared lines queues at those lines'
// memory channel, so what is polled is published once per XCD: the writer
// stores eight copies, and the workgroups of XCD x poll copy x only.  The
// logits are published as 64-bit (value, tag) words, the data being its own
// flag.  For the h hand-off a workgroup whose stores have all completed
// (s_waitcnt) writes the tag into its slot of each flag copy; waiters read
// their copy's slots with one load per lane.  No atomics, no counters: the
// tag is call-unique (the host's epoch, low word never 0), so words left by
// earlier calls never match and nothing has to be cleared first.  Every wait
// is bounded in time (see wait_until), so the grid always drains.
#include <type_traits>

#include "kernels.hpp"
#include "handoff.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxT = kDecodeMaxT;       // tokens (columns of every tile)
constexpr int kMaxHSteps = 16;           // 32-wide k-steps in one wave's quarter of H (H <= 2048)
constexpr int kMaxISteps = 4;            // 32-wide k-steps in one wave's quarter of an inner dim (<= 512)
constexpr int kXStride = 2048 + 8;       // LDS row stride of x, bf16 elements (rows stay 16-byte aligned)
constexpr int kBDepth = 2;               // gate/up blocks in flight per wave
constexpr int kCDepth = 6;               // down-projection stages in flight per wave
constexpr int kMaxCStages = 1 + 8 * 8;   // shared expert + one stage per expert touched by 8 tokens
constexpr int kLateMaxPairs = 2;         // shared (gate, up) pairs per workgroup on the wave-3 path
constexpr int kLateRows = 1 + 2 * kLateMaxPairs;   // the gate row, then the pairs
constexpr int kLateChunks = 4;           // 512-element chunks of a row (H <= 2048)
static_assert(kDecodeCtlWords >= kCtlFlags + kDecodeReplicas * kDecodeFlagStride, "control block too small");

// Phase A weight fragment (plain load: the non-temporal hint measured slower
// here, 21.1 against 20.2 us at one token).
__device__ __forceinline__ u32x4 ldw(const bf16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 ld_lds16(const bf16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---- device-coherent accesses (see handoff.hpp) ----
// Published data is read with device-scope buffer loads (sc1): they bypass any
// XCD-local cached copy, so no L2 invalidate is needed after a hand-off.
// Buffer loads past the resource's size return zero, which masks fragments
// without a branch.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutside = 0x80000000u;   // out of range even after adding a k offset
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// h after its hand-off: an ordinary (L2-cacheable) load.  No CU reads h
// before the hand-off in a call, and the caches hold no copies from earlier
// launches, so the first reader in each XCD fetches the written-through data
// and the XCD's other workgroups hit in its L2.
__device__ __forceinline__ u32x4 ld_after16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// Weight fragment through a buffer resource; an offset outside the resource
// returns zeros without touching memory, so pipeline stages past the end of
// the work and k-steps past the contraction are issued unconditionally (the
// load counter then matches in every path) and add zero.
__device__ __forceinline__ u32x4 ldw_buf(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// The same, non-temporal (cache policy bit 1): the routed gate/up stream of
// phase B, read once per call and by one workgroup, stays out of the caches
// (one token: 21.6 -> 20.2 us).  The down-projection stream measured slower
// with the hint (20.7 us with both) and keeps plain loads.
__device__ __forceinline__ u32x4 ldw_buf_nt(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}

// Wave-wide inclusive prefix sum (DPP shifts inside each 16-lane row, then the
// row totals are added from scalar registers).
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
            r2 = __builtin_amdgcn_readlane(v, 47);
  return v + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}

__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  const LayerArgs& L = a.L;
  const int H = L.H, E = L.E, K = L.K, I = L.I, Is = L.Is, T = a.T;
  const int TK = T * K;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int G = gridDim.x, wg = blockIdx.x;
  const int m = lane & 15;            // A-operand row / B-operand column of this lane
  const int kq = (lane >> 4) * 8;     // this lane's 8 elements inside a 32-wide k-step
  const int nks = H / 128;            // k-steps in this wave's quarter of H
  const int kbeg = wave * (H / 4);
  uint32_t* ctl = a.ctl;
  const uint32_t tag = (uint32_t)a.epoch;
  // This workgroup's XCD picks the copy of published data it polls.
  const int xcc = (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 7);   // HW_REG_XCC_ID[3:0]
  const int lstride = decode_logit_stride(T);
  const f32x4 zf4 = {0.f, 0.f, 0.f, 0.f};

  __shared__ __attribute__((aligned(16))) bf16_t s_x[kMaxT * kXStride];   // x, one padded row per token
  __shared__ f32x4 s_red[2][kWaves][kWave];     // partial tiles of the four waves (two blocks in flight)
  __shared__ uint32_t s_mask[256];              // tokens that selected expert e (bit t)
  __shared__ int s_off[257];                    // pair-list offsets per expert
  __shared__ int s_touched[256];                // touched experts, ascending
  __shared__ int s_list[kMaxT * 8];             // pair ids grouped by expert, pair-id order inside
  __shared__ int s_tidx[kMaxT * 8];
  __shared__ float s_tw[kMaxT * 8];
  __shared__ int s_cq[kMaxCStages * 16];       // phase C: h row of each stage's tile column (-1: none)
  __shared__ int s_tl[2][64];                   // experts touched by tokens 0-7 / 8-15, ascending (T > 8)
  __shared__ int s_U, s_U01;

  // This call's tag goes into the control block's latest-call word; the error
  // word is never cleared: it names the call whose wait timed out, so the
  // latest call failed exactly when the two words are equal.
  if (wg == 0 && tid == 0) st_dev(ctl + kCtlLast, tag);
  for (int i = tid; i < 256; i += kThreads) s_mask[i] = 0u;

  // ---------------- phase A: router rows and shared-expert rows ----------------
  // Workgroup wg owns router rows [r_lo, r_hi) of E + 1 (row E: the shared
  // gate) and shared inner rows [s_lo, s_hi).  Tile rows: the router rows, the
  // shared gate row (when it owns inner rows), then (gate, up) row pairs; the
  // host guarantees they fit one 16-row tile.  The weight loads go out first,
  // then x is staged in LDS (every workgroup keeps all of x there).
  //
  // With fewer tokens than waves (T <= 3) wave 3 routes no token, so the
  // shared rows leave the tile: after the router tile, wave 3 requests them
  // (the gate row and the pairs, whole rows, coalesced) and forms h_sh with
  // VALU dot products while the other waves poll the logits.  The router
  // tile then waits for router rows only, which puts the logit exchange
  // earlier.
  const int s_lo = (int)((long long)wg * Is / G), s_hi = (int)((long long)(wg + 1) * Is / G);
  const int n_s = s_hi - s_lo;
  const bool late_shared = T < kWaves && n_s <= kLateMaxPairs;
  const bool late_wave = late_shared && wave == kWaves - 1 && n_s > 0;
  {
    const int r_lo = (int)((long long)wg * (E + 1) / G), r_hi = (int)((long long)(wg + 1) * (E + 1) / G);
    const int n_r = r_hi - r_lo;
    const int p0 = late_shared ? n_r : n_r + (n_s > 0 ? 1 : 0);   // first (gate, up) pair row
    const int nrow = late_shared ? n_r : p0 + 2 * n_s;
    u32x4 af[kMaxHSteps];
    if (nrow > 0) {
      const int mr = min(m, nrow - 1);
      const bf16_t* rp;
      if (mr < n_r) {
        const int e = r_lo + mr;
        rp = e < E ? L.router_w + (size_t)e * H : L.sh_expert_gate;
      } else if (mr < p0) {
        rp = L.sh_expert_gate;
      } else {
        const int p = (mr - p0) >> 1;
        rp = (((mr - p0) & 1) ? L.sh_up_w : L.sh_gate_w) + (size_t)(s_lo + p) * H;
      }
      rp += kbeg + kq;
#pragma unroll
      for (int ks = 0; ks < kMaxHSteps; ++ks) af[ks] = ldw(rp + 32 * min(ks, nks - 1));
    }
    {
      const int cpr = H / 8;   // 16-byte chunks per row of x
      u32x4 xr[kMaxT];
#pragma unroll
      for (int j = 0; j < kMaxT; ++j) {
        const int i = tid + j * kThreads;
        if (i < T * cpr) {
          const int t = i / cpr;
          xr[j] = ld16(a.x + (size_t)t * H + 8 * (i - t * cpr));
        }
      }
#pragma unroll
      for (int j = 0; j < kMaxT; ++j) {
        const int i = tid + j * kThreads;
        if (i < T * cpr) {
          const int t = i / cpr;
          *reinterpret_cast<u32x4*>(s_x + t * kXStride + 8 * (i - t * cpr)) = xr[j];
        }
      }
    }
    __syncthreads();
    if (a.norm_w) {
      // Sub-block form: x = bf16(RMSNorm(x)) in place, wave w taking tokens
      // w, w + 4, ... with the expression, chunk order and wave sum of the
      // standalone norm kernel.
      const int nch = H / 8;
      for (int t = wave; t < T; t += kWaves) {
        bf16_t* xr = s_x + t * kXStride;
        float ss = 0.f;
        for (int c = lane; c < nch; c += kWave) {
          const u32x4 v = ld_lds16(xr + 8 * c);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float p = bf16_to_f32(v[j] & 0xFFFFu), q = bf16_to_f32(v[j] >> 16);
            ss += p * p;
            ss += q * q;
          }
        }
        const float r = 1.0f / sqrtf(wave_sum_f32(ss) / (float)H + a.eps);
        for (int c = lane; c < nch; c += kWave) {
          const u32x4 v = ld_lds16(xr + 8 * c), wv = ld16(a.norm_w + 8 * c);
          u32x4 o;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            o[j] = pack_bf16x2(bf16_to_f32(v[j] & 0xFFFFu) * r * bf16_to_f32(wv[j] & 0xFFFFu),
                               bf16_to_f32(v[j] >> 16) * r * bf16_to_f32(wv[j] >> 16));
          *reinterpret_cast<u32x4*>(xr + 8 * c) = o;
        }
      }
      __syncthreads();
    }
    if (nrow > 0) {
      const bf16_t* xs = s_x + min(m, T - 1) * kXStride + kbeg + kq;
      const u32x4 z4 = {0u, 0u, 0u, 0u};
      u32x4 xb[kMaxHSteps];
#pragma unroll
      for (int ks = 0; ks < kMaxHSteps; ++ks) xb[ks] = ks < nks ? ld_lds16(xs + 32 * ks) : z4;
      f32x4 d = zf4;
#pragma unroll
      for (int ks = 0; ks < kMaxHSteps; ++ks) d = mfma16(af[ks], xb[ks], d);
      s_red[0][wave][lane] = d;
      __syncthreads();
      // Thread (row mm, column n) of the summed tile.
      const int mm = tid >> 4, n = tid & 15;
      auto tile = [&](int row) {
        const int ll = (row >> 2) * 16 + n, ii = row & 3;
        return (s_red[0][0][ll][ii] + s_red[0][1][ll][ii]) + (s_red[0][2][ll][ii] + s_red[0][3][ll][ii]);
      };
      if (n < T && mm < nrow) {
        if (mm < n_r) {
          const int e = r_lo + mm;
          // Scores typed bf16 (the layer's option) are rounded here, before
          // anything reads them.
          const float v = a.L.logits_bf16 ? round_bf16(tile(mm)) : tile(mm);
          if (e < E) {
            // Slot 64 (e % 4) + e / 4 of the token's row: the reader lane that
            // owns experts 4 l .. 4 l + 3 finds them 512 bytes apart, so each
            // of its four loads covers four whole lines.
            const uint64_t tv = ((uint64_t)__float_as_uint(v) << 32) | tag;
            uint64_t* dst = a.logits_t + (size_t)n * 256 + 64 * (e & 3) + (e >> 2);
#pragma unroll
            for (int x = 0; x < kDecodeReplicas; ++x) st_dev(dst + (size_t)x * lstride, tv);
            if (a.logits_out) a.logits_out[(size_t)n * E + e] = v;
          } else {
            st_dev(a.gate_s + n, sigmoidf_(v));
          }
        } else if (mm >= p0 && ((mm - p0) & 1) == 0) {
          const float zg = a.L.logits_bf16 ? round_bf16(tile(n_r)) : tile(n_r);
          const float hv = sigmoidf_(zg) * siluf_(tile(mm)) * tile(mm + 1);
          st_dev(a.h_sh + (size_t)n * Is + s_lo + ((mm - p0) >> 1), (bf16_t)f32_to_bf16(hv));
        }
      }
    }
  }

  // ---------------- wave 3: shared rows (T <= 3), requested ----------------
  // Requested only now, after this workgroup's router rows: the router loads
  // of every workgroup (up to ~1 us apart in start time) reach memory first,
  // and these 4 MB (over the grid) use the otherwise idle time of the logit
  // exchange.  Lane l reads elements 8 l + 512 j .. + 7 of each row.  They
  // are consumed at the start of phase B, so the lists barrier never waits
  // for them.
  u32x4 shw[kLateRows][kLateChunks];
  if (late_wave) {
    const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < kLateRows; ++r) {
      const int p = (r - 1) >> 1;
      const bf16_t* rp = r == 0 ? L.sh_expert_gate
                                : (((r - 1) & 1) ? L.sh_up_w : L.sh_gate_w) + (size_t)(s_lo + min(p, n_s - 1)) * H;
#pragma unroll
      for (int j = 0; j < kLateChunks; ++j) {
        const int e = 8 * lane + 512 * j;
        shw[r][j] = (r == 0 || p < n_s) && e < H ? ldw(rp + e) : z4;
      }
    }
  }
  // Dot products of the gate row and the (gate, up) pairs with each token's x
  // (fixed per-lane order, then a fixed-order wave sum), then
  // h_sh = sigma(zg) SiLU(g) u as in the tile path; published like the rest
  // of h (complete before the hand-off).
  auto late_shared_rows = [&] {
    float acc[kLateRows][kWaves - 1];
#pragma unroll
    for (int r = 0; r < kLateRows; ++r)
#pragma unroll
      for (int t = 0; t < kWaves - 1; ++t) acc[r][t] = 0.f;
#pragma unroll
    for (int j = 0; j < kLateChunks; ++j) {
      const int e = 8 * lane + 512 * j;
      if (e < H) {
#pragma unroll
        for (int t = 0; t < kWaves - 1; ++t) {
          if (t < T) {
            const u32x4 xv = ld_lds16(s_x + t * kXStride + e);
#pragma unroll
            for (int r = 0; r < kLateRows; ++r)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                acc[r][t] += bf16_to_f32(shw[r][j][i] & 0xFFFFu) * bf16_to_f32(xv[i] & 0xFFFFu);
                acc[r][t] += bf16_to_f32(shw[r][j][i] >> 16) * bf16_to_f32(xv[i] >> 16);
              }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kWaves - 1; ++t) {
      if (t < T) {
        float sum[kLateRows];
#pragma unroll
        for (int r = 0; r < kLateRows; ++r) sum[r] = wave_sum_f32(acc[r][t]);
        const float zg = a.L.logits_bf16 ? round_bf16(sum[0]) : sum[0];
#pragma unroll
        for (int p = 0; p < kLateMaxPairs; ++p)
          if (p < n_s && lane == p) {
            const float hv = sigmoidf_(zg) * siluf_(sum[1 + 2 * p]) * sum[2 + 2 * p];
            st_dev(a.h_sh + (size_t)t * Is + s_lo + p, (bf16_t)f32_to_bf16(hv));
          }
      }
    }
  };

  // ---------------- phase K: top-K selections into LDS ----------------
  // Wave w handles tokens w, w + 4, ... (NT of them, lane: experts 4 lane ..
  // 4 lane + 3): it polls their tagged logits (its XCD's copy) until every one
  // carries this call's tag, then selects the top-K of all of them together.
  {
    const rsrc_t r_lt = make_rsrc(a.logits_t + (size_t)xcc * lstride, (size_t)T * 256 * 8);
    auto run = [&](auto nt_tag) {
      constexpr int NT = decltype(nt_tag)::value;
      // Each poll also takes the logits out of the words it checks: the last
      // one, which succeeded (or gave up), leaves them in lv.
      float lv[NT][4];
      auto ready = [&] {
        bool ok = true;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int t = wave + kWaves * j;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int e = 4 * lane + c;
            const bool in = e < E && t < T;
            // One 64-bit load: value and tag come from the same store.
            const auto w2 = __builtin_amdgcn_raw_buffer_load_b64(
                r_lt, in ? 8u * (uint32_t)(t * 256 + 64 * c + lane) : kOutside, 0, 16);
            ok = ok && (!in || w2[0] == tag);
            lv[j][c] = __uint_as_float(w2[1]);
          }
        }
        return __ballot(!ok) == 0ull;
      };
      wait_until(ready, ctl, tag, a.wait_ticks);
      int ix[NT];
      float wv[NT];
      topk_select<NT>(lv, E, K, lane, ix, wv);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int t = wave + kWaves * j;
        if (t < T && lane < K) {
          s_tidx[t * K + lane] = ix[j];
          s_tw[t * K + lane] = wv[j];
          atomicOr(&s_mask[ix[j]], 1u << t);
        }
      }
    };
    if (wave < T) {
      if (T <= kWaves) run(std::integral_constant<int, 1>{});
      else if (T <= 2 * kWaves) run(std::integral_constant<int, 2>{});
      else run(std::integral_constant<int, 4>{});
    }
  }
  // One token of a forward call: wave 0 made every selection and builds the
  // lists itself (its own LDS writes are visible to its later reads), so no
  // barrier separates the two phases and wave 3's shared rows only have to be
  // done by the barrier after phase L.
  const bool solo = T == 1 && !a.route_only;
  if (!solo) __syncthreads();

  // ---------------- phase L: per-expert pair lists in LDS ----------------
  // From the token masks per expert (set with the selections), wave 0 forms
  // the offsets and the touched list (ascending expert) from one scan (low
  // half: pair counts, high half: touched flags), then each pair's slot: its
  // expert's offset plus the number of earlier tokens with that expert.
  //
  // One token (forward): the K selections are distinct and each holds one
  // pair, so the touched list is the selections in ascending order: lane k
  // (k < K) finds the rank of its expert among them, which is its slot; the
  // offsets of a touched expert and of the expert after it are that rank and
  // rank + 1 (the only offsets phases B and C read).
  if (solo && wave == 0) {
    const int ek = lane < K ? s_tidx[lane] : 0x7FFFFFFF;
    int rank = 0;
    for (int j = 0; j < K; ++j) rank += __builtin_amdgcn_readlane(ek, j) < ek ? 1 : 0;
    if (lane < K) {
      s_touched[rank] = ek;
      s_list[rank] = lane;
      s_off[ek] = rank;
    }
    if (lane < K) s_off[ek + 1] = rank + 1;
    if (lane == 0) { s_U = K; s_U01 = 0; }
  } else if (wave == 0) {
    // Second scan: touched flags per token group (tokens 0-7 low half, 8-15
    // high half) for phase C with T > 8.
    int v4[4], g4[4], run = 0, grun = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      const uint32_t mk = e < E ? s_mask[e] : 0u;
      const int c = __popc(mk);
      v4[j] = c | ((c > 0 ? 1 : 0) << 16);
      g4[j] = ((mk & 0xFFu) ? 1 : 0) | ((mk & 0xFF00u) ? 1 << 16 : 0);
      run += v4[j];
      grun += g4[j];
    }
    const int incl = wave_incl_scan(run, lane);
    const int gincl = wave_incl_scan(grun, lane);
    int ex = incl - run, gx = gincl - grun;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      if (e < E) {
        s_off[e] = ex & 0xFFFF;
        if (v4[j] & 0xFFFF) s_touched[ex >> 16] = e;
        if (g4[j] & 0xFFFF) s_tl[0][gx & 0xFFFF] = e;
        if (g4[j] >> 16) s_tl[1][gx >> 16] = e;
      }
      ex += v4[j];
      gx += g4[j];
    }
    if (lane == 63) { s_off[E] = incl & 0xFFFF; s_U = incl >> 16; s_U01 = gincl; }
    // The wave's own LDS writes above are visible to its reads below.
    for (int q = lane; q < TK; q += kWave) {
      const int e = s_tidx[q], t = q / K;
      s_list[s_off[e] + __popc(s_mask[e] & ((1u << t) - 1u))] = q;
    }
  }
  __syncthreads();

  if (a.route_only) {
    if (wg == 0) {
      for (int e = tid; e <= E; e += kThreads) a.offsets_out[e] = s_off[e];
      for (int q = tid; q < TK; q += kThreads) {
        a.perm_out[q] = s_list[q];
        a.topk_idx[q] = s_tidx[q];
        a.topk_w[q] = s_tw[q];
      }
    }
    return;
  }
  const int U = s_U;


  // Phase C geometry (its first weights are requested during phase B).
  // Workgroup wg owns output rows [row0, row0 + nrows), nrows <= 8.  Its down
  // projection is one contraction over (segment, inner index) -- segment 0 the
  // shared expert, segment 1 + u the u-th touched expert -- with tokens as
  // tile columns, so every stage adds into the same accumulator tile.  A tile
  // has two 8-row halves: row 8 h + r is output row r, column 8 h + j token
  // tb(h) + j, and only the two diagonal 8 x 8 blocks of the product are used.
  // With T <= 8 the halves take different experts (stage s >= 1: touched
  // experts 2 (s - 1) + h), tb = 0, and the diagonal blocks are added at the
  // end; with T > 8, tb(h) = 8 h and half h takes the (s - 1)-th expert
  // touched by its own eight tokens.  Stage 0 is the shared expert (with
  // T <= 8 in half 0 only; h_sh carries its gate, h the routing weight).
  // Wave w takes k-steps [4 w, 4 w + 4) of the inner dimension.
  const bool split_tok = T > 8;
  const int U0 = s_U01 & 0xFFFF, U1 = s_U01 >> 16;
  const int NS = 1 + (split_tok ? max(U0, U1) : (U + 1) / 2);
  // Expert of half h at stage s >= 1, or -1.
  auto stage_expert = [&](int s, int h) -> int {
    if (split_tok) {
      const int j = s - 1;
      return j < (h ? U1 : U0) ? s_tl[h][j] : -1;
    }
    const int j = 2 * (s - 1) + h;
    return j < U ? s_touched[j] : -1;
  };
  const int rpw = (H + G - 1) / G;
  const int row0 = wg * rpw, nrows = max(0, min(rpw, H - row0));
  const int hm = m >> 3, rm = m & 7;     // this lane's A-row (and B-column) half and index in it
  const bool row_ok = rm < nrows;
  const int crow = min(row0 + rm, H - 1);
  u32x4 ca[kCDepth][kMaxISteps], cb[kCDepth][kMaxISteps];
  const rsrc_t r_dn = make_rsrc(L.down_w, (size_t)E * H * I * 2);
  const rsrc_t r_sdn = make_rsrc(L.sh_down_w, (size_t)H * Is * 2);
  // Down-projection weights of stage s for this lane's row (zeros from
  // outside the resource for stages past the last, empty halves, rows past
  // nrows and k-steps past the inner size).
  // MFMA step ks (32 wide) is half ks & 1 of the 64-wide step ks >> 1, lane
  // quarter q holding its elements 16 q + 8 (ks & 1) .. + 7: in row-major
  // weights 16 bytes of the row, in the tile layout 16 bytes of the 1 KB that
  // half occupies.
  auto issue_a = [&](u32x4 (&st)[kMaxISteps], int s) {
    uint32_t off = kOutside, ks2 = 128u, ks1 = 16u;
    if (row_ok && s < NS) {
      if (s == 0) {
        if (split_tok || hm == 0) off = 2u * (uint32_t)(crow * Is + 2 * kq);
      } else {
        const int e = stage_expert(s, hm);
        if (e >= 0) {
          if (L.tiled) {
            off = 2u * (uint32_t)(e * H * I) + 2048u * (uint32_t)((crow >> 4) * (I / 64)) +
                  16u * (uint32_t)(2 * kq + (crow & 15));
            ks2 = 2048u;
            ks1 = 1024u;
          } else {
            off = 2u * (uint32_t)((e * H + crow) * I + 2 * kq);
          }
        }
      }
    }
    const rsrc_t rs = s == 0 ? r_sdn : r_dn;
    const int nk = (s == 0 ? Is : I) / 32;
#pragma unroll
    for (int s4 = 0; s4 < kMaxISteps; ++s4) {
      const int ks = kMaxISteps * wave + s4;
      st[s4] = ldw_buf(rs, ks < nk ? off + ks2 * (uint32_t)(ks >> 1) + ks1 * (uint32_t)(ks & 1) : kOutside);
    }
  };

  // ---------------- phase B: routed gate/up blocks ----------------
  // Block b = (touched expert u = b / (I/8), inner rows i0 = 8 (b % (I/8)) ..
  // i0 + 7); workgroup wg takes blocks wg, wg + G, ...  Tile row 4j + i holds
  // the gate row (i < 2) or the up row (i >= 2) of inner row i0 + 2j + (i & 1),
  // so a lane's four accumulator rows are (g_a, g_b, u_a, u_b) of two inner rows.
  {
    const int nbi = I / 8;
    const int NB = U * nbi;
    const int nmine = NB > wg ? (NB - wg + G - 1) / G : 0;
    u32x4 wa[kBDepth][kMaxHSteps];
    const rsrc_t r_gu = make_rsrc(L.gate_up_w, (size_t)E * 2 * I * H * 2);
    // Stage loads are issued unconditionally: past the last block, and for
    // k-steps past H / 4, the offsets fall outside the resource.
    // MFMA step ks is half ks & 1 of this wave's 64-wide step ks >> 1 (lane
    // quarter q: elements 16 q + 8 (ks & 1) .. + 7), for row-major and tiled
    // weights alike.
    const uint32_t ks2 = L.tiled ? 2048u : 128u, ks1 = L.tiled ? 1024u : 16u;
    auto issue = [&](u32x4 (&st)[kMaxHSteps], int i) {
      uint32_t off = kOutside;
      if (i < nmine) {
        const int b = wg + i * G, u = b / nbi, i0 = 8 * (b - u * nbi);
        const int e = s_touched[u];
        const int r = ((m & 2) ? I : 0) + i0 + 2 * (m >> 2) + (m & 1);   // row of the expert's [2I, H]
        if (L.tiled)
          off = 2u * (uint32_t)(e * 2 * I * H) + 2048u * (uint32_t)((r >> 4) * (H / 64) + kbeg / 64) +
                16u * (uint32_t)(2 * kq + (r & 15));
        else
          off = 2u * (uint32_t)((e * 2 * I + r) * H + kbeg + 2 * kq);
      }
#pragma unroll
      for (int ks = 0; ks < kMaxHSteps; ++ks)
        st[ks] = ldw_buf_nt(r_gu, ks < nks ? off + ks2 * (uint32_t)(ks >> 1) + ks1 * (uint32_t)(ks & 1) : kOutside);
    };
    auto compute = [&](u32x4 (&st)[kMaxHSteps], int i) {
      if (i < nmine) {
        const int b = wg + i * G, u = b / nbi, i0 = 8 * (b - u * nbi);
        const int e = s_touched[u], beg = s_off[e], cnt = s_off[e + 1] - beg;
        const int t = s_list[beg + min(m, cnt - 1)] / K;
        const bf16_t* xs = s_x + t * kXStride + kbeg + 2 * kq;
        u32x4 xb[kMaxHSteps];
#pragma unroll
        for (int ks = 0; ks < kMaxHSteps; ++ks) {
          const int kc = min(ks, nks - 1);
          xb[ks] = ld_lds16(xs + 64 * (kc >> 1) + 8 * (kc & 1));
        }
        f32x4 d = zf4;
#pragma unroll
        for (int ks = 0; ks < kMaxHSteps; ++ks) d = mfma16(st[ks], xb[ks], d);
        s_red[i & 1][wave][lane] = d;
        __syncthreads();
        if (wave == 0 && m < cnt) {
          const f32x4 p0 = s_red[i & 1][0][lane], p1 = s_red[i & 1][1][lane];
          const f32x4 p2 = s_red[i & 1][2][lane], p3 = s_red[i & 1][3][lane];
          const f32x4 sum = (p0 + p1) + (p2 + p3);
          const int q = s_list[beg + m];
          const float w = s_tw[q];
          const float ha = siluf_(sum[0]) * sum[2] * w, hb = siluf_(sum[1]) * sum[3] * w;
          st_dev(reinterpret_cast<uint32_t*>(a.h + (size_t)q * I + i0 + 2 * (lane >> 4)), pack_bf16x2(ha, hb));
        }
      }
    };
    static_assert(kBDepth == 2, "the loop below is unrolled for two stages");
    if (late_wave) late_shared_rows();
    issue(wa[0], 0);
    issue(wa[1], 1);
    // Phase C's B operands: for every stage and tile column the row of h
    // (routed: the pair of that expert and token) or of h_sh (stage 0), or -1.
    // Read after the hand-off barrier.
    for (int i = tid; i < NS * 16; i += kThreads) {
      const int sg = i >> 4, n = i & 15, hb = n >> 3;
      const int t = (split_tok ? 8 * hb : 0) + (n & 7);
      int q = -1;
      if (t < T) {
        if (sg == 0) {
          if (split_tok || hb == 0) q = t;
        } else {
          const int e = stage_expert(sg, hb);
          if (e >= 0) {
            const uint32_t mk = s_mask[e];
            if ((mk >> t) & 1u) q = s_list[s_off[e] + __popc(mk & ((1u << t) - 1u))];
          }
        }
      }
      s_cq[i] = q;
    }
    // The first down-projection stages do not depend on h and are needed
    // only after the hand-off: they are requested once this workgroup's first
    // gate/up block has arrived, so that they do not compete with the gate/up
    // streams that everything waits for.
    compute(wa[0], 0);
#pragma unroll
    for (int s = 0; s < kCDepth; ++s) issue_a(ca[s], s);
    issue(wa[0], 2);
    compute(wa[1], 1);
    issue(wa[1], 3);
    for (int i = 2; i < nmine; i += 2) {
      compute(wa[0], i);
      issue(wa[0], i + 2);
      compute(wa[1], i + 1);
      issue(wa[1], i + 3);
    }
  }

  // ---------------- h hand-off ----------------
  // Every wave's stores (h, and h_sh from phase A) are complete, then wave 0
  // writes the tag into this workgroup's slot of every flag copy and waits
  // until all G slots of its XCD's copy carry it (lane l reads slots
  // 4 l .. 4 l + 3); the barrier releases the other waves.
  stores_complete();
  __syncthreads();
  // Rows of h for the first stages of phase C, read while the hand-off waits
  // (the table was completed before the barrier above).
  auto cq = [&](int s) {
    const int q = s_cq[min(s, kMaxCStages - 1) * 16 + m];
    return s < NS ? q : -1;
  };
  int q0[kCDepth];
#pragma unroll
  for (int s = 0; s < kCDepth; ++s) q0[s] = cq(s);
  if (wave == 0) {
    if (lane < kDecodeReplicas) st_dev(ctl + kCtlFlags + lane * kDecodeFlagStride + wg, tag);
    const rsrc_t r_fl = make_rsrc(ctl + kCtlFlags + xcc * kDecodeFlagStride, (size_t)G * 4);
    wait_until(
        [&] {
          const auto f = __builtin_amdgcn_raw_buffer_load_b128(r_fl, 16u * (uint32_t)lane, 0, 16);
          bool ok = true;
#pragma unroll
          for (int c = 0; c < 4; ++c) ok = ok && (4 * lane + c >= G || f[c] == tag);
          return __ballot(!ok) == 0ull;
        },
        ctl, tag, a.wait_ticks);
  }
  __syncthreads();

  // ---------------- phase C: down projection and combine ----------------
  {
    const rsrc_t r_h = make_rsrc(a.h, (size_t)TK * I * 2);
    const rsrc_t r_hsh = make_rsrc(a.h_sh, (size_t)T * Is * 2);
    // h fragments of stage s for this lane's column (h row q, or none).
    auto issue_b = [&](u32x4 (&st)[kMaxISteps], int s, int q) {
      const int inner = s == 0 ? Is : I, nk = inner / 32;
      const uint32_t row = q >= 0 ? 2u * (uint32_t)(q * inner) : kOutside;
      const rsrc_t rs = s == 0 ? r_hsh : r_h;
#pragma unroll
      for (int s4 = 0; s4 < kMaxISteps; ++s4) {
        const int ks = kMaxISteps * wave + s4;
        st[s4] = ld_after16(rs, ks < nk ? row + 2u * (uint32_t)(64 * (ks >> 1) + 8 * (ks & 1) + 2 * kq) : kOutside);
      }
    };
    // Two accumulators (even and odd k-steps) halve the MFMA dependency chain.
    f32x4 acc0 = zf4, acc1 = zf4;
    static_assert(kMaxISteps == 4, "compute() below takes four k-steps");
    auto compute = [&](u32x4 (&sa)[kMaxISteps], u32x4 (&sb)[kMaxISteps]) {
      acc0 = mfma16(sa[0], sb[0], acc0);
      acc1 = mfma16(sa[1], sb[1], acc1);
      acc0 = mfma16(sa[2], sb[2], acc0);
      acc1 = mfma16(sa[3], sb[3], acc1);
    };
    static_assert(kCDepth == 6, "the loop below is unrolled for six stages");
#pragma unroll
    for (int s = 0; s < kCDepth; ++s) issue_b(cb[s], s, q0[s]);
    if (NS <= kCDepth) {
      // Every stage is already in flight (one or a few tokens).
#pragma unroll
      for (int s = 0; s < kCDepth; ++s) compute(ca[s], cb[s]);
    } else {
      for (int g0 = 0; g0 < NS; g0 += kCDepth) {
#pragma unroll
        for (int s = 0; s < kCDepth; ++s) {
          compute(ca[s], cb[s]);
          const int sn = g0 + s + kCDepth;
          issue_a(ca[s], sn);
          issue_b(cb[s], sn, cq(sn));
        }
      }
    }
    // The four waves' partial tiles, summed in a fixed order.  Element
    // (i, j) of a tile is component i % 4 of lane 16 (i / 4) + j.
    s_red[0][wave][lane] = acc0 + acc1;
    __syncthreads();
    if (tid < nrows * T) {
      const int rr = tid / T, t = tid - rr * T;
      auto el = [&](int i, int j) {
        const int l = 16 * (i >> 2) + j, c = i & 3;
        return (s_red[0][0][l][c] + s_red[0][1][l][c]) + (s_red[0][2][l][c] + s_red[0][3][l][c]);
      };
      float v = split_tok ? (t < 8 ? el(rr, t) : el(8 + rr, t)) : el(rr, t) + el(8 + rr, 8 + t);
      if (a.residual) v = bf16_to_f32(a.residual[(size_t)t * H + row0 + rr]) + v;   // sub-block residual
      a.out[(size_t)t * H + row0 + rr] = (bf16_t)f32_to_bf16(v);
    }
  }
}

}  // namespace

// Plain launch of one workgroup per CU: with the device otherwise idle every
// workgroup is resident at once.  Should some not be (other kernels holding
// CUs), the bounded waits still let every wave finish, and the control block
// records the call as timed out (moe_workspace_status reports it).  A
// cooperative launch would guarantee residency, but measured 38 us per
// one-token call against 20.4 us for this one on MI355X.
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

bool decode_fits(int H, int E, int Is, int grid) {
  if (grid < 1 || grid > kDecodeMaxGrid) return false;
  const int rows_a = (E + 1 + grid - 1) / grid + 1 + 2 * ((Is + grid - 1) / grid);
  const int rows_c = (H + grid - 1) / grid;
  return rows_a <= 16 && rows_c <= 8;
}

}  // namespace moe
