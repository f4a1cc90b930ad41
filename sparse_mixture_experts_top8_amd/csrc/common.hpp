// Shared device helpers for the gfx950 MoE kernels: bf16 codec, MFMA operand
// types, wave-level reductions and the workspace descriptor.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bfloat16 bit pattern
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float -> bf16 (inputs finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// The bf16 value nearest to f (ties to even), as a float.
__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }
__device__ __forceinline__ float siluf_(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// Orderable 32-bit key of a logit: a larger logit has a larger key, NaN counts
// as -inf and -0 as +0, so two keys are equal exactly when the logits compare
// equal.  Every key is >= key(-inf) = 0x007FFFFF, above the 0 used for
// experts that do not exist (and for candidates already taken).
__device__ __forceinline__ uint32_t logit_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (f != f) b = 0xFF800000u;
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
// Maximum of an unsigned value over the wave, in every lane: four DPP steps
// inside each 16-lane row (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror), then the four row results through scalar
// registers.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<0xB1>(v));
  v = max(v, dpp_u<0x4E>(v));
  v = max(v, dpp_u<0x141>(v));
  v = max(v, dpp_u<0x140>(v));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Sum of a float over the wave, in every lane, in a fixed order: four DPP
// steps inside each 16-lane row (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror), then the four row sums.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Top-K (K <= 8) of NT tokens by one wave (independent chains, interleaved),
// from each lane's four logits of experts 4 lane + c: order by descending
// logit, ties to the lower expert index; lane k < K receives the k-th index
// and its weight, the softmax over the selected logits (equal to the full
// softmax renormalised over them), its denominator summed in rank order
// (lanes >= K receive a weight they do not use).
//
// Each lane first sorts its four keys (descending, lower c first among equal
// keys), so its best remaining candidate is always its head.  A pick is the
// wave maximum of the heads; among equal heads the lowest lane wins, which is
// the lowest expert index (a lane holding that key anywhere holds it at its
// head).  The winner's head then moves on to its next key.
template <int NT>
__device__ __forceinline__ void topk_select(const float (&lv)[NT][4], int E, int K, int lane, int (&idx_out)[NT],
                                            float (&w_out)[NT]) {
  uint32_t hk[NT][4];   // this lane's keys, sorted; 0 once used up (below every key)
  uint32_t hc[NT];      // their c, two bits each, head in the low bits
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    uint32_t k[4];
    int c[4] = {0, 1, 2, 3};
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = 4 * lane + i < E ? logit_key(lv[j][i]) : 0u;
    // Five compare-exchanges; (key, c) compared as key descending, c ascending.
    auto cx = [&](int a, int b) {
      const bool sw = k[b] > k[a] || (k[b] == k[a] && c[b] < c[a]);
      const uint32_t ka = k[a], kb = k[b];
      const int ca = c[a], cb = c[b];
      k[a] = sw ? kb : ka; k[b] = sw ? ka : kb;
      c[a] = sw ? cb : ca; c[b] = sw ? ca : cb;
    };
    cx(0, 1); cx(2, 3); cx(0, 2); cx(1, 3); cx(1, 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) hk[j][i] = k[i];
    hc[j] = (uint32_t)(c[0] | (c[1] << 2) | (c[2] << 4) | (c[3] << 6));
  }
  uint32_t my_key[NT], my_idx[NT], first_key[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) { my_key[j] = 0u; my_idx[j] = 0u; first_key[j] = 0u; }
  for (int k = 0; k < K; ++k) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint32_t m = wave_max_u32(hk[j][0]);
      const int wl = (int)__builtin_ctzll(__ballot(hk[j][0] == m));
      const uint32_t wc = (uint32_t)__builtin_amdgcn_readlane((int)hc[j], wl) & 3u;
      const bool won = lane == wl;
      hk[j][0] = won ? hk[j][1] : hk[j][0];
      hk[j][1] = won ? hk[j][2] : hk[j][1];
      hk[j][2] = won ? hk[j][3] : hk[j][2];
      hk[j][3] = won ? 0u : hk[j][3];
      hc[j] = won ? hc[j] >> 2 : hc[j];
      if (k == 0) first_key[j] = m;
      if (lane == k) { my_key[j] = m; my_idx[j] = 4u * (uint32_t)wl + wc; }
    }
  }
  // Lane k < K holds the k-th pick: its softmax numerator is formed in every
  // lane at once, and the denominator summed in rank order from them (the
  // exponentials stay off the selection's dependent chain).
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const float num = lane < K ? __expf(key_logit(my_key[j]) - key_logit(first_key[j])) : 0.f;
    float den = 0.f;
    for (int k = 0; k < K; ++k) den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(num), k));
    idx_out[j] = clamp_expert((int)my_idx[j], E);
    w_out[j] = num / den;
  }
}

// 16-byte global load/store as four dwords.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// Device-side view of one layer and one call.
struct LayerArgs {
  int H, E, K, I, Is;
  const bf16_t* router_w;       // [E, H]
  const bf16_t* gate_up_w;      // [E, 2I, H]
  const bf16_t* down_w;         // [E, H, I]
  const bf16_t* sh_gate_w;      // [Is, H]
  const bf16_t* sh_up_w;        // [Is, H]
  const bf16_t* sh_down_w;      // [H, Is]
  const bf16_t* sh_expert_gate; // [H]
  int logits_bf16;              // 1: router and shared-gate scores rounded to bf16
  int tiled;                    // 1: routed expert weights in the MFMA-tile layout
};

// Carved workspace (all device pointers).
struct Work {
  int32_t* topk_idx;   // [T*K]
  float* topk_w;       // [T*K]
  float* gate_s;       // [T]
  float* rlog;         // [ksplit, T, router_cols(E)]  router partial sums (column E: shared gate)
  int32_t* blk_counts; // [nblk * E]  router-block histograms, then block bases
  int32_t* offsets;    // [E + 1]
  int32_t* tiles_gu;   // [E + 2]   prefix of gate_up tiles per group (group E = shared)
  int32_t* tiles_dn;   // [E + 2]   prefix of down tiles per group
  int32_t* claims;     // [2][8][32] persistent GEMMs' claim counters (gate_up, down), one per XCD, 128 bytes apart
  int4* tdesc_gu;      // per gate_up tile: group, first slot, rows, row tile | column tile << 16
  int4* tdesc_dn;      // per down tile, same
  int32_t* perm;       // [T*K]
  int32_t* slot_tok;   // [T*K]  token of each slot (perm / K)
  int32_t* slot_of;    // [T*K]
  bf16_t* h;           // [T*K, I]  (its first E words hold the pairs per expert during the multi-launch dispatch)
  bf16_t* h_sh;        // [T, Is]
  bf16_t* y;           // [T*K + T, H]  weighted expert outputs, routed slots then shared rows
  float* psum;         // [nblk * E]  per router block: sum over its tokens of each expert's softmax probability
  int32_t* st_list;    // [E + 1]  streamed experts: touched experts ascending, then their count
  int32_t* st_slot;    // [E]      cache slot of each touched expert (-1 if untouched)
  int32_t* st_win_gu;  // [E][4]   per round: routed tile range and shared tile range (gate_up)
  int32_t* st_win_dn;  // [E][4]   the same for the down projection
  bf16_t* xn;          // [T, H]  RMSNorm of the sub-block input (block form)
  uint32_t* ctl;       // control block at the start of the workspace (kCtlLast is written)
  uint64_t* lt;        // tagged exchange region after it (fused small-batch route: logits, selections)
  uint32_t call_tag;   // this call's tag
};

}  // namespace moe
