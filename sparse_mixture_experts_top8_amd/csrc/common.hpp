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

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }
__device__ __forceinline__ float siluf_(float z) { return z / (1.0f + __expf(-z)); }

// ---- wavefront reductions on DPP lane moves (no LDS traffic) ----
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror and row_mirror
// combine lanes inside each 16-lane row (after the four steps every lane of a
// row holds the row's result); the four row results are then read into
// scalar registers and combined, so every lane returns the same value.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
__device__ __forceinline__ float row_lane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return (row_lane_f(v, 0) + row_lane_f(v, 16)) + (row_lane_f(v, 32) + row_lane_f(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return fmaxf(fmaxf(row_lane_f(v, 0), row_lane_f(v, 16)), fmaxf(row_lane_f(v, 32), row_lane_f(v, 48)));
}

__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<0xB1>(v));
  v = min(v, dpp_i<0x4E>(v));
  v = min(v, dpp_i<0x141>(v));
  v = min(v, dpp_i<0x140>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Arg-max over the wave under the order (higher value, then lower index):
// lane-local candidates (bv, bi) in, the winner's value and index out (uniform).
__device__ __forceinline__ void wave_argmax(float bv, int bi, float* v_out, int* i_out) {
  const float m = wave_max(bv);
  *i_out = wave_min_i(bv == m ? bi : 0x7FFFFFFF);
  *v_out = m;
}

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// Top-K of NT tokens by one wave (independent chains, interleaved), from each
// lane's four logits of experts 4 lane + c: descending logit, ties to the
// lower expert index (the lowest lane among equal lane bests, the lowest c
// inside a lane); lane k < K receives the k-th index and its weight, the
// softmax over the selected logits (equal to the full softmax renormalised).
// A validity mask (experts < E, not yet taken) keeps every pick distinct even
// among equal or -inf values; NaN counts as -inf.
template <int NT>
__device__ __forceinline__ void topk_select(const float (&lv)[NT][4], int E, int K, int lane, int (&idx_out)[NT],
                                            float (&w_out)[NT]) {
  float v[NT][4];
  uint32_t valid[NT];
  float vmax[NT], den[NT], mine_v[NT];
  int mine_i[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    valid[j] = 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[j][c] = lv[j][c] == lv[j][c] ? lv[j][c] : -INFINITY;
      if (4 * lane + c < E) valid[j] |= 1u << c;
    }
    vmax[j] = 0.f;
    den[j] = 0.f;
    mine_v[j] = 0.f;
    mine_i[j] = 0;
  }
  for (int k = 0; k < K; ++k) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      float bv = -INFINITY;
      int bc = -1;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (((valid[j] >> c) & 1u) && (bc < 0 || v[j][c] > bv)) { bv = v[j][c]; bc = c; }
      const float mx = wave_max(bv);
      const unsigned long long win = __ballot(bc >= 0 && bv == mx);
      const int wl = (int)__builtin_ctzll(win);
      const int wc = __builtin_amdgcn_readlane(bc, wl);
      if (lane == wl) valid[j] &= ~(1u << wc);
      if (k == 0) vmax[j] = mx;
      den[j] += __expf(mx - vmax[j]);
      if (lane == k) { mine_v[j] = mx; mine_i[j] = 4 * wl + wc; }
    }
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    idx_out[j] = clamp_expert(mine_i[j], E);
    w_out[j] = __expf(mine_v[j] - vmax[j]) / den[j];
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
  int4* tdesc_gu;      // per gate_up tile: group, first slot, rows, row tile | column tile << 16
  int4* tdesc_dn;      // per down tile, same
  int32_t* perm;       // [T*K]
  int32_t* slot_tok;   // [T*K]  token of each slot (perm / K)
  int32_t* slot_of;    // [T*K]
  bf16_t* h;           // [T*K, I]
  bf16_t* h_sh;        // [T, Is]
  bf16_t* y;           // [T*K + T, H]  weighted expert outputs, routed slots then shared rows
};

}  // namespace moe
