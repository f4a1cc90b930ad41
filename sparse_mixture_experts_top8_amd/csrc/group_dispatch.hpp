// One group's share of the dispatch of a small batch: the workgroup of
// group g (E: the shared expert) holds all T K selections (kPer per thread,
// pair q = tid + 256 j; -1 past T K), builds the expert counts and the three
// exclusive prefix sums in LDS, then writes its own group's offset, tile
// counts and tile descriptors and, for a routed expert, places its pairs:
// tokens pick an expert at most once, so a pair's rank among the expert's
// pairs (in pair-id order) is the number of earlier tokens that picked the
// expert, the population of the expert's token mask below the token.  The
// slots equal those of the other dispatch paths.  Workgroup 0 also zeroes
// the persistent GEMMs' claim counters.  Used by the per-group dispatch
// kernel and by the fused small-batch route.
#pragma once

#include "kernels.hpp"

namespace moe {

constexpr int kGroupThreads = 256;
constexpr int kGroupTokens = 2048;   // token mask words: kGroupTokens / 32

template <int kPer>
__device__ void dispatch_group(const LayerArgs& L, int T, const Work& w, int g, const int (&idx)[kPer]) {
  __shared__ int s_cnt[256], s_off[257], s_tgu[258], s_tdn[258];
  __shared__ uint32_t s_tmask[kGroupTokens / 32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = L.E, K = L.K;
  const int bmg = gemm_bm(T, K, E, true), bng = gemm_bn(T, K, E, true);
  const int bmd = gemm_bm(T, K, E, false), bnd = gemm_bn(T, K, E, false);
  for (int e = tid; e < E; e += kGroupThreads) s_cnt[e] = 0;
  for (int i = tid; i < (T + 31) / 32; i += kGroupThreads) s_tmask[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (idx[j] < 0) continue;
    atomicAdd(&s_cnt[idx[j]], 1);
    if (idx[j] == g) {
      const int t = (tid + j * kGroupThreads) / K;
      atomicOr(&s_tmask[t >> 5], 1u << (t & 31));
    }
  }
  __syncthreads();
  // Segment offsets and tile prefix sums (one wave per quantity, 256 experts
  // as four per lane; group E is the shared expert with T rows).
  if (wave < 3) {
    int v[4], run = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      const int cnt = e < E ? s_cnt[e] : 0;
      v[j] = wave == 0 ? cnt
                       : (wave == 1 ? ((cnt + bmg - 1) / bmg) * ((2 * L.I + bng - 1) / bng)
                                    : ((cnt + bmd - 1) / bmd) * (L.H / bnd));
      run += v[j];
    }
    int incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(incl, o, 64);
      if (lane >= o) incl += n;
    }
    int ex = incl - run;
    int* dst = wave == 0 ? s_off : (wave == 1 ? s_tgu : s_tdn);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      if (e < E) dst[e] = ex;
      ex += v[j];
    }
    if (lane == 63) {
      dst[E] = incl;
      if (wave == 1) dst[E + 1] = incl + ((T + bmg - 1) / bmg) * ((2 * L.Is + bng - 1) / bng);
      if (wave == 2) dst[E + 1] = incl + ((T + bmd - 1) / bmd) * (L.H / bnd);
    }
  }
  __syncthreads();
  const bool shared = g == E;
  if (tid == 0) {
    w.offsets[g] = s_off[g];
    w.tiles_gu[g] = s_tgu[g];
    w.tiles_dn[g] = s_tdn[g];
    if (shared) {
      w.tiles_gu[E + 1] = s_tgu[E + 1];
      w.tiles_dn[E + 1] = s_tdn[E + 1];
    }
  }
  if (g == 0 && tid < 16) w.claims[32 * tid] = 0;   // claim counters of the persistent GEMMs
  // This group's tile descriptors, in gemm_tile_order.
  const int seg0 = shared ? 0 : s_off[g];
  const int nrows = shared ? T : s_cnt[g];
  const int mtg = (nrows + bmg - 1) / bmg, mtd = (nrows + bmd - 1) / bmd;
  const int ngu = (2 * (shared ? L.Is : L.I) + bng - 1) / bng, ndn = L.H / bnd;
  const int rbg = gemm_row_block(T, K, E, true), rbd = gemm_row_block(T, K, E, false);
  for (int i = tid; i < mtg * ngu; i += kGroupThreads) {
    int mi, nt;
    gemm_tile_order(i, mtg, ngu, rbg, mi, nt);
    w.tdesc_gu[s_tgu[g] + i] = make_int4(g, seg0, nrows, mi | (nt << 16));
  }
  for (int i = tid; i < mtd * ndn; i += kGroupThreads) {
    int mi, nt;
    gemm_tile_order(i, mtd, ndn, rbd, mi, nt);
    w.tdesc_dn[s_tdn[g] + i] = make_int4(g, seg0, nrows, mi | (nt << 16));
  }
  if (shared) return;
  // Placement of this expert's pairs.
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (idx[j] != g) continue;
    const int q = tid + j * kGroupThreads, t = q / K;
    int rank = __popc(s_tmask[t >> 5] & ((1u << (t & 31)) - 1u));
    for (int i = 0; i < (t >> 5); ++i) rank += __popc(s_tmask[i]);
    const int slot = seg0 + rank;
    w.perm[slot] = q;
    w.slot_of[q] = slot;
    w.slot_tok[slot] = t;
  }
}

}  // namespace moe
