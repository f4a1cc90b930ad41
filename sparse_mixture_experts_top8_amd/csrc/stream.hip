// Routed-expert streaming on gfx950: the routed experts' weights live in
// pinned host memory and only the experts a batch routes to are brought into
// a device cache of C slots, driven by the routing result on the device (no
// host round trip).
//
// Placement hierarchy: "One Token Through Qwen3.6" (InferedThoughts), Where
// the Weights Live (weights staged from storage through system RAM into GPU
// memory; later versions make that hierarchy explicit) and One Complete
// Decode Step (routing decides which expert weights a layer actually needs).
//
// After dispatch, stream_plan_kernel (one workgroup) lists the touched
// experts in ascending order (rank u = number of touched experts below e),
// gives expert e the slot u mod C, and cuts the touched list into rounds of
// C experts.  Round r's GEMM tiles are one contiguous range of the dispatch
// tile list (tiles are ordered by expert), written as a window {first tile,
// count, shared first tile, shared count}; round 0 also carries the shared
// expert's tiles.  stream_copy_kernel(r) copies round r's experts from host
// memory into their slots (32 KB per workgroup, 16-byte loads, all in flight
// before the stores); the grouped GEMMs of round r then read the slots.
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kCopyChunk = 32768;                 // bytes per workgroup
constexpr int kCopyPerThread = kCopyChunk / (256 * 16);

__global__ __launch_bounds__(256) void stream_plan_kernel(LayerArgs L, Work w, int C, int R) {
  __shared__ int s_scan[256];
  __shared__ int s_list[256];
  const int tid = threadIdx.x, E = L.E;
  const int touched = (tid < E && w.offsets[tid + 1] > w.offsets[tid]) ? 1 : 0;
  // Inclusive scan of the touched flags over the 256 threads.
  s_scan[tid] = touched;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const int v = tid >= d ? s_scan[tid - d] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  const int U = s_scan[255];
  const int u = s_scan[tid] - touched;
  if (tid < E) {
    w.st_slot[tid] = touched ? u % C : -1;
    if (touched) {
      w.st_list[u] = tid;
      s_list[u] = tid;
    }
  }
  if (tid == 0) w.st_list[E] = U;
  __syncthreads();
  // Round r: the experts of ranks [r C, min(r C + C, U)), whose tiles run from
  // the first tile of the lowest to the end of the highest.
  for (int r = tid; r < R; r += 256) {
    const int a = r * C, b = min(a + C, U);
    int lo_gu = 0, n_gu = 0, lo_dn = 0, n_dn = 0;
    if (a < b) {
      const int e_lo = s_list[a], e_hi = s_list[b - 1];
      lo_gu = w.tiles_gu[e_lo];
      n_gu = w.tiles_gu[e_hi + 1] - lo_gu;
      lo_dn = w.tiles_dn[e_lo];
      n_dn = w.tiles_dn[e_hi + 1] - lo_dn;
    }
    reinterpret_cast<int4*>(w.st_win_gu)[r] =
        make_int4(lo_gu, n_gu, w.tiles_gu[E], r == 0 ? w.tiles_gu[E + 1] - w.tiles_gu[E] : 0);
    reinterpret_cast<int4*>(w.st_win_dn)[r] =
        make_int4(lo_dn, n_dn, w.tiles_dn[E], r == 0 ? w.tiles_dn[E + 1] - w.tiles_dn[E] : 0);
  }
}

// Round r: workgroup (j, i) copies chunk j of the i-th expert of the round
// (gate_up bytes first, then down) from host memory into slot i.
__global__ __launch_bounds__(256) void stream_copy_kernel(const char* __restrict__ host_gu,
                                                          const char* __restrict__ host_dn, char* __restrict__ slot_gu,
                                                          char* __restrict__ slot_dn, const int* __restrict__ list,
                                                          int E, int C, int r, size_t gu_bytes, size_t dn_bytes) {
  const int i = blockIdx.y;
  const int rank = r * C + i;
  if (rank >= list[E]) return;   // fewer experts in this round
  const int e = list[rank];
  const size_t off = (size_t)blockIdx.x * kCopyChunk;
  const char* src;
  char* dst;
  if (off < gu_bytes) {
    src = host_gu + (size_t)e * gu_bytes + off;
    dst = slot_gu + (size_t)i * gu_bytes + off;
  } else {
    src = host_dn + (size_t)e * dn_bytes + (off - gu_bytes);
    dst = slot_dn + (size_t)i * dn_bytes + (off - gu_bytes);
  }
  u32x4 v[kCopyPerThread];
#pragma unroll
  for (int k = 0; k < kCopyPerThread; ++k) v[k] = ld16(src + 16 * (threadIdx.x + 256 * k));
#pragma unroll
  for (int k = 0; k < kCopyPerThread; ++k) st16(dst + 16 * (threadIdx.x + 256 * k), v[k]);
}

}  // namespace

hipError_t launch_stream_plan(const LayerArgs& L, const Work& w, int C, int R, hipStream_t s) {
  hipLaunchKernelGGL(stream_plan_kernel, dim3(1), dim3(256), 0, s, L, w, C, R);
  return hipGetLastError();
}

hipError_t launch_stream_copy(const LayerArgs& L, const void* host_gu, const void* host_dn, void* slot_gu,
                              void* slot_dn, const Work& w, int C, int r, hipStream_t s) {
  const size_t gu = (size_t)2 * L.I * L.H * 2, dn = (size_t)L.H * L.I * 2;
  const unsigned chunks = (unsigned)((gu + dn) / kCopyChunk);
  hipLaunchKernelGGL(stream_copy_kernel, dim3(chunks, C), dim3(256), 0, s, (const char*)host_gu,
                     (const char*)host_dn, (char*)slot_gu, (char*)slot_dn, (const int*)w.st_list, L.E, C, r, gu, dn);
  return hipGetLastError();
}

}  // namespace moe
