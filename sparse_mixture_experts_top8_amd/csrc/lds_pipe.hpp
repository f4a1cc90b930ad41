// Pieces shared by the kernels that stage an activation tile in LDS with
// direct-to-LDS loads and feed v_mfma_f32_16x16x32_bf16 from it (the grouped
// GEMMs and the router's logits): the LDS row swizzle, LDS reads in inline
// asm with explicit, tied waits, and vmcnt waits the compiler can see.
//
// LDS rows of an activation tile are 128 bytes (one 64-wide k-step of bf16);
// the 16-byte chunk c of row r is stored at chunk c ^ swz(r),
// swz(r) = (r & 7) ^ ((r >> 3) & 1).  A ds_read_b128 of an MFMA operand reads
// rows 0 .. 15 of a block, one chunk column each: with 64 four-byte banks two
// consecutive rows share the bank space, and the term from bit 3 gives rows r
// and r + 8 different chunks.
#pragma once

#include <utility>

#include "common.hpp"

namespace moe {
namespace pipe {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutside = 0x80000000u;

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
// Stored chunk of chunk 0 of activation-tile row r (the same in every 16-row block).
__device__ __forceinline__ int lds_swizzle(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int OFF>
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF) : "memory");
  return v;
}
// Operands of G consecutive 16-row blocks I0 .. I0 + G - 1: one base address
// per lane, the blocks 2048 bytes apart (16 rows of 128 bytes; the chunk
// swizzle depends on row % 8 only, which is the same in every block).
template <int I0, int G, int... I>
__device__ __forceinline__ void lds_read_group(u32x4 (&a)[G], uint32_t addr, std::integer_sequence<int, I...>) {
  ((a[I] = lds_read16<2048 * (I0 + I)>(addr)), ...);
}
// Waits until at most N LDS reads are outstanding and ties the group's
// registers to the wait, so that no use of them can be scheduled before it
// (the group is older than the last N reads).
template <int N>
__device__ __forceinline__ void wait_lds_keep(u32x4 (&a)[2]) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a[0]), "+v"(a[1]) : "n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_lds_keep(u32x4 (&a)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]) : "n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_lds_keep(u32x4 (&a)[5]) {
  asm volatile("s_waitcnt lgkmcnt(%5)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]) : "n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_lds_keep(u32x4 (&a)[6]) {
  asm volatile("s_waitcnt lgkmcnt(%6)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]) : "n"(N)
               : "memory");
}
template <int N>
__device__ __forceinline__ void wait_lds_keep(u32x4 (&a)[8]) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
               : "n"(N)
               : "memory");
}
// s_waitcnt vmcnt(N) through the builtin, which the compiler's own wait
// insertion takes into account (it cannot see inside inline asm, and would
// otherwise add a wait for zero outstanding loads before the first use of a
// weight register in every unrolled iteration).  gfx9 encoding: vmcnt bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

}  // namespace pipe
}  // namespace moe
