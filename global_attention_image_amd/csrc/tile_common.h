// Device helpers shared by the attention kernels (forward and backward): tile layouts in
// LDS, direct-to-LDS tile copies, the wave-pair reductions and the workgroup order.
#pragma once
#include "uhla_internal.h"

namespace uhla {

constexpr int kKeyTile = 64;  // rows per K/V (or Q/dO) tile

// Position of key `kappa` (0..63) of a tile inside the stored V^T row: within each group
// of 16 keys the two middle quads are swapped (bits 2 and 3 of the index exchanged), so
// that the 8 keys one lane feeds into a 32x32x16 MFMA sit in 16 contiguous bytes.
__device__ __forceinline__ int v_slot(int kappa) {
  return (kappa & ~12) | ((kappa & 4) << 1) | ((kappa & 8) >> 1);
}

// Workgroups are dealt round-robin to the 8 XCDs; remap so that each XCD works on a
// contiguous range of (b, h, window): neighbouring windows and the guide K/V of one head
// then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int i, int G) {
  const int x = i & 7, j = i >> 3;
  const int per = G >> 3, rem = G & 7;
  return x < rem ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
}

// Lanes l and l ^ 32 hold the same query (different keys).  v_permlane32_swap exchanges
// the upper half of its first operand with the lower half of its second: with both
// operands = x, the two results hold x[l] and x[l ^ 32] in some order on every lane.
__device__ __forceinline__ float max_with_partner32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_with_partner32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <int D>
__device__ __forceinline__ int k_swizzle(int row) {
  // 16-byte chunk XOR swizzle so 16 lanes reading the same chunk of 16 rows hit 16
  // distinct bank groups.
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
__device__ __forceinline__ int v_swizzle(int row) { return (row >> 1) & 7; }

// 32-bit LDS address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(p)));
}

// Asynchronous 16-byte global -> LDS copy per lane (global_load_lds_dwordx4): lane l
// reads gbase + voff and writes LDS bytes [lds + 16 l, lds + 16 l + 16).  gbase and lds
// are wave-uniform.  The instruction has no register results (data goes to LDS), and it
// is issued from asm so that the compiler does not treat every later LDS read as
// possibly overlapping it (it cannot tell the ring stages apart and would wait for all
// in-flight tiles); completion is awaited explicitly by wait_vm_and_barrier.  M0 is
// written by the compiler just before the block, hence the wait state.
__device__ __forceinline__ void dma_16b(const char* gbase, int voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "{m0}"(lds)
               : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding, then
// barrier.  The direct-to-LDS tile loads are vector-memory operations, so this makes the
// older tiles visible to the whole workgroup while the newest ones stay in flight.  The
// "memory" clobber keeps the compiler from moving LDS accesses across the barrier.
template <int N>
__device__ __forceinline__ void wait_vm_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

}  // namespace uhla
