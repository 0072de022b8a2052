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

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// 16-byte chunk swizzle of row-major LDS tiles that are also read transposed (the
// backward's tiles, the V tiles of the permute-free forward): physical chunk = logical
// chunk ^ bwd_swizzle<D>(row).  The tiles are read two ways: 16 lanes reading one chunk of 16
// consecutive rows (the row fragments) need 16 distinct values over any 16 consecutive
// rows, and the transposed reads below, where each 32-lane half addresses 4 rows x 4
// consecutive chunks, need those 16 (row, chunk) pairs in 16 distinct bank groups.  The
// swizzle puts row bits 0-1 into chunk bits 2-3 and row bits 2-3 into chunk bits 0-1
// (D = 64: the same on row / 2, two rows sharing a 256-byte bank line), which meets both;
// XOR with the plain row % 16 would leave chunk bits 2-3 fixed within a half, 4 bank
// groups for 16 pairs.
template <int D>
__device__ __forceinline__ int bwd_swizzle(int row) {
  const int e = D == 128 ? (row & 15) : ((row >> 1) & 7);
  return D == 128 ? (((e & 3) << 2) | (e >> 2)) : (((e & 1) << 2) | (e >> 1));
}

// Transposed MFMA operands from a row-major LDS tile (rows of D bf16, chunks swizzled by
// bwd_swizzle<D>): A[i][k] = tile[row(k)][32 dt + i], i = lane % 32, for the 16 rows of
// reduction step ks, in the order of an accumulator converted in place (element jj of
// lane group g = lane / 32 is row 16 ks + 8 (jj / 4) + 4 g + jj % 4).  Two
// ds_read_b64_tr_b16 per fragment: within each 16-lane group, lane i' receives element
// i' % 4 of the 8 bytes addressed by lane 4 j + i' / 4 (j = 0..3), so the group's lanes
// address 4 rows x 16 consecutive columns and each lane receives one column of those rows.
// Lane l addresses row 16 ks + 8 b + R0 (R0 = 4 g + r, r = (l % 16) / 4) at logical chunk
// 4 dt + c (D = 128; D = 64: 4 dt + c as well, chunks of a 128-byte row) with
// c = 2 ((l / 16) % 2) + (l % 4) / 2, byte 8 (l % 2) of it.  Under the swizzle the byte
// offset is x ^ (64 dt + 32 b) plus 2048 b + 4096 ks (D = 64: 1024 b + 2048 ks) for a
// per-lane x: the XOR touches only bits 5-7 of x, so it costs one VALU op per (dt, b).
template <int D>
struct TrAddr {
  int x;  // per-lane byte offset of (ks, dt, b) = (0, 0, 0)
  __device__ __forceinline__ explicit TrAddr(int lane) {
    const int g = lane >> 5, r = (lane & 15) >> 2, r0 = 4 * g + r;
    const int c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    x = (D == 128 ? 256 * r0 + 64 * r : 128 * r0 + 64 * (r >> 1)) + 16 * (c ^ g) + 8 * (lane & 1);
  }
  // `xb` is x, made opaque by the caller where the XORs are to be recomputed
  __device__ __forceinline__ static bf16x8 frag(const char* tile, int xb, int ks, int dt) {
    bf16x8 out;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int off = (xb ^ (64 * dt + 32 * b)) + (D == 128 ? 2048 : 1024) * (b + 2 * ks);
      const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4*)(tile + off));
#pragma unroll
      for (int e = 0; e < 4; ++e) out[4 * b + e] = v[e];
    }
    return out;
  }
};

}  // namespace uhla
