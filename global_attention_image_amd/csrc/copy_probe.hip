// Copies of a known byte count through each global-memory load path the library's kernels
// use, so that memory-traffic counters (bytes fetched from and written to HBM) can be
// read against a known amount for each path:
//   mode 0: plain 16-byte vector loads and stores;
//   mode 1: nontemporal 16-byte loads and stores (the window permutation's path);
//   mode 2: 16-byte loads straight into LDS (global_load_lds_dwordx4, the path the
//           attention kernels stage their K and V tiles with), then LDS reads and plain
//           stores.
// A workgroup of 256 threads copies one 16 KiB block; every load of a thread is issued
// before its first store.
#include "tile_common.h"

namespace uhla {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;
constexpr int kProbeBlockBytes = kProbeThreads * kProbeUnroll * 16;  // 16 KiB

template <int MODE>
__global__ __launch_bounds__(kProbeThreads) void copy_probe_kernel(const char* __restrict__ src,
                                                                   char* __restrict__ dst) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kProbeBlockBytes;
  const char* s = src + base;
  char* d = dst + base;
  if constexpr (MODE == 2) {
    // wave w fills LDS bytes [4 KiB w, 4 KiB (w + 1)) with four 1 KiB loads, lane l's
    // 16 bytes of load i landing at 1 KiB i + 16 l
    __shared__ __attribute__((aligned(16))) char buf[kProbeBlockBytes];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int wave_off = wave * (kProbeUnroll * 1024);
#pragma unroll
    for (int i = 0; i < kProbeUnroll; ++i)
      dma_16b(s + wave_off + i * 1024, lane * 16,
              __builtin_amdgcn_readfirstlane(lds_addr(buf + wave_off + i * 1024)));
    wait_vm_and_barrier<0>();
    u32x4 r[kProbeUnroll];
#pragma unroll
    for (int i = 0; i < kProbeUnroll; ++i)
      r[i] = *reinterpret_cast<const u32x4*>(buf + wave_off + i * 1024 + lane * 16);
#pragma unroll
    for (int i = 0; i < kProbeUnroll; ++i)
      *reinterpret_cast<u32x4*>(d + wave_off + i * 1024 + lane * 16) = r[i];
  } else {
    const u32x4* sv = reinterpret_cast<const u32x4*>(s);
    u32x4* dv = reinterpret_cast<u32x4*>(d);
    u32x4 r[kProbeUnroll];
#pragma unroll
    for (int i = 0; i < kProbeUnroll; ++i) {
      const int u = threadIdx.x + i * kProbeThreads;
      r[i] = MODE == 1 ? __builtin_nontemporal_load(sv + u) : sv[u];
    }
#pragma unroll
    for (int i = 0; i < kProbeUnroll; ++i) {
      const int u = threadIdx.x + i * kProbeThreads;
      if (MODE == 1) __builtin_nontemporal_store(r[i], dv + u);
      else dv[u] = r[i];
    }
  }
}

}  // namespace uhla

extern "C" int uhla_copy_probe(const void* src, void* dst, int64_t bytes, int mode,
                               void* stream) {
  using namespace uhla;
  if (!src || !dst) return fail_arg("null pointer");
  if (bytes <= 0 || bytes % kProbeBlockBytes) return fail_arg("bytes must be a positive multiple of 16384");
  if (mode < 0 || mode > 2) return fail_arg("mode must be 0, 1 or 2");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16)
    return fail_arg("pointers must be 16-byte aligned");
  if (ranges_overlap(src, static_cast<size_t>(bytes), dst, static_cast<size_t>(bytes)))
    return fail_arg("src and dst overlap");
  const int64_t blocks = bytes / kProbeBlockBytes;
  if (blocks > 0x7fffffff) return fail_unsupported("copy too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* sp = static_cast<const char*>(src);
  char* dp = static_cast<char*>(dst);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kProbeThreads);
  if (mode == 0) hipLaunchKernelGGL(copy_probe_kernel<0>, grid, block, 0, s, sp, dp);
  else if (mode == 1) hipLaunchKernelGGL(copy_probe_kernel<1>, grid, block, 0, s, sp, dp);
  else hipLaunchKernelGGL(copy_probe_kernel<2>, grid, block, 0, s, sp, dp);
  return check_launch("copy_probe_kernel");
}
