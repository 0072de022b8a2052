// Window-first permutation of the hi-res token segment and its inverse.
//
// [UltraGen/it §2], [UltraGen/fr §2.A], [UltraGen/ar §2.A]: hi-res tokens are reordered
// window by window so each attention block is one spatial window.  One window row
// (w consecutive tokens) is contiguous in both the raster and the window-first order, so
// the permutation is a gather of contiguous "segments" of w * row_bytes bytes.  Each
// workgroup copies one slice of one segment with wide vector loads; all loads of a
// thread are issued before its stores, so many bytes are in flight per CU.
#include "uhla_internal.h"

namespace uhla {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

template <typename U>
__global__ __launch_bounds__(kCopyThreads) void window_copy_kernel(
    const char* __restrict__ src, char* __restrict__ dst, int W, int w, int n_wx,
    int64_t row_bytes, int64_t src_batch_bytes, int64_t dst_batch_bytes, int seg_units,
    int chunks_per_seg, int inverse) {
  const int seg = blockIdx.x / chunks_per_seg;
  const int chunk = blockIdx.x - seg * chunks_per_seg;
  const int win = seg / w, iy = seg - win * w;
  const int wy = win / n_wx, wx = win - wy * n_wx;
  const int64_t raster_tok = static_cast<int64_t>(wy * w + iy) * W + wx * w;
  const int64_t wf_tok = static_cast<int64_t>(win) * w * w + static_cast<int64_t>(iy) * w;
  const int64_t b = blockIdx.y;
  const U* s = reinterpret_cast<const U*>(src + b * src_batch_bytes +
                                          (inverse ? wf_tok : raster_tok) * row_bytes);
  U* d = reinterpret_cast<U*>(dst + b * dst_batch_bytes +
                              (inverse ? raster_tok : wf_tok) * row_bytes);
  const int base = chunk * kCopyThreads * kCopyUnroll + threadIdx.x;
  U r[kCopyUnroll];
#pragma unroll
  for (int i = 0; i < kCopyUnroll; ++i) {
    const int u = base + i * kCopyThreads;
    if (u < seg_units) r[i] = __builtin_nontemporal_load(s + u);
  }
#pragma unroll
  for (int i = 0; i < kCopyUnroll; ++i) {
    const int u = base + i * kCopyThreads;
    if (u < seg_units) __builtin_nontemporal_store(r[i], d + u);
  }
}

// Enqueues the segment copy; arguments already validated.
int launch_window_copy(const void* src, void* dst, int B, int H, int W, int w,
                       int64_t row_bytes, int64_t src_tpb, int64_t dst_tpb, int inverse,
                       hipStream_t stream) {
  const int n_wx = W / w, n_wy = H / w;
  const int64_t seg_bytes = static_cast<int64_t>(w) * row_bytes;
  const uintptr_t align = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst);
  int unit = 2;
  if (row_bytes % 16 == 0 && align % 16 == 0) unit = 16;
  else if (row_bytes % 4 == 0 && align % 4 == 0) unit = 4;
  const int64_t seg_units = seg_bytes / unit;
  if (seg_units > (int64_t(1) << 30)) return fail_unsupported("window row too large");
  const int64_t per_chunk = static_cast<int64_t>(kCopyThreads) * kCopyUnroll;
  const int chunks = static_cast<int>((seg_units + per_chunk - 1) / per_chunk);
  const int64_t n_seg = static_cast<int64_t>(n_wy) * n_wx * w;
  const int64_t gx = n_seg * chunks;
  if (gx > 0x7fffffff || B > 65535) return fail_unsupported("grid too large");
  const dim3 grid(static_cast<unsigned>(gx), B), block(kCopyThreads);
  const int64_t sb = src_tpb * row_bytes, db = dst_tpb * row_bytes;
  const char* s = static_cast<const char*>(src);
  char* d = static_cast<char*>(dst);
  const int su = static_cast<int>(seg_units);
  if (unit == 16)
    hipLaunchKernelGGL(window_copy_kernel<u32x4>, grid, block, 0, stream, s, d, W, w, n_wx,
                       row_bytes, sb, db, su, chunks, inverse);
  else if (unit == 4)
    hipLaunchKernelGGL(window_copy_kernel<uint32_t>, grid, block, 0, stream, s, d, W, w, n_wx,
                       row_bytes, sb, db, su, chunks, inverse);
  else
    hipLaunchKernelGGL(window_copy_kernel<uint16_t>, grid, block, 0, stream, s, d, W, w, n_wx,
                       row_bytes, sb, db, su, chunks, inverse);
  return check_launch("window_copy_kernel");
}

static int permute_common(const void* src, void* dst, int B, int H, int W, int w, int heads,
                          int head_dim, int elem_bytes, int64_t src_tpb, int64_t dst_tpb,
                          void* stream, int inverse) {
  if (!src || !dst) return fail_arg("null pointer");
  if (B < 1 || H < 1 || W < 1 || w < 1 || heads < 1 || head_dim < 1)
    return fail_arg("sizes must be >= 1");
  if (H % w || W % w) return fail_arg("w must divide H and W");
  if (elem_bytes != 2 && elem_bytes != 4) return fail_unsupported("elem_bytes must be 2 or 4");
  const int64_t N = static_cast<int64_t>(H) * W;
  if (src_tpb < N || dst_tpb < N) return fail_arg("batch stride smaller than H*W");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % elem_bytes)
    return fail_arg("pointers not aligned to elem_bytes");
  const int64_t row_bytes = static_cast<int64_t>(heads) * head_dim * elem_bytes;
  const size_t src_span = static_cast<size_t>(((B - 1) * src_tpb + N) * row_bytes);
  const size_t dst_span = static_cast<size_t>(((B - 1) * dst_tpb + N) * row_bytes);
  if (ranges_overlap(src, src_span, dst, dst_span)) return fail_arg("src and dst overlap");
  return launch_window_copy(src, dst, B, H, W, w, row_bytes, src_tpb, dst_tpb, inverse,
                            static_cast<hipStream_t>(stream));
}

}  // namespace uhla

extern "C" int uhla_window_permute(const void* src, void* dst, int B, int H, int W, int w,
                                   int heads, int head_dim, int elem_bytes,
                                   int64_t src_tokens_per_batch, int64_t dst_tokens_per_batch,
                                   void* stream) {
  return uhla::permute_common(src, dst, B, H, W, w, heads, head_dim, elem_bytes,
                              src_tokens_per_batch, dst_tokens_per_batch, stream, 0);
}

extern "C" int uhla_window_unpermute(const void* src, void* dst, int B, int H, int W, int w,
                                     int heads, int head_dim, int elem_bytes,
                                     int64_t src_tokens_per_batch,
                                     int64_t dst_tokens_per_batch, void* stream) {
  return uhla::permute_common(src, dst, B, H, W, w, heads, head_dim, elem_bytes,
                              src_tokens_per_batch, dst_tokens_per_batch, stream, 1);
}
