// Standalone 2D axial RoPE over a bf16 [B, L, heads, head_dim] tensor.
//
// Guide positions are scaled by rho onto the hi-res grid ([UltraGen/ar §2.B]); RoPE is the
// relative positional embedding the window-first order keeps in range ([UltraGen/fr §2.A]).
// A workgroup handles kRopeTok tokens: it first evaluates the fp64 cos/sin factors of
// those tokens (shared by all heads) into LDS, then rotates 16-byte chunks (4 pairs) in
// fp64 with one correct rounding to bf16.
#include "uhla_internal.h"

namespace uhla {

constexpr int kRopeThreads = 256;
constexpr int kRopeTok = 4;

struct GridPos {
  int y, x;
};

// Position (y, x) of joint-sequence row `tok` (see uhla.h for the conventions).
__device__ __forceinline__ GridPos token_position(int tok, int N, int W, int w, int n_wx,
                                                  int hi_order, int W_lr, int rho) {
  if (tok < N) {
    const int r = hi_order ? window_first_to_raster(tok, W, w, n_wx) : tok;
    return GridPos{r / W, r - (r / W) * W};
  }
  const int s = tok - N;
  return GridPos{rho * (s / W_lr), rho * (s - (s / W_lr) * W_lr)};
}

__global__ __launch_bounds__(kRopeThreads) void rope_apply_kernel(
    const bf16_t* src, bf16_t* dst, int L, int N, int W, int w, int n_wx, int hi_order,
    int W_lr, int rho, int heads, int D, double log2_theta) {
  extern __shared__ double2 cs[];  // [kRopeTok][D / 2]
  const int tok0 = blockIdx.x * kRopeTok;
  const int64_t b = blockIdx.y;
  const int half = D / 2, quarter = D / 4;
  for (int i = threadIdx.x; i < kRopeTok * half; i += kRopeThreads) {
    const int t = i / half, pr = i - t * half;
    const int tok = tok0 + t;
    if (tok >= L) continue;
    const GridPos pos = token_position(tok, N, W, w, n_wx, hi_order, W_lr, rho);
    const int axis = pr / quarter, k = pr - axis * quarter;  // axis 0 = y, 1 = x
    cs[i] = rope_cos_sin(axis ? pos.x : pos.y, k, half, log2_theta);
  }
  __syncthreads();
  const int chunks_per_head = D / 8;
  const int chunks_per_tok = heads * chunks_per_head;
  for (int i = threadIdx.x; i < kRopeTok * chunks_per_tok; i += kRopeThreads) {
    const int t = i / chunks_per_tok, c = i - t * chunks_per_tok;
    const int tok = tok0 + t;
    if (tok >= L) continue;
    const int h = c / chunks_per_head, j = c - h * chunks_per_head;
    const int64_t off = ((b * L + tok) * heads + h) * static_cast<int64_t>(D) + j * 8;
    const uint4 in = *reinterpret_cast<const uint4*>(src + off);
    const uint32_t wi[4] = {in.x, in.y, in.z, in.w};
    uint32_t wo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wo[e] = rope_rotate_word(wi[e], cs[t * half + j * 4 + e]);
    }
    *reinterpret_cast<uint4*>(dst + off) = make_uint4(wo[0], wo[1], wo[2], wo[3]);
  }
}

}  // namespace uhla

extern "C" int uhla_rope_apply(const void* src, void* dst, int B, int H, int W, int w,
                               int hi_order, int H_lr, int W_lr, int rho, int heads,
                               int head_dim, float theta, void* stream) {
  using namespace uhla;
  if (!src || !dst) return fail_arg("null pointer");
  if (B < 1 || H < 1 || W < 1 || heads < 1 || head_dim < 1 || H_lr < 0 || W_lr < 0)
    return fail_arg("sizes out of range");
  if (hi_order != 0 && hi_order != 1) return fail_arg("hi_order must be 0 or 1");
  if (hi_order == 1 && (w < 1 || H % w || W % w)) return fail_arg("w must divide H and W");
  if ((H_lr == 0) != (W_lr == 0)) return fail_arg("H_lr and W_lr must both be zero or not");
  const int64_t M = static_cast<int64_t>(H_lr) * W_lr;
  if (M > 0 && rho < 1) return fail_arg("rho must be >= 1 with guide tokens");
  if (head_dim % 8) return fail_unsupported("head_dim must be a multiple of 8");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16)
    return fail_arg("pointers must be 16-byte aligned");
  const int64_t N = static_cast<int64_t>(H) * W, L = N + M;
  if (L > 0x7fffffff - kRopeTok) return fail_unsupported("too many tokens");
  const size_t bytes = static_cast<size_t>(B * L * heads * head_dim * 2);
  if (src != dst && ranges_overlap(src, bytes, dst, bytes)) return fail_arg("partial overlap");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!(theta > 0.0f)) {
    if (src == dst) return UHLA_OK;
    const hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) {
      set_hip_detail("hipMemcpyAsync", e);
      return UHLA_ERR_HIP;
    }
    return UHLA_OK;
  }
  if (B > 65535) return fail_unsupported("batch too large");
  const int ww = hi_order ? w : 1;
  const dim3 grid(static_cast<unsigned>((L + kRopeTok - 1) / kRopeTok), B);
  const size_t shmem = sizeof(double2) * kRopeTok * (head_dim / 2);
  hipLaunchKernelGGL(rope_apply_kernel, grid, dim3(kRopeThreads), shmem, s,
                     static_cast<const bf16_t*>(src), static_cast<bf16_t*>(dst),
                     static_cast<int>(L), static_cast<int>(N), W, ww, W / ww, hi_order, W_lr,
                     rho, heads, head_dim, static_cast<double>(log2(static_cast<double>(theta))));
  return check_launch("rope_apply_kernel");
}
