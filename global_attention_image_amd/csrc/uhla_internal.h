// Internal helpers shared by the HIP translation units of libuhla (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "uhla.h"

namespace uhla {

typedef uint16_t bf16_t;  // storage type: raw bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- error reporting

void set_detail(const char* msg);
void set_hip_detail(const char* where, hipError_t e);
int fail_arg(const char* msg);
int fail_unsupported(const char* msg);

// Checks the launch just enqueued; returns UHLA_OK or UHLA_ERR_HIP with the detail.
int check_launch(const char* where);

// ---------------------------------------------------------------- numeric helpers

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Two floats -> two bf16 (round to nearest even) packed in one 32-bit word (lo = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// cos/sin of pos * theta^(-2k / d_axis) in fp64.  Every RoPE code path in the library
// calls this one function, so the same (pos, k) always gives bit-identical factors.
__device__ __forceinline__ double2 rope_cos_sin(int pos, int k, int d_axis, double log2_theta) {
  const double omega = exp2(-(2.0 * k / d_axis) * log2_theta);
  const double phi = static_cast<double>(pos) * omega;
  double s, c;
  sincos(phi, &s, &c);
  return make_double2(c, s);
}

// fp64 -> bf16 bits with a single correct rounding (nearest, ties to even): round to
// fp32 by round-to-odd (truncate toward zero, set the last bit if anything was lost),
// then round the fp32 value to bf16.  Round-to-odd at 24 bits followed by rounding at 8
// bits equals rounding the fp64 value directly.  Inputs are finite.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x) {
  const float f = static_cast<float>(x);
  uint32_t u = __float_as_uint(f);
  const double back = static_cast<double>(f);
  if (back != x) {
    if (fabs(back) > fabs(x)) u -= 1;  // sign-magnitude: one step toward zero
    u |= 1u;
  }
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Rotates the pair (a, b) packed as two bf16 in one word (a in the low half) by the
// factors cs = (cos, sin): (a cos - b sin, a sin + b cos) times `scale`, computed in fp64
// and rounded once to bf16 (scale = 1 is the plain rotation).
__device__ __forceinline__ uint32_t rope_rotate_word(uint32_t word, double2 cs, double scale = 1.0) {
  const double a = static_cast<double>(__uint_as_float(word << 16));
  const double b = static_cast<double>(__uint_as_float(word & 0xffff0000u));
  const double ra = fma(a, cs.x, -(b * cs.y)) * scale;
  const double rb = fma(a, cs.y, b * cs.x) * scale;
  return f64_to_bf16_bits(ra) | (f64_to_bf16_bits(rb) << 16);
}

// Both bf16 halves of a word times `scale`, in fp64, rounded once to bf16.
__device__ __forceinline__ uint32_t scale_word(uint32_t word, double scale) {
  const double a = static_cast<double>(__uint_as_float(word << 16)) * scale;
  const double b = static_cast<double>(__uint_as_float(word & 0xffff0000u)) * scale;
  return f64_to_bf16_bits(a) | (f64_to_bf16_bits(b) << 16);
}

// Raster index of the token at window-first position p (hi-res grid of width W,
// windows of w x w, n_wx = W / w windows per window row).
__device__ __forceinline__ int window_first_to_raster(int p, int W, int w, int n_wx) {
  const int ww = w * w;
  const int win = p / ww, t = p - win * ww;
  const int wy = win / n_wx, wx = win - wy * n_wx;
  const int iy = t / w, ix = t - iy * w;
  return (wy * w + iy) * W + (wx * w + ix);
}

inline bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- the forward (attention.hip)

// Host-side argument checks of the forward entry points (no device call).
int validate_forward(const void* q, const void* k, const void* v, void* o, int B, int64_t T,
                     int H, int W, int w, int H_lr, int W_lr, int rho, int heads, int D,
                     int radius, int guide_mode);
// Workspace bytes of the forward for this geometry (0 on invalid geometry).
size_t workspace_bytes(int B, int64_t T, int H, int W, int w, int H_lr, int W_lr, int rho,
                       int heads, int head_dim, int radius, int guide_mode);
// The forward: validation, then every launch on `stream`, scratch in `workspace`.
int forward_impl(const void* q, const void* k, const void* v, void* o, int B, int64_t T, int H,
                 int W, int w, int H_lr, int W_lr, int rho, int heads, int D, float scale,
                 float theta, int radius, int guide_mode, void* workspace,
                 size_t workspace_bytes, void* stream, uhla_timer* timer,
                 float* lse = nullptr, bool rope_k_at_load = false);

}  // namespace uhla
