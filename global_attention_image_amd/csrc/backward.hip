// Hierarchical local attention backward on gfx950: dQ, dK, dV for every mask of the
// forward (any neighbourhood radius; all guide tokens visible to hi-res queries, or in
// guide modes 1 and 2 only those of the query's window or neighbourhood; guide queries
// seeing guide keys only) and optional text tokens (text queries see every key, every
// query sees the text keys), from Q, K, V, O, dO and the forward's per-row log-sum-exp.
//
// Math per (batch, head), rotated Q~ K~, scale s: P = exp(s Q~ K~^T - lse) on the allowed
// pairs, dV = P^T dO, dP = dO V^T, dS = P (dP - D) with D = rowsum(dO O), dQ~ = s dS K~,
// dK~ = s dS^T Q~; dQ and dK rotate dQ~ and dK~ back (the transpose of RoPE).
//
// Pipeline (caller's stream, no allocation):
//   1. fp64 cos/sin table (as the forward);
//   2. bwd_rows_kernel: per (b, h) buffers with hi rows window-first, then guide rows and
//      then text rows, each of the last two padded to 256: Qb = rope(Q) * s * log2 e (the
//      forward's base-2 query), Kb = rope(K), Vb, dOb; bwd_aux_kernel: per 64-row tile,
//      -lse2 = -lse * log2 e (pad rows -inf) and -D; in guide modes 1 and 2
//      bwd_cellblock_kernel copies the guide K~ and V rows into 8x8 cell blocks;
//   3. bwd_dq_kernel (query-outer, the forward's tile lists): per key tile S, dP (two
//      32x32x16 MFMA chains from K and V tiles), dS, and dQ^T += K^T dS^T;
//   4. bwd_dkv_kernel (key-outer, the transposed mask: a hi window's keys are seen by the
//      queries of its neighbour windows, a guide key by every hi and guide query that
//      sees it): per query tile S, dP, dS and dV^T += dO^T P, dK^T += Q^T dS.
// Tiles are row-major in LDS; the transposed operands (K^T, Q^T, dO^T) are read from the
// same tiles with the gfx950 transposing LDS read, so each tile is copied once.  Both
// kernels keep a 4-stage ring of tiles, copied three tiles ahead, and write bf16
// gradients in the caller's raster layout, undoing RoPE in the epilogue.
#include <algorithm>

#include "tile_common.h"

namespace uhla {

namespace {

constexpr int kBwdRowsPerBlock = 4;
constexpr int kBwdThreads = 256;
constexpr int kBwdMaxTiles = 1024;  // neighbour-window tiles per window (table in LDS)
constexpr int kAuxBytes = 2 * kKeyTile * 4;  // per tile: 64 -lse2 then 64 -D values
constexpr int kBwdStages = 4;                 // LDS ring of tiles; copies run 3 tiles ahead
constexpr int kBwdWaves = 8;                  // guide-row workgroups: 8 waves x 32 rows
constexpr int kBwdGuideRows = kBwdWaves * 32;

struct BwdGeom {
  int B, H, W, w, H_lr, W_lr, rho, heads, D, radius, guide_mode;
  int nbi, nbjp;  // guide modes 1, 2: blocks of 8x8 guide cells, block rows padded to 4 blocks
  int64_t Mb;     // cell-block rows (nbi * nbjp * 64), 0 in guide mode 0
  int64_t T, N, M, Mp, Tp, R;  // R: rows per (b, h) = N + Mp + Tp (guide / text rows padded)
  int n_wx, n_wy, P;
  int splits;  // text row blocks: tile-range splits (0 without text tokens)
};

BwdGeom make_bwd_geom(int B, int64_t T, int H, int W, int w, int H_lr, int W_lr, int rho,
                      int heads, int D, int radius, int guide_mode) {
  BwdGeom g;
  g.B = B; g.H = H; g.W = W; g.w = w; g.H_lr = H_lr; g.W_lr = W_lr; g.rho = rho;
  g.heads = heads; g.D = D; g.radius = radius; g.guide_mode = guide_mode;
  g.nbi = (H_lr + 7) / 8;
  g.nbjp = ((W_lr + 7) / 8 + 3) / 4 * 4;
  g.Mb = (guide_mode != 0 && static_cast<int64_t>(H_lr) * W_lr > 0)
             ? static_cast<int64_t>(g.nbi) * g.nbjp * kKeyTile : 0;
  g.T = T;
  g.N = static_cast<int64_t>(H) * W;
  g.M = static_cast<int64_t>(H_lr) * W_lr;
  g.Mp = (g.M + kBwdGuideRows - 1) / kBwdGuideRows * kBwdGuideRows;
  g.Tp = (T + kBwdGuideRows - 1) / kBwdGuideRows * kBwdGuideRows;
  g.R = g.N + g.Mp + g.Tp;
  // Text row blocks walk every tile of the other side: few blocks, long lists.  Split each
  // list so that the GPU gets about 1024 workgroups, each split at least 8 tiles long.
  g.splits = 0;
  if (T > 0) {
    const int64_t blocks = static_cast<int64_t>(B) * heads * (g.Tp / kBwdGuideRows);
    const int64_t tiles = g.R / kKeyTile;
    int64_t sp = (1024 + blocks - 1) / blocks;
    sp = std::min(sp, std::max<int64_t>(1, tiles / 8));
    g.splits = static_cast<int>(std::max<int64_t>(1, sp));
  }
  g.n_wx = W / w; g.n_wy = H / w;
  g.P = H > W ? H : W;
  return g;
}

struct BwdWorkspace {
  double2* cs;
  bf16_t *qb, *kb, *vb, *dob;  // [B*heads][R][D]
  float* aux;                  // [B*heads][R/64][128]
  float *part0, *part1;        // [splits][B*heads][Tp][D] text row blocks' partial sums
  bf16_t *kgb, *vgb;           // [B*heads][Mb][D] guide K~, V in 8x8 cell blocks (modes 1, 2)
  size_t bytes;
};

BwdWorkspace carve_bwd(const BwdGeom& g, void* base) {
  BwdWorkspace ws;
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off = align_up(off + n, 256);
    return o;
  };
  const size_t rows = static_cast<size_t>(g.B) * g.heads * g.R;
  const size_t mat = rows * g.D * sizeof(bf16_t);
  const size_t o_cs = take(sizeof(double2) * g.P * (g.D / 4));
  size_t o_m[4];
  for (auto& x : o_m) x = take(mat);
  const size_t o_aux = take(rows / kKeyTile * kAuxBytes);
  const size_t part = static_cast<size_t>(g.splits) * g.B * g.heads * g.Tp * g.D * sizeof(float);
  const size_t o_p0 = take(part), o_p1 = take(part);
  const size_t cells = static_cast<size_t>(g.B) * g.heads * g.Mb * g.D * sizeof(bf16_t);
  const size_t o_kg = take(cells), o_vg = take(cells);
  char* b = static_cast<char*>(base);
  ws.cs = reinterpret_cast<double2*>(b + o_cs);
  bf16_t** mats[4] = {&ws.qb, &ws.kb, &ws.vb, &ws.dob};
  for (int i = 0; i < 4; ++i) *mats[i] = reinterpret_cast<bf16_t*>(b + o_m[i]);
  ws.aux = reinterpret_cast<float*>(b + o_aux);
  ws.part0 = reinterpret_cast<float*>(b + o_p0);
  ws.part1 = reinterpret_cast<float*>(b + o_p1);
  ws.kgb = reinterpret_cast<bf16_t*>(b + o_kg);
  ws.vgb = reinterpret_cast<bf16_t*>(b + o_vg);
  ws.bytes = off;
  return ws;
}

}  // namespace

__global__ void bwd_cos_sin_kernel(double2* cs, int P, int D, double log2_theta) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int quarter = D / 4;
  if (i >= P * quarter) return;
  const int pos = i / quarter, k = i - pos * quarter;
  cs[i] = rope_cos_sin(pos, k, D / 2, log2_theta);
}

// Token (row of the caller's [text | hi | guide] tensors) and RoPE position of buffer row
// `row`: hi rows window-first, then guide rows (padded to Mp), then text rows (padded, at
// position (0, 0)); -1 for padding rows.
__device__ __forceinline__ int64_t bwd_source(int64_t row, int64_t T, int64_t N, int64_t M,
                                              int64_t Mp, int W, int w, int n_wx, int W_lr,
                                              int rho, int& py, int& px) {
  py = px = 0;
  if (row < N) {
    const int r = window_first_to_raster(static_cast<int>(row), W, w, n_wx);
    py = r / W;
    px = r - py * W;
    return T + r;
  }
  if (row < N + Mp) {
    const int64_t s = row - N;
    if (s >= M) return -1;
    const int sy = static_cast<int>(s / W_lr);
    py = rho * sy;
    px = rho * static_cast<int>(s - static_cast<int64_t>(sy) * W_lr);
    return T + N + s;
  }
  const int64_t x = row - N - Mp;
  return x < T ? x : -1;
}

// Q, K, V, dO rows -> per (b, h) buffers [R][D]: Q rotated and scaled by q_scale in fp64
// and rounded once (as the forward), K rotated, V and dO copied; zero padding rows.
template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_rows_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, bf16_t* __restrict__ qb, bf16_t* __restrict__ kb,
    bf16_t* __restrict__ vb, bf16_t* __restrict__ dob, const double2* __restrict__ cs, int P,
    double log2_theta, int64_t T, int64_t N, int64_t M, int64_t Mp, int64_t R, int W, int w,
    int n_wx, int W_lr, int rho, int heads, int rope_on, double q_scale) {
  constexpr int CPH = D / 8, QUARTER = D / 4;
  __shared__ int64_t src_s[kBwdRowsPerBlock];
  __shared__ int pos_s[kBwdRowsPerBlock][2];
  __shared__ double2 cs_s[kBwdRowsPerBlock][2][QUARTER];
  const int64_t L = T + N + M, b = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid < kBwdRowsPerBlock) {
    int py, px;
    src_s[tid] = bwd_source(static_cast<int64_t>(blockIdx.x) * kBwdRowsPerBlock + tid, T, N, M, Mp,
                            W, w, n_wx, W_lr, rho, py, px);
    pos_s[tid][0] = py;
    pos_s[tid][1] = px;
  }
  __syncthreads();
  if (rope_on) {
    for (int e = tid; e < kBwdRowsPerBlock * 2 * QUARTER; e += kBwdThreads) {
      const int rt = e / (2 * QUARTER), axis = (e / QUARTER) & 1, kk = e % QUARTER;
      const int pos = pos_s[rt][axis];
      cs_s[rt][axis][kk] = pos < P ? cs[pos * QUARTER + kk] : rope_cos_sin(pos, kk, D / 2, log2_theta);
    }
    __syncthreads();
  }
  const int cpr = heads * CPH;
  for (int i = tid; i < kBwdRowsPerBlock * cpr; i += kBwdThreads) {
    const int t = i / cpr, c = i - t * cpr;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kBwdRowsPerBlock + t;
    if (row >= R) continue;
    const int h = c / CPH, j = c % CPH;
    const int64_t src = src_s[t];
    uint4 qo = make_uint4(0, 0, 0, 0), ko = qo, vo = qo, go = qo;
    if (src >= 0) {
      const int64_t so = ((b * L + src) * heads + h) * D + j * 8;
      const uint4 qi = *reinterpret_cast<const uint4*>(q + so);
      const uint4 ki = *reinterpret_cast<const uint4*>(k + so);
      vo = *reinterpret_cast<const uint4*>(v + so);
      go = *reinterpret_cast<const uint4*>(dout + so);
      if (rope_on) {
        const int axis = (4 * j) / QUARTER, k0 = 4 * j - axis * QUARTER;
        const double2* f = &cs_s[t][axis][k0];
        qo = make_uint4(rope_rotate_word(qi.x, f[0], q_scale), rope_rotate_word(qi.y, f[1], q_scale),
                        rope_rotate_word(qi.z, f[2], q_scale), rope_rotate_word(qi.w, f[3], q_scale));
        ko = make_uint4(rope_rotate_word(ki.x, f[0]), rope_rotate_word(ki.y, f[1]),
                        rope_rotate_word(ki.z, f[2]), rope_rotate_word(ki.w, f[3]));
      } else {
        qo = make_uint4(scale_word(qi.x, q_scale), scale_word(qi.y, q_scale),
                        scale_word(qi.z, q_scale), scale_word(qi.w, q_scale));
        ko = ki;
      }
    }
    const int64_t o = ((b * heads + h) * R + row) * D + j * 8;
    *reinterpret_cast<uint4*>(qb + o) = qo;
    *reinterpret_cast<uint4*>(kb + o) = ko;
    *reinterpret_cast<uint4*>(vb + o) = vo;
    *reinterpret_cast<uint4*>(dob + o) = go;
  }
}

// Per buffer row: lse2 = lse * log2 e (+inf for padding, so those rows get P = 0) and
// D = sum_d dO * O in fp32, stored negated per 64-row tile as [64 -lse2][64 -D] (the
// dK/dV kernel starts its S and dP accumulators from them).  D / 8 lanes read
// one (token, head) row of O and dO in raster memory order (coalesced) and reduce across
// lanes; threads past the B * L * heads rows fill the padding rows.
__global__ __launch_bounds__(kBwdThreads) void bwd_aux_kernel(
    const bf16_t* __restrict__ o, const bf16_t* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ aux, int64_t T, int64_t N, int64_t M, int64_t Mp, int64_t R, int W,
    int w, int n_wx, int heads, int D, int64_t bh_total) {
  const int cpr = D / 8;  // 16-byte chunks per row: 16 or 8, a power of two dividing 64
  const int64_t L = T + N + M;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t rows = bh_total * L;  // (b, token, head) rows, raster memory order
  const int64_t gi = i / cpr;
  const int c = static_cast<int>(i - gi * cpr);
  if (gi < rows) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + gi * D + c * 8);
    const uint4 g = *reinterpret_cast<const uint4*>(dout + gi * D + c * 8);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, gw[4] = {g.x, g.y, g.z, g.w};
    float dd = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dd += __uint_as_float(aw[e] << 16) * __uint_as_float(gw[e] << 16) +
            __uint_as_float(aw[e] & 0xffff0000u) * __uint_as_float(gw[e] & 0xffff0000u);
    for (int m = 1; m < cpr; m <<= 1) dd += __shfl_xor(dd, m, 64);
    if (c) return;
    const int64_t bt = gi / heads, h = gi - bt * heads;  // bt = b * L + token
    const int64_t b = bt / L, src = bt - b * L;
    int64_t row;
    if (src < T) {
      row = N + Mp + src;
    } else if (src < T + N) {  // raster -> window-first
      const int64_t r = src - T;
      const int y = static_cast<int>(r / W), x = static_cast<int>(r - static_cast<int64_t>(y) * W);
      const int wy = y / w, wx = x / w;
      row = (static_cast<int64_t>(wy) * n_wx + wx) * w * w + (y - wy * w) * w + (x - wx * w);
    } else {
      row = src - T;  // guide s = src - T - N sits at buffer row N + s
    }
    const int64_t bh = b * heads + h;
    float* t = aux + (bh * (R / kKeyTile) + row / kKeyTile) * (2 * kKeyTile);
    t[row % kKeyTile] = -(lse[bh * L + src] * 1.4426950408889634f);
    t[kKeyTile + row % kKeyTile] = -dd;
    return;
  }
  // padding rows: guide rows [N + M, N + Mp) and text rows [N + Mp + T, R)
  const int64_t pad_g = Mp - M, pad = pad_g + (R - N - Mp - T);
  const int64_t j = i - rows * cpr;
  if (j >= bh_total * pad) return;
  const int64_t bh = j / pad, jj = j - bh * pad;
  const int64_t row = jj < pad_g ? N + M + jj : N + Mp + T + (jj - pad_g);
  float* t = aux + (bh * (R / kKeyTile) + row / kKeyTile) * (2 * kKeyTile);
  t[row % kKeyTile] = -INFINITY;
  t[kKeyTile + row % kKeyTile] = 0.0f;
}

// Guide modes 1 and 2: guide K~ and V rows copied into 8x8 cell blocks (slot s: block s/64
// = (bi, bj) over an nbjp-wide block grid, cell (8 bi + (s%64)/8, 8 bj + s%8)), zero for
// cells outside the guide grid.  One thread per 16-byte chunk.
__global__ __launch_bounds__(kBwdThreads) void bwd_cellblock_kernel(
    const bf16_t* __restrict__ kb, const bf16_t* __restrict__ vb, bf16_t* __restrict__ kgb,
    bf16_t* __restrict__ vgb, int64_t N, int64_t R, int64_t Mb, int H_lr, int W_lr, int nbjp,
    int D, int64_t bh_total) {
  const int cpr = D / 8;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= bh_total * Mb * cpr) return;
  const int64_t row = i / cpr, bh = row / Mb, slot = row - bh * Mb;
  const int c = static_cast<int>(i - row * cpr);
  const int blk = static_cast<int>(slot / kKeyTile), k = static_cast<int>(slot % kKeyTile);
  const int bi = blk / nbjp, bj = blk - bi * nbjp;
  const int ci = 8 * bi + (k >> 3), cj = 8 * bj + (k & 7);
  uint4 kx = make_uint4(0, 0, 0, 0), vx = kx;
  if (ci < H_lr && cj < W_lr) {
    const int64_t src = (bh * R + N + static_cast<int64_t>(ci) * W_lr + cj) * D + c * 8;
    kx = *reinterpret_cast<const uint4*>(kb + src);
    vx = *reinterpret_cast<const uint4*>(vb + src);
  }
  const int64_t dst = (bh * Mb + slot) * D + c * 8;
  *reinterpret_cast<uint4*>(kgb + dst) = kx;
  *reinterpret_cast<uint4*>(vgb + dst) = vx;
}

struct BwdArgs {
  const bf16_t *qb, *kb, *vb, *dob;
  const bf16_t *kgb, *vgb;  // guide modes 1, 2: guide K~, V in cell blocks [B*heads][Mb][D]
  const float* aux;
  const double2* cs;
  bf16_t* out0;  // dQ (dq kernel) or dK (dkv kernel), the caller's [B][L][heads][D]
  bf16_t* out1;  // dV (dkv kernel)
  int64_t T, N, M, Mp, R, L;  // L = T + N + M tokens per batch
  int heads, w2, W, w, n_wx, n_wy, radius, rho, W_lr, P;
  int rope_on;
  double log2_theta;
  float out_scale;  // scale (dQ) or ln 2 (dK)
  int blocks_per_bh, total_blocks;
  int splits;             // text row blocks: tile-range splits per block
  float *part0, *part1;   // text row blocks: fp32 partial sums [splits][B*heads][Tp][D]
  int64_t Tp;
  int reach, H_lr, nbjp;  // guide modes 1, 2: a hi query sees the guide cells whose scaled
  int64_t Mb;             // position lies in a window within `reach` of its own window
};

// Guide cells [i0, i1) x [j0, j1) visible to the queries of window (wy, wx) in guide modes
// 1 and 2: cell (i, j) is visible when (rho i, rho j) lies in a window within `reach`.
__device__ __forceinline__ void window_cells(const BwdArgs& A, int wy, int wx, int& i0, int& i1,
                                             int& j0, int& j1) {
  const int gy0 = max(0, wy - A.reach), gy1 = min(A.n_wy - 1, wy + A.reach);
  const int gx0 = max(0, wx - A.reach), gx1 = min(A.n_wx - 1, wx + A.reach);
  i0 = (gy0 * A.w + A.rho - 1) / A.rho;
  i1 = min(A.H_lr, ((gy1 + 1) * A.w + A.rho - 1) / A.rho);
  j0 = (gx0 * A.w + A.rho - 1) / A.rho;
  j1 = min(A.W_lr, ((gx1 + 1) * A.w + A.rho - 1) / A.rho);
}

// Tile range [t0, t1) of split `split` of a list of n tiles (splits of equal length)
__device__ __forceinline__ void split_range(int n, int splits, int split, int& t0, int& t1) {
  const int per = (n + splits - 1) / splits;
  t0 = min(n, split * per);
  t1 = min(n, t0 + per);
}

// Sum of the text row blocks' split partials in a fixed order, scaled and stored as bf16
// in the caller's layout (text rows sit at position (0, 0), where RoPE is the identity).
// One thread per pair of dims of one (b, h, text row); part1 / out1 are optional.
__global__ void bwd_text_combine_kernel(const float* __restrict__ part0, const float* __restrict__ part1,
                                        bf16_t* out0, bf16_t* out1, float scale0, int splits,
                                        int64_t bh_total, int64_t Tp, int64_t T, int64_t L,
                                        int heads, int D) {
  const int64_t x = blockIdx.x, bh = blockIdx.y;
  const int d = 2 * threadIdx.x;
  if (x >= T || d >= D) return;
  float a0 = 0.0f, a1 = 0.0f, c0 = 0.0f, c1 = 0.0f;
  for (int sp = 0; sp < splits; ++sp) {
    const int64_t o = ((sp * bh_total + bh) * Tp + x) * D + d;
    a0 += part0[o];
    a1 += part0[o + 1];
    if (part1) {
      c0 += part1[o];
      c1 += part1[o + 1];
    }
  }
  const int64_t b = bh / heads, h = bh - b * heads;
  const int64_t ro = ((b * L + x) * heads + h) * D + d;
  *reinterpret_cast<uint32_t*>(out0 + ro) = pack_bf16x2(scale0 * a0, scale0 * a1);
  if (part1) *reinterpret_cast<uint32_t*>(out1 + ro) = pack_bf16x2(c0, c1);
}

// Inverse-RoPE factors of the D/4 pairs one lane stores: pairs d0/2 and d0/2 + 1 of each
// d0 = dt*32 + 8 rg + 4 g, factor i = 2 (4 dt + rg) + e, for a row at position (py, px):
// the fp64 factors rounded to fp32.  All table loads are issued before the first use (one
// wait); a position past the table (a guide row of a guide grid reaching beyond the
// hi-res extent) reads a clamped entry first and is then evaluated directly, with the
// function that fills the table.
template <int D>
__device__ __forceinline__ void lane_factors(int g, int py, int px, const BwdArgs& A, float2 (&cf)[D / 4]) {
  constexpr int QUARTER = D / 4;
  double2 f[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) {
    const int pr = (i >> 3) * 16 + 4 * ((i >> 1) & 3) + 2 * g + (i & 1);
    const int axis = pr / QUARTER, kk = pr - axis * QUARTER;
    const int pos = axis ? px : py, pc = pos < A.P ? pos : A.P - 1;
    f[i] = A.cs[pc * QUARTER + kk];
  }
#pragma unroll
  for (int i = 0; i < D / 4; ++i) {
    const int pr = (i >> 3) * 16 + 4 * ((i >> 1) & 3) + 2 * g + (i & 1);
    const int axis = pr / QUARTER, kk = pr - axis * QUARTER;
    const int pos = axis ? px : py;
    if (pos >= A.P) f[i] = rope_cos_sin(pos, kk, D / 2, A.log2_theta);
  }
#pragma unroll
  for (int i = 0; i < D / 4; ++i) cf[i] = make_float2(static_cast<float>(f[i].x), static_cast<float>(f[i].y));
}

// Inverse RoPE of the pair (a, b) with factors (cos, sin), in fp32, then bf16.
__device__ __forceinline__ uint32_t unrotate_pair(float a, float b, float2 cs) {
  return pack_bf16x2(a * cs.x + b * cs.y, b * cs.x - a * cs.y);
}

// One lane's part of an output row (lane: row ql, dims dt*32 + 8 (r/4) + 4 g + r%4 of
// v[dt][r]), times sc, inverse-rotated for a row at (py, px) when RoPE is on, as bf16.
template <int D>
__device__ __forceinline__ void store_row_part(const f32x16 (&v)[D / 32], float sc, int g, int py, int px,
                                               const BwdArgs& A, bf16_t* orow) {
  float2 cf[D / 4];
  if (A.rope_on) lane_factors<D>(g, py, px, A, cf);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = dt * 32 + 8 * rg + 4 * g, i = 2 * (4 * dt + rg);
      const float a0 = sc * v[dt][4 * rg], a1 = sc * v[dt][4 * rg + 1];
      const float a2 = sc * v[dt][4 * rg + 2], a3 = sc * v[dt][4 * rg + 3];
      const uint32_t w0 = A.rope_on ? unrotate_pair(a0, a1, cf[i]) : pack_bf16x2(a0, a1);
      const uint32_t w1 = A.rope_on ? unrotate_pair(a2, a3, cf[i + 1]) : pack_bf16x2(a2, a3);
      *reinterpret_cast<uint2*>(orow + d0) = make_uint2(w0, w1);
    }
}

// Token (row of the caller's tensors) and position of valid buffer row `row`.
__device__ __forceinline__ int64_t raster_row(int64_t row, const BwdArgs& A, int& py, int& px) {
  return bwd_source(row, A.T, A.N, A.M, A.Mp, A.W, A.w, A.n_wx, A.W_lr, A.rho, py, px);
}

// Row blocks of the three kinds: hi rows (window-first), guide rows, text rows.
enum { kRowsHi = 0, kRowsGuide = 1, kRowsText = 2 };

// Tile list of a row block (key tiles for dQ, query tiles for dK/dV), in three segments:
// first the tiles of the windows within `radius` of a hi block's window (an LDS table;
// the mask is symmetric there) or every hi tile, then guide tiles, then text tiles.
//   dQ:    hi rows: neighbours, guide, text; guide rows: guide, text; text rows: all.
//   dK/dV: hi rows: neighbours, text; guide and text rows: all.
struct TileSegs {
  int n_first, n_g, n_t;  // tiles per segment
  bool table;             // first segment from the table (else every hi tile)
  bool g_table;           // guide segment from the table too: cell blocks (guide modes 1, 2)
  int hi_tiles, g_base, t_base;
  __device__ __forceinline__ int count() const { return n_first + n_g + n_t; }
  __device__ __forceinline__ bool in_cells(int t) const { return g_table && t >= n_first && t < n_first + n_g; }
  __device__ __forceinline__ int index(int t, const uint32_t* tab) const {
    if (t < n_first) return table ? static_cast<int>(__builtin_amdgcn_readfirstlane(tab[t])) : t;
    if (t < n_first + n_g)
      return g_table ? static_cast<int>(__builtin_amdgcn_readfirstlane(tab[t])) : g_base + (t - n_first);
    return t_base + (t - n_first - n_g);
  }
  // rows of tile t that exist (guide and text segments end in partial tiles; cell blocks
  // are masked by their cell masks)
  __device__ __forceinline__ int valid(int t, const BwdArgs& A) const {
    if (t < n_first || in_cells(t)) return kKeyTile;
    const int64_t rem = t < n_first + n_g ? A.M - static_cast<int64_t>(t - n_first) * kKeyTile
                                          : A.T - static_cast<int64_t>(t - n_first - n_g) * kKeyTile;
    return rem < kKeyTile ? static_cast<int>(rem) : kKeyTile;
  }
};

__device__ __forceinline__ TileSegs make_segs(const BwdArgs& A, int kind, bool key_outer, int n_local) {
  TileSegs s;
  const int n_g = static_cast<int>((A.M + kKeyTile - 1) / kKeyTile);
  const int n_t = static_cast<int>((A.T + kKeyTile - 1) / kKeyTile);
  s.hi_tiles = static_cast<int>(A.N / kKeyTile);
  s.g_base = s.hi_tiles;
  s.t_base = static_cast<int>((A.N + A.Mp) / kKeyTile);
  s.table = kind == kRowsHi;
  s.g_table = false;
  if (kind == kRowsHi) {
    s.n_first = n_local;
    s.n_g = key_outer ? 0 : n_g;
  } else {
    s.n_first = (kind == kRowsText || key_outer) ? s.hi_tiles : 0;
    s.n_g = n_g;
  }
  s.n_t = n_t;
  return s;
}

// First buffer row of row block `blk` of a kind (hi blocks hold `rows` rows, the others 256)
__device__ __forceinline__ int64_t block_row0(const BwdArgs& A, int kind, int blk, int rows) {
  if (kind == kRowsHi) return static_cast<int64_t>(blk) * rows;
  if (kind == kRowsGuide) return A.N + static_cast<int64_t>(blk) * rows;
  return A.N + A.Mp + static_cast<int64_t>(blk) * rows;
}
// Whether buffer row `row` of a block of this kind holds a token (not padding)
__device__ __forceinline__ bool row_exists(const BwdArgs& A, int kind, int64_t row) {
  if (kind == kRowsHi) return true;
  if (kind == kRowsGuide) return row - A.N < A.M;
  return row - A.N - A.Mp < A.T;
}

// Tile list of a block of rows (queries for dQ, keys for dK/dV): for hi rows the tiles of
// the windows within `radius` of the row's window (the mask is symmetric there), then for
// dQ the guide key tiles; for guide rows: dQ the guide key tiles, dK/dV every hi query tile
// and then the guide query tiles.  Local tiles come from an LDS table of tile indices.
template <int NT>
__device__ int build_local_table(const BwdArgs& A, int r0, uint32_t* tab) {
  const int tpw = A.w2 / kKeyTile;
  const int win = r0 / A.w2;
  const int wy = win / A.n_wx, wx = win - wy * A.n_wx;
  const int y0 = max(0, wy - A.radius), y1 = min(A.n_wy - 1, wy + A.radius);
  const int x0 = max(0, wx - A.radius), x1 = min(A.n_wx - 1, wx + A.radius);
  const int nx = x1 - x0 + 1;
  const int n = (y1 - y0 + 1) * nx * tpw;
  for (int i = threadIdx.x; i < n; i += NT) {
    const int j = i / tpw, sub = i - j * tpw;
    const int jy = j / nx, nw = (y0 + jy) * A.n_wx + x0 + (j - jy * nx);
    tab[i] = static_cast<uint32_t>(nw * tpw + sub);
  }
  return n;
}

// Wait until at most n tiles' copies (ops_per_tile DMA instructions each) of this wave are
// in flight, then barrier: the older tiles are then complete and visible.
template <int OPS>
__device__ __forceinline__ void wait_tiles(int n) {
  if (n >= 2) wait_vm_and_barrier<2 * OPS>();
  else if (n == 1) wait_vm_and_barrier<OPS>();
  else wait_vm_and_barrier<0>();
}

// ---------------------------------------------------------------- dQ (query-outer)
//
// Wave = 32 queries (lane & 31), as the forward: S^T = K Q^T and dP^T = V dO^T (A = K / V
// tile rows from LDS, B = Q / dO held in registers), so each lane holds one query's
// scores; dS^T converted to bf16 in place is the B operand of dQ^T += K~^T dS^T with A read
// transposed from the same K tile.
template <int D, int NWAVES, int KIND, bool RECT>
__global__ __launch_bounds__(NWAVES * 64) void bwd_dq_kernel(BwdArgs A) {
  constexpr bool HI = KIND == kRowsHi;
  static_assert(!RECT || HI, "cell blocks serve hi-res queries");
  constexpr int NT = NWAVES * 64;
  constexpr int TILE = kKeyTile * D * 2;
  constexpr int CPT = TILE / 16 / NT;
  constexpr int KCH = D / 8;
  constexpr int OPS = 2 * CPT;      // DMA instructions per wave per tile
  constexpr int STAGE = 2 * TILE;   // K rows, V rows
  constexpr int AH = kBwdStages - 1;
  __shared__ __attribute__((aligned(16))) char ring[kBwdStages * STAGE];
  __shared__ uint32_t tab[HI ? kBwdMaxTiles : 1];
  __shared__ uint32_t tmask[RECT ? kBwdMaxTiles : 1];  // cell-block tiles: row / column masks

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, g = lane >> 5;
  const int blk = xcd_remap(blockIdx.x, A.total_blocks);
  const int bh = blk / A.blocks_per_bh, rem_blk = blk - bh * A.blocks_per_bh;
  const int qb = KIND == kRowsText ? rem_blk / A.splits : rem_blk;
  const int split = KIND == kRowsText ? rem_blk - qb * A.splits : 0;
  const int b = bh / A.heads, h = bh - b * A.heads;
  const int64_t r0 = block_row0(A, KIND, qb, NWAVES * 32);
  int n_local = 0, n_rect = 0;
  if (HI) {
    n_local = build_local_table<NT>(A, static_cast<int>(r0), tab);
    if (RECT) {
      // the 8x8 cell blocks that meet the window's visible guide cells, with row / column
      // masks (bits 0-7 the block's cell rows, bits 8-15 its columns)
      const int win = static_cast<int>(r0 / A.w2), wy = win / A.n_wx, wx = win - wy * A.n_wx;
      int i0, i1, j0, j1;
      window_cells(A, wy, wx, i0, i1, j0, j1);
      if (i0 < i1 && j0 < j1) {
        const int bi0 = i0 >> 3, bj0 = j0 >> 3, nbx = ((j1 - 1) >> 3) - bj0 + 1;
        n_rect = (((i1 - 1) >> 3) - bi0 + 1) * nbx;
        for (int k = threadIdx.x; k < n_rect; k += NT) {
          const int ky = k / nbx, bi = bi0 + ky, bj = bj0 + (k - ky * nbx);
          uint32_t rows = 0, cols = 0;
          for (int e = 0; e < 8; ++e) {
            rows |= static_cast<uint32_t>(8 * bi + e >= i0 && 8 * bi + e < i1) << e;
            cols |= static_cast<uint32_t>(8 * bj + e >= j0 && 8 * bj + e < j1) << e;
          }
          tab[n_local + k] = static_cast<uint32_t>(bi * A.nbjp + bj);
          tmask[n_local + k] = rows | (cols << 8);
        }
      }
    }
    __syncthreads();
  }
  TileSegs segs = make_segs(A, KIND, false, n_local);
  if (RECT) {
    segs.n_g = n_rect;
    segs.g_table = true;
  }
  int t_first = 0, t_end = segs.count();
  if (KIND == kRowsText) split_range(segs.count(), A.splits, split, t_first, t_end);
  const int n_tiles = t_end - t_first;  // this workgroup's tiles t_first + [0, n_tiles)
  const int64_t mat = static_cast<int64_t>(bh) * A.R * D * 2;
  const char* kbase = reinterpret_cast<const char*>(A.kb) + mat;
  const char* vbase = reinterpret_cast<const char*>(A.vb) + mat;
  const int64_t cmat = static_cast<int64_t>(bh) * A.Mb * D * 2;
  const char* kgbase = reinterpret_cast<const char*>(A.kgb) + cmat;
  const char* vgbase = reinterpret_cast<const char*>(A.vgb) + cmat;
  auto tile_index = [&](int t) -> int { return segs.index(t_first + t, tab); };
  auto tile_valid = [&](int t) -> int { return segs.valid(t_first + t, A); };
  auto tile_cells = [&](int t) -> uint32_t {
    return RECT && segs.in_cells(t_first + t) ? __builtin_amdgcn_readfirstlane(tmask[t_first + t]) : 0xffffu;
  };
  int k_src[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int slot = (i * NWAVES + wave) * 64 + lane;
    const int kr = slot / KCH, kp = slot - kr * KCH;
    k_src[i] = kr * (D * 2) + ((kp ^ bwd_swizzle<D>(kr)) << 4);
  }
  auto issue = [&](int t) {
    const int64_t off = static_cast<int64_t>(tile_index(t)) * TILE;
    const bool cellt = RECT && segs.in_cells(t_first + t);
    const char* ks = (cellt ? kgbase : kbase) + off;
    const char* vs = (cellt ? vgbase : vbase) + off;
    const uint32_t base = lds_addr(ring + (t & (kBwdStages - 1)) * STAGE);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const uint32_t o = __builtin_amdgcn_readfirstlane(base + (i * NWAVES + wave) * 64 * 16);
      dma_16b(ks, k_src[i], o);
      dma_16b(vs, k_src[i], o + TILE);
    }
  };

  // query fragments (B operands): Q (base-2 scaled) and dO; per-lane -lse2 and -D
  const int64_t qrow = r0 + wave * 32 + ql;
  bf16x8 qf[D / 16], gf[D / 16];
  {
    const bf16_t* qp = A.qb + (static_cast<int64_t>(bh) * A.R + qrow) * D;
    const bf16_t* gp = A.dob + (static_cast<int64_t>(bh) * A.R + qrow) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qf[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk + 8 * g);
      gf[kk] = *reinterpret_cast<const bf16x8*>(gp + 16 * kk + 8 * g);
    }
  }
  const float* at = A.aux + (static_cast<int64_t>(bh) * (A.R / kKeyTile) + qrow / kKeyTile) * (2 * kKeyTile);
  const float nl2 = at[qrow % kKeyTile], nd = at[kKeyTile + qrow % kKeyTile];
  __builtin_amdgcn_s_waitcnt(0);

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;

  // Row fragment for reduction step kk: rows ql (half 0) and 32 + ql (half 1).  The
  // swizzled offset is row * 2D + (((2 kk + g) ^ swz(row)) << 4) = kfo ^ (kk << 5) (+ 64 D
  // for half 1: swz(row) is the same for both halves); kfo is made opaque once per tile
  // so that the XORs are recomputed there instead of held in registers across the loop.
  const int kfo0 = ql * (D * 2) + ((g ^ bwd_swizzle<D>(ql)) << 4);
  int kfo = kfo0;
  auto k_frag = [&](const char* tb, int kk, int half) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(tb + (kfo ^ (kk << 5)) + half * 32 * (D * 2));
  };
  const TrAddr<D> tra(lane);

  for (int p = 0; p < AH; ++p)
    if (p < n_tiles) issue(p);
  wait_tiles<OPS>(std::min(n_tiles, AH) - 1);
  for (int t = 0; t < n_tiles; ++t) {
    if (t + AH < n_tiles) issue(t + AH);
    kfo = kfo0;
    asm volatile("" : "+v"(kfo));
    const char* kt_ = ring + (t & (kBwdStages - 1)) * STAGE;
    const char* vt_ = kt_ + TILE;
    f32x16 s0 = {}, s1 = {}, p0 = {}, p1 = {};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(kt_, kk, 0), qf[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(kt_, kk, 1), qf[kk], s1, 0, 0, 0);
      p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(vt_, kk, 0), gf[kk], p0, 0, 0, 0);
      p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(vt_, kk, 1), gf[kk], p1, 0, 0, 0);
    }
    const int valid = tile_valid(t);
    // cell-block tiles: key k is cell (k / 8, k % 8) of the block, i.e. row r/4 (+4 in the
    // second half) and column 4g + r%4
    const uint32_t cells = tile_cells(t);
    if (valid < kKeyTile || cells != 0xffffu) {
      // partial or cell-block tile: scores of keys past the end or outside the cells -> -inf
      const uint32_t colm = (cells >> (8 + 4 * g)) & 15u;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * g + (r & 3);
        const bool c_ok = (colm >> (r & 3)) & 1u;
        if (!(key < valid && c_ok && ((cells >> (r >> 2)) & 1u))) s0[r] = -INFINITY;
        if (!(key + 32 < valid && c_ok && ((cells >> (4 + (r >> 2))) & 1u))) s1[r] = -INFINITY;
      }
    }
    bf16x8 dsb[4];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float a0 = __builtin_amdgcn_exp2f(s0[r] + nl2);
      const float a1 = __builtin_amdgcn_exp2f(s1[r] + nl2);
      dsb[r >> 3][r & 7] = static_cast<__bf16>(a0 * (p0[r] + nd));
      dsb[2 + (r >> 3)][r & 7] = static_cast<__bf16>(a1 * (p1[r] + nd));
    }
    int xb = tra.x;
    asm volatile("" : "+v"(xb));
    {
      // dQ^T += K~^T dS^T: MFMA i takes key-step i / DT and dims i % DT; its transposed
      // fragment is read two MFMAs ahead (S and dP are dead here)
      constexpr int DT = D / 32, NI = 4 * DT, AHD = 2;
      bf16x8 f[NI];
#pragma unroll
      for (int i = 0; i < AHD; ++i) f[i] = TrAddr<D>::frag(kt_, xb, i / DT, i % DT);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        acc[i % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i], dsb[i / DT], acc[i % DT], 0, 0, 0);
        if (i + AHD < NI) f[i + AHD] = TrAddr<D>::frag(kt_, xb, (i + AHD) / DT, (i + AHD) % DT);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_tiles<OPS>(std::min(n_tiles - 1, t + AH) - (t + 1));
  }

  // epilogue: dQ~ = scale * acc (lane: query ql, dims dt*32 + 8*(r/4) + 4g + r%4), unrotate;
  // text row blocks store their split's unscaled partial sums for bwd_text_combine_kernel
  if (KIND == kRowsText) {
    float* pp = A.part0 + ((static_cast<int64_t>(split) * A.total_blocks / A.blocks_per_bh + bh) * A.Tp +
                           (qrow - A.N - A.Mp)) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = dt * 32 + 8 * rg + 4 * g;
        *reinterpret_cast<f32x4*>(pp + d0) =
            f32x4{acc[dt][4 * rg], acc[dt][4 * rg + 1], acc[dt][4 * rg + 2], acc[dt][4 * rg + 3]};
      }
    return;
  }
  if (!row_exists(A, KIND, qrow)) return;
  int py, px;
  const int64_t rr = raster_row(qrow, A, py, px);
  bf16_t* orow = A.out0 + ((static_cast<int64_t>(b) * A.L + rr) * A.heads + h) * D;
  store_row_part<D>(acc, A.out_scale, g, py, px, A, orow);
}

// ---------------------------------------------------------------- dK, dV (key-outer)
//
// Wave = 32 keys (lane & 31).  Per 64-query tile, in halves of 32 queries: S = Q K~^T and
// dP = dO V^T (A = Q / dO tile rows from LDS, B = K / V held in registers), so a lane holds
// one key's scores for 16 queries; P and dS converted to bf16 in place are the B operands
// of dV^T += dO^T P and dK^T += Q^T dS with A read transposed from the same dO / Q tiles.
template <int D, int NWAVES, int KIND, bool RECT>
__global__ __launch_bounds__(NWAVES * 64) void bwd_dkv_kernel(BwdArgs A) {
  constexpr bool HI = KIND == kRowsHi;
  // RECT: guide keys of guide modes 1 and 2, in cell-block order (slot = block * 64 + cell)
  static_assert(!RECT || KIND == kRowsGuide, "cell blocks order guide keys");
  constexpr int NT = NWAVES * 64;
  constexpr int TILE = kKeyTile * D * 2;
  constexpr int CPT = TILE / 16 / NT;
  constexpr int KCH = D / 8;
  constexpr int AUX_LANES = kAuxBytes / 16 / NWAVES;  // lanes per wave copying the aux block
  constexpr int OPS = 2 * CPT + 1;                     // DMA instructions per wave per tile
  constexpr int STAGE = 2 * TILE + kAuxBytes;          // Q rows, dO rows, -lse2 / -D
  constexpr int AH = kBwdStages - 1;
  static_assert(AUX_LANES >= 1 && AUX_LANES * 16 * NWAVES == kAuxBytes, "aux split");
  __shared__ __attribute__((aligned(16))) char ring[kBwdStages * STAGE];
  __shared__ uint32_t tab[HI || RECT ? kBwdMaxTiles : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, g = lane >> 5;
  const int blk = xcd_remap(blockIdx.x, A.total_blocks);
  const int bh = blk / A.blocks_per_bh, rem_blk = blk - bh * A.blocks_per_bh;
  const int kb_ = KIND == kRowsText ? rem_blk / A.splits : rem_blk;
  const int split = KIND == kRowsText ? rem_blk - kb_ * A.splits : 0;
  const int b = bh / A.heads, h = bh - b * A.heads;
  // RECT: r0 is the first cell-block slot of the workgroup (4 blocks of one block row)
  const int64_t r0 = RECT ? static_cast<int64_t>(kb_) * NWAVES * 32 : block_row0(A, KIND, kb_, NWAVES * 32);
  int n_local = 0;
  if (HI) {
    n_local = build_local_table<NT>(A, static_cast<int>(r0), tab);
    __syncthreads();
  }
  if (RECT) {
    // query tiles of the windows that see any cell of the workgroup's blocks: the window
    // holding a visible cell's scaled position, widened by `reach` (a bounding box; the
    // per-key masks below drop the pairs it over-covers)
    const int blk0 = static_cast<int>(r0 / kKeyTile), bi = blk0 / A.nbjp, bj0 = blk0 - bi * A.nbjp;
    const int ci0 = 8 * bi, cj0 = 8 * bj0;
    const int ci1 = min(min(8 * bi + 7, A.H_lr - 1), (A.n_wy * A.w - 1) / A.rho);
    const int cj1 = min(min(8 * bj0 + 31, A.W_lr - 1), (A.n_wx * A.w - 1) / A.rho);
    if (ci0 <= ci1 && cj0 <= cj1) {
      const int y0 = max(0, A.rho * ci0 / A.w - A.reach), y1 = min(A.n_wy - 1, A.rho * ci1 / A.w + A.reach);
      const int x0 = max(0, A.rho * cj0 / A.w - A.reach), x1 = min(A.n_wx - 1, A.rho * cj1 / A.w + A.reach);
      const int tpw = A.w2 / kKeyTile, nx = x1 - x0 + 1;
      n_local = (y1 - y0 + 1) * nx * tpw;
      for (int i = threadIdx.x; i < n_local; i += NT) {
        const int j = i / tpw, sub = i - j * tpw;
        const int jy = j / nx, nw = (y0 + jy) * A.n_wx + x0 + (j - jy * nx);
        tab[i] = static_cast<uint32_t>(nw * tpw + sub);
      }
    }
    __syncthreads();
  }
  TileSegs segs = make_segs(A, KIND, true, n_local);
  if (RECT) {
    segs.n_first = n_local;
    segs.table = true;
  }
  int t_first = 0, t_end = segs.count();
  if (KIND == kRowsText) split_range(segs.count(), A.splits, split, t_first, t_end);
  const int n_tiles = t_end - t_first;  // this workgroup's tiles t_first + [0, n_tiles)
  const int64_t mat = static_cast<int64_t>(bh) * A.R * D * 2;
  const char* qbase = reinterpret_cast<const char*>(A.qb) + mat;
  const char* gbase = reinterpret_cast<const char*>(A.dob) + mat;
  const char* abase = reinterpret_cast<const char*>(A.aux) + static_cast<int64_t>(bh) * (A.R / kKeyTile) * kAuxBytes;
  auto tile_index = [&](int t) -> int { return segs.index(t_first + t, tab); };
  int k_src[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int slot = (i * NWAVES + wave) * 64 + lane;
    const int kr = slot / KCH, kp = slot - kr * KCH;
    k_src[i] = kr * (D * 2) + ((kp ^ bwd_swizzle<D>(kr)) << 4);
  }
  // every wave issues the same number of copies per tile (its share of the aux block
  // included), so the in-flight counts of wait_tiles hold for all waves
  auto issue = [&](int t) {
    const int ti = tile_index(t);
    const int64_t off = static_cast<int64_t>(ti) * TILE;
    const uint32_t base = lds_addr(ring + (t & (kBwdStages - 1)) * STAGE);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const uint32_t o = __builtin_amdgcn_readfirstlane(base + (i * NWAVES + wave) * 64 * 16);
      dma_16b(qbase + off, k_src[i], o);
      dma_16b(gbase + off, k_src[i], o + TILE);
    }
    if (lane < AUX_LANES)
      dma_16b(abase + static_cast<int64_t>(ti) * kAuxBytes, (wave * AUX_LANES + lane) * 16,
              __builtin_amdgcn_readfirstlane(base + 2 * TILE + wave * AUX_LANES * 16));
  };

  // key fragments (B operands): K~ and V rows of this lane's key
  const int64_t krow = r0 + wave * 32 + ql;  // RECT: cell-block slot
  int kci = 0, kcj = 0;                        // RECT: the key's guide cell
  if (RECT) {
    const int cb = static_cast<int>(krow / kKeyTile), cc = static_cast<int>(krow % kKeyTile);
    const int bi = cb / A.nbjp;
    kci = 8 * bi + (cc >> 3);
    kcj = 8 * (cb - bi * A.nbjp) + (cc & 7);
  }
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const bf16_t* kp = RECT ? A.kgb + (static_cast<int64_t>(bh) * A.Mb + krow) * D
                            : A.kb + (static_cast<int64_t>(bh) * A.R + krow) * D;
    const bf16_t* vp = RECT ? A.vgb + (static_cast<int64_t>(bh) * A.Mb + krow) * D
                            : A.vb + (static_cast<int64_t>(bh) * A.R + krow) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      kf[kk] = *reinterpret_cast<const bf16x8*>(kp + 16 * kk + 8 * g);
      vf[kk] = *reinterpret_cast<const bf16x8*>(vp + 16 * kk + 8 * g);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[dt][r] = dv[dt][r] = 0.0f;

  // Row fragment for reduction step kk: rows ql (half 0) and 32 + ql (half 1).  The
  // swizzled offset is row * 2D + (((2 kk + g) ^ swz(row)) << 4) = kfo ^ (kk << 5) (+ 64 D
  // for half 1: swz(row) is the same for both halves); kfo is made opaque once per tile
  // so that the XORs are recomputed there instead of held in registers across the loop.
  const int kfo0 = ql * (D * 2) + ((g ^ bwd_swizzle<D>(ql)) << 4);
  int kfo = kfo0;
  auto k_frag = [&](const char* tb, int kk, int half) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(tb + (kfo ^ (kk << 5)) + half * 32 * (D * 2));
  };
  const TrAddr<D> tra(lane);

  for (int p = 0; p < AH; ++p)
    if (p < n_tiles) issue(p);
  wait_tiles<OPS>(std::min(n_tiles, AH) - 1);
  for (int t = 0; t < n_tiles; ++t) {
    if (t + AH < n_tiles) issue(t + AH);
    kfo = kfo0;
    asm volatile("" : "+v"(kfo));
    const char* qt_ = ring + (t & (kBwdStages - 1)) * STAGE;
    const char* gt_ = qt_ + TILE;
    const float* aux = reinterpret_cast<const float*>(qt_ + 2 * TILE);
    // RECT: hi query tiles (first segment) see this lane's key only if the tile's window
    // sees its cell; guide and text queries see every guide key
    bool kvis = true;
    if (RECT && t_first + t < segs.n_first) {
      const int win = tile_index(t) / (A.w2 / kKeyTile), wy = win / A.n_wx, wx = win - wy * A.n_wx;
      int i0, i1, j0, j1;
      window_cells(A, wy, wx, i0, i1, j0, j1);
      kvis = kci >= i0 && kci < i1 && kcj >= j0 && kcj < j1;
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // S and dP start from -lse2 and -D of their query rows (rows are queries
      // 32 half + 8(r/4) + 4g + r%4 of the tile; lanes are keys), so P = exp2(S) and
      // dS = P dP come out of the accumulators directly
      f32x16 s, p;
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int q0 = 32 * half + 8 * rq + 4 * g;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(aux + q0);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(aux + kKeyTile + q0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[4 * rq + e] = l4[e];
          p[4 * rq + e] = d4[e];
        }
      }
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(qt_, kk, half), kf[kk], s, 0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(gt_, kk, half), vf[kk], p, 0, 0, 0);
      }
      bf16x8 pb[2], db[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = kvis ? __builtin_amdgcn_exp2f(s[r]) : 0.0f;
        pb[r >> 3][r & 7] = static_cast<__bf16>(pr);
        db[r >> 3][r & 7] = static_cast<__bf16>(pr * p[r]);
      }
      int xb = tra.x;
      asm volatile("" : "+v"(xb));
      {
        // dV^T += dO^T P and dK^T += Q^T dS: MFMA i takes key-step j = i / (2 DT) and dims
        // dt = (i / 2) % DT, dV for even i, dK for odd i.  Its transposed fragment is read two
        // MFMAs ahead (the scheduling barriers keep the reads there; S and dP are dead by
        // now, so the registers are free)
        constexpr int DT = D / 32, NI = 4 * DT, AHD = 2;
        auto frag = [&](int i) __attribute__((always_inline)) {
          return TrAddr<D>::frag((i & 1) ? qt_ : gt_, xb, 2 * half + i / (2 * DT), (i / 2) % DT);
        };
        bf16x8 f[NI];
#pragma unroll
        for (int i = 0; i < AHD; ++i) f[i] = frag(i);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          __builtin_amdgcn_sched_barrier(0);
          const int j = i / (2 * DT), dt = (i / 2) % DT;
          if (i & 1) dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i], db[j], dk[dt], 0, 0, 0);
          else dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i], pb[j], dv[dt], 0, 0, 0);
          if (i + AHD < NI) f[i + AHD] = frag(i + AHD);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_tiles<OPS>(std::min(n_tiles - 1, t + AH) - (t + 1));
  }

  // epilogue: dK~ = ln2 * dk (Q carried scale * log2 e), unrotated; dV = dv; text row
  // blocks store their split's unscaled partial sums for bwd_text_combine_kernel
  if (KIND == kRowsText) {
    const int64_t po = ((static_cast<int64_t>(split) * A.total_blocks / A.blocks_per_bh + bh) * A.Tp +
                        (krow - A.N - A.Mp)) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = dt * 32 + 8 * rg + 4 * g;
        *reinterpret_cast<f32x4*>(A.part0 + po + d0) =
            f32x4{dk[dt][4 * rg], dk[dt][4 * rg + 1], dk[dt][4 * rg + 2], dk[dt][4 * rg + 3]};
        *reinterpret_cast<f32x4*>(A.part1 + po + d0) =
            f32x4{dv[dt][4 * rg], dv[dt][4 * rg + 1], dv[dt][4 * rg + 2], dv[dt][4 * rg + 3]};
      }
    return;
  }
  int py, px;
  int64_t rr;
  if (RECT) {
    if (kci >= A.H_lr || kcj >= A.W_lr) return;
    py = A.rho * kci;
    px = A.rho * kcj;
    rr = A.T + A.N + static_cast<int64_t>(kci) * A.W_lr + kcj;
  } else {
    if (!row_exists(A, KIND, krow)) return;
    rr = raster_row(krow, A, py, px);
  }
  const int64_t ro = ((static_cast<int64_t>(b) * A.L + rr) * A.heads + h) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = dt * 32 + 8 * rg + 4 * g;
      *reinterpret_cast<uint2*>(A.out1 + ro + d0) =
          make_uint2(pack_bf16x2(dv[dt][4 * rg], dv[dt][4 * rg + 1]),
                     pack_bf16x2(dv[dt][4 * rg + 2], dv[dt][4 * rg + 3]));
    }
  store_row_part<D>(dk, A.out_scale, g, py, px, A, A.out0 + ro);
}

// ------------------------------------------------------------------ host side

namespace {

// Largest LDS tile tables of guide modes 1 and 2 (mirrors the kernels' constructions): per
// window its neighbour tiles plus the cell blocks of its visible cells (dQ), and per
// workgroup of 4 cell blocks the tiles of the windows that can see them (dK/dV).
int64_t max_rect_tables(const BwdGeom& g) {
  const int tpw = g.w * g.w / kKeyTile, n_wy = g.H / g.w, n_wx = g.W / g.w;
  const int reach = g.guide_mode == 1 ? 0 : g.radius;
  auto span = [](int c, int r, int n) { return std::min(n - 1, c + r) - std::max(0, c - r) + 1; };
  int64_t best = 0;
  for (int wy = 0; wy < n_wy; ++wy)
    for (int wx = 0; wx < n_wx; ++wx) {
      int64_t n = static_cast<int64_t>(span(wy, g.radius, n_wy)) * span(wx, g.radius, n_wx) * tpw;
      const int gy0 = std::max(0, wy - reach), gy1 = std::min(n_wy - 1, wy + reach);
      const int gx0 = std::max(0, wx - reach), gx1 = std::min(n_wx - 1, wx + reach);
      const int i0 = (gy0 * g.w + g.rho - 1) / g.rho, i1 = std::min(g.H_lr, ((gy1 + 1) * g.w + g.rho - 1) / g.rho);
      const int j0 = (gx0 * g.w + g.rho - 1) / g.rho, j1 = std::min(g.W_lr, ((gx1 + 1) * g.w + g.rho - 1) / g.rho);
      if (i0 < i1 && j0 < j1)
        n += static_cast<int64_t>(((i1 - 1) >> 3) - (i0 >> 3) + 1) * (((j1 - 1) >> 3) - (j0 >> 3) + 1);
      best = std::max(best, n);
    }
  for (int bi = 0; bi < g.nbi; ++bi)
    for (int bj0 = 0; bj0 < g.nbjp; bj0 += 4) {
      const int ci0 = 8 * bi, cj0 = 8 * bj0;
      const int ci1 = std::min(std::min(8 * bi + 7, g.H_lr - 1), (n_wy * g.w - 1) / g.rho);
      const int cj1 = std::min(std::min(8 * bj0 + 31, g.W_lr - 1), (n_wx * g.w - 1) / g.rho);
      if (ci0 > ci1 || cj0 > cj1) continue;
      const int y0 = std::max(0, g.rho * ci0 / g.w - reach), y1 = std::min(n_wy - 1, g.rho * ci1 / g.w + reach);
      const int x0 = std::max(0, g.rho * cj0 / g.w - reach), x1 = std::min(n_wx - 1, g.rho * cj1 / g.w + reach);
      best = std::max<int64_t>(best, static_cast<int64_t>(y1 - y0 + 1) * (x1 - x0 + 1) * tpw);
    }
  return best;
}


int validate_backward(const void* const* ptrs, int n_ptrs, int B, int T, int H, int W, int w,
                      int H_lr, int W_lr, int rho, int heads, int D, int radius, int guide_mode) {
  for (int i = 0; i < n_ptrs; ++i) {
    if (!ptrs[i]) return fail_arg("null pointer");
    if (reinterpret_cast<uintptr_t>(ptrs[i]) % 16) return fail_arg("tensors must be 16-byte aligned");
  }
  if (B < 1 || T < 0 || H < 1 || W < 1 || w < 1 || heads < 1 || H_lr < 0 || W_lr < 0)
    return fail_arg("sizes out of range");
  if (H % w || W % w) return fail_arg("w must divide H and W");
  if ((H_lr == 0) != (W_lr == 0)) return fail_arg("H_lr and W_lr must both be zero or not");
  if (static_cast<int64_t>(H_lr) * W_lr > 0 && rho < 1) return fail_arg("rho must be >= 1 with guide tokens");
  if (radius < 0) return fail_arg("radius must be >= 0");
  if (guide_mode < 0 || guide_mode > 2) return fail_arg("guide_mode must be 0, 1 or 2");
  if (D != 64 && D != 128) return fail_unsupported("head_dim must be 64 or 128");
  if (w % 8 || (w > 16 && w % 16)) return fail_unsupported("window size must be 8, 16 or a multiple of 16");
  if (B > 65535) return fail_unsupported("batch too large");
  const int64_t N = static_cast<int64_t>(H) * W, M = static_cast<int64_t>(H_lr) * W_lr;
  if (N > (int64_t(1) << 26) || M > (int64_t(1) << 26) || T > (int64_t(1) << 24) ||
      static_cast<int64_t>(B) * heads * ((N + M + T) / 64 + 10) > 0x7fffffff)
    return fail_unsupported("problem too large");
  const int r = std::min(radius, H / w + W / w);
  const int64_t tiles = static_cast<int64_t>(std::min(2 * r + 1, H / w)) * std::min(2 * r + 1, W / w) *
                        (w * w / kKeyTile);
  if (tiles > kBwdMaxTiles) return fail_unsupported("too many key tiles per window");
  if (guide_mode != 0 && M > 0 &&
      max_rect_tables(make_bwd_geom(B, T, H, W, w, H_lr, W_lr, rho, heads, D, r, guide_mode)) > kBwdMaxTiles)
    return fail_unsupported("too many tiles per window or cell-block group");
  return UHLA_OK;
}

// RECT (guide modes 1, 2) selects the cell-block variants: dQ of hi rows, dK/dV of guide rows
template <int D, int KIND, bool RECT>
void launch_dq(int nwaves, const BwdArgs& a, hipStream_t s) {
  constexpr bool R = RECT && KIND == kRowsHi;
  if (KIND != kRowsHi || nwaves == kBwdWaves)
    hipLaunchKernelGGL((bwd_dq_kernel<D, kBwdWaves, KIND, R>), dim3(a.total_blocks), dim3(kBwdWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, 2, kRowsHi, R>), dim3(a.total_blocks), dim3(128), 0, s, a);
}

template <int D, int KIND, bool RECT>
void launch_dkv(int nwaves, const BwdArgs& a, hipStream_t s) {
  constexpr bool R = RECT && KIND == kRowsGuide;
  if (KIND != kRowsHi || nwaves == kBwdWaves)
    hipLaunchKernelGGL((bwd_dkv_kernel<D, kBwdWaves, KIND, R>), dim3(a.total_blocks), dim3(kBwdWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dkv_kernel<D, 2, kRowsHi, false>), dim3(a.total_blocks), dim3(128), 0, s, a);
}

template <int KIND>
void launch_both(bool dkv, bool rect, int D, int nwaves, const BwdArgs& a, hipStream_t s) {
  if (rect) {
    if (dkv) D == 128 ? launch_dkv<128, KIND, true>(nwaves, a, s) : launch_dkv<64, KIND, true>(nwaves, a, s);
    else D == 128 ? launch_dq<128, KIND, true>(nwaves, a, s) : launch_dq<64, KIND, true>(nwaves, a, s);
  } else {
    if (dkv) D == 128 ? launch_dkv<128, KIND, false>(nwaves, a, s) : launch_dkv<64, KIND, false>(nwaves, a, s);
    else D == 128 ? launch_dq<128, KIND, false>(nwaves, a, s) : launch_dq<64, KIND, false>(nwaves, a, s);
  }
}

}  // namespace

}  // namespace uhla

extern "C" size_t uhla_backward_workspace_bytes(int B, int T, int H, int W, int w, int H_lr,
                                                int W_lr, int rho, int heads, int head_dim,
                                                int radius, int guide_mode) {
  if (B < 1 || T < 0 || H < 1 || W < 1 || w < 1 || heads < 1 || H_lr < 0 || W_lr < 0 || radius < 0 ||
      guide_mode < 0 || guide_mode > 2)
    return 0;
  if (H % w || W % w || (H_lr == 0) != (W_lr == 0)) return 0;
  if (head_dim != 64 && head_dim != 128) return 0;
  if (static_cast<int64_t>(H_lr) * W_lr > 0 && rho < 1) return 0;
  return uhla::carve_bwd(uhla::make_bwd_geom(B, T, H, W, w, H_lr, W_lr, rho, heads, head_dim, radius,
                                             guide_mode),
                         nullptr).bytes;
}

extern "C" int uhla_backward(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             int B, int T, int H, int W, int w, int H_lr, int W_lr, int rho,
                             int heads, int head_dim, float scale, float theta, int radius,
                             int guide_mode, void* workspace, size_t workspace_bytes,
                             void* stream) {
  using namespace uhla;
  const void* ptrs[9] = {q, k, v, o, dout, lse, dq, dk, dv};
  int st = validate_backward(ptrs, 9, B, T, H, W, w, H_lr, W_lr, rho, heads, head_dim, radius,
                             guide_mode);
  if (st) return st;
  radius = std::min(radius, H / w + W / w);
  const int D = head_dim;
  const BwdGeom g = make_bwd_geom(B, T, H, W, w, H_lr, W_lr, rho, heads, D, radius, guide_mode);
  const bool rect = g.Mb > 0;
  const BwdWorkspace need = carve_bwd(g, nullptr);
  if (!workspace || workspace_bytes < need.bytes)
    return (set_detail("workspace too small"), UHLA_ERR_WORKSPACE);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail_arg("workspace must be 256-byte aligned");
  const int64_t L = g.T + g.N + g.M;
  const size_t tb = static_cast<size_t>(B) * L * heads * D * 2;
  const void* ins[5] = {q, k, v, o, dout};
  void* outs[3] = {dq, dk, dv};
  for (void* x : outs) {
    for (const void* y : ins)
      if (ranges_overlap(x, tb, y, tb)) return fail_arg("a gradient overlaps an input");
    if (ranges_overlap(x, tb, workspace, need.bytes) ||
        ranges_overlap(x, tb, lse, static_cast<size_t>(B) * heads * L * 4))
      return fail_arg("a gradient overlaps the workspace or lse");
  }
  if (ranges_overlap(dq, tb, dk, tb) || ranges_overlap(dq, tb, dv, tb) || ranges_overlap(dk, tb, dv, tb))
    return fail_arg("gradients overlap each other");
  // the row-prep pass writes the workspace while the inputs are still being read
  for (const void* y : ins)
    if (ranges_overlap(workspace, need.bytes, y, tb)) return fail_arg("the workspace overlaps an input");
  if (ranges_overlap(workspace, need.bytes, lse, static_cast<size_t>(B) * heads * L * 4))
    return fail_arg("the workspace overlaps lse");
  const BwdWorkspace ws = carve_bwd(g, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool rope_on = theta > 0.0f;
  const float sc = scale > 0.0f ? scale : 1.0f / sqrtf(static_cast<float>(D));
  const double l2t = rope_on ? log2(static_cast<double>(theta)) : 0.0;
  const int64_t BH = static_cast<int64_t>(B) * heads;
  const int n_wx = W / w;

#define UHLA_BSTEP(call, name) \
  do {                         \
    call;                      \
    st = check_launch(name);   \
    if (st) return st;         \
  } while (0)

  if (rope_on) {
    const int n = g.P * (D / 4);
    UHLA_BSTEP(hipLaunchKernelGGL(bwd_cos_sin_kernel, dim3((n + 255) / 256), dim3(256), 0, s, ws.cs,
                                  g.P, D, l2t),
               "bwd_cos_sin_kernel");
  }
  {
    const dim3 grid(static_cast<unsigned>((g.R + kBwdRowsPerBlock - 1) / kBwdRowsPerBlock), B);
    const double qs = static_cast<double>(sc) * 1.4426950408889634;
    const bf16_t* qp = static_cast<const bf16_t*>(q);
    const bf16_t* kp = static_cast<const bf16_t*>(k);
    const bf16_t* vp = static_cast<const bf16_t*>(v);
    const bf16_t* gp = static_cast<const bf16_t*>(dout);
    if (D == 128)
      hipLaunchKernelGGL(bwd_rows_kernel<128>, grid, dim3(kBwdThreads), 0, s, qp, kp, vp, gp, ws.qb,
                         ws.kb, ws.vb, ws.dob, ws.cs, g.P, l2t, g.T, g.N, g.M, g.Mp, g.R, W, w, n_wx,
                         W_lr, rho, heads, rope_on ? 1 : 0, qs);
    else
      hipLaunchKernelGGL(bwd_rows_kernel<64>, grid, dim3(kBwdThreads), 0, s, qp, kp, vp, gp, ws.qb,
                         ws.kb, ws.vb, ws.dob, ws.cs, g.P, l2t, g.T, g.N, g.M, g.Mp, g.R, W, w, n_wx,
                         W_lr, rho, heads, rope_on ? 1 : 0, qs);
    st = check_launch("bwd_rows_kernel");
    if (st) return st;
    const int64_t aux_threads = BH * L * (D / 8) + BH * (g.R - L);  // rows, then padding rows
    UHLA_BSTEP(hipLaunchKernelGGL(bwd_aux_kernel, dim3(static_cast<unsigned>((aux_threads + kBwdThreads - 1) / kBwdThreads)),
                                  dim3(kBwdThreads), 0, s, static_cast<const bf16_t*>(o), gp, lse,
                                  ws.aux, g.T, g.N, g.M, g.Mp, g.R, W, w, n_wx, heads, D, BH),
               "bwd_aux_kernel");
    if (rect) {
      const int64_t n = BH * g.Mb * (D / 8);
      UHLA_BSTEP(hipLaunchKernelGGL(bwd_cellblock_kernel, dim3(static_cast<unsigned>((n + kBwdThreads - 1) / kBwdThreads)),
                                    dim3(kBwdThreads), 0, s, ws.kb, ws.vb, ws.kgb, ws.vgb, g.N, g.R, g.Mb,
                                    H_lr, W_lr, g.nbjp, D, BH),
                 "bwd_cellblock_kernel");
    }
  }

  BwdArgs a{};
  a.qb = ws.qb; a.kb = ws.kb; a.vb = ws.vb; a.dob = ws.dob;
  a.aux = ws.aux; a.cs = ws.cs;
  a.T = g.T; a.N = g.N; a.M = g.M; a.Mp = g.Mp; a.R = g.R; a.L = L;
  a.heads = heads; a.w2 = w * w; a.W = W; a.w = w; a.n_wx = n_wx; a.n_wy = H / w;
  a.radius = radius; a.rho = rho; a.W_lr = W_lr; a.P = g.P;
  a.rope_on = rope_on ? 1 : 0; a.log2_theta = l2t;
  a.splits = g.splits; a.part0 = ws.part0; a.part1 = ws.part1; a.Tp = g.Tp;
  a.kgb = ws.kgb; a.vgb = ws.vgb; a.Mb = g.Mb; a.nbjp = g.nbjp; a.H_lr = H_lr;
  a.reach = guide_mode == 1 ? 0 : radius;
  const int nw_hi = std::min(kBwdWaves, w * w / 32);  // w * w is 64 or a multiple of 256

  // dQ, then dK / dV, each over hi rows, guide rows and text rows
  for (int pass = 0; pass < 2; ++pass) {
    const bool dkv = pass == 1;
    a.out0 = static_cast<bf16_t*>(dkv ? dk : dq);
    a.out1 = static_cast<bf16_t*>(dv);
    a.out_scale = dkv ? 0.69314718055994531f : sc;
    a.blocks_per_bh = static_cast<int>(g.N / (nw_hi * 32));
    a.total_blocks = static_cast<int>(BH * a.blocks_per_bh);
    UHLA_BSTEP(launch_both<kRowsHi>(dkv, rect, D, nw_hi, a, s), dkv ? "bwd_dkv_kernel(hi)" : "bwd_dq_kernel(hi)");
    if (g.M > 0) {
      // guide keys of modes 1, 2 are processed in cell-block order
      a.blocks_per_bh = static_cast<int>((dkv && rect ? g.Mb : g.Mp) / kBwdGuideRows);
      a.total_blocks = static_cast<int>(BH * a.blocks_per_bh);
      UHLA_BSTEP(launch_both<kRowsGuide>(dkv, rect, D, kBwdWaves, a, s),
                 dkv ? "bwd_dkv_kernel(guide)" : "bwd_dq_kernel(guide)");
    }
    if (g.T > 0) {
      a.blocks_per_bh = static_cast<int>(g.Tp / kBwdGuideRows) * g.splits;
      a.total_blocks = static_cast<int>(BH * a.blocks_per_bh);
      UHLA_BSTEP(launch_both<kRowsText>(dkv, rect, D, kBwdWaves, a, s),
                 dkv ? "bwd_dkv_kernel(text)" : "bwd_dq_kernel(text)");
      UHLA_BSTEP(hipLaunchKernelGGL(bwd_text_combine_kernel, dim3(static_cast<unsigned>(g.T), static_cast<unsigned>(BH)),
                                    dim3(D / 2), 0, s, ws.part0, dkv ? ws.part1 : nullptr, a.out0,
                                    dkv ? a.out1 : nullptr, a.out_scale, g.splits, BH, g.Tp, g.T, L,
                                    heads, D),
                 "bwd_text_combine_kernel");
    }
  }
#undef UHLA_BSTEP
  return UHLA_OK;
}
