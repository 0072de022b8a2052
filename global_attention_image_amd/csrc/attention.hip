// Hierarchical local attention forward on gfx950 (bf16 MFMA, fp32 softmax).
//
// Mask ([UltraGen/ar §2.B], [UltraGen/es §2]): each hi-res window attends to itself, to
// its clipped 3x3 neighbourhood of windows and to every guide token; guide tokens attend
// to each other.  Blocks are spatial windows in window-first order ([UltraGen/it §2],
// [UltraGen/fr §2.A]).
//
// Pipeline (all on the caller's stream, no allocation):
//   1. the fp64 RoPE cos/sin table [P][head_dim/4]
//   2. prep: window-first permutation of the hi rows of K and V, fused with RoPE on K;
//      K lands head-major [B*heads][rows][D]; V lands in 64-key tiles transposed to
//      [D][64] so the P.V contraction reads it with one 16-byte LDS load per operand.
//      Guide rows are rotated / re-laid out the same way (no permutation).  Q is not
//      prepared: each wave reads its query rows from the caller's Q and rotates them.
//   3. hi pass: one workgroup per (b, h, window, 256-query chunk); it computes its
//      window's neighbour tiles, streams the K/V tiles of its neighbour windows, then of
//      all guide tokens, through LDS, and stores each output row at its raster position
//      (the inverse permutation, fused).
//   4. guide pass: one workgroup per (b, h, 256 guide queries) over all guide keys.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, wave64).  Each wave owns 32 queries.
// S^T = K Q^T: A = 32 keys x 16 dims from LDS, B = Q^T held in registers, so each lane
// holds the scores of ONE query (lane & 31) for 16 keys: softmax statistics stay in the
// lane, plus one exchange with lane ^ 32 (v_permlane32_swap).  O^T = V^T P^T: A = V^T (32 dims x 16 keys)
// from LDS, B = P^T, which is the S^T accumulator converted to bf16 in place.
#include <algorithm>

#include "tile_common.h"

namespace uhla {

constexpr int kMaxQuery = 256;   // queries per workgroup (8 waves x 32)
constexpr int kMaxTableTiles = 1024;  // table-driven key tiles (neighbour + cell-block) per window

// ------------------------------------------------------------------ geometry / layout

struct Geom {
  int B, H, W, w, H_lr, W_lr, rho, heads, D;
  int radius, guide_mode;  // neighbourhood radius in windows; guide tokens seen (0 all, 1, 2)
  int64_t T;               // text tokens at the front of the joint sequence
  int64_t N, M, Mk, Mq;    // Mk: guide rows padded to the key tile; Mq: to the query block
  int64_t Tk, Tq;          // text rows padded to the key tile / the query block
  int64_t Mg;              // rows of the global-key buffer: guide (Mk) then text (Tk)
  int n_wx, n_wy, nW, P;   // P: positions covered by the cos/sin table (max(H, W))
  int nbi, nbj;            // guide grid in 8x8 cell blocks (rows, columns)
  int64_t Mb;              // guide cells in block order, padded: nbi * nbj * 64 (0 if unused)
  int64_t Mbg;             // rows of the cell-block buffer: Mb then (if Mb > 0) the text rows
  int splits;              // key-range splits of the text-query pass
};

static Geom make_geom(int B, int H, int W, int w, int H_lr, int W_lr, int rho, int heads,
                      int D, int radius, int guide_mode, int64_t T) {
  Geom g;
  g.B = B; g.H = H; g.W = W; g.w = w; g.H_lr = H_lr; g.W_lr = W_lr; g.rho = rho;
  g.heads = heads; g.D = D; g.radius = radius; g.guide_mode = guide_mode; g.T = T;
  g.N = static_cast<int64_t>(H) * W;
  g.M = static_cast<int64_t>(H_lr) * W_lr;
  g.Mk = (g.M + kKeyTile - 1) / kKeyTile * kKeyTile;
  g.Mq = (g.M + kMaxQuery - 1) / kMaxQuery * kMaxQuery;
  g.Tk = (T + kKeyTile - 1) / kKeyTile * kKeyTile;
  g.Tq = (T + kMaxQuery - 1) / kMaxQuery * kMaxQuery;
  g.Mg = g.Mk + g.Tk;
  g.n_wx = W / w; g.n_wy = H / w; g.nW = g.n_wx * g.n_wy;
  // The cos/sin table covers hi-res positions; guide positions beyond it (a guide grid
  // reaching past the hi-res extent) are evaluated directly with the same function.
  const int p = H > W ? H : W;
  g.P = p;
  g.nbi = (H_lr + 7) / 8;
  g.nbj = (W_lr + 7) / 8;
  g.Mb = (guide_mode != 0 && g.M > 0) ? static_cast<int64_t>(g.nbi) * g.nbj * kKeyTile : 0;
  g.Mbg = g.Mb > 0 ? g.Mb + g.Tk : 0;
  // Text queries attend to all N + M + T keys: few query blocks, so the key range is split
  // to give the GPU about 1024 workgroups, each split at least 8 tiles long.
  g.splits = 0;
  if (T > 0) {
    const int64_t qblocks = static_cast<int64_t>(B) * heads * (g.Tq / kMaxQuery);
    const int64_t tiles = (g.N + g.Mg) / kKeyTile;
    int64_t sp = (1024 + qblocks - 1) / qblocks;
    sp = std::min(sp, std::max<int64_t>(1, tiles / 8));
    g.splits = static_cast<int>(std::max<int64_t>(1, sp));
  }
  return g;
}

struct Workspace {
  double2* cs;    // [P][D/4]
  bf16_t* k_hi;   // [B*heads][N][D]   window-first, rotated
  bf16_t* v_hi;   // [B*heads][N/64][D][64]  window-first, transposed tiles
  bf16_t* k_lr;   // [B*heads][Mg][D]  global keys: guide rows (Mk, zero padded), text rows (Tk)
  bf16_t* v_lr;   // [B*heads][Mg/64][D][64]
  bf16_t* k_gb;   // [B*heads][Mbg][D] guide K in 8x8 cell blocks, then text (guide modes 1, 2)
  bf16_t* v_gb;   // [B*heads][Mbg/64][D][64]
  float* o_part;  // [splits][B*heads][Tq][D]  text-query partial outputs (unnormalised)
  float2* ml_part;  // [splits][B*heads][Tq]   their (running max, sum)
  bf16_t* q_hi;   // guide modes 1, 2: [B*heads][N][D] window-first Q, rotated and scaled
  bf16_t* q_lr;   // guide modes 1, 2: [B*heads][M][D] guide Q, rotated and scaled
  size_t bytes;
};

static Workspace carve(const Geom& g, void* base) {
  Workspace ws;
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off = align_up(off + n, 256);
    return o;
  };
  const size_t bh = static_cast<size_t>(g.B) * g.heads;
  const size_t e = sizeof(bf16_t);
  const size_t o_cs = take(sizeof(double2) * g.P * (g.D / 4));
  const size_t o_kh = take(bh * g.N * g.D * e);
  const size_t o_vh = take(bh * g.N * g.D * e);
  const size_t o_kl = take(bh * g.Mg * g.D * e);
  const size_t o_vl = take(bh * g.Mg * g.D * e);
  const size_t o_kb = take(bh * g.Mbg * g.D * e);
  const size_t o_vb = take(bh * g.Mbg * g.D * e);
  const size_t o_op = take(static_cast<size_t>(g.splits) * bh * g.Tq * g.D * sizeof(float));
  const size_t o_ml = take(static_cast<size_t>(g.splits) * bh * g.Tq * sizeof(float2));
  // With the guide-locality masks a workgroup has few key tiles (5 at radius 0), so the
  // latency of gathering its query rows from the raster layout (one workgroup per CU) is
  // not hidden by its loop: there Q is prepared like K.
  const bool q_pre = g.guide_mode != 0 && g.M > 0;
  const size_t o_qh = take(q_pre ? bh * g.N * g.D * e : 0);
  const size_t o_ql = take(q_pre ? bh * g.M * g.D * e : 0);
  char* b = static_cast<char*>(base);
  ws.cs = reinterpret_cast<double2*>(b + o_cs);
  ws.k_hi = reinterpret_cast<bf16_t*>(b + o_kh);
  ws.v_hi = reinterpret_cast<bf16_t*>(b + o_vh);
  ws.k_lr = reinterpret_cast<bf16_t*>(b + o_kl);
  ws.v_lr = reinterpret_cast<bf16_t*>(b + o_vl);
  ws.k_gb = reinterpret_cast<bf16_t*>(b + o_kb);
  ws.v_gb = reinterpret_cast<bf16_t*>(b + o_vb);
  ws.o_part = reinterpret_cast<float*>(b + o_op);
  ws.ml_part = reinterpret_cast<float2*>(b + o_ml);
  ws.q_hi = q_pre ? reinterpret_cast<bf16_t*>(b + o_qh) : nullptr;
  ws.q_lr = q_pre ? reinterpret_cast<bf16_t*>(b + o_ql) : nullptr;
  ws.bytes = off;
  return ws;
}

// Guide cell of slot `slot` in block order: block slot/64 = (BI, BJ) row-major over an
// nbj-wide block grid, cell (8 BI + k/8, 8 BJ + k%8) with k = slot % 64.
__device__ __forceinline__ void block_cell(int64_t slot, int nbj, int& i, int& j) {
  const int blk = static_cast<int>(slot / kKeyTile), k = static_cast<int>(slot % kKeyTile);
  const int bi = blk / nbj, bj = blk - bi * nbj;
  i = 8 * bi + (k >> 3);
  j = 8 * bj + (k & 7);
}

// ------------------------------------------------------------------ step 1: tables

__global__ void cos_sin_table_kernel(double2* cs, int P, int D, double log2_theta) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int quarter = D / 4;
  if (i >= P * quarter) return;
  const int pos = i / quarter, k = i - pos * quarter;
  cs[i] = rope_cos_sin(pos, k, D / 2, log2_theta);
}

// ------------------------------------------------------------------ step 2: prep

constexpr int kPrepThreads = 256;
constexpr int kPrepRows = 4;

// K rows -> head-major, rotated.  The input rows are [text | hi | guide].  Prep rows of a
// batch:
//   [0, N)            hi-res rows in window-first order (source row T + r(p)) -> k_hi;
//   [N, N + Mk)       guide rows s (source T + N + s, zero beyond M) -> k_lr row s;
//   [.., + Mb)        guide cells in 8x8 block order (zero outside the grid) -> k_gb, used
//                     by the guide-locality masks;
//   [.., + Tk)        text rows x (source x, zero beyond T; position (0, 0), so RoPE is the
//                     identity) -> k_lr row Mk + x and, with cell blocks, k_gb row Mb + x.
// Q is normally not prepared (the attention kernel rotates its query rows as it loads
// them); with q_hi non-null (guide modes 1, 2) the hi and guide rows of Q are also written,
// rotated and multiplied by q_scale in fp64 and rounded once, to q_hi / q_lr.
template <int D>
__global__ __launch_bounds__(kPrepThreads) void prep_k_kernel(
    const bf16_t* __restrict__ k, bf16_t* __restrict__ k_hi, bf16_t* __restrict__ k_lr,
    bf16_t* __restrict__ k_gb, const double2* __restrict__ cs, int P, double log2_theta,
    int64_t T, int64_t N, int64_t M, int64_t Mk, int64_t Mg, int64_t Mb, int64_t Mbg,
    int64_t Tk, int W, int w, int n_wx, int H_lr, int W_lr, int nbj, int rho, int heads,
    int rope_on, const bf16_t* __restrict__ q, bf16_t* __restrict__ q_hi,
    bf16_t* __restrict__ q_lr, double q_scale) {
  constexpr int CPH = D / 8;      // 16-byte chunks per head row
  constexpr int QUARTER = D / 4;  // rotation pairs per axis
  // Per row of this block: source row (-1: zero row), destinations (buffer row offsets in
  // elements of one head row, null: none), and the RoPE factors of its y and x positions.
  __shared__ int64_t src_s[kPrepRows];
  __shared__ bf16_t* dk_s[kPrepRows];
  __shared__ bf16_t* dk2_s[kPrepRows];
  __shared__ bf16_t* dq_s[kPrepRows];
  __shared__ int64_t kst_s[kPrepRows], k2st_s[kPrepRows], qst_s[kPrepRows];  // per-head strides
  __shared__ int pos_s[kPrepRows][2];
  // RoPE factors of pair 4j + e (pairs of both axes in one list, y first) at [row][e][j]:
  // the 16-byte reads of the lanes that rotate chunks j = 0, 1, ... are consecutive
  __shared__ double2 cs_s[kPrepRows][4][CPH];
  const int64_t L = T + N + M;
  const int64_t b = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid < kPrepRows) {
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kPrepRows + tid;
    const int64_t bh0 = b * heads;  // first (b, h) of this batch
    int64_t src = -1;
    bf16_t* dk = nullptr;
    bf16_t* dk2 = nullptr;
    bf16_t* dq = nullptr;
    int64_t kst = 0, k2st = 0, qst = 0;
    int py = 0, px = 0;
    if (row < N) {
      const int r = window_first_to_raster(static_cast<int>(row), W, w, n_wx);
      src = T + r;
      py = r / W;
      px = r - py * W;
      dk = k_hi + (bh0 * N + row) * D;  kst = N * D;
      if (q_hi) { dq = q_hi + (bh0 * N + row) * D;  qst = N * D; }
    } else if (row < N + Mk) {
      const int64_t s = row - N;
      if (s < M) {
        src = T + N + s;
        const int sy = static_cast<int>(s / W_lr);
        py = rho * sy;
        px = rho * static_cast<int>(s - static_cast<int64_t>(sy) * W_lr);
        if (q_lr) { dq = q_lr + (bh0 * M + s) * D;  qst = M * D; }
      }
      dk = k_lr + (bh0 * Mg + s) * D;  kst = Mg * D;
    } else if (row < N + Mk + Mb) {
      const int64_t slot = row - N - Mk;
      int ci, cj;
      block_cell(slot, nbj, ci, cj);
      if (ci < H_lr && cj < W_lr) src = T + N + static_cast<int64_t>(ci) * W_lr + cj;
      py = rho * ci;
      px = rho * cj;
      dk = k_gb + (bh0 * Mbg + slot) * D;  kst = Mbg * D;
    } else if (row < N + Mk + Mb + Tk) {
      const int64_t x = row - N - Mk - Mb;
      if (x < T) src = x;
      dk = k_lr + (bh0 * Mg + Mk + x) * D;  kst = Mg * D;
      if (Mb > 0) { dk2 = k_gb + (bh0 * Mbg + Mb + x) * D;  k2st = Mbg * D; }
    }
    src_s[tid] = src;
    dk_s[tid] = dk;  kst_s[tid] = kst;
    dk2_s[tid] = dk2;  k2st_s[tid] = k2st;
    dq_s[tid] = dq;  qst_s[tid] = qst;
    pos_s[tid][0] = py;
    pos_s[tid][1] = px;
  }
  __syncthreads();
  if (rope_on) {
    for (int e = tid; e < kPrepRows * 2 * QUARTER; e += kPrepThreads) {
      const int rt = e / (2 * QUARTER), axis = (e / QUARTER) & 1, kk = e % QUARTER;
      const int pos = pos_s[rt][axis];
      cs_s[rt][kk % 4][(axis * QUARTER + kk) / 4] =
          pos < P ? cs[pos * QUARTER + kk] : rope_cos_sin(pos, kk, D / 2, log2_theta);
    }
    __syncthreads();
  }

  const int cpr = heads * CPH;  // chunks per row
  // task i = (row t, chunk c); t and c advance without divisions.  K is read and written
  // with nontemporal loads and stores: each byte is touched once here.
  int t = tid / cpr, c = tid - (tid / cpr) * cpr;
  for (; t < kPrepRows; ) {
    const int h = c / CPH, j = c % CPH;
    const int64_t src = src_s[t];
    uint4 ko = make_uint4(0, 0, 0, 0), qo = ko;
    bf16_t* dq = dq_s[t];
    if (src >= 0) {
      const int64_t so = ((b * L + src) * heads + h) * D + j * 8;
      const u32x4 kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + so));
      const uint4 ki = make_uint4(kv[0], kv[1], kv[2], kv[3]);
      if (rope_on) {
        // pairs 4j .. 4j+3 lie on one axis (y for the first D/4 pairs)
        const double2 f[4] = {cs_s[t][0][j], cs_s[t][1][j], cs_s[t][2][j], cs_s[t][3][j]};
        ko = make_uint4(rope_rotate_word(ki.x, f[0]), rope_rotate_word(ki.y, f[1]),
                        rope_rotate_word(ki.z, f[2]), rope_rotate_word(ki.w, f[3]));
        if (dq) {
          const uint4 qi = *reinterpret_cast<const uint4*>(q + so);
          qo = make_uint4(rope_rotate_word(qi.x, f[0], q_scale), rope_rotate_word(qi.y, f[1], q_scale),
                          rope_rotate_word(qi.z, f[2], q_scale), rope_rotate_word(qi.w, f[3], q_scale));
        }
      } else {
        ko = ki;
        if (dq) {
          const uint4 qi = *reinterpret_cast<const uint4*>(q + so);
          qo = make_uint4(scale_word(qi.x, q_scale), scale_word(qi.y, q_scale),
                          scale_word(qi.z, q_scale), scale_word(qi.w, q_scale));
        }
      }
    }
    if (dq) *reinterpret_cast<uint4*>(dq + h * qst_s[t] + j * 8) = qo;
    bf16_t* dk = dk_s[t];
    bf16_t* dk2 = dk2_s[t];
    if (dk) __builtin_nontemporal_store(u32x4{ko.x, ko.y, ko.z, ko.w}, reinterpret_cast<u32x4*>(dk + h * kst_s[t] + j * 8));
    if (dk2) *reinterpret_cast<uint4*>(dk2 + h * k2st_s[t] + j * 8) = ko;
    c += kPrepThreads;
    while (c >= cpr) {
      c -= cpr;
      ++t;
    }
  }
}

// V rows -> 64-key tiles transposed to [D][64] (key order by v_slot); one (tile, head, batch)
// per workgroup (grid: tiles * heads, B).  Tiles of a batch:
// [0, N/64) window-first hi rows -> v_hi; the next Mg/64 the global keys -> v_lr (guide
// rows in raster order, zero padded to Mk, then text rows); the last Mbg/64 the cell-block
// buffer -> v_gb (guide cells in 8x8 block order, then text rows).  Input rows are
// [text | hi | guide].
__global__ __launch_bounds__(kPrepThreads) void prep_v_kernel(
    const bf16_t* __restrict__ v, bf16_t* v_hi, bf16_t* v_lr, bf16_t* v_gb, int64_t T,
    int64_t N, int64_t M, int64_t Mk, int64_t Mg, int64_t Mb, int64_t Mbg, int W, int w,
    int n_wx, int H_lr, int W_lr, int nbj, int heads, int D) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[kKeyTile][128 + 2];
  const int64_t L = T + N + M;
  const int64_t b = blockIdx.y;
  // heads vary fastest over the grid, so the workgroups reading the same raster rows
  // (one head's 256-byte slice each) run together
  const int h = static_cast<int>(blockIdx.x % heads);
  const int64_t tile_id = blockIdx.x / heads;
  const int64_t n_hi = N / kKeyTile, n_g = Mg / kKeyTile;
  const int chunks_per_row = D / 8;
  // source row (or -1) of key kr of this tile
  auto source = [&](int kr) -> int64_t {
    if (tile_id < n_hi) return T + window_first_to_raster(static_cast<int>(tile_id * kKeyTile + kr), W, w, n_wx);
    if (tile_id < n_hi + n_g) {
      const int64_t r = (tile_id - n_hi) * kKeyTile + kr;
      if (r < Mk) return r < M ? T + N + r : -1;
      return r - Mk < T ? r - Mk : -1;
    }
    const int64_t r = (tile_id - n_hi - n_g) * kKeyTile + kr;
    if (r >= Mb) return r - Mb < T ? r - Mb : -1;
    int ci, cj;
    block_cell(r, nbj, ci, cj);
    return (ci < H_lr && cj < W_lr) ? T + N + static_cast<int64_t>(ci) * W_lr + cj : -1;
  };
  // load 64 rows x D of head h (16-byte chunks; all of a thread's loads before its stores;
  // nontemporal, as every byte is read and written once here)
  constexpr int kLoads = kKeyTile * 16 / kPrepThreads;  // chunks per thread for D = 128
  uint4 x[kLoads];
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int i = threadIdx.x + u * kPrepThreads;
    x[u] = make_uint4(0, 0, 0, 0);
    if (i < kKeyTile * chunks_per_row) {
      const int kr = i / chunks_per_row, j = i - kr * chunks_per_row;
      const int64_t src_row = source(kr);
      if (src_row >= 0) {
        const u32x4 xv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + ((b * L + src_row) * heads + h) * D + j * 8));
        x[u] = make_uint4(xv[0], xv[1], xv[2], xv[3]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int i = threadIdx.x + u * kPrepThreads;
    if (i < kKeyTile * chunks_per_row) {
      const int kr = i / chunks_per_row, j = i - kr * chunks_per_row;
      // row stride 260 bytes: the four words of a chunk are 4-byte aligned
      uint32_t* tw = reinterpret_cast<uint32_t*>(&tile[kr][j * 8]);
      tw[0] = x[u].x;
      tw[1] = x[u].y;
      tw[2] = x[u].z;
      tw[3] = x[u].w;
    }
  }
  __syncthreads();
  // write D rows x 64 keys; each task takes 8 consecutive slots of two adjacent d-rows:
  // it reads 4-byte words (dims d, d + 1 of one key) and splits them into the two rows
  const int64_t bh = b * heads + h, tsz = static_cast<int64_t>(D) * kKeyTile;
  bf16_t* dst;
  if (tile_id < n_hi) dst = v_hi + (bh * n_hi + tile_id) * tsz;
  else if (tile_id < n_hi + n_g) dst = v_lr + (bh * n_g + (tile_id - n_hi)) * tsz;
  else dst = v_gb + (bh * (Mbg / kKeyTile) + (tile_id - n_hi - n_g)) * tsz;
  for (int i = threadIdx.x; i < (D / 2) * (kKeyTile / 8); i += kPrepThreads) {
    const int dp = i / (kKeyTile / 8), s8 = (i - dp * (kKeyTile / 8)) * 8;
    const int d = 2 * dp;
    uint32_t r0[4], r1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // slot s holds key v_slot(s) (the mapping is its own inverse)
      const uint32_t lo = *reinterpret_cast<const uint32_t*>(&tile[v_slot(s8 + 2 * e)][d]);
      const uint32_t hi = *reinterpret_cast<const uint32_t*>(&tile[v_slot(s8 + 2 * e + 1)][d]);
      r0[e] = (lo & 0xffffu) | (hi << 16);
      r1[e] = (lo >> 16) | (hi & 0xffff0000u);
    }
    bf16_t* row = dst + static_cast<int64_t>(d) * kKeyTile + s8;
    __builtin_nontemporal_store(u32x4{r0[0], r0[1], r0[2], r0[3]}, reinterpret_cast<u32x4*>(row));
    __builtin_nontemporal_store(u32x4{r1[0], r1[1], r1[2], r1[3]},
                                reinterpret_cast<u32x4*>(row + kKeyTile));
  }
}

// ------------------------------------------------------------------ steps 3-4: attention

struct AttnArgs {
  const bf16_t* q;        // the caller's token-major Q [B][out_rows][heads][D]; query row i of
                          // the pass is token out_row0 + (hi pass: r(i), else i)
  int64_t q_rows;         // query rows per (b, h) of the pass (a multiple of the block)
  const bf16_t* q_pre;    // or, when non-null, Q rows prepared (rotated, scaled) [B*heads][q_valid][D]
  const double2* cs;      // fp64 RoPE factors [P][D/4]
  double log2_theta;      // for positions >= P
  double q_scale;         // softmax scale * log2 e, applied to Q before its rounding to bf16
  int P, rope_on;
  const bf16_t* k_hi;     // [B*heads][N][D]
  const bf16_t* v_hi;     // [B*heads][N/64][D][64]
  const bf16_t* k_lr;     // [B*heads][Mg][D]        global keys: guide rows, then text rows
  const bf16_t* v_lr;     // [B*heads][Mg/64][D][64] (RECT: the cell-block buffer, Mg = Mbg)
  bf16_t* out;            // token-major [B][out_rows][heads][D]
  int64_t out_rows;       // rows per batch of out
  int64_t out_row0;       // first row of this pass inside a batch of out
  int64_t N, M, Mk, Mg, T, Mb;
  int heads, w2;
  int W, w, n_wx, n_wy;   // hi pass: query row p (window-first) is written to raster row r(p)
  int radius;             // hi pass: windows within this distance (per axis) are visible
  int reach;              // RECT: the guide cells whose scaled position lies within `reach`
                          // windows of the query window are visible
  int rho, H_lr, W_lr, nbj;
  int q_valid;            // valid query rows per (b, h)
  int blocks_per_bh;
  int total_blocks;
  int splits;             // TEXT: key-range splits per query block
  float* o_part;          // TEXT: [splits][B*heads][q_rows][D] unnormalised partial outputs
  float2* ml_part;        // TEXT: [splits][B*heads][q_rows] (running max, sum)
  float* lse;             // optional [B*heads][out_rows]: natural-log sum of exp(scaled scores)
  const bf16_t* k_raw;    // RAW: the caller's K and V [B][out_rows][heads][D], read in place
  const bf16_t* v_raw;
};

constexpr int kStages = 4;  // LDS ring: tiles t, t+1 are read while t+2, t+3 land
constexpr int kQkAhead = 2;  // K fragment reads in flight ahead of the QK^T MFMAs (steps)
constexpr int kPvAhead = 4;  // V fragment reads in flight ahead of the PV MFMAs

// One workgroup = NWAVES waves x 32 queries.  Waves [0, NWAVES/2) ("A") and
// [NWAVES/2, NWAVES) ("B") are offset by half an iteration: in iteration t, A runs
// PV_{t-1}, QK^T_t, softmax_t and B runs softmax_t, PV_t, QK^T_{t+1}.  Waves w and
// w + NWAVES/2 share a SIMD, so while one runs its block of MFMAs the other runs its
// softmax on the VALU.
//
// K/V tiles are copied global -> LDS by the DMA path of global_load_lds_dwordx4 (lane l of
// a load writes LDS bytes [16 l, 16 l + 16) above the wave's base), two iterations ahead of
// their first use.  Each lane picks the global 16-byte chunk that belongs at its LDS slot
// under the XOR swizzle, so the LDS layout is the one the fragment reads expect.  Every
// iteration issues the same copies (past the last tile it copies a tile again into a stage
// nobody reads any more), so the loop has no per-copy branches and one fixed wait.  The
// first V fragments of each PV block are read ahead of it (wave A before the barrier that
// ends the previous iteration, wave B right after its softmax), and the first K fragments
// of each QK^T block before the PV block that precedes it, so neither block's first MFMA
// waits for LDS.
//
// ROTK (uhla_forward_rope_at_load): K arrives unrotated and every workgroup rotates each K
// tile in LDS after it lands (RoPE fused into the K tile load), instead of K being rotated
// once by the prep pass.  Each thread rotates its own DMA chunks of the tile: cos/sin of
// the key's position times the chunk's four frequencies from the hardware sin/cos (angle
// in revolutions, reduced with fract), the rotation in fp32, one rounding to bf16.  Tile
// t+1 is rotated in iteration t before a mid-iteration barrier, ahead of its first reader
// (wave B's QK^T_{t+1} in the second half of that iteration).
//
// RAW (uhla_forward_permute_free): no prep pass at all.  Tiles are copied straight from the
// caller's raster K and V: a 64-key hi tile is 64 / w window rows of w tokens (or a
// 64-token piece of one row of a wider window), so this lane's source chunk sits at the
// same offset from the tile's first token in every hi tile, and a guide tile is 64
// consecutive guide tokens (the missing keys of the last one re-read its last token and
// are masked).  K is rotated at load as with ROTK; V lands row-major (chunks swizzled for
// the transposing LDS read) and its V^T fragments are read with ds_read_b64_tr_b16.
template <int D, int NWAVES, bool HI, bool RECT, bool TEXT, bool ROTK = false, bool RAW = false>
__global__ __launch_bounds__(NWAVES * 64) void attn_fwd_kernel(AttnArgs a) {
  constexpr int NT = NWAVES * 64;
  constexpr int TILE_BYTES = kKeyTile * D * 2;       // one K or V tile
  constexpr int CHUNKS = TILE_BYTES / 16;
  constexpr int CPT = CHUNKS / NT;                     // 16-byte chunks per thread
  static_assert(CHUNKS % NT == 0, "tile must split evenly");
  constexpr int KCH = D / 8;                           // 16-byte chunks per K row
  constexpr int LOADS_PER_TILE = 2 * CPT;              // DMA instructions per thread per tile
  // Four separate stage buffers (K tile then V tile), always addressed with a static
  // stage index: the compiler can then tell the stage being read from the stage the
  // DMA is writing, and does not wait for in-flight tile loads before LDS reads.
  __shared__ __attribute__((aligned(16))) char stage0[2 * TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char stage1[2 * TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char stage2[2 * TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char stage3[2 * TILE_BYTES];
  __shared__ uint32_t tile_off_s[HI ? kMaxTableTiles : 1];
  __shared__ uint32_t tile_mask_s[RECT ? kMaxTableTiles : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, g = lane >> 5;
  const bool wave_b = wave >= NWAVES / 2;
  const int blk = xcd_remap(blockIdx.x, a.total_blocks);
  const int bh = blk / a.blocks_per_bh;
  const int rem_blk = blk - bh * a.blocks_per_bh;
  const int qb = TEXT ? rem_blk / a.splits : rem_blk;
  const int split = TEXT ? rem_blk - qb * a.splits : 0;
  const int b = bh / a.heads, h = bh - b * a.heads;
  const int q0 = qb * (NWAVES * 32);

  // Tile list.  Hi pass: the key tiles (w2/64 each) of the windows within `radius` of the
  // query window, clipped to the grid, row-major; then the global tiles: guide tiles (all
  // of them in raster order, or with RECT the 8x8 cell blocks that meet the window's
  // guide rectangle, each with a row/column mask), then text tiles.  Guide pass: the
  // global tiles.  Text pass: this split's share of all hi tiles followed by the global
  // tiles.  Byte offsets of the table-driven tiles are staged in LDS once, so that
  // picking a tile costs one LDS read and the loop keeps few scalars live.
  const int n_hi_tiles = static_cast<int>(a.N / kKeyTile);
  const int n_text_tiles = static_cast<int>((a.T + kKeyTile - 1) / kKeyTile);
  int n_local = 0, n_rect = 0, n_guide = static_cast<int>(a.Mg / kKeyTile), t_base = 0;
  if (TEXT) {
    const int total = n_hi_tiles + static_cast<int>(a.Mg / kKeyTile);
    t_base = static_cast<int>(static_cast<int64_t>(split) * total / a.splits);
    n_guide = static_cast<int>(static_cast<int64_t>(split + 1) * total / a.splits) - t_base;
  }
  // Query rows: loaded first, so that their latency overlaps the table set-up below.
  // Lane (ql, g) holds query ql's dims 16kk + 8g .. +8 (the B operand layout of S^T = K Q^T).
  // Hi queries sit at their raster position, guide query s at (rho * (s / W_lr),
  // rho * (s % W_lr)), text queries at (0, 0); rows past the pass's valid rows are zero.
  constexpr int QUARTER = D / 4;
  const int qi = q0 + wave * 32 + ql;
  const bool qvalid = qi < a.q_valid;
  bf16x8 qf[D / 16];
  uint4 raw[D / 16];
  int py = 0, px = 0;
  if (a.q_pre) {
    const bf16_t* qrow = a.q_pre + (static_cast<int64_t>(bh) * a.q_valid + (qvalid ? qi : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qf[kk] = qvalid ? *reinterpret_cast<const bf16x8*>(qrow + 16 * kk + 8 * g) : bf16x8{};
  } else if (qvalid) {
    int tok = qi;
    if (HI) {
      tok = window_first_to_raster(qi, a.W, a.w, a.n_wx);
      py = tok / a.W;
      px = tok - py * a.W;
    } else if (!TEXT) {
      const int sy = qi / a.W_lr;
      py = a.rho * sy;
      px = a.rho * (qi - sy * a.W_lr);
    }
    const bf16_t* qrow = a.q + ((static_cast<int64_t>(b) * a.out_rows + a.out_row0 + tok) * a.heads + h) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) raw[kk] = *reinterpret_cast<const uint4*>(qrow + 16 * kk + 8 * g);
  }
  // Hi pass: the RoPE factors of the workgroup's query positions (ny window rows from
  // ry0, and every column of the window), rounded to fp32 and multiplied by the Q scale,
  // are staged once in LDS (stage 3, which the tile ring first writes in iteration 0), so
  // that each lane reads its 2 x D/4 factors from LDS instead of the fp64 table.  Rows are
  // FRS bytes apart (16 bytes of padding spread the column rows over the banks).  A window
  // too wide for the stage falls back to the table reads.
  constexpr int FRS = QUARTER * 8 + 16;
  int ry0 = 0, ny = 0;
  bool lds_rope = false;
  if (HI) {
    const int tiles_per_win = a.w2 / kKeyTile;
    const int win = q0 / a.w2;
    const int wy = win / a.n_wx, wx = win - wy * a.n_wx;
    {
      const int p0 = q0 - win * a.w2;
      ry0 = p0 / a.w;
      ny = (p0 + NWAVES * 32 - 1) / a.w - ry0 + 1;
      lds_rope = a.rope_on && !a.q_pre && (ny + a.w) * FRS <= 2 * TILE_BYTES;
      if (lds_rope) {
        const float qs = static_cast<float>(a.q_scale);
        for (int i = tid; i < (ny + a.w) * QUARTER; i += NT) {
          const int row = i / QUARTER, k = i - row * QUARTER;
          const int pos = row < ny ? wy * a.w + ry0 + row : wx * a.w + (row - ny);
          const double2 f = a.cs[pos * QUARTER + k];
          *reinterpret_cast<float2*>(stage3 + row * FRS + k * 8) =
              make_float2(static_cast<float>(f.x) * qs, static_cast<float>(f.y) * qs);
        }
      }
    }
    const int y0 = max(0, wy - a.radius), y1 = min(a.n_wy - 1, wy + a.radius);
    const int x0 = max(0, wx - a.radius), x1 = min(a.n_wx - 1, wx + a.radius);
    const int nx = x1 - x0 + 1;
    n_local = (y1 - y0 + 1) * nx * tiles_per_win;
    for (int i = tid; i < n_local; i += NT) {
      const int j = i / tiles_per_win, sub = i - j * tiles_per_win;
      const int jy = j / nx, nw = (y0 + jy) * a.n_wx + x0 + (j - jy * nx);
      tile_off_s[i] = static_cast<uint32_t>(nw * a.w2 + sub * kKeyTile) * (D * 2);
    }
    if (RECT) {
      // guide cells (i, j) whose scaled position (rho i, rho j) lies in the windows within
      // `reach` of the query window: i in [ceil(gy0 w / rho), ceil((gy1 + 1) w / rho))
      const int gy0 = max(0, wy - a.reach), gy1 = min(a.n_wy - 1, wy + a.reach);
      const int gx0 = max(0, wx - a.reach), gx1 = min(a.n_wx - 1, wx + a.reach);
      const int i0 = (gy0 * a.w + a.rho - 1) / a.rho, i1 = min(a.H_lr, ((gy1 + 1) * a.w + a.rho - 1) / a.rho);
      const int j0 = (gx0 * a.w + a.rho - 1) / a.rho, j1 = min(a.W_lr, ((gx1 + 1) * a.w + a.rho - 1) / a.rho);
      int ng = 0;
      if (i0 < i1 && j0 < j1) {
        const int bi0 = i0 >> 3, bj0 = j0 >> 3, nbx = ((j1 - 1) >> 3) - bj0 + 1;
        ng = (((i1 - 1) >> 3) - bi0 + 1) * nbx;
        for (int k = tid; k < ng; k += NT) {
          const int ky = k / nbx, bi = bi0 + ky, bj = bj0 + (k - ky * nbx);
          uint32_t rows = 0, cols = 0;
          for (int e = 0; e < 8; ++e) {
            rows |= static_cast<uint32_t>(8 * bi + e >= i0 && 8 * bi + e < i1) << e;
            cols |= static_cast<uint32_t>(8 * bj + e >= j0 && 8 * bj + e < j1) << e;
          }
          tile_off_s[n_local + k] = static_cast<uint32_t>(bi * a.nbj + bj) * TILE_BYTES;
          tile_mask_s[n_local + k] = rows | (cols << 8);
        }
      }
      // the text tiles follow the cell blocks in the same buffer
      for (int x = tid; x < n_text_tiles; x += NT) {
        tile_off_s[n_local + ng + x] = static_cast<uint32_t>(a.Mb / kKeyTile + x) * TILE_BYTES;
        tile_mask_s[n_local + ng + x] = 0xffffu;
      }
      n_rect = ng;
      n_guide = ng + n_text_tiles;
    }
    __syncthreads();
  }
  const int n_tiles = n_local + n_guide;

  // Per-lane source offsets (bytes inside a tile) for this thread's DMA slots.
  int k_src[CPT], v_src[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int slot = (i * NWAVES + wave) * 64 + lane;  // 16-byte LDS slot in the tile
    const int kr = slot / KCH, kp = slot - kr * KCH;
    k_src[i] = kr * (D * 2) + ((kp ^ k_swizzle<D>(kr)) << 4);
    const int vr = slot >> 3, vp = slot & 7;
    v_src[i] = vr * (kKeyTile * 2) + ((vp ^ v_swizzle(vr)) << 4);
  }
  static_assert(!RAW || (ROTK && !RECT && !TEXT), "raster tiles: K rotated at load, default mask");
  // RAW: this lane's chunk offsets from a tile's first token in the caller's K and V, for
  // hi tiles (h) and guide tiles (g)
  int kh_src[RAW ? CPT : 1], kg_src[RAW ? CPT : 1], vh_src[RAW ? CPT : 1], vg_src[RAW ? CPT : 1];
  const int rowb = a.heads * (D * 2);  // bytes between consecutive tokens of one head
  if constexpr (RAW) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int slot = (i * NWAVES + wave) * 64 + lane;
      const int kr = slot / KCH, kp = slot - kr * KCH;
      const int rel = a.w <= kKeyTile ? (kr / a.w) * a.W + (kr % a.w) : kr;
      kh_src[i] = rel * rowb + ((kp ^ k_swizzle<D>(kr)) << 4);
      kg_src[i] = kr * rowb + ((kp ^ k_swizzle<D>(kr)) << 4);
      vh_src[i] = rel * rowb + ((kp ^ bwd_swizzle<D>(kr)) << 4);
      vg_src[i] = kr * rowb + ((kp ^ bwd_swizzle<D>(kr)) << 4);
    }
  }
  // Global sources of tile t (K tile, V^T tile).  A V^T tile of 64 keys holds as many bytes
  // as the K tile of the same keys, so one offset serves both.
  const char* k_hi_b = reinterpret_cast<const char*>(a.k_hi) + static_cast<int64_t>(bh) * a.N * (D * 2);
  const char* v_hi_b = reinterpret_cast<const char*>(a.v_hi) + static_cast<int64_t>(bh) * a.N * (D * 2);
  const char* k_lr_b = reinterpret_cast<const char*>(a.k_lr) + static_cast<int64_t>(bh) * a.Mg * (D * 2);
  const char* v_lr_b = reinterpret_cast<const char*>(a.v_lr) + static_cast<int64_t>(bh) * a.Mg * (D * 2);
  // Keys of tile t that exist (a prefix): only the last guide tile and the last text tile
  // of the global buffer can be partial, so their tile indices (-1: none) and key counts
  // are found once and the loop tests two scalars per tile ...
  int part_t0 = -1, part_v0 = kKeyTile, part_t1 = -1, part_v1 = kKeyTile;
  if (RECT) {
    if (a.T % kKeyTile) {
      part_t1 = n_local + n_rect + static_cast<int>(a.T / kKeyTile);
      part_v1 = static_cast<int>(a.T % kKeyTile);
    }
  } else {
    const int goff = TEXT ? n_hi_tiles - t_base : n_local;  // tile t = global tile t - goff
    if (a.M % kKeyTile) {
      part_t0 = static_cast<int>(a.M / kKeyTile) + goff;
      part_v0 = static_cast<int>(a.M % kKeyTile);
    }
    if (a.T % kKeyTile) {
      part_t1 = static_cast<int>(a.Mk / kKeyTile + a.T / kKeyTile) + goff;
      part_v1 = static_cast<int>(a.T % kKeyTile);
    }
  }
  // (with RECT, k_lr / v_lr / Mg describe the cell-block buffer)
  // RAW tiles also report their kind (0: hi, 1: guide) and how many of their keys exist.
  const int64_t g_row0 = HI ? a.out_row0 + a.N : a.out_row0;  // row of guide token 0 (RAW)
  auto tile_src = [&](int t, const char*& kp, const char*& vp, int& kind, int& valid) __attribute__((always_inline)) {
    kind = 0;
    valid = kKeyTile;
    if constexpr (RAW) {
      int64_t row;  // row of the tile's first token within batch b of the caller's tensors
      if (HI && t < n_local) {
        const int p0 = static_cast<int>(__builtin_amdgcn_readfirstlane(tile_off_s[t]) / (D * 2));
        row = a.out_row0 + window_first_to_raster(p0, a.W, a.w, a.n_wx);
      } else {
        row = g_row0 + static_cast<int64_t>(t - (HI ? n_local : 0)) * kKeyTile;
        kind = 1;
        valid = t == part_t0 ? part_v0 : kKeyTile;
      }
      const int64_t off = ((static_cast<int64_t>(b) * a.out_rows + row) * a.heads + h) * (D * 2);
      kp = reinterpret_cast<const char*>(a.k_raw) + off;
      vp = reinterpret_cast<const char*>(a.v_raw) + off;
      return;
    }
    if (HI && t < n_local) {
      const uint32_t off = __builtin_amdgcn_readfirstlane(tile_off_s[t]);
      kp = k_hi_b + off;
      vp = v_hi_b + off;
    } else if (RECT) {
      const uint32_t off = __builtin_amdgcn_readfirstlane(tile_off_s[t]);
      kp = k_lr_b + off;
      vp = v_lr_b + off;
    } else if (TEXT && t + t_base < n_hi_tiles) {
      const uint32_t off = static_cast<uint32_t>(t + t_base) * TILE_BYTES;
      kp = k_hi_b + off;
      vp = v_hi_b + off;
    } else {
      const uint32_t off = static_cast<uint32_t>(t + t_base - (TEXT ? n_hi_tiles : n_local)) * TILE_BYTES;
      kp = k_lr_b + off;
      vp = v_lr_b + off;
    }
  };
  // DMA instructions [p0, p1) of this thread's share of one K tile and one V tile:
  // instruction p copies K chunk p/2 (p even) from kp into the K half of stage `kdst`, or
  // V chunk p/2 (p odd) from vp into the V half of stage `vdst`; a null source is skipped.
  // Source offset of this lane's chunk of DMA instruction i (K or V half) for a tile of the
  // given kind; RAW guide tiles with fewer than 64 keys re-read their last key.
  auto src_off = [&](int i, bool is_v, int kind, int valid) __attribute__((always_inline)) -> int {
    if constexpr (!RAW) {
      return is_v ? v_src[i] : k_src[i];
    } else {
      if (kind == 0) return is_v ? vh_src[i] : kh_src[i];
      if (valid >= kKeyTile) return is_v ? vg_src[i] : kg_src[i];
      const int slot = (i * NWAVES + wave) * 64 + lane, kr = slot / KCH, kp = slot - kr * KCH;
      return min(kr, valid - 1) * rowb + ((kp ^ (is_v ? bwd_swizzle<D>(kr) : k_swizzle<D>(kr))) << 4);
    }
  };
  auto issue_parts = [&](const char* kp, const char* vp, char* kdst, char* vdst, int p0, int p1,
                         int kind, int valid) __attribute__((always_inline)) {
    const uint32_t klds = lds_addr(kdst), vlds = lds_addr(vdst) + TILE_BYTES;
#pragma unroll
    for (int p = 0; p < LOADS_PER_TILE; ++p) {
      if (p < p0 || p >= p1) continue;
      const int i = p >> 1;
      const uint32_t off = (i * NWAVES + wave) * 64 * 16;
      if (p & 1) {
        if (vp) dma_16b(vp, src_off(i, true, kind, valid), __builtin_amdgcn_readfirstlane(vlds + off));
      } else {
        if (kp) dma_16b(kp, src_off(i, false, kind, valid), __builtin_amdgcn_readfirstlane(klds + off));
      }
    }
  };
  auto issue_k = [&](int t, char* dst) __attribute__((always_inline)) {
    const char* kp;
    const char* vp;
    int kind, valid;
    tile_src(t, kp, vp, kind, valid);
    issue_parts(kp, nullptr, dst, dst, 0, LOADS_PER_TILE, kind, valid);
  };
  auto issue_v = [&](int t, char* dst) __attribute__((always_inline)) {
    const char* kp;
    const char* vp;
    int kind, valid;
    tile_src(t, kp, vp, kind, valid);
    issue_parts(nullptr, vp, dst, dst, 0, LOADS_PER_TILE, kind, valid);
  };
  auto tile_valid = [&](int t) __attribute__((always_inline)) -> int {
    return t == part_t0 ? part_v0 : t == part_t1 ? part_v1 : kKeyTile;
  };
  // ... and, for a cell-block guide tile, which of its 8x8 cells are visible: bits 0-7 the
  // rows, bits 8-15 the columns (0xffff: all).
  auto tile_mask = [&](int t) __attribute__((always_inline)) -> uint32_t {
    if (RECT && t >= n_local) return __builtin_amdgcn_readfirstlane(tile_mask_s[t]);
    return 0xffffu;
  };

  // ROTK: this thread's chunk slots of a K tile.  With 8 waves every thread's slots hold
  // the same 16-byte dims chunk (rows 32 apart, same swizzle), so one set of four pair
  // frequencies (in revolutions per position step) serves them all.
  static_assert(!ROTK || (NWAVES == 8 && !RECT && !TEXT), "K rotation at load: 8 waves, default mask");
  int rk_row[CPT];
  float rk_fr[4];
  int rk_axis = 0;
  if constexpr (ROTK) {
    int chunk = 0;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int slot = (i * NWAVES + wave) * 64 + lane;
      rk_row[i] = slot / KCH;
      chunk = (slot - rk_row[i] * KCH) ^ k_swizzle<D>(rk_row[i]);
    }
    const int pr = 4 * chunk;  // first of the chunk's four rotation pairs
    rk_axis = pr / (D / 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kq = pr + e - rk_axis * (D / 4);
      rk_fr[e] = static_cast<float>(exp2(-(2.0 * kq / (D / 2)) * a.log2_theta) * 0.15915494309189535);
    }
  }
  // Position (py, px) of key `kr` of tile t (hi tiles: window-first rows; global tiles:
  // guide rows, padding rows at (0, 0)).
  auto key_pos = [&](int t, int kr, int& py, int& px) __attribute__((always_inline)) {
    py = 0;
    px = 0;
    if (HI && t < n_local) {
      const int row = static_cast<int>(tile_off_s[t] / TILE_BYTES) * kKeyTile + kr;
      const int r = window_first_to_raster(row, a.W, a.w, a.n_wx);
      py = r / a.W;
      px = r - py * a.W;
    } else {
      const int64_t srow = static_cast<int64_t>(t - n_local) * kKeyTile + kr;
      if (srow < a.M) {
        const int sr = static_cast<int>(srow), sy = sr / a.W_lr;
        py = a.rho * sy;
        px = a.rho * (sr - sy * a.W_lr);
      }
    }
  };
  // Rotate this thread's chunks of K tile t in the stage buffer kbuf (LDS, in place).
  auto rotate_k = [&](char* kbuf, int t) __attribute__((always_inline)) {
    if (!a.rope_on) return;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      int py, px;
      key_pos(t, rk_row[i], py, px);
      const float pos = static_cast<float>(rk_axis ? px : py);
      const int slot = (i * NWAVES + wave) * 64 + lane;
      uint4* cp = reinterpret_cast<uint4*>(kbuf + slot * 16);
      const uint4 wv = *cp;
      const uint32_t win[4] = {wv.x, wv.y, wv.z, wv.w};
      uint32_t wout[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float rev = __builtin_amdgcn_fractf(pos * rk_fr[e]);
        const float c = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
        const float x = __uint_as_float(win[e] << 16), y = __uint_as_float(win[e] & 0xffff0000u);
        wout[e] = pack_bf16x2(x * c - y * sn, x * sn + y * c);
      }
      *cp = make_uint4(wout[0], wout[1], wout[2], wout[3]);
    }
  };
  // LDS writes done and visible to the workgroup (no wait on the in-flight tile copies)
  auto lds_barrier = []() __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  // Q rotation (RoPE fused into the Q load): the fp64 cos/sin factors rounded to fp32 and
  // multiplied by the softmax scale * log2 e, the rotation in fp32 and one rounding to
  // bf16, so the scores come out in base-2 logits (the result differs from a correctly
  // rounded fp64 rotation in rare last-bit cases).  With q_pre (guide modes 1, 2, whose
  // workgroups have few tiles) the rows come prepared by the prep pass instead (rotated
  // and scaled in fp64, one rounding).
  if (!a.q_pre) {
    // pairs 8kk + 4g .. +3 lie on one axis (y for the first D/4 pairs)
    auto rotate = [&](int kk, const float (&c)[4], const float (&sn)[4]) __attribute__((always_inline)) {
      const uint32_t wi[4] = {raw[kk].x, raw[kk].y, raw[kk].z, raw[kk].w};
      uint32_t wo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = lo_bf16(wi[e]), y0 = hi_bf16(wi[e]);
        wo[e] = pack_bf16x2(x0 * c[e] - y0 * sn[e], x0 * sn[e] + y0 * c[e]);
      }
      const uint4 qo = make_uint4(wo[0], wo[1], wo[2], wo[3]);
      qf[kk] = *reinterpret_cast<const bf16x8*>(&qo);
    };
    if (!qvalid) {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) qf[kk] = bf16x8{};
    } else if (!a.rope_on) {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const uint4 qo = make_uint4(scale_word(raw[kk].x, a.q_scale), scale_word(raw[kk].y, a.q_scale),
                                    scale_word(raw[kk].z, a.q_scale), scale_word(raw[kk].w, a.q_scale));
        qf[kk] = *reinterpret_cast<const bf16x8*>(&qo);
      }
    } else if (HI && lds_rope) {
      const int p = qi % a.w2, ry = p / a.w - ry0, cx = p % a.w;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const int pr = 8 * kk + 4 * g, axis = pr / QUARTER, k0 = pr - axis * QUARTER;
        const char* fp = stage3 + (axis ? ny + cx : ry) * FRS + k0 * 8;
        const float4 f01 = *reinterpret_cast<const float4*>(fp);
        const float4 f23 = *reinterpret_cast<const float4*>(fp + 16);
        const float c[4] = {f01.x, f01.z, f23.x, f23.z}, sn[4] = {f01.y, f01.w, f23.y, f23.w};
        rotate(kk, c, sn);
      }
    } else {
      // All factor loads are issued before any is used.  Hi and text positions always lie
      // inside the table; a guide position past it (a guide grid reaching beyond the
      // hi-res extent) reads a clamped entry first and is then evaluated directly, with
      // the same function that fills the table.
      double2 f[D / 16][4];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const int pr = 8 * kk + 4 * g, axis = pr / QUARTER, k0 = pr - axis * QUARTER;
        const int pos = axis ? px : py, pc = pos < a.P ? pos : a.P - 1;
#pragma unroll
        for (int e = 0; e < 4; ++e) f[kk][e] = a.cs[pc * QUARTER + k0 + e];
      }
      if (!HI && !TEXT) {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const int pr = 8 * kk + 4 * g, axis = pr / QUARTER, k0 = pr - axis * QUARTER;
          const int pos = axis ? px : py;
          if (pos >= a.P) {
#pragma unroll
            for (int e = 0; e < 4; ++e) f[kk][e] = rope_cos_sin(pos, k0 + e, D / 2, a.log2_theta);
          }
        }
      }
      const float qs = static_cast<float>(a.q_scale);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        float c[4], sn[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c[e] = static_cast<float>(f[kk][e].x) * qs;
          sn[e] = static_cast<float>(f[kk][e].y) * qs;
        }
        rotate(kk, c, sn);
      }
    }
  }
  // Let the Q loads complete here, in a wait the compiler sees: it cannot see the
  // tile DMA below, and would otherwise wait for "the Q loads" inside the loop by
  // counting vector-memory operations, which would drain the in-flight tiles.
  __builtin_amdgcn_s_waitcnt(0);

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  // Scores are base-2 logits (Q carries softmax scale * log2 e) measured from the running
  // row maximum m_run: the QK^T accumulators start at -m_run (neg_m), so exp2 takes S as is.
  float m_run = 0.0f, l_run = 0.0f;
  bool first = true;  // no running maximum yet
  f32x16 neg_m;
#pragma unroll
  for (int r = 0; r < 16; ++r) neg_m[r] = 0.0f;
  asm volatile("" : "+v"(neg_m));
  f32x16 s0, s1;  // S^T of the current tile: lane = query ql; keys 8(r/4) + 4g + r%4 (+32)

  // K fragment for reduction step kk: keys ql (half 0) and 32 + ql (half 1)
  auto k_frag = [&](const char* kb, int kk, int half) __attribute__((always_inline)) -> bf16x8 {
    const int row = half * 32 + ql;
    return *reinterpret_cast<const bf16x8*>(kb + row * (D * 2) + (((2 * kk + g) ^ k_swizzle<D>(row)) << 4));
  };
  // S^T = K Q^T - m.  K fragments are read kQkAhead reduction steps ahead of their MFMAs;
  // the scheduling barriers keep the compiler from sinking each read next to its use,
  // which would expose the full LDS latency at every step.
  constexpr int QKS = D / 16, QAH = kQkAhead < QKS ? kQkAhead : QKS;
  // the first QAH K fragment pairs of a QK^T block, read ahead of the block
  auto qk_pre = [&](const char* kb, bf16x8 (&a0)[QAH], bf16x8 (&a1)[QAH]) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < QAH; ++kk) {
      a0[kk] = k_frag(kb, kk, 0);
      a1[kk] = k_frag(kb, kk, 1);
    }
  };
  auto qk_run = [&](const char* kb, const bf16x8 (&a0)[QAH], const bf16x8 (&a1)[QAH]) __attribute__((always_inline)) {
    bf16x8 f0[QKS], f1[QKS];
#pragma unroll
    for (int kk = 0; kk < QAH; ++kk) {
      f0[kk] = a0[kk];
      f1[kk] = a1[kk];
    }
    s0 = neg_m;
    s1 = neg_m;
#pragma unroll
    for (int kk = 0; kk < QKS; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0[kk], qf[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1[kk], qf[kk], s1, 0, 0, 0);
      if (kk + QAH < QKS) {
        f0[kk + QAH] = k_frag(kb, kk + QAH, 0);
        f1[kk + QAH] = k_frag(kb, kk + QAH, 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Raise the running max by delta (per lane): rescale O and l by alpha, shift the live
  // scores, and re-seed the QK^T accumulator start value.
  auto rescale = [&](float delta, float alpha) __attribute__((always_inline)) {
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] -= delta;
      s1[r] -= delta;
    }
    m_run += delta;
#pragma unroll
    for (int r = 0; r < 16; ++r) neg_m[r] = -m_run;
    asm volatile("" : "+v"(neg_m));
  };
  auto row_max = [&]() __attribute__((always_inline)) -> float {
    float m3[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      m3[i] = fmaxf(fmaxf(fmaxf(s0[4 * i], s0[4 * i + 1]), fmaxf(s0[4 * i + 2], s0[4 * i + 3])),
                    fmaxf(fmaxf(s1[4 * i], s1[4 * i + 1]), fmaxf(s1[4 * i + 2], s1[4 * i + 3])));
    return max_with_partner32(fmaxf(fmaxf(m3[0], m3[1]), fmaxf(m3[2], m3[3])));
  };
  // P = exp2(S) as bf16 B operands; returns this lane's partial row sum.  The softmax uses
  // only one- and two-operand VALU instructions (exp, add, cvt): on gfx950 these issue
  // beside the SIMD partner's MFMAs, while three-operand ones (fma, dot2) mostly wait.
  auto expo = [&](bf16x8 (&pf)[4]) __attribute__((always_inline)) -> float {
    float ps0 = 0.0f, ps1 = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float e0 = __builtin_amdgcn_exp2f(s0[r]), e1 = __builtin_amdgcn_exp2f(s0[r + 1]);
      const float e2 = __builtin_amdgcn_exp2f(s1[r]), e3 = __builtin_amdgcn_exp2f(s1[r + 1]);
      const bf16x2 a = {static_cast<__bf16>(e0), static_cast<__bf16>(e1)};
      const bf16x2 c = {static_cast<__bf16>(e2), static_cast<__bf16>(e3)};
      ps0 += e0 + e1;
      ps1 += e2 + e3;
      // key-step ks = 2*half + r/8; slot j = r % 8
      pf[r >> 3][r & 7] = a[0];
      pf[r >> 3][(r & 7) + 1] = a[1];
      pf[2 + (r >> 3)][r & 7] = c[0];
      pf[2 + (r >> 3)][(r & 7) + 1] = c[1];
    }
    return ps0 + ps1;
  };

  // Online softmax (base 2) of the current S.  The first tile sets the running maximum.
  // Later tiles exponentiate against the stale maximum and only look at the row max when
  // a lane's partial sum exceeds 2^20 (some score grew by more than ~2^15 over it, or
  // overflowed): then the maximum is raised, O and l rescaled, and P recomputed.  P stays
  // below 2^20, far inside fp32 and bf16 range.  Produces P^T as four bf16 B operands.
  auto softmax = [&](int valid, uint32_t cells, bf16x8 (&pf)[4]) __attribute__((always_inline)) {
    if (valid < kKeyTile) {
      // key 8(r/4) + 4g + r%4 (+32) is past the end iff its g-free part reaches valid - 4g;
      // comparing against that compile-time part keeps 32 key indices out of registers
      const int lim = valid - 4 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kc = 8 * (r >> 2) + (r & 3);
        if (kc >= lim) s0[r] = -INFINITY;
        if (kc + 32 >= lim) s1[r] = -INFINITY;
      }
    } else if (cells != 0xffffu) {
      // cell-block tile: key k is cell (k / 8, k % 8) of the block, i.e. row r/4 (+4 in the
      // second half) and column 4g + r%4
      const uint32_t cols = (cells >> (8 + 4 * g)) & 15u;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool col_ok = (cols >> (r & 3)) & 1u;
        if (!(col_ok && ((cells >> (r >> 2)) & 1u))) s0[r] = -INFINITY;
        if (!(col_ok && ((cells >> (4 + (r >> 2))) & 1u))) s1[r] = -INFINITY;
      }
    }
    if (first) {
      rescale(row_max(), 0.0f);
      first = false;
    }
    float ps = expo(pf);
    if (__builtin_amdgcn_ballot_w64(!(ps <= 1048576.0f)) != 0) {
      const float delta = fmaxf(row_max(), 0.0f);
      rescale(delta, __builtin_amdgcn_exp2f(-delta));
      ps = expo(pf);
    }
    l_run += ps;
  };

  // V^T fragment for key-step ks, output dims 32 dt + ql
  const TrAddr<D> tra(lane);  // RAW: transposed V^T fragments from the row-major V tile
  auto v_frag = [&](const char* vb, int ks, int dt) __attribute__((always_inline)) -> bf16x8 {
    if constexpr (RAW) return TrAddr<D>::frag(vb, tra.x, ks, dt);
    const int vr = dt * 32 + ql;
    return *reinterpret_cast<const bf16x8*>(vb + vr * (kKeyTile * 2) + (((2 * ks + g) ^ v_swizzle(vr)) << 4));
  };
  constexpr int PDT = D / 32, PNI = 4 * PDT, PAH = kPvAhead < PNI ? kPvAhead : PNI;
  // the first PAH V fragments of a PV block, read ahead of the block
  auto pv_pre = [&](const char* vb, bf16x8 (&a)[PAH]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PAH; ++i) a[i] = v_frag(vb, i / PDT, i % PDT);
  };
  // O^T += V^T P^T over 4 key-steps of 16 keys; V fragments are read kPvAhead MFMAs ahead
  auto pv_run = [&](const char* vb, const bf16x8 (&pf)[4], const bf16x8 (&a)[PAH]) __attribute__((always_inline)) {
    bf16x8 f[PNI];
#pragma unroll
    for (int i = 0; i < PAH; ++i) f[i] = a[i];
#pragma unroll
    for (int i = 0; i < PNI; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      o[i % PDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i], pf[i / PDT], o[i % PDT], 0, 0, 0);
      if (i + PAH < PNI) {
        f[i + PAH] = v_frag(vb, (i + PAH) / PDT, (i + PAH) % PDT);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  auto stage = [&](int i) __attribute__((always_inline)) -> char* {
    return i == 0 ? stage0 : i == 1 ? stage1 : i == 2 ? stage2 : stage3;
  };

  // Iteration t (one barrier each): wave A runs PV_{t-1}, QK^T_t, softmax_t and carries P_t
  // to the next iteration; wave B runs softmax_t, PV_t, QK^T_{t+1} and carries S.  Each wave
  // thus alternates one block of 32 MFMAs with one softmax, half an iteration apart from its
  // SIMD partner, so one wave's softmax runs under the other wave's MFMAs.
  // Iteration t reads K_t, K_{t+1}, V_{t-1}, V_t; it copies K_{t+3} into the K half of stage
  // (t+3) % 4 (K_{t-1} was last read before the previous barrier) and V_{t+2} into the V
  // half of stage (t+2) % 4 (V_{t-2} likewise), and at its barrier waits for the copies
  // issued one iteration earlier (K_{t+2}, V_{t+1}).
  // Prologue: K_0, V_0, K_1 must land before iteration 0; K_2 and V_1 stay in flight.
  issue_k(0, stage0);
  issue_v(0, stage0);
  if (n_tiles > 1) issue_k(1, stage1);
  if (n_tiles > 2) issue_k(2, stage2);
  if (n_tiles > 1) issue_v(1, stage1);
  if (n_tiles > 2) wait_vm_and_barrier<LOADS_PER_TILE>();
  else if (n_tiles > 1) wait_vm_and_barrier<LOADS_PER_TILE / 2>();
  else wait_vm_and_barrier<0>();
  if constexpr (ROTK) {
    rotate_k(stage0, 0);
    lds_barrier();
  }
  bf16x8 pa[4];  // wave A: P of the previous tile, consumed by the next iteration's PV
  bf16x8 va[PAH];  // V fragments read ahead of the next PV block
  bf16x8 ka0[QAH], ka1[QAH];  // K fragments read ahead of the next QK^T block
  // One copy of the loop per role (B = wave B), so that neither carries the other's state.
  auto run = [&]<bool B>() __attribute__((always_inline)) {
    if (B) {
      qk_pre(stage0, ka0, ka1);
      qk_run(stage0, ka0, ka1);
    }
    // Tile t lives in stage t % 4; S is the (compile-time) stage of tile t.
    auto step = [&]<int S>(int t) __attribute__((always_inline)) {
      char* cur = stage(S);
      // K_{t+3} and V_{t+2}; past the last tile, tile t is copied again instead: the
      // stages written then hold K_{t-1} and V_{t-2}, which are never read again, so every
      // iteration issues the same copies and waits the same way
      const char* kp;
      const char* vp;
      const char* unused;
      int k_kind, k_valid, v_kind, v_valid;
      tile_src(t + 3 < n_tiles ? t + 3 : t, kp, unused, k_kind, k_valid);
      tile_src(t + 2 < n_tiles ? t + 2 : t, unused, vp, v_kind, v_valid);
      char* kdst = stage((S + 3) & 3);
      char* vdst = stage((S + 2) & 3);
      auto dma_slot = [&](int slot) __attribute__((always_inline)) {
        const uint32_t klds = lds_addr(kdst), vlds = lds_addr(vdst) + TILE_BYTES;
#pragma unroll
        for (int p = slot * LOADS_PER_TILE / 4; p < (slot + 1) * LOADS_PER_TILE / 4; ++p) {
          const int i = p >> 1;
          const uint32_t off = (i * NWAVES + wave) * 64 * 16;
          if (p & 1) dma_16b(vp, src_off(i, true, v_kind, v_valid), __builtin_amdgcn_readfirstlane(vlds + off));
          else dma_16b(kp, src_off(i, false, k_kind, k_valid), __builtin_amdgcn_readfirstlane(klds + off));
        }
      };
      dma_slot(0);
      if constexpr (!B) {
        // PV_{t-1} (its first V fragments were read at the end of the previous iteration),
        // with K_t's first fragments read before it so that they land during it; K_t and V_t
        // are visible in iteration t
        __builtin_amdgcn_s_setprio(1);
        qk_pre(cur, ka0, ka1);
        if (t > 0) pv_run(stage((S + 3) & 3) + TILE_BYTES, pa, va);
        dma_slot(1);
        qk_run(cur, ka0, ka1);
        __builtin_amdgcn_s_setprio(0);
        if constexpr (ROTK) {
          if (t + 1 < n_tiles) rotate_k(stage((S + 1) & 3), t + 1);
          lds_barrier();
        }
        dma_slot(2);
        softmax(tile_valid(t), tile_mask(t), pa);
        pv_pre(cur + TILE_BYTES, va);  // V_t, for PV_t in the next iteration
      } else {
        // V_t's first fragments are read right after the softmax and K_{t+1}'s before PV_t
        // (both tiles are visible in iteration t; past the last tile the K reads fetch a stale
        // stage and go unused)
        bf16x8 pf[4];
        softmax(tile_valid(t), tile_mask(t), pf);
        pv_pre(cur + TILE_BYTES, va);
        if constexpr (ROTK) {
          if (t + 1 < n_tiles) rotate_k(stage((S + 1) & 3), t + 1);
          lds_barrier();
        }
        __builtin_amdgcn_s_setprio(1);
        dma_slot(1);
        qk_pre(stage((S + 1) & 3), ka0, ka1);
        pv_run(cur + TILE_BYTES, pf, va);
        dma_slot(2);
        if (t + 1 < n_tiles) qk_run(stage((S + 1) & 3), ka0, ka1);
        __builtin_amdgcn_s_setprio(0);
      }
      dma_slot(3);
      wait_vm_and_barrier<LOADS_PER_TILE>();
    };
    int t = 0;
    for (; t + 4 <= n_tiles; t += 4) {
      step.template operator()<0>(t);
      step.template operator()<1>(t + 1);
      step.template operator()<2>(t + 2);
      step.template operator()<3>(t + 3);
    }
    if (t < n_tiles) step.template operator()<0>(t);
    if (t + 1 < n_tiles) step.template operator()<1>(t + 1);
    if (t + 2 < n_tiles) step.template operator()<2>(t + 2);
    // the last iteration's copies (of tiles never read) land before the workgroup ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!B) {
      // PV of the last tile (its V fragments were read at the end of the last iteration)
      switch ((n_tiles - 1) & 3) {
        case 0: pv_run(stage0 + TILE_BYTES, pa, va); break;
        case 1: pv_run(stage1 + TILE_BYTES, pa, va); break;
        case 2: pv_run(stage2 + TILE_BYTES, pa, va); break;
        default: pv_run(stage3 + TILE_BYTES, pa, va); break;
      }
    }
  };
  if (wave_b) run.template operator()<true>();
  else run.template operator()<false>();

  // ---- epilogue (lane: query ql, dims dt*32 + 8*(r/4) + 4g + r%4)
  const float lt = sum_with_partner32(l_run);
  const int qrow = q0 + wave * 32 + ql;
  if (TEXT) {
    // partial result of this key range: unnormalised O, the running max and the sum, all
    // relative to that max (base-2 logits); text_combine_kernel merges the splits
    const int64_t prow = (static_cast<int64_t>(split) * a.total_blocks / a.blocks_per_bh + bh) *
                             a.q_rows + qrow;
    float* op = a.o_part + prow * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = dt * 32 + 8 * rg + 4 * g;
        *reinterpret_cast<f32x4*>(op + d0) =
            f32x4{o[dt][4 * rg], o[dt][4 * rg + 1], o[dt][4 * rg + 2], o[dt][4 * rg + 3]};
      }
    if (g == 0) a.ml_part[prow] = make_float2(m_run, lt);
    return;
  }
  const float inv = 1.0f / lt;
  // The hi pass undoes the window-first permutation here: window-first row qrow goes to
  // its raster row, so O needs no separate inverse-permutation pass.
  auto out_row = [&](int qr) __attribute__((always_inline)) {
    return HI ? window_first_to_raster(qr, a.W, a.w, a.n_wx) : qr;
  };
  const int my_orow = qrow < a.q_valid ? out_row(qrow) : -1;  // -1: padding row
  if (a.lse && g == 0 && my_orow >= 0)  // scores are base-2 logits: ln(sum e^s) = ln 2 (m + log2 l)
    a.lse[static_cast<int64_t>(bh) * a.out_rows + a.out_row0 + my_orow] =
        (m_run + __log2f(lt)) * 0.69314718055994531f;
  // O goes out through LDS so that the stores are whole rows: each wave writes its 32 rows
  // (bf16, 16-byte chunks XOR-swizzled by row) into its own slice of the stage buffers,
  // then every store instruction covers 64 / (D / 8) complete rows.  The barrier makes sure
  // no wave still reads a stage or has a tile copy landing in one.
  constexpr int OCH = D / 8;  // 16-byte chunks per row
  static_assert(NWAVES <= 16, "O staging: four waves per stage buffer");
  __syncthreads();
  char* obuf = stage(wave >> 2) + (wave & 3) * (32 * D * 2);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int c = 4 * dt + rg;  // chunk of dims dt*32 + 8rg .. +8; this lane holds half g
      const uint32_t w0 = pack_bf16x2(o[dt][4 * rg] * inv, o[dt][4 * rg + 1] * inv);
      const uint32_t w1 = pack_bf16x2(o[dt][4 * rg + 2] * inv, o[dt][4 * rg + 3] * inv);
      *reinterpret_cast<uint2*>(obuf + ql * (D * 2) + ((c ^ (ql & (OCH - 1))) << 4) + 8 * g) = make_uint2(w0, w1);
    }
  constexpr int RPI = 64 / OCH;  // rows per store instruction
#pragma unroll
  for (int u = 0; u < 32 / RPI; ++u) {
    const int r = u * RPI + lane / OCH, c = lane % OCH;
    const uint4 val = *reinterpret_cast<const uint4*>(obuf + r * (D * 2) + ((c ^ (r & (OCH - 1))) << 4));
    const int orr = __shfl(my_orow, r);  // the output row of query r, from lane r
    if (orr >= 0) {
      bf16_t* orow = a.out + ((static_cast<int64_t>(b) * a.out_rows + a.out_row0 + orr) * a.heads + h) * D;
      *reinterpret_cast<uint4*>(orow + 8 * c) = val;
    }
  }
}

// Merges the key-range splits of the text-query pass: with m* the largest running max,
// O = sum_s 2^(m_s - m*) O_s / sum_s 2^(m_s - m*) l_s, stored as bf16 in text row x of
// (b, h).  One thread per pair of dims.
__global__ void text_combine_kernel(const float* __restrict__ o_part, const float2* __restrict__ ml,
                                    bf16_t* out, float* lse, int splits, int64_t bh_total,
                                    int64_t Tq, int64_t out_rows, int heads, int D) {
  const int64_t x = blockIdx.x, bh = blockIdx.y;
  const int d = 2 * threadIdx.x;
  if (d >= D) return;
  float mx = -INFINITY;
  for (int sp = 0; sp < splits; ++sp) mx = fmaxf(mx, ml[(sp * bh_total + bh) * Tq + x].x);
  float l = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int sp = 0; sp < splits; ++sp) {
    const int64_t prow = (sp * bh_total + bh) * Tq + x;
    const float2 m = ml[prow];
    const float f = exp2f(m.x - mx);
    l += f * m.y;
    o0 += f * o_part[prow * D + d];
    o1 += f * o_part[prow * D + d + 1];
  }
  const int64_t b = bh / heads, h = bh - b * heads;
  *reinterpret_cast<uint32_t*>(out + ((b * out_rows + x) * heads + h) * D + d) = pack_bf16x2(o0 / l, o1 / l);
  if (lse && d == 0) lse[bh * out_rows + x] = (mx + __log2f(l)) * 0.69314718055994531f;
}

template <int D, int NWAVES, bool HI, bool RECT, bool TEXT, bool ROTK = false, bool RAW = false>
static void launch_attn(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, NWAVES, HI, RECT, TEXT, ROTK, RAW>), dim3(a.total_blocks),
                     dim3(NWAVES * 64), 0, s, a);
}

enum PassKind { kPassHi = 0, kPassHiRect = 1, kPassGuide = 2, kPassText = 3, kPassHiRotK = 4,
                kPassGuideRotK = 5, kPassHiRaw = 6, kPassGuideRaw = 7 };

template <int D>
static void dispatch_attn_d(int nwaves, PassKind kind, const AttnArgs& a, hipStream_t s) {
  switch (kind) {
    case kPassGuide: launch_attn<D, 8, false, false, false>(a, s); break;
    case kPassText: launch_attn<D, 8, false, false, true>(a, s); break;
    case kPassHiRotK: launch_attn<D, 8, true, false, false, true>(a, s); break;
    case kPassGuideRotK: launch_attn<D, 8, false, false, false, true>(a, s); break;
    case kPassHiRaw: launch_attn<D, 8, true, false, false, true, true>(a, s); break;
    case kPassGuideRaw: launch_attn<D, 8, false, false, false, true, true>(a, s); break;
    case kPassHiRect:
      nwaves == 8 ? launch_attn<D, 8, true, true, false>(a, s) : launch_attn<D, 2, true, true, false>(a, s);
      break;
    default:
      nwaves == 8 ? launch_attn<D, 8, true, false, false>(a, s) : launch_attn<D, 2, true, false, false>(a, s);
  }
}

static void dispatch_attn(int D, int nwaves, PassKind kind, const AttnArgs& a, hipStream_t s) {
  if (D == 128) dispatch_attn_d<128>(nwaves, kind, a, s);
  else dispatch_attn_d<64>(nwaves, kind, a, s);
}

// ------------------------------------------------------------------ host side

int timer_begin(uhla_timer* t, int stage, hipStream_t s);
int timer_end(uhla_timer* t, int stage, hipStream_t s);
int timer_commit(uhla_timer* t);

// Largest number of table-driven tiles (neighbour-window tiles plus cell-block guide
// tiles) over all windows; mirrors the tile-list construction of the hi pass.
static int64_t max_table_tiles(const Geom& g) {
  const int tpw = g.w * g.w / kKeyTile;
  const int reach = g.guide_mode == 1 ? 0 : g.radius;
  const bool rect = g.guide_mode != 0 && g.M > 0;
  int64_t best = 0;
  for (int wy = 0; wy < g.n_wy; ++wy)
    for (int wx = 0; wx < g.n_wx; ++wx) {
      auto span = [](int c, int r, int n) { return std::min(n - 1, c + r) - std::max(0, c - r) + 1; };
      int64_t n = static_cast<int64_t>(span(wy, g.radius, g.n_wy)) * span(wx, g.radius, g.n_wx) * tpw;
      if (rect) {
        const int gy0 = std::max(0, wy - reach), gy1 = std::min(g.n_wy - 1, wy + reach);
        const int gx0 = std::max(0, wx - reach), gx1 = std::min(g.n_wx - 1, wx + reach);
        const int i0 = (gy0 * g.w + g.rho - 1) / g.rho, i1 = std::min(g.H_lr, ((gy1 + 1) * g.w + g.rho - 1) / g.rho);
        const int j0 = (gx0 * g.w + g.rho - 1) / g.rho, j1 = std::min(g.W_lr, ((gx1 + 1) * g.w + g.rho - 1) / g.rho);
        if (i0 < i1 && j0 < j1)
          n += static_cast<int64_t>(((i1 - 1) >> 3) - (i0 >> 3) + 1) * (((j1 - 1) >> 3) - (j0 >> 3) + 1);
        n += g.Tk / kKeyTile;  // text tiles follow the cell blocks in the table
      }
      best = std::max(best, n);
    }
  return best;
}

int validate_forward(const void* q, const void* k, const void* v, void* o, int B,
                            int64_t T, int H, int W, int w, int H_lr, int W_lr, int rho,
                            int heads, int D, int radius, int guide_mode) {
  if (!q || !k || !v || !o) return fail_arg("null pointer");
  if (B < 1 || H < 1 || W < 1 || w < 1 || heads < 1 || D < 1 || H_lr < 0 || W_lr < 0 || T < 0)
    return fail_arg("sizes out of range");
  if (H % w || W % w) return fail_arg("w must divide H and W");
  if ((H_lr == 0) != (W_lr == 0)) return fail_arg("H_lr and W_lr must both be zero or not");
  if (static_cast<int64_t>(H_lr) * W_lr > 0 && rho < 1)
    return fail_arg("rho must be >= 1 with guide tokens");
  if (radius < 0) return fail_arg("radius must be >= 0");
  if (guide_mode < 0 || guide_mode > 2) return fail_arg("guide_mode must be 0, 1 or 2");
  if (D != 64 && D != 128) return fail_unsupported("head_dim must be 64 or 128");
  if (w % 8 || (w > 16 && w % 16)) return fail_unsupported("window size must be 8, 16 or a multiple of 16");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
       reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o)) % 16)
    return fail_arg("tensors must be 16-byte aligned");
  if (B > 65535) return fail_unsupported("batch too large");
  if (heads > 65535) return fail_unsupported("too many heads");
  const int64_t N = static_cast<int64_t>(H) * W, M = static_cast<int64_t>(H_lr) * W_lr;
  const int64_t bh = static_cast<int64_t>(B) * heads;
  // 32-bit row indices and tile byte offsets inside the kernels; 32-bit workgroup counts
  if (N > (int64_t(1) << 26) || M > (int64_t(1) << 26) || T > (int64_t(1) << 24) ||
      bh * ((N + M + T) / 64 + 1) > 0x7fffffff)
    return fail_unsupported("problem too large");
  {
    // The attention kernels address a K or V tile by its 32-bit byte offset inside the
    // (batch, head) region of its buffer: hi rows (N), global keys (guide rows padded to
    // the key tile, then text rows) and, in guide modes 1 and 2, the cell-block copy.
    const Geom g = make_geom(B, H, W, w, H_lr, W_lr, rho > 0 ? rho : 1, heads, D, 1, guide_mode, T);
    const int64_t row_bytes = static_cast<int64_t>(D) * 2, lim = int64_t(1) << 32;
    if (g.N * row_bytes > lim || g.Mg * row_bytes > lim || g.Mbg * row_bytes > lim)
      return fail_unsupported("a (batch, head) K or V region exceeds 4 GiB");
  }
  // radius capped so that the neighbourhood span stays far inside int range
  if (max_table_tiles(make_geom(B, H, W, w, H_lr, W_lr, rho, heads, D,
                                std::min(radius, H / w + W / w), guide_mode, T)) > kMaxTableTiles)
    return fail_unsupported("too many key tiles per window (window size, radius or text too large)");
  return UHLA_OK;
}

int forward_impl(const void* q, const void* k, const void* v, void* o, int B, int64_t T,
                        int H, int W, int w, int H_lr, int W_lr, int rho, int heads, int D,
                        float scale, float theta, int radius, int guide_mode, void* workspace,
                        size_t workspace_bytes, void* stream, uhla_timer* timer,
                        float* lse, bool rope_k_at_load) {
  int st = validate_forward(q, k, v, o, B, T, H, W, w, H_lr, W_lr, rho, heads, D, radius, guide_mode);
  if (st) return st;
  if (rope_k_at_load && w * w < kMaxQuery)
    return fail_unsupported("K rotation at tile load needs windows of at least 256 tokens");
  // a radius reaching past the grid is the whole grid
  radius = std::min(radius, H / w + W / w);
  const Geom g = make_geom(B, H, W, w, H_lr, W_lr, rho, heads, D, radius, guide_mode, T);
  const Workspace need = carve(g, nullptr);
  if (!workspace || workspace_bytes < need.bytes)
    return (set_detail("workspace too small"), UHLA_ERR_WORKSPACE);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail_arg("workspace must be 256-byte aligned");
  const int64_t L = T + g.N + g.M;
  const size_t tensor_bytes = static_cast<size_t>(B) * L * heads * D * 2;
  if (ranges_overlap(o, tensor_bytes, q, tensor_bytes) ||
      ranges_overlap(o, tensor_bytes, k, tensor_bytes) ||
      ranges_overlap(o, tensor_bytes, v, tensor_bytes) ||
      ranges_overlap(o, tensor_bytes, workspace, need.bytes))
    return fail_arg("o overlaps an input or the workspace");
  // the prep pass writes the workspace while the inputs are still being read
  for (const void* x : {q, k, v})
    if (ranges_overlap(workspace, need.bytes, x, tensor_bytes))
      return fail_arg("the workspace overlaps an input");
  const size_t lse_bytes = static_cast<size_t>(B) * heads * L * sizeof(float);
  if (lse && (reinterpret_cast<uintptr_t>(lse) % 4 || ranges_overlap(lse, lse_bytes, o, tensor_bytes) ||
              ranges_overlap(lse, lse_bytes, workspace, need.bytes) ||
              ranges_overlap(lse, lse_bytes, q, tensor_bytes) ||
              ranges_overlap(lse, lse_bytes, k, tensor_bytes) ||
              ranges_overlap(lse, lse_bytes, v, tensor_bytes)))
    return fail_arg("lse misaligned or overlapping o, an input or the workspace");
  const Workspace ws = carve(g, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool rope_on = theta > 0.0f;
  const float sc = scale > 0.0f ? scale : 1.0f / sqrtf(static_cast<float>(D));
  const int w2 = w * w;

#define UHLA_STEP(call, name)          \
  do {                                 \
    call;                              \
    st = check_launch(name);           \
    if (st) return st;                 \
  } while (0)

  // 1. tables (the neighbour windows are a clipped rectangle, computed in the hi pass)
  if (timer) timer_begin(timer, UHLA_STAGE_TABLES, s);
  if (rope_on) {
    const int n = g.P * (D / 4);
    UHLA_STEP(hipLaunchKernelGGL(cos_sin_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s,
                                 ws.cs, g.P, D, log2(static_cast<double>(theta))),
              "cos_sin_table_kernel");
  }
  if (timer) timer_end(timer, UHLA_STAGE_TABLES, s);

  // 2. prep: permutation + RoPE (K) and permutation + tile transpose (V); Q is rotated
  //    as the attention kernel loads it
  const double l2t = rope_on ? log2(static_cast<double>(theta)) : 0.0;
  const bf16_t* kb = static_cast<const bf16_t*>(k);
  const bf16_t* vb = static_cast<const bf16_t*>(v);
  const double qs = static_cast<double>(sc) * 1.4426950408889634;  // scale * log2 e
  if (timer) timer_begin(timer, UHLA_STAGE_PREP_HI, s);
  {
    const int64_t rows = g.N + g.Mk + g.Mb + g.Tk;
    const dim3 grid(static_cast<unsigned>((rows + kPrepRows - 1) / kPrepRows), B);
    if (D == 128)
      hipLaunchKernelGGL(prep_k_kernel<128>, grid, dim3(kPrepThreads), 0, s, kb, ws.k_hi, ws.k_lr,
                         ws.k_gb, ws.cs, g.P, l2t, T, g.N, g.M, g.Mk, g.Mg, g.Mb, g.Mbg, g.Tk, W,
                         w, g.n_wx, H_lr, W_lr, g.nbj, rho, heads, rope_on && !rope_k_at_load ? 1 : 0,
                         static_cast<const bf16_t*>(q), ws.q_hi, ws.q_lr, qs);
    else
      hipLaunchKernelGGL(prep_k_kernel<64>, grid, dim3(kPrepThreads), 0, s, kb, ws.k_hi, ws.k_lr,
                         ws.k_gb, ws.cs, g.P, l2t, T, g.N, g.M, g.Mk, g.Mg, g.Mb, g.Mbg, g.Tk, W,
                         w, g.n_wx, H_lr, W_lr, g.nbj, rho, heads, rope_on && !rope_k_at_load ? 1 : 0,
                         static_cast<const bf16_t*>(q), ws.q_hi, ws.q_lr, qs);
    st = check_launch("prep_k_kernel");
    if (st) return st;
    const int64_t tiles = (g.N + g.Mg + g.Mbg) / kKeyTile;
    if (tiles * heads > 0x7fffffff) return fail_unsupported("problem too large");
    UHLA_STEP(hipLaunchKernelGGL(prep_v_kernel, dim3(static_cast<unsigned>(tiles * heads), B), dim3(kPrepThreads), 0, s,
                                 vb, ws.v_hi, ws.v_lr, ws.v_gb, T, g.N, g.M, g.Mk, g.Mg, g.Mb, g.Mbg,
                                 W, w, g.n_wx, H_lr, W_lr, g.nbj, heads, D),
              "prep_v_kernel");
  }
  if (timer) timer_end(timer, UHLA_STAGE_PREP_HI, s);
  if (timer) timer_begin(timer, UHLA_STAGE_PREP_LR, s);  // guide rows are folded into step 2
  if (timer) timer_end(timer, UHLA_STAGE_PREP_LR, s);

  AttnArgs a{};
  a.q = static_cast<const bf16_t*>(q);
  a.cs = ws.cs; a.log2_theta = l2t; a.P = g.P; a.rope_on = rope_on ? 1 : 0;
  a.q_scale = qs;
  a.rho = rho; a.H_lr = H_lr; a.W_lr = W_lr; a.nbj = g.nbj;  // guide query positions
  a.k_hi = ws.k_hi; a.v_hi = ws.v_hi; a.k_lr = ws.k_lr; a.v_lr = ws.v_lr;
  a.N = g.N; a.M = g.M; a.Mk = g.Mk; a.Mg = g.Mg; a.T = T; a.Mb = g.Mb;
  a.heads = heads; a.w2 = w2;
  a.out = static_cast<bf16_t*>(o); a.out_rows = L;
  a.lse = lse;
  const int64_t BH = static_cast<int64_t>(B) * heads;

  // 3. hi pass
  if (timer) timer_begin(timer, UHLA_STAGE_ATTN_HI, s);
  {
    const int nwaves = w2 >= kMaxQuery ? 8 : w2 / 32;
    const int qt = nwaves * 32;
    AttnArgs h = a;
    h.q_rows = g.N;
    h.q_pre = ws.q_hi;  // non-null in guide modes 1, 2
    h.out_row0 = T;
    h.W = W; h.w = w; h.n_wx = g.n_wx; h.n_wy = g.n_wy;
    h.radius = radius;
    const bool rect = guide_mode != 0 && g.M > 0;
    if (rect) {
      h.k_lr = ws.k_gb; h.v_lr = ws.v_gb; h.Mg = g.Mbg;
    }
    h.reach = guide_mode == 1 ? 0 : radius;
    h.q_valid = static_cast<int>(g.N);
    h.blocks_per_bh = static_cast<int>(g.N / qt);
    h.total_blocks = static_cast<int>(BH * h.blocks_per_bh);
    const PassKind kind = rope_k_at_load ? kPassHiRotK : rect ? kPassHiRect : kPassHi;
    UHLA_STEP(dispatch_attn(D, nwaves, kind, h, s), "attn_fwd_kernel(hi)");
  }
  if (timer) timer_end(timer, UHLA_STAGE_ATTN_HI, s);

  // 4. guide pass (guide keys, then text keys)
  if (timer) timer_begin(timer, UHLA_STAGE_ATTN_LR, s);
  if (g.M > 0) {
    AttnArgs l = a;
    l.q_rows = g.Mq;
    l.q_pre = ws.q_lr;
    l.out_row0 = T + g.N;
    l.q_valid = static_cast<int>(g.M);
    l.blocks_per_bh = static_cast<int>(g.Mq / kMaxQuery);
    l.total_blocks = static_cast<int>(BH * l.blocks_per_bh);
    UHLA_STEP(dispatch_attn(D, 8, rope_k_at_load ? kPassGuideRotK : kPassGuide, l, s), "attn_fwd_kernel(guide)");
  }
  if (timer) timer_end(timer, UHLA_STAGE_ATTN_LR, s);

  // 5. the inverse permutation of O is fused into the hi pass's stores (stage left empty)
  if (timer) timer_begin(timer, UHLA_STAGE_UNPERMUTE, s);
  if (timer) timer_end(timer, UHLA_STAGE_UNPERMUTE, s);

  // 6. text queries: every key, split over the key range, then merged
  if (timer) timer_begin(timer, UHLA_STAGE_ATTN_TEXT, s);
  if (T > 0) {
    AttnArgs x = a;
    x.q_rows = g.Tq;
    x.q_valid = static_cast<int>(T);
    x.splits = g.splits;
    x.blocks_per_bh = static_cast<int>(g.Tq / kMaxQuery) * g.splits;
    x.total_blocks = static_cast<int>(BH * x.blocks_per_bh);
    x.o_part = ws.o_part; x.ml_part = ws.ml_part;
    UHLA_STEP(dispatch_attn(D, 8, kPassText, x, s), "attn_fwd_kernel(text)");
    UHLA_STEP(hipLaunchKernelGGL(text_combine_kernel, dim3(static_cast<unsigned>(T), static_cast<unsigned>(BH)),
                                 dim3(D / 2), 0, s, ws.o_part, ws.ml_part, static_cast<bf16_t*>(o),
                                 lse, g.splits, BH, g.Tq, L, heads, D),
              "text_combine_kernel");
  }
  if (timer) timer_end(timer, UHLA_STAGE_ATTN_TEXT, s);
#undef UHLA_STEP
  if (timer) return timer_commit(timer);
  return UHLA_OK;
}

size_t workspace_bytes(int B, int64_t T, int H, int W, int w, int H_lr, int W_lr, int rho,
                              int heads, int head_dim, int radius, int guide_mode) {
  if (B < 1 || H < 1 || W < 1 || w < 1 || heads < 1 || H_lr < 0 || W_lr < 0 || T < 0) return 0;
  if (H % w || W % w || (H_lr == 0) != (W_lr == 0)) return 0;
  if (head_dim != 64 && head_dim != 128) return 0;
  if (radius < 0 || guide_mode < 0 || guide_mode > 2) return 0;
  if (static_cast<int64_t>(H_lr) * W_lr > 0 && rho < 1) return 0;
  return carve(make_geom(B, H, W, w, H_lr, W_lr, rho, heads, head_dim, radius, guide_mode, T),
               nullptr).bytes;
}

// Permute-free forward (uhla_forward_permute_free): no K/V prep pass; the attention
// kernels copy their tiles straight from the caller's raster K and V, rotate K at load and
// read V transposed from LDS.  Workspace: the cos/sin table only.
static size_t permute_free_workspace(const Geom& g) {
  return (static_cast<size_t>(g.P) * (g.D / 4) * sizeof(double2) + 255) / 256 * 256;
}

static int validate_permute_free(const void* q, const void* k, const void* v, void* o, int B,
                                 int H, int W, int w, int H_lr, int W_lr, int rho, int heads,
                                 int D) {
  int st = validate_forward(q, k, v, o, B, 0, H, W, w, H_lr, W_lr, rho, heads, D, 1, 0);
  if (st) return st;
  // a 64-key tile must be whole window rows (64 / w of them) or a 64-token piece of one
  if (w < 16 || (kKeyTile % w != 0 && w % kKeyTile != 0))
    return fail_unsupported("permute-free forward: window size must be 16, 32, 64 or a multiple of 64");
  // per-lane chunk offsets from a tile's first token are 32-bit
  const int64_t rowb = static_cast<int64_t>(heads) * D * 2;
  const int64_t rows = w <= kKeyTile ? static_cast<int64_t>(kKeyTile / w) * W : kKeyTile;
  if (rows * rowb >= (int64_t(1) << 31))
    return fail_unsupported("permute-free forward: rows of the tensors too long for 32-bit tile offsets");
  return UHLA_OK;
}

static int forward_permute_free_impl(const void* q, const void* k, const void* v, void* o, int B,
                                     int H, int W, int w, int H_lr, int W_lr, int rho, int heads,
                                     int D, float scale, float theta, void* workspace,
                                     size_t workspace_bytes, void* stream, uhla_timer* timer) {
  int st = validate_permute_free(q, k, v, o, B, H, W, w, H_lr, W_lr, rho, heads, D);
  if (st) return st;
  const Geom g = make_geom(B, H, W, w, H_lr, W_lr, rho, heads, D, 1, 0, 0);
  const size_t need = permute_free_workspace(g);
  if (!workspace || workspace_bytes < need) return (set_detail("workspace too small"), UHLA_ERR_WORKSPACE);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail_arg("workspace must be 256-byte aligned");
  const int64_t L = g.N + g.M;
  const size_t tensor_bytes = static_cast<size_t>(B) * L * heads * D * 2;
  if (ranges_overlap(o, tensor_bytes, q, tensor_bytes) || ranges_overlap(o, tensor_bytes, k, tensor_bytes) ||
      ranges_overlap(o, tensor_bytes, v, tensor_bytes) || ranges_overlap(o, tensor_bytes, workspace, need))
    return fail_arg("o overlaps an input or the workspace");
  for (const void* x : {q, k, v})
    if (ranges_overlap(workspace, need, x, tensor_bytes)) return fail_arg("the workspace overlaps an input");
  hipStream_t s = static_cast<hipStream_t>(stream);
  double2* cs = static_cast<double2*>(workspace);
  const bool rope_on = theta > 0.0f;
  const float sc = scale > 0.0f ? scale : 1.0f / sqrtf(static_cast<float>(D));
  const double l2t = rope_on ? log2(static_cast<double>(theta)) : 0.0;
  if (timer) timer_begin(timer, UHLA_STAGE_TABLES, s);
  if (rope_on) {
    const int n = g.P * (D / 4);
    hipLaunchKernelGGL(cos_sin_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, cs, g.P, D, l2t);
    st = check_launch("cos_sin_table_kernel");
    if (st) return st;
  }
  if (timer) {  // no prep and no separate unpermute: their stages stay empty
    timer_end(timer, UHLA_STAGE_TABLES, s);
    for (int stage : {UHLA_STAGE_PREP_HI, UHLA_STAGE_PREP_LR}) {
      timer_begin(timer, stage, s);
      timer_end(timer, stage, s);
    }
  }
  AttnArgs a{};
  a.q = static_cast<const bf16_t*>(q);
  a.k_raw = static_cast<const bf16_t*>(k);
  a.v_raw = static_cast<const bf16_t*>(v);
  a.k_hi = a.k_lr = a.k_raw;  // unused by the raster-tile kernels
  a.v_hi = a.v_lr = a.v_raw;
  a.cs = cs; a.log2_theta = l2t; a.P = g.P; a.rope_on = rope_on ? 1 : 0;
  a.q_scale = static_cast<double>(sc) * 1.4426950408889634;
  a.rho = rho; a.H_lr = H_lr; a.W_lr = W_lr; a.nbj = g.nbj;
  a.N = g.N; a.M = g.M; a.Mk = g.Mk; a.Mg = g.Mk; a.T = 0; a.Mb = 0;
  a.heads = heads; a.w2 = w * w;
  a.out = static_cast<bf16_t*>(o); a.out_rows = L;
  const int64_t BH = static_cast<int64_t>(B) * heads;
  if (timer) timer_begin(timer, UHLA_STAGE_ATTN_HI, s);
  {
    AttnArgs h = a;
    h.q_rows = g.N;
    h.out_row0 = 0;
    h.W = W; h.w = w; h.n_wx = g.n_wx; h.n_wy = g.n_wy;
    h.radius = 1;
    h.q_valid = static_cast<int>(g.N);
    h.blocks_per_bh = static_cast<int>(g.N / kMaxQuery);
    h.total_blocks = static_cast<int>(BH * h.blocks_per_bh);
    dispatch_attn(D, 8, kPassHiRaw, h, s);
    st = check_launch("attn_fwd_kernel(hi, raster tiles)");
    if (st) return st;
  }
  if (timer) {
    timer_end(timer, UHLA_STAGE_ATTN_HI, s);
    timer_begin(timer, UHLA_STAGE_ATTN_LR, s);
  }
  if (g.M > 0) {
    AttnArgs l = a;
    l.q_rows = g.Mq;
    l.out_row0 = g.N;
    l.q_valid = static_cast<int>(g.M);
    l.blocks_per_bh = static_cast<int>(g.Mq / kMaxQuery);
    l.total_blocks = static_cast<int>(BH * l.blocks_per_bh);
    dispatch_attn(D, 8, kPassGuideRaw, l, s);
    st = check_launch("attn_fwd_kernel(guide, raster tiles)");
    if (st) return st;
  }
  if (timer) {
    timer_end(timer, UHLA_STAGE_ATTN_LR, s);
    for (int stage : {UHLA_STAGE_UNPERMUTE, UHLA_STAGE_ATTN_TEXT}) {
      timer_begin(timer, stage, s);
      timer_end(timer, stage, s);
    }
    return timer_commit(timer);
  }
  return UHLA_OK;
}

}  // namespace uhla

extern "C" size_t uhla_forward_workspace_bytes(int B, int H, int W, int w, int H_lr, int W_lr,
                                               int heads, int head_dim) {
  return uhla::workspace_bytes(B, 0, H, W, w, H_lr, W_lr, 1, heads, head_dim, 1, 0);
}

extern "C" size_t uhla_forward_masked_workspace_bytes(int B, int H, int W, int w, int H_lr,
                                                      int W_lr, int rho, int heads, int head_dim,
                                                      int radius, int guide_mode) {
  return uhla::workspace_bytes(B, 0, H, W, w, H_lr, W_lr, rho, heads, head_dim, radius, guide_mode);
}

extern "C" size_t uhla_forward_text_workspace_bytes(int B, int T, int H, int W, int w, int H_lr,
                                                    int W_lr, int rho, int heads, int head_dim,
                                                    int radius, int guide_mode) {
  return uhla::workspace_bytes(B, T, H, W, w, H_lr, W_lr, rho, heads, head_dim, radius, guide_mode);
}

extern "C" int uhla_forward(const void* q, const void* k, const void* v, void* o, int B, int H,
                            int W, int w, int H_lr, int W_lr, int rho, int heads, int head_dim,
                            float scale, float theta, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return uhla::forward_impl(q, k, v, o, B, 0, H, W, w, H_lr, W_lr, rho, heads, head_dim, scale,
                            theta, 1, 0, workspace, workspace_bytes, stream, nullptr);
}

extern "C" int uhla_forward_masked(const void* q, const void* k, const void* v, void* o, int B,
                                   int H, int W, int w, int H_lr, int W_lr, int rho, int heads,
                                   int head_dim, float scale, float theta, int radius,
                                   int guide_mode, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return uhla::forward_impl(q, k, v, o, B, 0, H, W, w, H_lr, W_lr, rho, heads, head_dim, scale,
                            theta, radius, guide_mode, workspace, workspace_bytes, stream, nullptr);
}

extern "C" int uhla_forward_text(const void* q, const void* k, const void* v, void* o, int B,
                                 int T, int H, int W, int w, int H_lr, int W_lr, int rho,
                                 int heads, int head_dim, float scale, float theta, int radius,
                                 int guide_mode, void* workspace, size_t workspace_bytes,
                                 void* stream, uhla_timer* timer) {
  return uhla::forward_impl(q, k, v, o, B, T, H, W, w, H_lr, W_lr, rho, heads, head_dim, scale,
                            theta, radius, guide_mode, workspace, workspace_bytes, stream, timer);
}

extern "C" int uhla_forward_timed(const void* q, const void* k, const void* v, void* o, int B,
                                  int H, int W, int w, int H_lr, int W_lr, int rho, int heads,
                                  int head_dim, float scale, float theta, void* workspace,
                                  size_t workspace_bytes, void* stream, uhla_timer* timer) {
  if (!timer) return uhla::fail_arg("null timer");
  return uhla::forward_impl(q, k, v, o, B, 0, H, W, w, H_lr, W_lr, rho, heads, head_dim, scale,
                            theta, 1, 0, workspace, workspace_bytes, stream, timer);
}

extern "C" int uhla_forward_masked_timed(const void* q, const void* k, const void* v, void* o,
                                         int B, int H, int W, int w, int H_lr, int W_lr, int rho,
                                         int heads, int head_dim, float scale, float theta,
                                         int radius, int guide_mode, void* workspace,
                                         size_t workspace_bytes, void* stream, uhla_timer* timer) {
  if (!timer) return uhla::fail_arg("null timer");
  return uhla::forward_impl(q, k, v, o, B, 0, H, W, w, H_lr, W_lr, rho, heads, head_dim, scale,
                            theta, radius, guide_mode, workspace, workspace_bytes, stream, timer);
}

extern "C" int uhla_forward_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int T, int H, int W, int w, int H_lr, int W_lr, int rho,
                                int heads, int head_dim, float scale, float theta, int radius,
                                int guide_mode, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (!lse) return uhla::fail_arg("null lse");
  return uhla::forward_impl(q, k, v, o, B, T, H, W, w, H_lr, W_lr, rho, heads, head_dim, scale,
                            theta, radius, guide_mode, workspace, workspace_bytes, stream, nullptr,
                            lse);
}

extern "C" int uhla_forward_rope_at_load(const void* q, const void* k, const void* v, void* o,
                                         int B, int H, int W, int w, int H_lr, int W_lr, int rho,
                                         int heads, int head_dim, float scale, float theta,
                                         void* workspace, size_t workspace_bytes, void* stream,
                                         uhla_timer* timer) {
  return uhla::forward_impl(q, k, v, o, B, 0, H, W, w, H_lr, W_lr, rho, heads, head_dim, scale,
                            theta, 1, 0, workspace, workspace_bytes, stream, timer, nullptr, true);
}


extern "C" size_t uhla_forward_permute_free_workspace_bytes(int B, int H, int W, int w, int H_lr,
                                                           int W_lr, int rho, int heads,
                                                           int head_dim) {
  // 0 for the sizes uhla_forward_permute_free rejects on their own (its pointer checks aside)
  if (uhla::workspace_bytes(B, 0, H, W, w, H_lr, W_lr, rho, heads, head_dim, 1, 0) == 0) return 0;
  if (w < 16 || (uhla::kKeyTile % w != 0 && w % uhla::kKeyTile != 0)) return 0;
  return uhla::permute_free_workspace(uhla::make_geom(B, H, W, w, H_lr, W_lr, rho > 0 ? rho : 1,
                                                      heads, head_dim, 1, 0, 0));
}

extern "C" int uhla_forward_permute_free(const void* q, const void* k, const void* v, void* o,
                                         int B, int H, int W, int w, int H_lr, int W_lr, int rho,
                                         int heads, int head_dim, float scale, float theta,
                                         void* workspace, size_t workspace_bytes, void* stream,
                                         uhla_timer* timer) {
  return uhla::forward_permute_free_impl(q, k, v, o, B, H, W, w, H_lr, W_lr, rho, heads,
                                         head_dim, scale, theta, workspace, workspace_bytes,
                                         stream, timer);
}
