/*
 * uhla.h -- C ABI of the MI355X (gfx950) hierarchical local attention library.
 *
 * The method is UltraGen's hierarchical local attention.  Citation keys:
 * [UltraGen/<lang> §n] is the gist.science summary page "UltraGen: Efficient
 * Ultra-High-Resolution Image Generation with Hierarchical Local Attention" in the
 * named language edition (it, fr, es, ar, ko), section n of its technical summary.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Token-major layout [B, L, heads, head_dim], contiguous, L = N + M.  Rows 0..N-1 are
 *   the hi-res tokens of an H x W grid in raster order (row y = index / W); rows N..L-1
 *   are the low-res guide tokens of an H_lr x W_lr grid in raster order.  This is the
 *   joint [hi | guide] part of the text | image | guide sequence of [UltraGen/it §2].
 * - Device pointers are HIP device memory owned by the caller.  The library never
 *   allocates, frees or synchronises (except uhla_timer_read), keeps no global mutable
 *   state (except the static scratch of uhla_forward_noalloc) and may be called from
 *   several host threads on different streams.
 * - `stream` is a hipStream_t (NULL = the legacy default stream).  All work is enqueued
 *   asynchronously on it.
 * - Every function returns a uhla_status; nothing throws across the ABI.  Argument
 *   errors are detected on the host before anything is enqueued.  UHLA_ERR_HIP means a
 *   HIP call failed; uhla_last_error_detail() then returns the HIP message for the
 *   calling thread.
 * - bf16 is IEEE bfloat16 stored as 16-bit words; rounding to bf16 is round to nearest
 *   even.
 */
#ifndef UHLA_H_
#define UHLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  UHLA_OK = 0,
  UHLA_ERR_ARG = 1,          /* invalid argument (null pointer, bad size, aliasing) */
  UHLA_ERR_UNSUPPORTED = 2,  /* valid but not built: head_dim, elem_bytes, window size */
  UHLA_ERR_WORKSPACE = 3,    /* workspace pointer null or smaller than required */
  UHLA_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} uhla_status;

/* Stage timer (measurement only; see uhla_timer_create below). */
typedef struct uhla_timer uhla_timer;

/*
 * Window-first permutation of the hi-res segment, and its exact inverse.
 *
 * Defined in [UltraGen/it §2], [UltraGen/fr §2.A] and [UltraGen/ar §2.A]: hi-res
 * tokens are split into fixed, non-overlapping w x w windows and reordered window by
 * window, so that each attention block is one spatial window.  Windows are enumerated
 * row-major over the (H/w) x (W/w) window grid; tokens are raster inside a window:
 *   p = win * w*w + iy * w + ix,  win = wy * (W/w) + wx,
 *   r(p) = (wy*w + iy) * W + (wx*w + ix).
 * uhla_window_permute:   dst[b, p] = src[b, r(p)]   for p in 0..H*W-1
 * uhla_window_unpermute: dst[b, r(p)] = src[b, p]
 * A "row" is heads * head_dim elements of elem_bytes bytes (2 = bf16/fp16, 4 = fp32);
 * rows are copied bit-exactly.  Batch b of src starts at row b * src_tokens_per_batch,
 * of dst at row b * dst_tokens_per_batch (both >= H*W), so the hi segment of a
 * [B, N + M, heads, head_dim] tensor can be permuted in place of a copy; rows at and
 * beyond H*W in each batch are neither read nor written.  src and dst must not overlap.
 * Errors: UHLA_ERR_ARG for null pointers, B/H/W/w/heads/head_dim < 1, w not dividing
 * H or W, a batch stride < H*W, overlapping src/dst; UHLA_ERR_UNSUPPORTED for
 * elem_bytes not in {2, 4}.
 */
int uhla_window_permute(const void* src, void* dst, int B, int H, int W, int w,
                        int heads, int head_dim, int elem_bytes,
                        int64_t src_tokens_per_batch, int64_t dst_tokens_per_batch,
                        void* stream);
int uhla_window_unpermute(const void* src, void* dst, int B, int H, int W, int w,
                          int heads, int head_dim, int elem_bytes,
                          int64_t src_tokens_per_batch, int64_t dst_tokens_per_batch,
                          void* stream);

/*
 * 2D axial RoPE on a bf16 [B, L, heads, head_dim] tensor (src may equal dst; partial
 * overlap is an error).
 *
 * Positions: guide-token indices are scaled by rho onto the hi-res grid
 * ([UltraGen/ar §2.B]): guide raster token s sits at (rho * (s / W_lr), rho * (s % W_lr)).
 * Hi-res row i sits at (r / W, r % W) with r = i (hi_order = 0, raster) or r = r(i)
 * of the window-first map above (hi_order = 1).
 * Rotation: d_axis = head_dim / 2; dims [0, d_axis) rotate by y, dims [d_axis, head_dim)
 * by x; inside an axis block the pair (2k, 2k+1) = (a, b) becomes
 * (a cos phi - b sin phi, a sin phi + b cos phi), phi = pos * theta^(-2k / d_axis).
 * cos/sin and the rotation are evaluated in fp64 and each result is rounded once to bf16
 * (round to nearest even).  theta <= 0 copies src to dst unchanged.
 * Errors: UHLA_ERR_ARG (null pointers, sizes < 1, w not dividing H or W when
 * hi_order = 1, exactly one of H_lr/W_lr zero, rho < 1 with guide tokens, hi_order not
 * 0/1, partial overlap); UHLA_ERR_UNSUPPORTED when head_dim % 8 != 0.
 */
int uhla_rope_apply(const void* src, void* dst, int B, int H, int W, int w, int hi_order,
                    int H_lr, int W_lr, int rho, int heads, int head_dim, float theta,
                    void* stream);

/*
 * Workspace bytes uhla_forward needs for this geometry (0 on invalid geometry).
 */
size_t uhla_forward_workspace_bytes(int B, int H, int W, int w, int H_lr, int W_lr,
                                    int heads, int head_dim);

/*
 * Hierarchical local attention forward.
 *
 * Q, K, V, O: bf16 [B, N + M, heads, head_dim] in the layout above.  The result is
 *   O = softmax(rope(Q) rope(K)^T * scale + mask) V   per (batch, head),
 * with the mask of [UltraGen/ar §2.B] and [UltraGen/es §2]: a hi-res token attends to
 * every token of its own window and of the clipped 3x3 neighbourhood of windows, and to
 * all M guide tokens; a guide token attends to all guide tokens and to no hi-res token.
 * Steps: window-first permutation of the hi segment of K and V, fused with RoPE on K
 * (guide rows rotated in place of permuting); block-sparse attention of each window over
 * its neighbour windows and the guide tokens (bf16 MFMA, fp32 accumulation and softmax),
 * which reads its query rows from Q in raster order and rotates them as it loads them,
 * and whose stores put each output row back at its raster position (the inverse
 * permutation, fused); guide-only attention.
 * scale <= 0 selects 1/sqrt(head_dim); theta <= 0 switches RoPE off; H_lr = W_lr = 0
 * means no guide tokens.  Deterministic: no atomics, fixed reduction order.
 * workspace: device memory of at least uhla_forward_workspace_bytes(...) bytes, 256-byte
 *   aligned, owned by the caller; its contents are scratch.
 * Errors: UHLA_ERR_ARG (null pointers, sizes < 1, w not dividing H or W, rho < 1 with
 * guide tokens, exactly one of H_lr/W_lr zero, O overlapping Q, K, V or the workspace,
 * the workspace overlapping Q, K or V);
 * UHLA_ERR_UNSUPPORTED (head_dim not in {64, 128}; w not a multiple of 8, or w > 16
 * and not a multiple of 16; more than 1024 key tiles of 64 keys per window, counting
 * the neighbour windows' tiles and, in the masked variant, the guide cell blocks; B or
 * heads above 65535; grids, guide grids or text too large for 32-bit row and workgroup
 * indices; a (batch, head) region of K or V rows above 4 GiB, i.e. H*W rows, or the guide
 * rows rounded up to 64 plus the text rows rounded up to 64, times head_dim * 2 bytes,
 * above 2^32); UHLA_ERR_WORKSPACE; UHLA_ERR_HIP.
 */
int uhla_forward(const void* q, const void* k, const void* v, void* o,
                 int B, int H, int W, int w, int H_lr, int W_lr, int rho,
                 int heads, int head_dim, float scale, float theta,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Mask variants the pages leave open ([UltraGen/it §2]: a window looks at the guide
 * tokens that correspond to it; [UltraGen/ar §2.B]: the neighbourhood of adjacent
 * windows).  Same as uhla_forward except for the hi-res rows of the mask:
 *   radius >= 0: a hi-res token sees the windows within `radius` windows along each axis
 *     (clipped to the grid; 1 is the 3x3 neighbourhood of uhla_forward, 0 its own window);
 *   guide_mode 0: every guide token (as uhla_forward);
 *   guide_mode 1: the guide tokens (i, j) whose scaled position (rho*i, rho*j) lies in the
 *     query's window;
 *   guide_mode 2: those whose scaled position lies in one of the query's `radius`
 *     neighbourhood windows.
 *   A scaled position outside the hi-res grid lies in no window.  Guide rows of O are as
 *   in uhla_forward.  uhla_forward(...) == uhla_forward_masked(..., 1, 0, ...).
 * workspace: at least uhla_forward_masked_workspace_bytes(...) bytes (0 on invalid
 *   arguments); guide modes 1 and 2 add a cell-block copy of the guide K and V.
 * Errors: as uhla_forward, plus UHLA_ERR_ARG for radius < 0 or guide_mode not in {0,1,2}.
 */
size_t uhla_forward_masked_workspace_bytes(int B, int H, int W, int w, int H_lr, int W_lr,
                                           int rho, int heads, int head_dim, int radius,
                                           int guide_mode);
int uhla_forward_masked(const void* q, const void* k, const void* v, void* o,
                        int B, int H, int W, int w, int H_lr, int W_lr, int rho,
                        int heads, int head_dim, float scale, float theta,
                        int radius, int guide_mode,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Text tokens in the joint sequence ([UltraGen/it §2], [UltraGen/fr §2.C]: the DiT input is
 * text | hi-res | guide).  Q, K, V, O: bf16 [B, T + N + M, heads, head_dim], rows 0..T-1
 * the text tokens, then the hi-res rows and the guide rows as in uhla_forward.  The mask
 * of uhla_forward_masked (radius, guide_mode) is extended by the plain joint-attention
 * reading: a text query attends to every key, and every query attends to every text key.
 * Text tokens sit at position (0, 0), so RoPE leaves them unrotated.  T = 0 is
 * uhla_forward_masked.  The text queries run as one extra pass over all keys, split into
 * key ranges whose partial results are merged (log-sum-exp) before the bf16 store.
 * timer: NULL, or a timer as for uhla_forward_timed (stage UHLA_STAGE_ATTN_TEXT times the
 *   text pass).
 * workspace: at least uhla_forward_text_workspace_bytes(...) bytes (0 on invalid
 *   arguments).
 * Errors: as uhla_forward_masked, plus UHLA_ERR_ARG for T < 0 and UHLA_ERR_UNSUPPORTED for
 * T > 2^24.
 */
size_t uhla_forward_text_workspace_bytes(int B, int T, int H, int W, int w, int H_lr,
                                         int W_lr, int rho, int heads, int head_dim, int radius,
                                         int guide_mode);
int uhla_forward_text(const void* q, const void* k, const void* v, void* o,
                      int B, int T, int H, int W, int w, int H_lr, int W_lr, int rho,
                      int heads, int head_dim, float scale, float theta,
                      int radius, int guide_mode,
                      void* workspace, size_t workspace_bytes, void* stream,
                      uhla_timer* timer);

/*
 * Training support ([UltraGen/it §2], [UltraGen/ar §2.C]: the guide path is fine-tuned with
 * LoRA, which needs the attention's gradients).
 *
 * uhla_forward_lse: uhla_forward_text (T = 0: uhla_forward_masked) that also writes lse,
 *   fp32 [B, heads, T + N + M] in the same row order as O: the natural log of each row's
 *   sum of exp(scale * q.k) over the keys the row sees.  Errors: as uhla_forward_text, plus
 *   UHLA_ERR_ARG for a null or misaligned lse or one overlapping O, Q, K, V or the
 *   workspace.
 *
 * uhla_backward: gradients dQ, dK, dV (bf16, layout of Q) of O = uhla_forward_text(Q, K,
 *   V; T, radius, guide_mode) (T = 0: uhla_forward_masked) for the output gradient dO,
 *   given O and the lse written by uhla_forward_lse for the same inputs.  Q, K, V, O, dO:
 *   bf16 [B, T + N + M, heads, head_dim], text rows first.  Per (batch, head), with rotated
 *   Q~, K~ and P = exp(scale Q~ K~^T - lse) on the allowed pairs: dV = P^T dO,
 *   dS = P (dO V^T - D), D = rowsum(dO O), dQ~ = scale dS K~, dK~ = scale dS^T Q~, and dQ,
 *   dK rotate dQ~, dK~ back (the transpose of RoPE).  Computed as the forward: bf16 MFMA,
 *   fp32 accumulation, P and dS rounded to bf16 for their products.  Deterministic (no
 *   atomics).
 *   workspace: at least uhla_backward_workspace_bytes(...) bytes, 256-byte aligned.
 *   Errors: UHLA_ERR_ARG (null or misaligned pointers, sizes < 1, T < 0, w not dividing H
 *   or W, radius < 0, guide_mode outside 0..2, gradients overlapping an input, lse, the
 *   workspace or each other, the workspace overlapping an input or lse); UHLA_ERR_UNSUPPORTED (head_dim not in {64, 128}, w as in
 *   uhla_forward, more than 1024 key tiles per window or, in guide modes 1 and 2, more
 *   than 1024 tiles in a window's or a cell-block group's tile list, T > 2^24);
 *   UHLA_ERR_WORKSPACE; UHLA_ERR_HIP.
 */
int uhla_forward_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int T, int H, int W, int w, int H_lr, int W_lr, int rho,
                     int heads, int head_dim, float scale, float theta, int radius,
                     int guide_mode, void* workspace, size_t workspace_bytes, void* stream);
size_t uhla_backward_workspace_bytes(int B, int T, int H, int W, int w, int H_lr, int W_lr,
                                     int rho, int heads, int head_dim, int radius,
                                     int guide_mode);
int uhla_backward(const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, void* dq, void* dk, void* dv,
                  int B, int T, int H, int W, int w, int H_lr, int W_lr, int rho, int heads,
                  int head_dim, float scale, float theta, int radius, int guide_mode,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* uhla_strerror(int status);

/* Detail of the last UHLA_ERR_HIP / argument error on the calling thread ("" if none). */
const char* uhla_last_error_detail(void);

/*
 * Stage timing with HIP events (measurement only).
 *
 * uhla_forward_timed runs exactly uhla_forward (uhla_forward_masked_timed exactly
 * uhla_forward_masked) and records a start/stop event pair on
 * `stream` around each stage; a timer holds pairs for up to max_calls calls.
 * uhla_timer_read waits for the recorded events and writes, for each stage s <
 * n_stages, the summed milliseconds over the recorded calls into stage_ms[s], and the
 * number of recorded calls into *calls.  Stages are enumerated by uhla_stage.
 * uhla_timer_reset forgets recorded calls.  A call beyond max_calls is not timed.
 * uhla_timer_destroy frees the timer and all its events (NULL: no-op); it returns
 * UHLA_ERR_HIP if destroying an event failed, the timer being freed all the same.
 */
typedef enum {
  UHLA_STAGE_TABLES = 0,    /* RoPE cos/sin table */
  UHLA_STAGE_PREP_HI = 1,   /* window-first permutation of K, V fused with RoPE on K */
  UHLA_STAGE_PREP_LR = 2,   /* guide-token RoPE / V re-layout */
  UHLA_STAGE_ATTN_HI = 3,   /* hi-res block-sparse attention */
  UHLA_STAGE_ATTN_LR = 4,   /* guide-only attention */
  UHLA_STAGE_UNPERMUTE = 5, /* inverse permutation of O (fused into the hi pass: empty) */
  UHLA_STAGE_ATTN_TEXT = 6, /* text queries over all keys (uhla_forward_text), merge */
  UHLA_NUM_STAGES = 7
} uhla_stage;

int uhla_timer_create(int max_calls, uhla_timer** out);
int uhla_timer_destroy(uhla_timer* timer);
int uhla_timer_reset(uhla_timer* timer);
int uhla_timer_read(uhla_timer* timer, double* stage_ms, int n_stages, int* calls);
int uhla_forward_timed(const void* q, const void* k, const void* v, void* o,
                       int B, int H, int W, int w, int H_lr, int W_lr, int rho,
                       int heads, int head_dim, float scale, float theta,
                       void* workspace, size_t workspace_bytes, void* stream,
                       uhla_timer* timer);
/* uhla_forward_masked with the same stage timing. */
int uhla_forward_masked_timed(const void* q, const void* k, const void* v, void* o,
                              int B, int H, int W, int w, int H_lr, int W_lr, int rho,
                              int heads, int head_dim, float scale, float theta,
                              int radius, int guide_mode,
                              void* workspace, size_t workspace_bytes, void* stream,
                              uhla_timer* timer);

/*
 * uhla_forward with RoPE on K fused into the K tile loads instead of applied once by the
 * prep pass (the alternative design, kept to measure against): the prep pass only
 * permutes K, and every attention workgroup rotates each K tile in LDS after it lands,
 * in fp32 from the hardware sin/cos of the key's position (2D axial RoPE, guide positions
 * scaled by rho, [UltraGen/ar §2.B]) with one rounding to bf16.  Same arguments,
 * layouts, workspace (uhla_forward_workspace_bytes) and errors as uhla_forward, plus
 * UHLA_ERR_UNSUPPORTED for windows of fewer than 256 tokens.  The result equals
 * uhla_forward's up to the rounding of rotated K (not bit for bit).  timer may be NULL;
 * otherwise stages are recorded as in uhla_forward_timed.
 */
int uhla_forward_rope_at_load(const void* q, const void* k, const void* v, void* o,
                              int B, int H, int W, int w, int H_lr, int W_lr, int rho,
                              int heads, int head_dim, float scale, float theta,
                              void* workspace, size_t workspace_bytes, void* stream,
                              uhla_timer* timer);

/*
 * Permute-free forward: the result of uhla_forward without the window-first copies of K
 * and V.  The window-first order exists to make every attention block one spatial window
 * ([UltraGen/it §2], [UltraGen/fr §2.A]); here the attention kernels copy each 64-key tile
 * straight from the caller's raster K and V (a tile of a w-wide window is 64 / w window
 * rows, or a 64-token piece of one row when w > 64; a guide tile is 64 consecutive guide
 * tokens), rotate the K tile in LDS as uhla_forward_rope_at_load does, and read the V^T
 * operand transposed from the row-major V tile.  Q and O stay in raster order as in
 * uhla_forward.  Same arguments, layouts and errors as uhla_forward, plus
 * UHLA_ERR_UNSUPPORTED for a window size other than 16, 32, 64 or a multiple of 64, or for
 * rows too long for 32-bit offsets within a tile (the tokens a tile spans in the raster
 * tensor, (64 / w) * W for w <= 64 and 64 for w > 64, times heads * head_dim * 2 bytes,
 * reaching 2^31).
 * workspace: at least uhla_forward_permute_free_workspace_bytes(...) bytes (the fp64 RoPE
 * table only; 0 on invalid sizes), 256-byte aligned.  The result equals uhla_forward's up to
 * the rounding of rotated K (not bit for bit).  timer may be NULL; otherwise stages are
 * recorded as in uhla_forward_timed (the prep and unpermute stages stay empty).
 */
size_t uhla_forward_permute_free_workspace_bytes(int B, int H, int W, int w, int H_lr,
                                                 int W_lr, int rho, int heads, int head_dim);
int uhla_forward_permute_free(const void* q, const void* k, const void* v, void* o,
                              int B, int H, int W, int w, int H_lr, int W_lr, int rho,
                              int heads, int head_dim, float scale, float theta,
                              void* workspace, size_t workspace_bytes, void* stream,
                              uhla_timer* timer);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): uhla_forward without a workspace
 * argument.  Its scratch memory is a 64 MiB (67108864-byte) array in the library's device
 * code, one per GPU, held until the process ends; the call allocates nothing and calls no
 * allocating routine.  The first call on a device looks up that device's array with the
 * device current (the stream must belong to the current device).  Every call on one GPU
 * shares its array and rewrites what it reads of it, so calls in stream order are
 * independent, but calls that overlap on one GPU (other streams or host threads) race.
 * Same arguments (without workspace), result (bit for bit) and errors as uhla_forward,
 * plus UHLA_ERR_WORKSPACE when uhla_forward_workspace_bytes(...) of the problem exceeds
 * 64 MiB.
 */
int uhla_forward_noalloc(const void* q, const void* k, const void* v, void* o,
                         int B, int H, int W, int w, int H_lr, int W_lr, int rho,
                         int heads, int head_dim, float scale, float theta, void* stream);

/*
 * Measurement aid: copies `bytes` bytes from src to dst (device memory, 16-byte aligned,
 * not overlapping) through one of the global-memory load paths the library's kernels use,
 * so that memory-traffic counters can be read against a known byte count per path:
 *   mode 0: plain 16-byte vector loads and stores;
 *   mode 1: nontemporal 16-byte loads and stores (the path of uhla_window_permute);
 *   mode 2: 16-byte loads straight into LDS (global_load_lds_dwordx4, the path the
 *           attention kernels stage their K and V tiles with), then LDS reads and plain
 *           stores.
 * The copy is bit-exact.  Errors: UHLA_ERR_ARG for null or misaligned pointers, bytes not a
 * positive multiple of 16384, mode outside 0..2, overlapping buffers;
 * UHLA_ERR_UNSUPPORTED above 2^31 blocks of 16384 bytes; UHLA_ERR_HIP.
 */
int uhla_copy_probe(const void* src, void* dst, int64_t bytes, int mode, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* UHLA_H_ */
