/*
 * bsattn -- block-sparse softmax self-attention over video tokens, for
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The problem (LVSA page, "Meccanismo Core"; CalibAtt page, "A. Fase di
 * Calibrazione" and "B. Fase di Inferenza"): Q, K, V of shape [B, H, N, d]
 * hold the tokens of a video latent of T frames on a grid_h x grid_w grid,
 * flattened frame-major (token n = f*P + y*grid_w + x, P = grid_h*grid_w,
 * N = T*P).  The attention matrix is cut into square tiles of `tile` tokens;
 * a tile mask says which key tiles each query tile reads, and only those
 * tiles are computed.  The output O has the shape of Q.
 *
 * Pipeline: bsattn_build_mask -> bsattn_compact -> bsattn_fwd (or
 * bsattn_fwd_plan once per list set, then bsattn_fwd_planned).  A static mask
 * can instead be calibrated: bsattn_block_energy -> bsattn_select_blocks ->
 * bsattn_aggregate_masks, then bsattn_compact -> bsattn_fwd.
 *
 * Conventions shared by every call:
 *   - Every pointer argument named "device" is device memory on the current
 *     HIP device, owned by the caller.  The library never allocates, frees or
 *     copies caller memory and never synchronises.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued asynchronously; results are valid in stream order.
 *   - Every call validates its arguments on the host first.  On error it
 *     enqueues nothing and returns a negative bsattn_status; the detail is
 *     available from bsattn_last_error() (per thread).
 *   - Results are deterministic: repeated calls on the same inputs give
 *     bitwise-identical outputs.
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSATTN_API __attribute__((visibility("default")))

typedef enum {
  BSATTN_OK = 0,
  BSATTN_ERR_INVALID_ARG = -1, /* null pointer, inconsistent sizes, Hm not in {1,H} */
  BSATTN_ERR_UNSUPPORTED = -2, /* head dim, tile or dtype outside the built set */
  BSATTN_ERR_HIP = -3          /* the HIP runtime rejected a launch */
} bsattn_status;

typedef enum { BSATTN_DTYPE_BF16 = 0, BSATTN_DTYPE_F32 = 1 } bsattn_dtype;

typedef enum {
  BSATTN_MASK_WINDOW_ANCHOR = 0, /* LVSA local window + rotating global anchors */
  BSATTN_MASK_STATIC_RANDOM = 1, /* seeded stand-in for a calibrated static mask */
  BSATTN_MASK_DENSE = 2,         /* all tiles active (full attention) */
  BSATTN_MASK_WINDOW_ANCHOR_EXPANDED = 3, /* LVSA window grown to a frame budget + anchors */
  BSATTN_MASK_BLOCK_DIAGONAL = 4,         /* SQuad passes: square blocks of block_tiles tiles */
  BSATTN_MASK_DENSE_ROWS = 5,             /* query tiles < query_tiles dense, the rest empty */
  BSATTN_MASK_DENSE_ROWS_SPREAD = 6       /* query_tiles dense tiles in blocks spread evenly */
} bsattn_mask_kind;

/* Token geometry of the video latent.  N = frames*grid_h*grid_w; the number
 * of query tiles and of key tiles is Tq = Tk = ceil(N / tile). */
typedef struct {
  int32_t frames; /* T >= 1 */
  int32_t grid_h; /* >= 1 */
  int32_t grid_w; /* >= 1 */
  int32_t tile;   /* BT, in tokens, >= 1 (bsattn_fwd supports 64 and 128) */
} bsattn_layout;

/* Mask parameters; fields a mode does not use are ignored.
 *
 * WINDOW_ANCHOR (LVSA page, "Meccanismo Core"): query frame t attends to
 *   A(t) = G u W(t), W(t) = {f in [0,T) : |f - t| <= window} and
 *   G = {(r + floor(k*T/num_anchors)) mod T : 0 <= k < num_anchors}, with
 *   r = rotation reduced mod T (the caller picks r per denoising step and
 *   layer; the page shifts the anchors with the step).  Tile pair (i, j) is
 *   active when some frame covered by query tile i attends to some frame
 *   covered by key tile j.  All mask_heads slices are identical.
 * WINDOW_ANCHOR_EXPANDED (LVSA page, "Meccanismo Core", expanded adaptive
 *   windows): as WINDOW_ANCHOR, but each query frame's window grows until
 *   |G u W(t)| >= min(budget, T).  Growth starts from the plain window and
 *   adds the nearest frame not yet in it, the earlier of two equally near
 *   frames first and never a frame outside [0, T); an anchor frame it reaches
 *   adds nothing to the count.  W(t) stays one run of frames around t, and
 *   budget = num_anchors + 2*window + 1 makes up exactly for the frames the
 *   window shares with G and for the clipped window at the video's ends.
 *   A budget no larger than |G u W(t)| leaves the window as it is.
 * STATIC_RANDOM (CalibAtt page, "B. Fase di Inferenza": a precomputed,
 *   deterministic per-head block list): cell c = (h*Tq + i)*Tk + j is active
 *   when the top 24 bits of the (c+1)-th SplitMix64 output for `seed` are
 *   below thresh24 (thresh24 = floor(p * 2^24) for density p), or when i == j
 *   and force_diagonal != 0.
 * DENSE: every cell active.
 * BLOCK_DIAGONAL (SQuad page, "1. Operatore di Attenzione SQuad": each pass
 *   is softmax attention inside disjoint groups of tokens): cell (i, j) is
 *   active when i / block_tiles == j / block_tiles (integer division), so
 *   runs of block_tiles * tile consecutive tokens attend only among
 *   themselves.  The frame layout is irrelevant to this mode.
 * DENSE_ROWS (CalibAtt page, "B. Fase di Inferenza": a repetitive head
 *   computes its anchor rows only): query tiles i < query_tiles read every
 *   key tile, the others none, for anchor rows packed at the front of Q
 *   (bsattn_anchor_rows with block_rows = 0).
 * DENSE_ROWS_SPREAD (same passage): the Ta = query_tiles dense query tiles
 *   come in Rg = ceil(Ta / block_tiles) blocks of block_tiles tiles, the
 *   last one holding the Ta - (Rg - 1) * block_tiles left over; of the
 *   Pg = ceil(Tq / block_tiles) block slots, block g takes slot
 *   floor(g * Pg / Rg), i.e. query tiles from floor(g * Pg / Rg) *
 *   block_tiles on.  Those tiles read every key tile, all others none.
 *   Rg <= Pg is required.  This is the layout bsattn_anchor_rows writes with
 *   block_rows = block_tiles * tile; the dense tiles then spread evenly over
 *   each head, and bsattn_fwd's workgroups load the GPU evenly (packed at
 *   the front, half of every head's workgroups would have no work). */
typedef struct {
  int32_t kind;           /* bsattn_mask_kind */
  int32_t window;         /* w >= 0, in frames */
  int32_t num_anchors;    /* 0 <= n_a <= T */
  int32_t rotation;       /* any integer; reduced mod T */
  uint64_t seed;          /* STATIC_RANDOM */
  uint32_t thresh24;      /* STATIC_RANDOM, <= 2^24 */
  int32_t force_diagonal; /* STATIC_RANDOM */
  int32_t mask_heads;     /* Hm >= 1: number of mask slices (1 = shared by all heads) */
  int32_t budget;         /* WINDOW_ANCHOR_EXPANDED: C >= 0 frames per query frame */
  int32_t block_tiles;    /* BLOCK_DIAGONAL: b >= 1 tiles per diagonal block;
                             DENSE_ROWS_SPREAD: >= 1 tiles per block */
  int32_t query_tiles;    /* DENSE_ROWS(_SPREAD): >= 0 query tiles with every key tile */
} bsattn_mask_params;

/* Library version as MAJOR*10000 + MINOR*100 + PATCH (a library utility,
 * not a step of the method). */
BSATTN_API int bsattn_version(void);

/* Short static text for a status code (library utility). */
BSATTN_API const char* bsattn_status_string(int status);

/* Detail of the last error on the calling thread ("" if none; library
 * utility). */
BSATTN_API const char* bsattn_last_error(void);

/* Number of tiles along one side: ceil(tokens / tile); -1 on bad input (the
 * 128x128 blocks of CalibAtt page, "A. Fase di Calibrazione"). */
BSATTN_API int32_t bsattn_num_tiles(int64_t tokens, int32_t tile);

/* Build the tile mask of one of the kinds above, each defined by the passage
 * cited on it (LVSA page, "Meccanismo Core"; CalibAtt page, "B. Fase di
 * Inferenza"; SQuad page, "1. Operatore di Attenzione SQuad").
 *   layout, params: host structs (read during the call only).
 *   mask: device uint8 [Hm, Tq, Tk], row-major, Hm = params->mask_heads;
 *         every byte is written (0 or 1).
 * Errors: INVALID_ARG on null pointers, non-positive sizes, window < 0,
 * num_anchors outside [0, T], budget < 0 (expanded mode), block_tiles < 1
 * (block-diagonal and spread dense-rows modes), query_tiles < 0 (dense-rows
 * modes), spread blocks that do not fit (Rg > Pg), thresh24 > 2^24,
 * mask_heads < 1, an unknown kind, or Hm*Tq*Tk >= 2^31. */
BSATTN_API int bsattn_build_mask(const bsattn_layout* layout,
                                 const bsattn_mask_params* params,
                                 uint8_t* mask, void* stream);

/* Turn a tile mask into per-query-tile lists of active key tiles (CSR over
 * the mask viewed as a [rows, Tk] matrix, rows = Hm*Tq, row r = h*Tq + i).
 *   mask:    device uint8 [rows, Tk]; any nonzero byte counts as active.
 *   row_ptr: device int32 [rows + 1]; row_ptr[0] = 0, row_ptr[r+1] =
 *            row_ptr[r] + (active tiles of row r); row_ptr[rows] = nnz.
 *   col_idx: device int32, capacity >= nnz (rows*Tk always suffices);
 *            entries row_ptr[r] .. row_ptr[r+1]-1 hold row r's active key
 *            tiles in ascending order.
 * CalibAtt page, "B. Fase di Inferenza" (precomputed block lists); the list
 * stores the active tiles, the complement of the page's skip list.
 * Errors: INVALID_ARG on null pointers, rows < 0, Tk < 0, rows*Tk >= 2^31. */
BSATTN_API int bsattn_compact(int32_t rows, int32_t Tk, const uint8_t* mask,
                              int32_t* row_ptr, int32_t* col_idx, void* stream);

/* Block-sparse attention forward: softmax attention of every query row over
 * the keys of its query tile's active key tiles only (CalibAtt page, "B. Fase
 * di Inferenza": only the selected 128x128 blocks are computed; LVSA page,
 * "Meccanismo Core": each query attends to its frame set A(t)).
 *   q, k, v: device [B, H, N, d] contiguous, element type `dtype`
 *            (BF16 or F32; F32 inputs are rounded to bf16 for the matrix
 *            products, which accumulate in fp32).
 *   o:       device [B, H, N, d] of the same dtype (written).
 *   lse:     device float [B, H, N] or NULL; natural-log sum of exp of the
 *            scaled scores over the active keys (-inf for a row with none).
 *   mask_heads: Hm, 1 or H; head h reads CSR slice (Hm == H ? h : 0).  All
 *            batch entries share the CSR.
 *   row_ptr, col_idx: device CSR from bsattn_compact for rows = Hm*Tq,
 *            Tk = Tq = ceil(N/tile).  Key-tile indices outside [0, Tk) are
 *            skipped; row_ptr values are read as written by bsattn_compact.
 *   scale:   softmax scale; <= 0 selects 1/sqrt(d).
 * For each query row n: O[n] = softmax(scale * q_n K_A^T) V_A over the keys A
 * of its active tiles (keys >= N never enter); O[n] = 0 when A is empty.
 * Supported: d in {64, 128}, tile in {64, 128}.  B*H*N == 0 is a no-op.
 * Errors: INVALID_ARG (null pointers, negative sizes, Hm not in {1, H},
 * B*H*N*d >= 2^31 elements per tensor), UNSUPPORTED (d, tile, dtype),
 * HIP (launch failure). */
BSATTN_API int bsattn_fwd(int32_t B, int32_t H, int32_t N, int32_t d,
                          int32_t tile, int32_t dtype, const void* q,
                          const void* k, const void* v, void* o, float* lse,
                          int32_t mask_heads, const int32_t* row_ptr,
                          const int32_t* col_idx, float scale, void* stream);

/* The forward on the grouped view of the tokens: SQuad's global pass
 * (SQuad page, "1. Operatore di Attenzione SQuad": the tokens at the same
 * position inside every window of w tokens attend to one another).  With
 * G = N / window, position-major index p = r * G + c (window c, position r)
 * stands for buffer row n(p) = c * window + r.  The call computes, for every
 * p, O[n(p)] = softmax(scale * q[n(p)] K^T) V over the keys n(p') whose
 * position-major tiles p' / 128 are active for tile p / 128 in the CSR,
 * which therefore describes the position-major order (for SQuad's global
 * pass: a block-diagonal mask of G / 128 tiles per block).  It equals
 * bsattn_window_reorder of q, k and v, then bsattn_fwd, then the inverse
 * reorder of o (and lse), bit for bit, without the reorders' traffic.
 * Arguments as bsattn_fwd, plus window (w >= 1).  Supported: bf16, d = 128,
 * tile = 128, N a multiple of w with G a multiple of 128.
 * Errors: as bsattn_fwd; UNSUPPORTED for other dtypes or sizes, INVALID_ARG
 * for window < 1 or N not of that form. */
BSATTN_API int bsattn_fwd_grouped(int32_t B, int32_t H, int32_t N, int32_t d, int32_t tile,
                                  int32_t dtype, const void* q, const void* k, const void* v,
                                  void* o, float* lse, int32_t mask_heads,
                                  const int32_t* row_ptr, const int32_t* col_idx,
                                  int32_t window, float scale, void* stream);

/* ---- Planned forward.  The active lists are fixed inputs of the forward
 * (CalibAtt page, "B. Fase di Inferenza": inference follows per-block lists
 * worked out beforehand, with no decision left to the attention kernel), so
 * the work schedule is worked out once per list set too: which query-tile
 * pairs each worker (one persistent workgroup per compute unit) computes, in
 * which order, and every pair's merged key-tile list.  The planned forward
 * then moves from one pair to the next without draining its pipeline, the
 * per-workgroup set-up of bsattn_fwd gone.  A pair whose two lists largely
 * coincide is computed as bsattn_fwd computes it (bitwise-identical O and
 * LSE); a pair that bsattn_fwd splits (5 I < n0 + n1, I common key tiles of
 * lists of n0 and n1 entries, or an empty list) becomes two single tiles,
 * each walked by one group of waves over its own list, item after item:
 * the same softmax arithmetic as a tile in pair mode, different from
 * bsattn_fwd's split mode only by rounding (both within the output bar).
 *
 * Supported: bf16, d = 128, tile = 128, Tq <= 4096, B*H <= 65535.  Workers
 * is a multiple of 8 in [8, 512] (worker w is taken to run on XCD w % 8);
 * 0 selects the current device's compute units (256 on MI355X). */

/* Bytes of a plan buffer (the plan of bsattn_fwd_plan, for block lists fixed
 * before inference: CalibAtt page, "B. Fase di Inferenza") for these sizes:
 * a fixed part, plus 8 bytes per
 * step; the steps number at most the smaller of B * (H / mask_heads) *
 * (nnz_bound + mask_heads * ceil(Tq / 2)) and B * H * ceil(Tq / 2) * Tk,
 * nnz_bound an upper bound on the CSR's entries (< 0 or above
 * mask_heads*Tq*Tk selects mask_heads*Tq*Tk).  Returns the size (> 0), or a
 * negative bsattn_status (sizes as for bsattn_fwd_plan). */
BSATTN_API int64_t bsattn_fwd_plan_bytes(int32_t B, int32_t H, int32_t N, int32_t tile,
                                         int32_t mask_heads, int64_t nnz_bound,
                                         int32_t workers);

/* Build the plan of a CSR (CalibAtt page, "B. Fase di Inferenza": the block
 * lists are fixed before inference, so the forward's scheduling can be
 * worked out once per list set) (as written by bsattn_compact for rows =
 * mask_heads*Tq, Tk = Tq = ceil(N / tile)) into `plan`: device memory of
 * plan_bytes bytes, 16-byte aligned, owned by the caller; its contents are
 * the library's own (three launches on `stream`).  Key-tile indices outside
 * [0, Tk) are left out; entries beyond the plan's step capacity (a
 * plan_bytes below what bsattn_fwd_plan_bytes gives for the CSR's entry
 * count) are dropped, and the forward then misses them.  The plan stays
 * valid as long as the CSR does not change.  How the work is shared out
 * follows the speeds of the GPU's eight XCDs as the last planned forward on
 * the current device measured them (a small table of the library's, one
 * per GPU): ranges of work go to the XCDs in proportion to their measured
 * speeds, or evenly before any planned forward has run.  That moves work
 * between compute units only: the outputs never depend on it.
 * Errors: INVALID_ARG (sizes, mask_heads not in {1, H}, null or unaligned
 * pointers, plan_bytes below the fixed part, bad workers), UNSUPPORTED
 * (tile, Tq, B*H), HIP.  B*H*N == 0 is a no-op. */
BSATTN_API int bsattn_fwd_plan(int32_t B, int32_t H, int32_t N, int32_t tile,
                               int32_t mask_heads, const int32_t* row_ptr,
                               const int32_t* col_idx, int32_t workers, void* plan,
                               int64_t plan_bytes, void* stream);

/* The forward through a plan: the attention bsattn_fwd computes (CalibAtt
 * page, "B. Fase di Inferenza"; LVSA page, "Meccanismo Core"), with
 * arguments as bsattn_fwd, plus the plan buffer
 * (plan, plan_bytes and workers as given to bsattn_fwd_plan, whose CSR must
 * be row_ptr / col_idx) and window: 0 for contiguous tokens, w > 0 for the
 * grouped view of bsattn_fwd_grouped.  Launches `workers` workgroups.  The
 * kernel checks the plan's header (B, H, N, Tq, mask_heads, workers); a
 * plan built for other sizes makes it return without writing O or LSE.  The
 * plan is only read; each workgroup also records how long it ran, with its
 * share of the work, in the library's per-GPU table that the next
 * bsattn_fwd_plan on the device reads (calls racing on one GPU write the
 * same entries; either record serves).
 * Errors: as bsattn_fwd and bsattn_fwd_plan; UNSUPPORTED for other dtypes,
 * head dims or tiles; INVALID_ARG for window < 0 or N not of the grouped
 * form. */
BSATTN_API int bsattn_fwd_planned(int32_t B, int32_t H, int32_t N, int32_t d, int32_t tile,
                                  int32_t dtype, const void* q, const void* k, const void* v,
                                  void* o, float* lse, int32_t mask_heads,
                                  const int32_t* row_ptr, const int32_t* col_idx,
                                  const void* plan, int64_t plan_bytes, int32_t workers,
                                  int32_t window, float scale, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * forward of bsattn_fwd, with its arguments.  For bf16, d = 128, tile = 128
 * (Tq <= 4096, B*H <= 65535) it plans the lists (bsattn_fwd_plan, three
 * launches) into a static device array of the library's own and runs
 * bsattn_fwd_planned from it (the same output, bit for bit, as those two
 * calls with a buffer of the caller's); every other supported shape runs
 * bsattn_fwd's kernels, which need no memory beyond the arguments.  It
 * calls no allocator.  The array holds 96 MiB per GPU, kept until the
 * process ends (the worst-case plan for B = 1, H = 12, 131 072 tokens needs
 * about 68 MiB); a plan larger than that is rejected with INVALID_ARG
 * before anything is enqueued.  Every call on a GPU shares that GPU's
 * array: calls that overlap in time on one GPU (on different streams) race,
 * so order them on one stream.  Errors: as bsattn_fwd; INVALID_ARG for a
 * plan above the array's size; HIP. */
BSATTN_API int bsattn_fwd_noalloc(int32_t B, int32_t H, int32_t N, int32_t d, int32_t tile,
                                  int32_t dtype, const void* q, const void* k, const void* v,
                                  void* o, float* lse, int32_t mask_heads,
                                  const int32_t* row_ptr, const int32_t* col_idx, float scale,
                                  void* stream);

/* Reorder token rows between window-major and position-major order (SQuad
 * page, "1. Operatore di Attenzione SQuad": the global pass groups the
 * tokens at the same position inside every window).  With G = N / w:
 *   inverse == 0:  dst[b, h, r*G + a, :] = src[b, h, a*w + r, :]
 *   inverse != 0:  dst[b, h, a*w + r, :] = src[b, h, r*G + a, :]
 * for a < G, r < w.  After the forward reorder, each position group is a
 * contiguous run of G tokens, so the global pass is a BLOCK_DIAGONAL mask
 * with G / tile tiles per block.
 *   src, dst: device [B, H, N, d] contiguous, element type `dtype`, distinct
 *             buffers (dst written; src read only).
 * Errors: INVALID_ARG (null or equal pointers, negative sizes, w < 1, N not
 * a multiple of w, unaligned buffers, B*H*N*d >= 2^40), UNSUPPORTED (dtype),
 * HIP.  B*H*N == 0 is a no-op. */
BSATTN_API int bsattn_window_reorder(int32_t B, int32_t H, int32_t N, int32_t d, int32_t w,
                                     int32_t dtype, const void* src, void* dst, int32_t inverse,
                                     void* stream);

/* ---- Spatial repetition (CalibAtt page, "A. Fase di Calibrazione" step 3
 * and "B. Fase di Inferenza").  In a repetitive head the spatial rows of a
 * frame attend alike: attention is computed for the anchor rows only (every
 * stride-th latent row, y = 0, s, 2s, ...) and copied to the rows between.
 * Tokens are frame-major, n = f*P + y*grid_w + x, N = T*grid_h*grid_w; row
 * y copies from its anchor a(y) = s*floor(y/s). */

/* Row similarity (CalibAtt page, "A. Fase di Calibrazione", step 3):
 *   cos[b, h, f, y] = sum_x <p_(y,x), p_(a,x)> /
 *                     sqrt(sum_x |p_(y,x)|^2 * sum_x |p_(a,x)|^2),
 * p_n the full-attention softmax probabilities of query n over all N keys
 * (scale <= 0 selects 1/sqrt(d)); anchor rows get 1.
 *   q, k: device [B, H, N, d], dtype BF16 (or F32 rounded to bf16).
 *   cos:  device float [B, H, T, grid_h], written.
 *   workspace: null, or device memory of at least
 *              bsattn_row_cosines_workspace_bytes(...) bytes, 4-byte
 *              aligned, owned by the caller and overwritten.  With bf16 and
 *              d = 128 it lets the kernel pack the columns of all rows into
 *              full waves (per-column sums go there, a second kernel adds
 *              them per row); otherwise, or when null, it is not used.
 * Supported: d in {64, 128}, grid_w <= 256.  B*H*T == 0 is a no-op.
 * Errors: INVALID_ARG (null pointers, sizes, B or H > 65535, unaligned q or
 * k, non-finite scale, workspace_bytes below the size asked for),
 * UNSUPPORTED (d, dtype, grid_w), HIP. */
BSATTN_API int bsattn_row_cosines(int32_t B, int32_t H, int32_t T, int32_t grid_h,
                                  int32_t grid_w, int32_t d, int32_t stride, int32_t dtype,
                                  const void* q, const void* k, float* cos, float scale,
                                  void* workspace, int64_t workspace_bytes, void* stream);

/* Bytes of the workspace bsattn_row_cosines packs with (row similarity:
 * CalibAtt page, "A. Fase di Calibrazione", step 3): 12 * B * H * T *
 * (non-anchor rows per frame) * grid_w; 0 when there is no non-anchor row.
 * Negative on invalid sizes (B, H, T < 0, grid_h, grid_w, stride < 1). */
BSATTN_API int64_t bsattn_row_cosines_workspace_bytes(int32_t B, int32_t H, int32_t T,
                                                      int32_t grid_h, int32_t grid_w,
                                                      int32_t stride);

/* Repetitive heads (CalibAtt page, "A. Fase di Calibrazione", step 3):
 * flags[h] = 1 when the mean of cos over the
 * prompts b, frames f and non-anchor rows y (float64, summed in that
 * order) is >= gamma, or when no row is a non-anchor row.
 *   cos:   device float [B, H, T, grid_h] (as written by bsattn_row_cosines).
 *   flags: device uint8 [H], written.
 * Errors: INVALID_ARG (negative sizes, grid_h or stride < 1, null pointers,
 * non-finite gamma), HIP. */
BSATTN_API int bsattn_repetitive_heads(int32_t B, int32_t H, int32_t T, int32_t grid_h,
                                       int32_t stride, const float* cos, double gamma,
                                       uint8_t* flags, void* stream);

/* Anchor-row gather and broadcast (CalibAtt page, "B. Fase di Inferenza": a
 * repetitive head computes its anchor rows and copies them to the rows
 * between), on [B, H, N, d] buffers.
 * The anchor rows' tokens, frame by frame, row by row, have packed indices
 * a = 0 .. Na-1 (Na = T * ceil(grid_h/stride) * grid_w); packed index a is
 * stored at buffer row a when block_rows == 0, else at row
 *   floor(g * Pg / Rg) * block_rows + (a mod block_rows),
 *   g = a / block_rows, Rg = ceil(Na / block_rows), Pg = ceil(N / block_rows)
 * (blocks of block_rows rows spread evenly; every such row lies below N).
 *   broadcast == 0: the anchor tokens are written to their buffer rows of
 *                   dst; the other rows of dst are not written.
 *   broadcast != 0: every row n of dst receives the src buffer row of n's
 *                   anchor-row token.
 * With the gathered Q, a DENSE_ROWS mask of ceil(Na/tile) query tiles (or,
 * for block_rows = b * tile, a DENSE_ROWS_SPREAD mask with block_tiles = b),
 * bsattn_fwd, then the broadcast of its output, a repetitive head costs
 * about Na/N of full attention.
 *   src, dst: distinct device buffers, element type `dtype`, 16-byte aligned,
 *             rows of d elements a multiple of 16 bytes (any such d).
 * Errors: INVALID_ARG (null or aliased buffers, sizes, row length,
 * block_rows < 0), UNSUPPORTED (dtype), HIP. */
BSATTN_API int bsattn_anchor_rows(int32_t B, int32_t H, int32_t T, int32_t grid_h,
                                  int32_t grid_w, int32_t d, int32_t stride, int32_t dtype,
                                  const void* src, void* dst, int32_t broadcast,
                                  int32_t block_rows, void* stream);

/* As bsattn_anchor_rows, head by head (CalibAtt page, "B. Fase di
 * Inferenza": in one layer the repetitive heads compute their anchor rows
 * and copy them, the other heads follow their block lists): heads with
 * flags[h] != 0 are gathered (broadcast == 0) or broadcast as
 * bsattn_anchor_rows does; heads with flags[h] == 0 are copied row for row
 * (dst row n = src row n, every row).  In a gathered head the rows that do
 * not hold an anchor token are not written.
 *   flags: device uint8 [H] (as written by bsattn_repetitive_heads).
 * Other arguments and errors as bsattn_anchor_rows; INVALID_ARG for null
 * flags. */
BSATTN_API int bsattn_anchor_rows_heads(int32_t B, int32_t H, int32_t T, int32_t grid_h,
                                        int32_t grid_w, int32_t d, int32_t stride,
                                        int32_t dtype, const void* src, void* dst,
                                        int32_t broadcast, int32_t block_rows,
                                        const uint8_t* flags, void* stream);

/* Per-head choice between two tile masks (CalibAtt page, "B. Fase di
 * Inferenza": in its inference layer the repetitive heads take the
 * anchor-row mask, the others their calibrated block lists):
 *   out[h] = flags[h] != 0 ? set_mask[set_heads == 1 ? 0 : h]
 *                          : clear_mask[clear_heads == 1 ? 0 : h],
 * each slice uint8 [Tq, Tk].
 *   flags: device uint8 [H]; set_mask: device uint8 [set_heads, Tq, Tk];
 *   clear_mask: device uint8 [clear_heads, Tq, Tk]; out: device uint8
 *   [H, Tq, Tk], written (not aliasing the inputs).
 * Errors: INVALID_ARG (negative sizes, mask heads not in {1, H}, null
 * pointers, H*Tq*Tk >= 2^31), HIP.  H*Tq*Tk == 0 is a no-op. */
BSATTN_API int bsattn_mask_select(int32_t H, int32_t Tq, int32_t Tk, const uint8_t* flags,
                                  const uint8_t* set_mask, int32_t set_heads,
                                  const uint8_t* clear_mask, int32_t clear_heads,
                                  uint8_t* out, void* stream);

/* ---- Static-mask calibration (CalibAtt page, "A. Fase di Calibrazione").
 * The calibration runs full attention on a few prompts, measures how much
 * attention every block receives, keeps per query block the fewest key
 * blocks that carry a fraction eps of it, and keeps a block in the final
 * static mask when enough prompts agree.  The result feeds bsattn_compact and
 * bsattn_fwd like any other tile mask. */

/* Block energies of full softmax attention (CalibAtt page, "A. Fase di
 * Calibrazione", step 1):
 *   E[b, h, i, j] = sum over query rows n of tile i and key columns m of
 *   tile j of softmax_m(scale * q_n . k_m), the softmax over all N keys.
 * Each row of E sums to the number of query rows in tile i.
 *   q, k:    device [B, H, N, d] contiguous, element type `dtype` (BF16, or
 *            F32 rounded to bf16 for the products, which accumulate in fp32).
 *   energy:  device float [B, H, T, T], T = ceil(N / tile), written.
 *   scale:   softmax scale; <= 0 selects 1/sqrt(d).
 *   workspace: null, or device memory of at least
 *            bsattn_block_energy_workspace_bytes(...) bytes, 16-byte aligned,
 *            owned by the caller and overwritten.  With bf16, d = 128 and
 *            tile = 128 it lets the kernel make one sweep over the keys
 *            instead of two (every row's per-tile sums wait there until the
 *            row's normaliser is known); otherwise, or when null, it is not
 *            used.
 * The batch index plays the role of the calibration prompt.  Supported:
 * d in {64, 128}, tile in {64, 128}.  B*H*N == 0 is a no-op.
 * Errors: INVALID_ARG (null pointers, negative sizes, B or H > 65535,
 * unaligned q, k or workspace, non-finite scale, B*H*T*T >= 2^31,
 * workspace_bytes below the size asked for), UNSUPPORTED (d, tile, dtype),
 * HIP. */
BSATTN_API int bsattn_block_energy(int32_t B, int32_t H, int32_t N, int32_t d, int32_t tile,
                                   int32_t dtype, const void* q, const void* k, float* energy,
                                   float scale, void* workspace, int64_t workspace_bytes,
                                   void* stream);

/* Bytes of the workspace of bsattn_block_energy's one-sweep kernel (block
 * energies: CalibAtt page, "A. Fase di Calibrazione", step 1):
 * 1024 * min(512, B * H * ceil(T / 2)) * T for tile 128 (512 persistent
 * workgroups at most, each with 2 query tiles x 128 rows x T floats), 0 for
 * other tiles.  Negative on invalid sizes. */
BSATTN_API int64_t bsattn_block_energy_workspace_bytes(int32_t B, int32_t H, int32_t N,
                                                       int32_t tile);

/* Energy-based block selection (CalibAtt page, "A. Fase di Calibrazione",
 * step 1), one row at a time:
 *   energy: device float [rows, Tk], finite and >= 0 (as written by
 *           bsattn_block_energy, viewed as [B*H*T, T]).
 *   mask:   device uint8 [rows, Tk], written: 1 for the kept key blocks.
 * Per row the key blocks are ordered by decreasing energy (the lower index
 * first on equal energy) and the shortest prefix whose cumulative energy is
 * >= eps * (row total) is kept; the sums are float64, added one at a time in
 * that order, the total included.  eps <= 0 keeps nothing, eps > 1 keeps
 * every block.  The threshold eps(t) of the page varies with the timestep:
 * the caller passes the value for the step being calibrated.
 * Errors: INVALID_ARG (negative sizes, null pointers, non-finite eps,
 * rows*Tk >= 2^31), UNSUPPORTED (Tk > 4096), HIP. */
BSATTN_API int bsattn_select_blocks(int32_t rows, int32_t Tk, const float* energy, double eps,
                                    uint8_t* mask, void* stream);

/* Cross-prompt agreement (CalibAtt page, "A. Fase di Calibrazione", step 2):
 *   masks: device uint8 [P, cells] (P prompt masks, any nonzero = selected).
 *   out:   device uint8 [cells], written: 1 where the number of prompts that
 *          selected the cell is >= rho * P (float64), else 0.
 * Errors: INVALID_ARG (P < 1, cells < 0, null pointers, non-finite rho),
 * HIP. */
BSATTN_API int bsattn_aggregate_masks(int32_t P, int64_t cells, const uint8_t* masks, double rho,
                                      uint8_t* out, void* stream);

/* Diagnostic, not a step of any page's method: the achievable bf16
 * matrix-core rate of the device, against
 * which the forward's throughput is read (next to the vendor's dense peak).
 * Enqueues `blocks` workgroups of 512 threads that each run `iters` loop
 * trips of 16 register-only v_mfma_f32_32x32x16_bf16 per wave (four
 * independent accumulator chains); no memory is read.
 *   sink: device float [blocks], written (one value per workgroup, keeps the
 *         work from being optimised away; the values mean nothing).
 * Returns the number of floating-point operations enqueued (> 0), or a
 * negative bsattn_status: INVALID_ARG for blocks < 1, iters < 1 or a null
 * sink, HIP on a launch failure.  Time it with events on `stream`. */
BSATTN_API int64_t bsattn_mfma_ceiling(int32_t blocks, int32_t iters, float* sink,
                                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_H */
