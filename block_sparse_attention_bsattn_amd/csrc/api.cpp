// Host side of the C ABI declared in include/bsattn.h: argument validation,
// error reporting and dispatch to the kernel launchers.  Nothing is enqueued
// unless every check passes; no device memory is allocated here.
#include "bsattn.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "bsattn_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return BSATTN_OK;
}

int hip_status(int err, const char* what) {
  if (err == 0) return ok();
  return fail(BSATTN_ERR_HIP, "%s: HIP error %d", what, err);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxCells = (int64_t)1 << 31;

}  // namespace

extern "C" {

BSATTN_API int bsattn_version(void) { return 100; }

BSATTN_API const char* bsattn_status_string(int status) {
  switch (status) {
    case BSATTN_OK: return "ok";
    case BSATTN_ERR_INVALID_ARG: return "invalid argument";
    case BSATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case BSATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

BSATTN_API const char* bsattn_last_error(void) { return g_last_error.c_str(); }

BSATTN_API int32_t bsattn_num_tiles(int64_t tokens, int32_t tile) {
  if (tokens < 0 || tile <= 0) return -1;
  const int64_t t = (tokens + tile - 1) / tile;
  return t > INT32_MAX ? -1 : (int32_t)t;
}

BSATTN_API int bsattn_build_mask(const bsattn_layout* layout,
                                 const bsattn_mask_params* params,
                                 uint8_t* mask, void* stream) {
  if (!layout || !params || !mask)
    return fail(BSATTN_ERR_INVALID_ARG, "build_mask: null pointer");
  const bsattn_layout L = *layout;
  const bsattn_mask_params M = *params;
  if (L.frames < 1 || L.grid_h < 1 || L.grid_w < 1 || L.tile < 1)
    return fail(BSATTN_ERR_INVALID_ARG,
                "build_mask: frames, grid_h, grid_w and tile must be >= 1");
  const int64_t per_frame = (int64_t)L.grid_h * L.grid_w;
  const int64_t tokens = per_frame * L.frames;
  if (tokens > INT32_MAX)
    return fail(BSATTN_ERR_INVALID_ARG, "build_mask: more than 2^31-1 tokens");
  if (M.kind < BSATTN_MASK_WINDOW_ANCHOR || M.kind > BSATTN_MASK_DENSE_ROWS_SPREAD)
    return fail(BSATTN_ERR_INVALID_ARG, "build_mask: unknown mask kind %d", M.kind);
  if (M.mask_heads < 1)
    return fail(BSATTN_ERR_INVALID_ARG, "build_mask: mask_heads must be >= 1");
  const bool frame_rule = M.kind == BSATTN_MASK_WINDOW_ANCHOR ||
                          M.kind == BSATTN_MASK_WINDOW_ANCHOR_EXPANDED;
  if (frame_rule) {
    if (M.window < 0)
      return fail(BSATTN_ERR_INVALID_ARG, "build_mask: window must be >= 0");
    if (M.num_anchors < 0 || M.num_anchors > L.frames)
      return fail(BSATTN_ERR_INVALID_ARG,
                  "build_mask: num_anchors must lie in [0, frames]");
  }
  if (M.kind == BSATTN_MASK_WINDOW_ANCHOR_EXPANDED && M.budget < 0)
    return fail(BSATTN_ERR_INVALID_ARG, "build_mask: budget must be >= 0");
  if (M.kind == BSATTN_MASK_BLOCK_DIAGONAL && M.block_tiles < 1)
    return fail(BSATTN_ERR_INVALID_ARG, "build_mask: block_tiles must be >= 1");
  const bool dense_rows =
      M.kind == BSATTN_MASK_DENSE_ROWS || M.kind == BSATTN_MASK_DENSE_ROWS_SPREAD;
  if (dense_rows && M.query_tiles < 0)
    return fail(BSATTN_ERR_INVALID_ARG, "build_mask: query_tiles must be >= 0");
  if (M.kind == BSATTN_MASK_STATIC_RANDOM && M.thresh24 > (1u << 24))
    return fail(BSATTN_ERR_INVALID_ARG, "build_mask: thresh24 exceeds 2^24");
  const int32_t tiles = bsattn_num_tiles(tokens, L.tile);
  if (M.kind == BSATTN_MASK_DENSE_ROWS_SPREAD) {
    if (M.block_tiles < 1)
      return fail(BSATTN_ERR_INVALID_ARG, "build_mask: block_tiles must be >= 1");
    const int64_t rg = ((int64_t)M.query_tiles + M.block_tiles - 1) / M.block_tiles;
    const int64_t pg = ((int64_t)tiles + M.block_tiles - 1) / M.block_tiles;
    if (rg > pg)
      return fail(BSATTN_ERR_INVALID_ARG,
                  "build_mask: %d query tiles in blocks of %d do not fit %lld block slots",
                  M.query_tiles, M.block_tiles, (long long)pg);
  }
  const int64_t cells = (int64_t)M.mask_heads * tiles * tiles;
  if (cells >= kMaxCells)
    return fail(BSATTN_ERR_INVALID_ARG, "build_mask: mask has >= 2^31 cells");

  bsattn::MaskLaunch a;
  a.kind = M.kind;
  a.frames = L.frames;
  a.tokens_per_frame = (int32_t)per_frame;
  a.tokens = (int32_t)tokens;
  a.tile = L.tile;
  a.tq = tiles;
  a.tk = tiles;
  a.mask_heads = M.mask_heads;
  a.window = frame_rule ? (M.window < L.frames ? M.window : L.frames) : 0;
  a.budget = M.kind == BSATTN_MASK_WINDOW_ANCHOR_EXPANDED
                 ? (M.budget < L.frames ? M.budget : L.frames)
                 : 0;
  a.num_anchors = M.num_anchors;
  a.rotation = ((M.rotation % L.frames) + L.frames) % L.frames;
  a.block_tiles = (M.kind == BSATTN_MASK_BLOCK_DIAGONAL || M.kind == BSATTN_MASK_DENSE_ROWS_SPREAD)
                     ? M.block_tiles
                     : 1;
  a.query_tiles = dense_rows ? M.query_tiles : 0;
  a.seed = M.seed;
  a.thresh24 = M.thresh24;
  a.force_diagonal = M.force_diagonal != 0;
  return hip_status(bsattn::launch_build_mask(a, mask, stream), "build_mask");
}

BSATTN_API int bsattn_compact(int32_t rows, int32_t Tk, const uint8_t* mask,
                              int32_t* row_ptr, int32_t* col_idx, void* stream) {
  if (rows < 0 || Tk < 0)
    return fail(BSATTN_ERR_INVALID_ARG, "compact: rows and Tk must be >= 0");
  if ((int64_t)rows * Tk >= kMaxCells)
    return fail(BSATTN_ERR_INVALID_ARG, "compact: mask has >= 2^31 cells");
  if (!row_ptr) return fail(BSATTN_ERR_INVALID_ARG, "compact: null row_ptr");
  if ((int64_t)rows * Tk > 0 && (!mask || !col_idx))
    return fail(BSATTN_ERR_INVALID_ARG, "compact: null mask or col_idx");
  return hip_status(bsattn::launch_compact(rows, Tk, mask, row_ptr, col_idx, stream),
                    "compact");
}

// Validation shared by the two forward entry points; fills `a` on success.
// A no-op call (B*H*N == 0) returns OK with *noop set.
static int fwd_args(const char* who, int32_t B, int32_t H, int32_t N, int32_t d, int32_t tile,
                    int32_t dtype, const void* q, const void* k, const void* v, void* o,
                    float* lse, int32_t mask_heads, const int32_t* row_ptr,
                    const int32_t* col_idx, float scale, bsattn::FwdLaunch& a, bool* noop) {
  *noop = false;
  if (B < 0 || H < 0 || N < 0 || d < 0)
    return fail(BSATTN_ERR_INVALID_ARG, "%s: B, H, N and d must be >= 0", who);
  if (d != 64 && d != 128)
    return fail(BSATTN_ERR_UNSUPPORTED, "%s: head dim %d (supported: 64, 128)", who, d);
  if (tile != 64 && tile != 128)
    return fail(BSATTN_ERR_UNSUPPORTED, "%s: tile %d (supported: 64, 128)", who, tile);
  if (dtype != BSATTN_DTYPE_BF16 && dtype != BSATTN_DTYPE_F32)
    return fail(BSATTN_ERR_UNSUPPORTED, "%s: dtype %d", who, dtype);
  if ((int64_t)B * H * N == 0) {
    *noop = true;
    return BSATTN_OK;
  }
  if (B > 65535 || H > 65535)
    return fail(BSATTN_ERR_INVALID_ARG, "%s: B and H must be <= 65535", who);
  if (mask_heads != 1 && mask_heads != H)
    return fail(BSATTN_ERR_INVALID_ARG, "%s: mask_heads %d must be 1 or H=%d", who,
                mask_heads, H);
  if (!q || !k || !v || !o || !row_ptr || !col_idx)
    return fail(BSATTN_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(BSATTN_ERR_INVALID_ARG, "%s: q, k, v, o must be 16-byte aligned", who);
  if (!(scale == scale) || isinf(scale))
    return fail(BSATTN_ERR_INVALID_ARG, "%s: scale must be finite", who);
  const int32_t tiles = bsattn_num_tiles(N, tile);
  const int64_t cells = (int64_t)mask_heads * tiles * tiles;
  if (cells >= kMaxCells)
    return fail(BSATTN_ERR_INVALID_ARG, "%s: tile mask has >= 2^31 cells", who);
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.tile = tile;
  a.dtype = dtype;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.mask_heads = mask_heads;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.tiles = tiles;
  a.col_cap = cells;
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
  a.scale_log2 = sc * 1.4426950408889634f;
  a.window = 0;
  a.plan = nullptr;
  a.pl = bsattn::PlanLayout{};
  return BSATTN_OK;
}

BSATTN_API int bsattn_fwd(int32_t B, int32_t H, int32_t N, int32_t d,
                          int32_t tile, int32_t dtype, const void* q,
                          const void* k, const void* v, void* o, float* lse,
                          int32_t mask_heads, const int32_t* row_ptr,
                          const int32_t* col_idx, float scale, void* stream) {
  bsattn::FwdLaunch a;
  bool noop;
  const int st = fwd_args("fwd", B, H, N, d, tile, dtype, q, k, v, o, lse, mask_heads, row_ptr,
                          col_idx, scale, a, &noop);
  if (st != BSATTN_OK) return st;
  if (noop) return ok();
  return hip_status(bsattn::launch_fwd(a, stream), "fwd");
}

BSATTN_API int bsattn_fwd_grouped(int32_t B, int32_t H, int32_t N, int32_t d, int32_t tile,
                                  int32_t dtype, const void* q, const void* k, const void* v,
                                  void* o, float* lse, int32_t mask_heads,
                                  const int32_t* row_ptr, const int32_t* col_idx,
                                  int32_t window, float scale, void* stream) {
  bsattn::FwdLaunch a;
  bool noop;
  const int st = fwd_args("fwd_grouped", B, H, N, d, tile, dtype, q, k, v, o, lse, mask_heads,
                          row_ptr, col_idx, scale, a, &noop);
  if (st != BSATTN_OK) return st;
  if (d != 128 || tile != 128 || dtype != BSATTN_DTYPE_BF16)
    return fail(BSATTN_ERR_UNSUPPORTED, "fwd_grouped: bf16, d 128 and tile 128 only");
  if (window < 1)
    return fail(BSATTN_ERR_INVALID_ARG, "fwd_grouped: window must be >= 1");
  if (noop) return ok();
  if (N % window != 0 || (N / window) % 128 != 0)
    return fail(BSATTN_ERR_INVALID_ARG,
                "fwd_grouped: N=%d must be window=%d times a multiple of 128", N, window);
  if ((int64_t)N * 256 >= ((int64_t)1 << 31))
    return fail(BSATTN_ERR_INVALID_ARG, "fwd_grouped: N * 256 bytes must stay below 2^31");
  a.window = window;
  return hip_status(bsattn::launch_fwd(a, stream), "fwd_grouped");
}

// ---- planned forward

// Validation shared by the three planned calls; fills *workers (0 selects
// the device's compute units, rounded down to a multiple of 8).
static int plan_args(const char* who, int32_t B, int32_t H, int32_t N, int32_t tile,
                     int32_t mask_heads, int32_t* workers) {
  if (B < 0 || H < 0 || N < 0)
    return fail(BSATTN_ERR_INVALID_ARG, "%s: B, H and N must be >= 0", who);
  if (tile != 128)
    return fail(BSATTN_ERR_UNSUPPORTED, "%s: tile %d (the planned path: 128)", who, tile);
  if (mask_heads != 1 && mask_heads != H)
    return fail(BSATTN_ERR_INVALID_ARG, "%s: mask_heads %d must be 1 or H=%d", who,
                mask_heads, H);
  const int32_t tiles = bsattn_num_tiles(N, tile);
  if (tiles > bsattn::kPlanMaxTiles)
    return fail(BSATTN_ERR_UNSUPPORTED, "%s: %d tiles (at most %d)", who, tiles,
                bsattn::kPlanMaxTiles);
  if ((int64_t)B * H > 65535)
    return fail(BSATTN_ERR_UNSUPPORTED, "%s: B*H must be <= 65535", who);
  int32_t w = *workers;
  if (w == 0) {
    const int cu = bsattn::device_compute_units();
    if (cu < 1) return fail(BSATTN_ERR_HIP, "%s: cannot query the device", who);
    w = cu - cu % bsattn::kPlanXcds;
    const int most = bsattn::kPlanXcds * bsattn::kPlanMaxWorkersPerXcd;
    if (w > most) w = most;
    if (w < bsattn::kPlanXcds) w = bsattn::kPlanXcds;
  }
  if (w < bsattn::kPlanXcds || w % bsattn::kPlanXcds != 0 ||
      w > bsattn::kPlanXcds * bsattn::kPlanMaxWorkersPerXcd)
    return fail(BSATTN_ERR_INVALID_ARG, "%s: workers %d must be a multiple of %d in [%d, %d]",
                who, w, bsattn::kPlanXcds, bsattn::kPlanXcds,
                bsattn::kPlanXcds * bsattn::kPlanMaxWorkersPerXcd);
  *workers = w;
  return BSATTN_OK;
}

// The plan layout for a buffer of plan_bytes bytes (the step capacity is
// whatever follows the fixed part); INVALID_ARG when it is too small.
static int plan_fit(const char* who, int32_t B, int32_t H, int32_t N, int32_t mask_heads,
                    int32_t workers, const void* plan, int64_t plan_bytes,
                    bsattn::PlanLayout& L) {
  L = bsattn::plan_layout(B, H, N, 128, mask_heads, 0, workers);
  if (!plan) return fail(BSATTN_ERR_INVALID_ARG, "%s: null plan", who);
  if (!aligned16(plan)) return fail(BSATTN_ERR_INVALID_ARG, "%s: plan not 16-byte aligned", who);
  if (plan_bytes < L.bytes)
    return fail(BSATTN_ERR_INVALID_ARG, "%s: plan_bytes %lld below the minimum %lld", who,
                (long long)plan_bytes, (long long)L.bytes);
  L.step_cap = (plan_bytes - L.off_steps) / 8;
  L.bytes = plan_bytes;
  return BSATTN_OK;
}

BSATTN_API int64_t bsattn_fwd_plan_bytes(int32_t B, int32_t H, int32_t N, int32_t tile,
                                         int32_t mask_heads, int64_t nnz_bound,
                                         int32_t workers) {
  const int st = plan_args("fwd_plan_bytes", B, H, N, tile, mask_heads, &workers);
  if (st != BSATTN_OK) return st;
  const int32_t tiles = bsattn_num_tiles(N, tile);
  const int64_t full = (int64_t)mask_heads * tiles * tiles;
  if (nnz_bound < 0 || nnz_bound > full) nnz_bound = full;
  ok();
  return bsattn::plan_layout(B, H, N, tile, mask_heads, nnz_bound, workers).bytes;
}

BSATTN_API int bsattn_fwd_plan(int32_t B, int32_t H, int32_t N, int32_t tile,
                               int32_t mask_heads, const int32_t* row_ptr,
                               const int32_t* col_idx, int32_t workers, void* plan,
                               int64_t plan_bytes, void* stream) {
  int st = plan_args("fwd_plan", B, H, N, tile, mask_heads, &workers);
  if (st != BSATTN_OK) return st;
  if ((int64_t)B * H * N == 0) return ok();
  if (!row_ptr || !col_idx) return fail(BSATTN_ERR_INVALID_ARG, "fwd_plan: null CSR");
  bsattn::PlanLayout L;
  st = plan_fit("fwd_plan", B, H, N, mask_heads, workers, plan, plan_bytes, L);
  if (st != BSATTN_OK) return st;
  const int64_t cap = (int64_t)mask_heads * L.tiles * L.tiles;
  return hip_status(bsattn::launch_fwd_plan(L, row_ptr, col_idx, cap, (char*)plan, stream),
                    "fwd_plan");
}

BSATTN_API int bsattn_fwd_planned(int32_t B, int32_t H, int32_t N, int32_t d, int32_t tile,
                                  int32_t dtype, const void* q, const void* k, const void* v,
                                  void* o, float* lse, int32_t mask_heads,
                                  const int32_t* row_ptr, const int32_t* col_idx,
                                  const void* plan, int64_t plan_bytes, int32_t workers,
                                  int32_t window, float scale, void* stream) {
  bsattn::FwdLaunch a;
  bool noop;
  int st = fwd_args("fwd_planned", B, H, N, d, tile, dtype, q, k, v, o, lse, mask_heads,
                    row_ptr, col_idx, scale, a, &noop);
  if (st != BSATTN_OK) return st;
  if (d != 128 || tile != 128 || dtype != BSATTN_DTYPE_BF16)
    return fail(BSATTN_ERR_UNSUPPORTED, "fwd_planned: bf16, d 128 and tile 128 only");
  st = plan_args("fwd_planned", B, H, N, tile, mask_heads, &workers);
  if (st != BSATTN_OK) return st;
  if (window < 0) return fail(BSATTN_ERR_INVALID_ARG, "fwd_planned: window must be >= 0");
  if (noop) return ok();
  if (window > 0 && (N % window != 0 || (N / window) % 128 != 0))
    return fail(BSATTN_ERR_INVALID_ARG,
                "fwd_planned: N=%d must be window=%d times a multiple of 128", N, window);
  if ((int64_t)N * 256 >= ((int64_t)1 << 31))
    return fail(BSATTN_ERR_INVALID_ARG, "fwd_planned: N * 256 bytes must stay below 2^31");
  st = plan_fit("fwd_planned", B, H, N, mask_heads, workers, plan, plan_bytes, a.pl);
  if (st != BSATTN_OK) return st;
  a.plan = static_cast<const char*>(plan);
  a.window = window;
  return hip_status(bsattn::launch_fwd(a, stream), "fwd_planned");
}

BSATTN_API int bsattn_fwd_noalloc(int32_t B, int32_t H, int32_t N, int32_t d, int32_t tile,
                                  int32_t dtype, const void* q, const void* k, const void* v,
                                  void* o, float* lse, int32_t mask_heads,
                                  const int32_t* row_ptr, const int32_t* col_idx, float scale,
                                  void* stream) {
  bsattn::FwdLaunch a;
  bool noop;
  int st = fwd_args("fwd_noalloc", B, H, N, d, tile, dtype, q, k, v, o, lse, mask_heads,
                    row_ptr, col_idx, scale, a, &noop);
  if (st != BSATTN_OK) return st;
  if (noop) return ok();
  // shapes outside the planned path run bsattn_fwd's kernels, which use no
  // memory beyond their arguments
  const bool planned = d == 128 && tile == 128 && dtype == BSATTN_DTYPE_BF16 &&
                       a.tiles <= bsattn::kPlanMaxTiles && (int64_t)B * H <= 65535 &&
                       (int64_t)N * 256 < ((int64_t)1 << 31);
  if (!planned) return hip_status(bsattn::launch_fwd(a, stream), "fwd_noalloc");
  int32_t workers = 0;
  st = plan_args("fwd_noalloc", B, H, N, tile, mask_heads, &workers);
  if (st != BSATTN_OK) return st;
  const int64_t full = (int64_t)mask_heads * a.tiles * a.tiles;
  bsattn::PlanLayout L = bsattn::plan_layout(B, H, N, tile, mask_heads, full, workers);
  if (L.bytes > bsattn::kNoAllocScratchBytes)
    return fail(BSATTN_ERR_INVALID_ARG,
                "fwd_noalloc: a plan for B=%d H=%d N=%d mask_heads=%d needs %lld bytes, above "
                "the library's %lld-byte device scratch (use bsattn_fwd_plan with a buffer "
                "of the caller's)",
                B, H, N, mask_heads, (long long)L.bytes,
                (long long)bsattn::kNoAllocScratchBytes);
  char* plan = nullptr;
  int e = bsattn::noalloc_scratch(&plan);
  if (e != 0) return hip_status(e, "fwd_noalloc: device scratch");
  e = bsattn::launch_fwd_plan(L, row_ptr, col_idx, full, plan, stream);
  if (e != 0) return hip_status(e, "fwd_noalloc: plan");
  a.plan = plan;
  a.pl = L;
  return hip_status(bsattn::launch_fwd(a, stream), "fwd_noalloc");
}

BSATTN_API int bsattn_window_reorder(int32_t B, int32_t H, int32_t N, int32_t d, int32_t w,
                                     int32_t dtype, const void* src, void* dst, int32_t inverse,
                                     void* stream) {
  if (B < 0 || H < 0 || N < 0 || d < 1 || w < 1)
    return fail(BSATTN_ERR_INVALID_ARG, "window_reorder: B, H, N >= 0 and d, w >= 1 required");
  if (dtype != BSATTN_DTYPE_BF16 && dtype != BSATTN_DTYPE_F32)
    return fail(BSATTN_ERR_UNSUPPORTED, "window_reorder: dtype %d", dtype);
  if ((int64_t)B * H * N == 0) return ok();
  if (N % w != 0)
    return fail(BSATTN_ERR_INVALID_ARG, "window_reorder: N=%d is not a multiple of w=%d", N, w);
  if (!src || !dst || src == dst)
    return fail(BSATTN_ERR_INVALID_ARG, "window_reorder: null or aliased buffers");
  const int32_t elt = dtype == BSATTN_DTYPE_BF16 ? 2 : 4;
  const int64_t row_bytes = (int64_t)d * elt;
  if (row_bytes % 16 != 0 || !aligned16(src) || !aligned16(dst))
    return fail(BSATTN_ERR_INVALID_ARG,
                "window_reorder: rows must be 16-byte multiples on 16-byte aligned buffers");
  if ((double)B * H * N * row_bytes >= 1.0e12)
    return fail(BSATTN_ERR_INVALID_ARG, "window_reorder: tensor too large");
  return hip_status(bsattn::launch_window_reorder((int64_t)B * H, N, (int32_t)row_bytes, w, src,
                                                  dst, inverse != 0, stream),
                    "window_reorder");
}

static int check_grid(const char* who, int32_t B, int32_t H, int32_t T, int32_t gh, int32_t gw,
                      int32_t d, int32_t stride, int32_t dtype, bool mfma_dims) {
  if (B < 0 || H < 0 || T < 0 || gh < 1 || gw < 1 || stride < 1 || d < 1)
    return fail(BSATTN_ERR_INVALID_ARG,
                "%s: B, H, T >= 0 and grid_h, grid_w, stride, d >= 1 required", who);
  if (mfma_dims && d != 64 && d != 128)
    return fail(BSATTN_ERR_UNSUPPORTED, "%s: head dim %d (supported: 64, 128)", who, d);
  if (dtype != BSATTN_DTYPE_BF16 && dtype != BSATTN_DTYPE_F32)
    return fail(BSATTN_ERR_UNSUPPORTED, "%s: dtype %d", who, dtype);
  if (B > 65535 || H > 65535)
    return fail(BSATTN_ERR_INVALID_ARG, "%s: B and H must be <= 65535", who);
  if ((int64_t)T * gh * gw > INT32_MAX)
    return fail(BSATTN_ERR_INVALID_ARG, "%s: more than 2^31-1 tokens", who);
  return BSATTN_OK;
}

BSATTN_API int64_t bsattn_row_cosines_workspace_bytes(int32_t B, int32_t H, int32_t T,
                                                      int32_t grid_h, int32_t grid_w,
                                                      int32_t stride) {
  if (B < 0 || H < 0 || T < 0 || grid_h < 1 || grid_w < 1 || stride < 1) return -1;
  return bsattn::row_cos_workspace_bytes(B, H, T, grid_h, grid_w, stride);
}

BSATTN_API int bsattn_row_cosines(int32_t B, int32_t H, int32_t T, int32_t grid_h,
                                  int32_t grid_w, int32_t d, int32_t stride, int32_t dtype,
                                  const void* q, const void* k, float* cos, float scale,
                                  void* workspace, int64_t workspace_bytes, void* stream) {
  const int st = check_grid("row_cosines", B, H, T, grid_h, grid_w, d, stride, dtype, true);
  if (st != BSATTN_OK) return st;
  if (grid_w > 256) return fail(BSATTN_ERR_UNSUPPORTED, "row_cosines: grid_w %d > 256", grid_w);
  if ((int64_t)B * H * T == 0) return ok();
  if (!q || !k || !cos) return fail(BSATTN_ERR_INVALID_ARG, "row_cosines: null pointer");
  if (!aligned16(q) || !aligned16(k))
    return fail(BSATTN_ERR_INVALID_ARG, "row_cosines: q and k must be 16-byte aligned");
  if (!(scale == scale) || isinf(scale))
    return fail(BSATTN_ERR_INVALID_ARG, "row_cosines: scale must be finite");
  if ((int64_t)T * grid_h > INT32_MAX / 2)
    return fail(BSATTN_ERR_INVALID_ARG, "row_cosines: too many rows");
  if (workspace != nullptr) {
    const int64_t need = bsattn::row_cos_workspace_bytes(B, H, T, grid_h, grid_w, stride);
    if (workspace_bytes < need)
      return fail(BSATTN_ERR_INVALID_ARG, "row_cosines: workspace of %lld bytes, %lld needed",
                  (long long)workspace_bytes, (long long)need);
    if ((reinterpret_cast<uintptr_t>(workspace) & 3) != 0)
      return fail(BSATTN_ERR_INVALID_ARG, "row_cosines: workspace must be 4-byte aligned");
  }
  bsattn::RowCosLaunch a;
  a.B = B;
  a.H = H;
  a.T = T;
  a.gh = grid_h;
  a.gw = grid_w;
  a.N = T * grid_h * grid_w;
  a.d = d;
  a.dtype = dtype;
  a.stride = stride;
  a.q = q;
  a.k = k;
  a.cos = cos;
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
  a.scale_log2 = sc * 1.4426950408889634f;
  a.ws = static_cast<float*>(workspace);
  return hip_status(bsattn::launch_row_cosines(a, stream), "row_cosines");
}

BSATTN_API int bsattn_repetitive_heads(int32_t B, int32_t H, int32_t T, int32_t grid_h,
                                       int32_t stride, const float* cos, double gamma,
                                       uint8_t* flags, void* stream) {
  if (B < 0 || H < 0 || T < 0 || grid_h < 1 || stride < 1)
    return fail(BSATTN_ERR_INVALID_ARG,
                "repetitive_heads: B, H, T >= 0 and grid_h, stride >= 1 required");
  if (!(gamma == gamma) || isinf(gamma))
    return fail(BSATTN_ERR_INVALID_ARG, "repetitive_heads: gamma must be finite");
  if (H == 0) return ok();
  if (!flags || ((int64_t)B * T > 0 && !cos))
    return fail(BSATTN_ERR_INVALID_ARG, "repetitive_heads: null pointer");
  return hip_status(bsattn::launch_repetitive_heads(B, H, T, grid_h, stride, cos, gamma, flags,
                                                    stream),
                    "repetitive_heads");
}

static int anchor_rows_call(const char* who, int32_t B, int32_t H, int32_t T, int32_t grid_h,
                            int32_t grid_w, int32_t d, int32_t stride, int32_t dtype,
                            const void* src, void* dst, int32_t broadcast, int32_t block_rows,
                            const uint8_t* flags, bool need_flags, void* stream);

BSATTN_API int bsattn_anchor_rows(int32_t B, int32_t H, int32_t T, int32_t grid_h,
                                  int32_t grid_w, int32_t d, int32_t stride, int32_t dtype,
                                  const void* src, void* dst, int32_t broadcast,
                                  int32_t block_rows, void* stream) {
  return anchor_rows_call("anchor_rows", B, H, T, grid_h, grid_w, d, stride, dtype, src, dst,
                          broadcast, block_rows, nullptr, false, stream);
}

BSATTN_API int bsattn_anchor_rows_heads(int32_t B, int32_t H, int32_t T, int32_t grid_h,
                                        int32_t grid_w, int32_t d, int32_t stride,
                                        int32_t dtype, const void* src, void* dst,
                                        int32_t broadcast, int32_t block_rows,
                                        const uint8_t* flags, void* stream) {
  return anchor_rows_call("anchor_rows_heads", B, H, T, grid_h, grid_w, d, stride, dtype, src,
                          dst, broadcast, block_rows, flags, true, stream);
}

BSATTN_API int bsattn_mask_select(int32_t H, int32_t Tq, int32_t Tk, const uint8_t* flags,
                                  const uint8_t* set_mask, int32_t set_heads,
                                  const uint8_t* clear_mask, int32_t clear_heads,
                                  uint8_t* out, void* stream) {
  if (H < 0 || Tq < 0 || Tk < 0)
    return fail(BSATTN_ERR_INVALID_ARG, "mask_select: H, Tq and Tk must be >= 0");
  if ((set_heads != 1 && set_heads != H) || (clear_heads != 1 && clear_heads != H))
    return fail(BSATTN_ERR_INVALID_ARG, "mask_select: mask heads must be 1 or H=%d", H);
  const int64_t cells = (int64_t)Tq * Tk;
  if ((int64_t)H * cells >= kMaxCells)
    return fail(BSATTN_ERR_INVALID_ARG, "mask_select: mask has >= 2^31 cells");
  if ((int64_t)H * cells == 0) return ok();
  if (!flags || !set_mask || !clear_mask || !out)
    return fail(BSATTN_ERR_INVALID_ARG, "mask_select: null pointer");
  return hip_status(bsattn::launch_mask_select(H, cells, flags, set_mask, set_heads, clear_mask,
                                               clear_heads, out, stream),
                    "mask_select");
}

static int anchor_rows_call(const char* who, int32_t B, int32_t H, int32_t T, int32_t grid_h,
                            int32_t grid_w, int32_t d, int32_t stride, int32_t dtype,
                            const void* src, void* dst, int32_t broadcast, int32_t block_rows,
                            const uint8_t* flags, bool need_flags, void* stream) {
  const int st = check_grid(who, B, H, T, grid_h, grid_w, d, stride, dtype, false);
  if (st != BSATTN_OK) return st;
  if ((d * (dtype == BSATTN_DTYPE_BF16 ? 2 : 4)) % 16 != 0)
    return fail(BSATTN_ERR_INVALID_ARG, "%s: rows must be 16-byte multiples", who);
  if (block_rows < 0)
    return fail(BSATTN_ERR_INVALID_ARG, "%s: block_rows must be >= 0", who);
  if (block_rows > 0) {
    const int64_t n = (int64_t)T * grid_h * grid_w;
    const int64_t packed = (int64_t)T * ((grid_h + stride - 1) / stride) * grid_w;
    if ((packed + block_rows - 1) / block_rows > (n + block_rows - 1) / block_rows)
      return fail(BSATTN_ERR_INVALID_ARG,
                  "%s: %lld anchor rows in blocks of %d do not fit %lld block slots", who,
                  (long long)packed, block_rows, (long long)((n + block_rows - 1) / block_rows));
  }
  if ((int64_t)B * H * T == 0) return ok();
  if (!src || !dst || src == dst)
    return fail(BSATTN_ERR_INVALID_ARG, "%s: null or aliased buffers", who);
  if (!aligned16(src) || !aligned16(dst))
    return fail(BSATTN_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", who);
  if (need_flags && !flags) return fail(BSATTN_ERR_INVALID_ARG, "%s: null flags", who);
  const int32_t row_bytes = d * (dtype == BSATTN_DTYPE_BF16 ? 2 : 4);
  return hip_status(bsattn::launch_anchor_rows((int64_t)B * H, T * grid_h * grid_w, row_bytes,
                                               grid_h, grid_w, stride, broadcast != 0,
                                               block_rows, src, dst, flags, H, stream),
                    who);
}

BSATTN_API int64_t bsattn_block_energy_workspace_bytes(int32_t B, int32_t H, int32_t N,
                                                       int32_t tile) {
  if (B < 0 || H < 0 || N < 0 || (tile != 64 && tile != 128)) return -1;
  return bsattn::energy_workspace_bytes(B, H, N, tile);
}

BSATTN_API int bsattn_block_energy(int32_t B, int32_t H, int32_t N, int32_t d, int32_t tile,
                                   int32_t dtype, const void* q, const void* k, float* energy,
                                   float scale, void* workspace, int64_t workspace_bytes,
                                   void* stream) {
  if (B < 0 || H < 0 || N < 0 || d < 0)
    return fail(BSATTN_ERR_INVALID_ARG, "block_energy: B, H, N and d must be >= 0");
  if (d != 64 && d != 128)
    return fail(BSATTN_ERR_UNSUPPORTED, "block_energy: head dim %d (supported: 64, 128)", d);
  if (tile != 64 && tile != 128)
    return fail(BSATTN_ERR_UNSUPPORTED, "block_energy: tile %d (supported: 64, 128)", tile);
  if (dtype != BSATTN_DTYPE_BF16 && dtype != BSATTN_DTYPE_F32)
    return fail(BSATTN_ERR_UNSUPPORTED, "block_energy: dtype %d", dtype);
  if ((int64_t)B * H * N == 0) return ok();
  if (B > 65535 || H > 65535)
    return fail(BSATTN_ERR_INVALID_ARG, "block_energy: B and H must be <= 65535");
  if (!q || !k || !energy) return fail(BSATTN_ERR_INVALID_ARG, "block_energy: null pointer");
  if (!aligned16(q) || !aligned16(k))
    return fail(BSATTN_ERR_INVALID_ARG, "block_energy: q and k must be 16-byte aligned");
  if (!(scale == scale) || isinf(scale))
    return fail(BSATTN_ERR_INVALID_ARG, "block_energy: scale must be finite");
  const int32_t tiles = bsattn_num_tiles(N, tile);
  if ((int64_t)B * H * tiles * tiles >= kMaxCells)
    return fail(BSATTN_ERR_INVALID_ARG, "block_energy: energy tensor has >= 2^31 cells");
  if (workspace != nullptr) {
    const int64_t need = bsattn::energy_workspace_bytes(B, H, N, tile);
    if (workspace_bytes < need)
      return fail(BSATTN_ERR_INVALID_ARG, "block_energy: workspace of %lld bytes, %lld needed",
                  (long long)workspace_bytes, (long long)need);
    if (!aligned16(workspace))
      return fail(BSATTN_ERR_INVALID_ARG, "block_energy: workspace must be 16-byte aligned");
  }
  bsattn::EnergyLaunch a;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.tile = tile;
  a.dtype = dtype;
  a.q = q;
  a.k = k;
  a.energy = energy;
  a.tiles = tiles;
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
  a.scale_log2 = sc * 1.4426950408889634f;
  a.ws = static_cast<float*>(workspace);
  return hip_status(bsattn::launch_block_energy(a, stream), "block_energy");
}

BSATTN_API int bsattn_select_blocks(int32_t rows, int32_t Tk, const float* energy, double eps,
                                    uint8_t* mask, void* stream) {
  if (rows < 0 || Tk < 0)
    return fail(BSATTN_ERR_INVALID_ARG, "select_blocks: rows and Tk must be >= 0");
  if (Tk > 4096) return fail(BSATTN_ERR_UNSUPPORTED, "select_blocks: Tk %d > 4096", Tk);
  if ((int64_t)rows * Tk >= kMaxCells)
    return fail(BSATTN_ERR_INVALID_ARG, "select_blocks: >= 2^31 cells");
  if (!(eps == eps) || isinf(eps))
    return fail(BSATTN_ERR_INVALID_ARG, "select_blocks: eps must be finite");
  if ((int64_t)rows * Tk == 0) return ok();
  if (!energy || !mask) return fail(BSATTN_ERR_INVALID_ARG, "select_blocks: null pointer");
  return hip_status(bsattn::launch_select_blocks(rows, Tk, energy, eps, mask, stream),
                    "select_blocks");
}

BSATTN_API int bsattn_aggregate_masks(int32_t P, int64_t cells, const uint8_t* masks, double rho,
                                      uint8_t* out, void* stream) {
  if (P < 1 || cells < 0)
    return fail(BSATTN_ERR_INVALID_ARG, "aggregate_masks: P >= 1 and cells >= 0 required");
  if ((double)P * (double)cells >= 9.0e18)
    return fail(BSATTN_ERR_INVALID_ARG, "aggregate_masks: P * cells too large");
  if (!(rho == rho) || isinf(rho))
    return fail(BSATTN_ERR_INVALID_ARG, "aggregate_masks: rho must be finite");
  if (cells == 0) return ok();
  if (!masks || !out) return fail(BSATTN_ERR_INVALID_ARG, "aggregate_masks: null pointer");
  return hip_status(bsattn::launch_aggregate(P, cells, masks, rho, out, stream),
                    "aggregate_masks");
}

BSATTN_API int64_t bsattn_mfma_ceiling(int32_t blocks, int32_t iters, float* sink,
                                       void* stream) {
  if (blocks < 1 || iters < 1 || !sink)
    return fail(BSATTN_ERR_INVALID_ARG, "mfma_ceiling: blocks, iters >= 1 and sink required");
  const int err = bsattn::launch_mfma_ceiling(blocks, iters, sink, stream);
  if (err != 0) return hip_status(err, "mfma_ceiling");
  ok();
  return bsattn::mfma_ceiling_flops(blocks, iters);
}

}  // extern "C"
