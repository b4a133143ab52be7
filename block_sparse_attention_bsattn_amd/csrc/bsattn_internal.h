// Internal launch entry points shared by the host API layer and the kernel
// translation units.  Arguments are already validated by the caller.
#pragma once

#include <stdint.h>

namespace bsattn {

struct MaskLaunch {
  int32_t kind;
  int32_t frames, tokens_per_frame, tokens, tile;
  int32_t tq, tk, mask_heads;
  int32_t window, num_anchors, rotation;  // window <= frames, rotation in [0, frames)
  int32_t budget;                         // expanded mode: min(C, frames)
  int32_t block_tiles;                    // block-diagonal and spread dense-rows modes
  int32_t query_tiles;                    // dense-rows modes
  uint64_t seed;
  uint32_t thresh24;
  int32_t force_diagonal;
};

// Work plan of the planned forward (bf16, d 128, tile 128): built on the
// device from the CSR lists by launch_fwd_plan, read by the planned forward.
// All offsets are in bytes from the start of the caller's plan buffer.
struct PlanLayout {
  int32_t B, H, N, tiles, mask_heads, workers, pairs;
  int64_t items;      // B * H * pairs
  int64_t step_cap;   // capacity of the step array (8-byte entries)
  int64_t off_xw;     // int32 [8]: the XCD weights the ranges were cut by (byte 64)
  int64_t off_wstep;  // int32 [4 * workers]: each worker's pair stream, group 0's and
                      // group 1's single-tile streams: first step of each, then the end
  int64_t off_witem;  // int32 [2 * workers]: each worker's (first, count) in witems
  int64_t off_wcnt;   // int32 [3 * workers]: steps of each worker's three streams
  int64_t off_witems; // int32 [items]: item words in each worker's order (bit 31: split mode)
  int64_t off_pinfo;  // int32x8 [mask_heads * pairs]: union, common, raw lengths n0 and
                      // n1, valid lengths a and b, per list pair
  int64_t off_itmp;   // int32x4 [items]: worker, sequence number, step offset(s) (the
                      // last with bit 30 set when tile 2p + 1 goes to group 0)
  int64_t off_steps;  // int32x2 [step_cap]: (entry word, item word)
  int64_t bytes;
};
constexpr int32_t kPlanMagic = 0x42535031;
// XCD weights are in units of 1/4096 of the mean XCD speed
constexpr int kPlanWeightOne = 4096;
// header: magic, B, H, N, tiles, Hm, workers, pairs, then the section
// offsets / 16 (wstep, witem, wcnt, witems, pinfo, itmp, steps) and the step
// capacity (clamped to 2^31 - 1)
constexpr int kPlanHeaderInts = 16;
constexpr int kPlanXcds = 8;
constexpr int kPlanMaxTiles = 4096;
constexpr int kPlanMaxWorkersPerXcd = 64;
// Item words: in a pair stream (b * H + h) << 15 | pair, pair = query-tile
// pair index; in a single-tile stream (b * H + h) << 13 | query tile.
constexpr int kPlanPairBits = 15;
constexpr int kPlanTileBits = 13;

PlanLayout plan_layout(int32_t B, int32_t H, int32_t N, int32_t tile, int32_t mask_heads,
                       int64_t nnz_bound, int32_t workers);
// compute units of the current device (-1 on a runtime error)
int device_compute_units();
// The allocation-free forward's plan: a static device array of this many
// bytes per GPU; noalloc_scratch gives the current device's address (a
// hipError_t value, 0 = success).
constexpr int64_t kNoAllocScratchBytes = (int64_t)96 << 20;
int noalloc_scratch(char** ptr);
// The current device's XCD feedback table: one (busy ticks, planned load)
// pair of int32 per worker of the last planned forward on the device, written by
// that forward and read by the next plan (a hipError_t value, 0 = success).
int xcd_feedback(int32_t** ptr);

struct FwdLaunch {
  int32_t B, H, N, d, tile, dtype;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int32_t mask_heads;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int32_t tiles;      // Tq = Tk
  int64_t col_cap;    // entries of col_idx that may be read
  float scale_log2;   // softmax scale * log2(e)
  int32_t window;     // 0, or w > 0: the grouped view (bf16 / d 128 / tile 128 only)
  // planned forward only (plan == nullptr otherwise)
  const char* plan;
  PlanLayout pl;
  int32_t* xfb = nullptr;  // the device's XCD feedback table: int32 pairs (planned only)
};

// Each returns a hipError_t value (0 = success).
struct EnergyLaunch {
  int32_t B, H, N, d, tile, dtype;
  const void* q;
  const void* k;
  float* energy;      // [B, H, tiles, tiles]
  int32_t tiles;
  float scale_log2;   // softmax scale * log2(e)
  float* ws;          // null, or the one-sweep workspace (tuned instance)
};

// tuned forward for bf16, d = 64, tile = 64 (contiguous rows, no plan)
bool fwd_d64_t64_fits(const FwdLaunch& a);
int launch_fwd_d64_t64(const FwdLaunch& a, void* stream);

// tuned block energies (bf16, d = 128, tile = 128)
bool energy_tuned_fits(const EnergyLaunch& a);
int64_t energy_workspace_bytes(int64_t B, int64_t H, int64_t N, int32_t tile);
int launch_energy_tuned(const EnergyLaunch& a, void* stream);

int launch_build_mask(const MaskLaunch& a, uint8_t* mask, void* stream);
int launch_compact(int32_t rows, int32_t tk, const uint8_t* mask,
                   int32_t* row_ptr, int32_t* col_idx, void* stream);
// the work plan of the planned forward (three launches)
int launch_fwd_plan(const PlanLayout& L, const int32_t* row_ptr, const int32_t* col_idx,
                    int64_t col_cap, char* plan, void* stream);
int launch_fwd(const FwdLaunch& a, void* stream);
// tuned instance: bf16, head dim 128, 128x128 tiles, N * 256 < 2^31
int launch_fwd_bf16_t128_d128(const FwdLaunch& a, void* stream);

// token reorder between window-major and position-major order
int launch_window_reorder(int64_t BH, int32_t N, int32_t row_bytes, int32_t w, const void* src,
                          void* dst, int inverse, void* stream);

// spatial repetition
struct RowCosLaunch {
  int32_t B, H, T, gh, gw, N, d, dtype, stride;
  const void* q;
  const void* k;
  float* cos;         // [B, H, T, gh]
  float scale_log2;   // softmax scale * log2(e)
  float* ws;          // null, or per-column sums [B, H, T * nna * gw, 3] (tuned, packed)
};
int launch_row_cosines(const RowCosLaunch& a, void* stream);
// tuned instance (bf16, d = 128; without a workspace grid_w <= 128): non-anchor rows only
bool row_cos_tuned_fits(const RowCosLaunch& a);
int64_t row_cos_workspace_bytes(int64_t B, int64_t H, int64_t T, int32_t gh, int32_t gw,
                                int32_t stride);
int launch_row_cos_tuned(const RowCosLaunch& a, void* stream);
int launch_repetitive_heads(int32_t B, int32_t H, int32_t T, int32_t gh, int32_t stride,
                            const float* cos, double gamma, uint8_t* flags, void* stream);
// flags: null, or uint8 [H]: heads with flag 0 are copied row for row
int launch_anchor_rows(int64_t BH, int32_t N, int32_t row_bytes, int32_t gh, int32_t gw,
                       int32_t stride, int broadcast, int32_t block_rows, const void* src,
                       void* dst, const uint8_t* flags, int32_t H, void* stream);
// out[h] = flags[h] ? set[set_heads == 1 ? 0 : h] : clear[clear_heads == 1 ? 0 : h],
// each a [cells] byte slice
int launch_mask_select(int32_t H, int64_t cells, const uint8_t* flags, const uint8_t* set,
                       int32_t set_heads, const uint8_t* clear, int32_t clear_heads,
                       uint8_t* out, void* stream);

// static-mask calibration
int launch_block_energy(const EnergyLaunch& a, void* stream);
int launch_select_blocks(int32_t rows, int32_t tk, const float* energy, double eps,
                         uint8_t* mask, void* stream);
int launch_aggregate(int32_t P, int64_t cells, const uint8_t* masks, double rho, uint8_t* out,
                     void* stream);

// matrix-core ceiling microbenchmark
int64_t mfma_ceiling_flops(int blocks, int iters);
int launch_mfma_ceiling(int blocks, int iters, float* sink, void* stream);

}  // namespace bsattn
