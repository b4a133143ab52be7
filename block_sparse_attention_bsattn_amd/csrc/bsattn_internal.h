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
};

// Each returns a hipError_t value (0 = success).
struct EnergyLaunch {
  int32_t B, H, N, d, tile, dtype;
  const void* q;
  const void* k;
  float* energy;      // [B, H, tiles, tiles]
  int32_t tiles;
  float scale_log2;   // softmax scale * log2(e)
};

int launch_build_mask(const MaskLaunch& a, uint8_t* mask, void* stream);
int launch_compact(int32_t rows, int32_t tk, const uint8_t* mask,
                   int32_t* row_ptr, int32_t* col_idx, void* stream);
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
};
int launch_row_cosines(const RowCosLaunch& a, void* stream);
int launch_repetitive_heads(int32_t B, int32_t H, int32_t T, int32_t gh, int32_t stride,
                            const float* cos, double gamma, uint8_t* flags, void* stream);
int launch_anchor_rows(int64_t BH, int32_t N, int32_t row_bytes, int32_t gh, int32_t gw,
                       int32_t stride, int broadcast, int32_t block_rows, const void* src,
                       void* dst, void* stream);

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
