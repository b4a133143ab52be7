// Tile-mask builder.
//
// LVSA page, "Meccanismo Core": a query frame t attends to A(t) = G u W(t),
// the local window W(t) plus the rotating global anchor frames G.  The mask is
// built at tile granularity: tile pair (i, j) is active when some frame
// covered by query tile i may attend to some frame covered by key tile j.
//
// The frames a tile covers form a contiguous range [lo, hi], so the window
// part reduces to the gap between two integer intervals:
//   exists t in [a, b], f in [c, e] with |f - t| <= w
//   <=>  max(0, c - b, a - e) <= w.
// The anchor part is independent of the query tile: some anchor frame
// g_k = (r + floor(k*T/n_a)) mod T lies in the key tile's range.
//
// Expanded mode (same section, the expanded adaptive windows that hold |A(t)|
// near a frame budget C): the window of query frame t grows from [t-w, t+w]
// by the nearest missing frame, the earlier one on a tie and never past the
// video's ends, until |G u W(t)| >= min(C, T); an anchor frame it passes adds
// nothing.  W(t) stays one interval [lo(t), hi(t)], found by walking outward
// from the plain window while counting the non-anchor frames taken.  Whether
// a frame is an anchor is O(1): the offsets floor(k*T/n_a) strictly increase
// with k (n_a <= T), so frame f is an anchor exactly when k = ceil(g*n_a/T),
// g = (f - r) mod T, satisfies k < n_a and floor(k*T/n_a) == g.
//
// Block-diagonal mode (SQuad page, "1. Operatore di Attenzione SQuad": each
// pass attends inside disjoint runs of tokens): tile pair (i, j) is active
// when i and j fall in the same run of block_tiles tiles.
//
// Dense-rows mode (CalibAtt page, "B. Fase di Inferenza": a repetitive head
// computes its anchor rows only, packed into the first query tiles): query
// tiles below query_tiles read every key tile, the others none.
//
// Spread dense-rows mode (same passage, with the anchor rows laid out in
// blocks spread evenly over the sequence): the query_tiles anchor tiles form
// Rg = ceil(query_tiles / block_tiles) blocks of block_tiles tiles (the last
// one possibly shorter); block g sits at block slot floor(g * Pg / Rg) of the
// Pg = ceil(Tq / block_tiles) slots (the rows bsattn_anchor_rows writes for
// block_rows = block_tiles * tile).  The slot of g strictly increases with g
// (Rg <= Pg), so slot b holds block g = ceil(b * Rg / Pg) exactly when
// floor(g * Pg / Rg) == b; with Rg < Pg no block reaches the last slot.
//
// Static mode (CalibAtt page, "B. Fase di Inferenza": the block lists are
// precomputed and deterministic) draws one SplitMix64 value per cell
// c = (h*Tq + i)*Tk + j: the (c+1)-th output of the generator seeded with
// `seed` (Steele, Lea and Flood, OOPSLA 2014).  The cell is active when the
// output's top 24 bits are below thresh24, or on the diagonal when forced.
#include <hip/hip_runtime.h>

#include "bsattn_internal.h"

namespace bsattn {
namespace {

__device__ __forceinline__ uint64_t splitmix64_at(uint64_t seed, uint64_t n) {
  uint64_t z = seed + n * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ void frame_range(int tile_idx, int tile, int tokens,
                                            int per_frame, int& lo, int& hi) {
  const int first = tile_idx * tile;
  const int last = min(first + tile, tokens) - 1;
  lo = first / per_frame;
  hi = last / per_frame;
}

__device__ __forceinline__ int is_anchor(int f, const MaskLaunch& a) {
  if (a.num_anchors == 0) return 0;
  const int g = f >= a.rotation ? f - a.rotation : f - a.rotation + a.frames;
  const int64_t k = ((int64_t)g * a.num_anchors + a.frames - 1) / a.frames;
  return k < a.num_anchors && ((int64_t)k * a.frames) / a.num_anchors == g;
}

// [lo, hi]: the expanded window of query frame t.
__device__ void expanded_window(int t, const MaskLaunch& a, int& lo, int& hi) {
  const int T = a.frames;
  lo = max(0, t - a.window);
  hi = min(T - 1, t + a.window);
  int count = a.num_anchors;
  for (int f = lo; f <= hi; ++f) count += !is_anchor(f, a);
  // count reaches T once [lo, hi] = [0, T-1], and budget <= T, so the walk
  // stops by then; d < T bounds it regardless.
  for (int d = a.window + 1; count < a.budget && d < T; ++d) {
    if (t - d >= 0) {
      lo = t - d;
      count += !is_anchor(lo, a);
      if (count >= a.budget) break;
    }
    if (t + d < T) {
      hi = t + d;
      count += !is_anchor(hi, a);
    }
  }
}

__device__ __forceinline__ int anchor_in(int ka, int kb, const MaskLaunch& a) {
  for (int k = 0; k < a.num_anchors; ++k) {
    const int g = (int)((a.rotation + ((int64_t)k * a.frames) / a.num_anchors) %
                        a.frames);
    if (g >= ka && g <= kb) return 1;
  }
  return 0;
}

__global__ void build_mask_kernel(MaskLaunch a, uint8_t* __restrict__ mask) {
  const int64_t total = (int64_t)a.mask_heads * a.tq * a.tk;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += stride) {
    const int j = (int)(c % a.tk);
    const int64_t hi_row = c / a.tk;
    const int i = (int)(hi_row % a.tq);
    uint8_t on = 0;
    if (a.kind == 0 || a.kind == 3) {
      int qa, qb, ka, kb;
      frame_range(i, a.tile, a.tokens, a.tokens_per_frame, qa, qb);
      frame_range(j, a.tile, a.tokens, a.tokens_per_frame, ka, kb);
      if (a.kind == 0) {
        const int gap = max(0, max(ka - qb, qa - kb));
        on = gap <= a.window;
      } else {
        for (int t = qa; t <= qb && !on; ++t) {
          int lo, hi;
          expanded_window(t, a, lo, hi);
          on = lo <= kb && ka <= hi;
        }
      }
      if (!on) on = anchor_in(ka, kb, a);
    } else if (a.kind == 4) {
      on = (i / a.block_tiles) == (j / a.block_tiles);
    } else if (a.kind == 5) {
      on = i < a.query_tiles;
    } else if (a.kind == 6) {
      const int64_t bt = a.block_tiles;
      const int64_t rg = (a.query_tiles + bt - 1) / bt, pg = (a.tq + bt - 1) / bt;
      const int64_t b = i / bt;
      if (b < pg && rg > 0) {
        const int64_t g = (b * rg + pg - 1) / pg;
        if (g < rg && (g * pg) / rg == b) {
          const int64_t size = g < rg - 1 ? bt : a.query_tiles - (rg - 1) * bt;
          on = (i - b * bt) < size;
        }
      }
    } else if (a.kind == 1) {
      const uint64_t z = splitmix64_at(a.seed, (uint64_t)c + 1);
      on = ((uint32_t)(z >> 40) < a.thresh24) || (a.force_diagonal && i == j);
    } else {
      on = 1;
    }
    mask[c] = on;
  }
}

}  // namespace

int launch_build_mask(const MaskLaunch& a, uint8_t* mask, void* stream) {
  const int64_t total = (int64_t)a.mask_heads * a.tq * a.tk;
  if (total == 0) return hipSuccess;
  const int block = 256;
  int64_t grid = (total + block - 1) / block;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(build_mask_kernel, dim3((unsigned)grid), dim3(block), 0,
                     (hipStream_t)stream, a, mask);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256)
mask_select_kernel(int32_t H, int64_t cells, const uint8_t* __restrict__ flags,
                   const uint8_t* __restrict__ set, int32_t set_heads,
                   const uint8_t* __restrict__ clear, int32_t clear_heads,
                   uint8_t* __restrict__ out) {
  const int64_t total = (int64_t)H * cells;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int h = (int)(i / cells);
    const int64_t c = i - (int64_t)h * cells;
    out[i] = flags[h] ? set[(set_heads == 1 ? 0 : (int64_t)h) * cells + c]
                      : clear[(clear_heads == 1 ? 0 : (int64_t)h) * cells + c];
  }
}

int launch_mask_select(int32_t H, int64_t cells, const uint8_t* flags, const uint8_t* set,
                       int32_t set_heads, const uint8_t* clear, int32_t clear_heads,
                       uint8_t* out, void* stream) {
  const int64_t total = (int64_t)H * cells;
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  if (grid > 1 << 16) grid = 1 << 16;
  hipLaunchKernelGGL(mask_select_kernel, dim3((unsigned)grid), dim3(256), 0,
                     (hipStream_t)stream, H, cells, flags, set, set_heads, clear, clear_heads,
                     out);
  return hipGetLastError();
}

}  // namespace bsattn
