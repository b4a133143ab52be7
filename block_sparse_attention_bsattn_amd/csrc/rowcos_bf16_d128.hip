// Row cosines of the spatial repetition test, tuned instance: bf16 Q and K,
// head dim 128 (CalibAtt page, "A. Fase di Calibrazione" step 3).
//
// For a non-anchor spatial row (f, y) and a column x, the two queries
// q1 = (f, y, x) and q2 = (f, a(y), x) (a(y) the anchor row) attend over
// all N keys.  One sweep keeps, per query, a running max m and relative to
// it the normaliser z = sum_k e (e = 2^(s scale log2(e) - m)) and, per
// column, the raw sums sum e1 e2, sum e1^2 and sum e2^2; dividing by z1 z2,
// z1^2 and z2^2 at the end gives <p1, p2>, |p1|^2 and |p2|^2 of the two
// probability rows, and the row's cosine is
//   cos(y) = sum_x <p1, p2> / sqrt(sum_x |p1|^2 * sum_x |p2|^2).
//
// Lazy max.  The exponentials of a 64-key tile are taken against the
// current m.  Only when a lane's tile sums of squares exceed 2^64 (some
// score lies over 32 above m) or are not finite (the first tile, m still
// -inf) does the wave take the tile's exact max, rescale its sums and redo
// the tile's exponentials.  Every e stays below 2^32, so no sum overflows,
// and all terms share one scale per query, so the ratios are those of
// exact-max arithmetic up to rounding.  After the first tile this is rare
// (the max has to jump by 32 in log2 units), so the vector work per score
// is the exponential, its argument and five sums, with no max.
//
// Mapping onto CDNA4 (gfx950)
// ---------------------------
//  * Per pair of scores (both queries, one key) the vector work is two
//    exponentials (8 cycles a wave each on gfx950, twice an FMA) and seven
//    other instructions, about 45 cycles, against a quarter of a 32x32x16
//    MFMA (8 cycles): the vector ALU bounds the kernel.  MFMA and vector
//    work of two waves on one SIMD overlap (each MFMA still holds the other
//    wave's vector issue for about 11 cycles), within a wave they
//    serialise.  Workgroup = 8 waves,
//    two groups of 4 (waves w and w + 4 share a SIMD), in a ping-pong: in
//    phase 2t group 0 computes the scores of key tile t (matrix phase) while
//    group 1 runs the exponentials and sums of tile t - 1 (vector phase); in
//    phase 2t + 1 the roles swap.
//  * A wave holds 32 columns, lane (column, half) both queries of its column
//    and half of each tile's keys (S^T = K Q^T on v_mfma_f32_32x32x16_bf16,
//    A = K rows from LDS, B = Q^T in VGPRs); each K operand read feeds the
//    MFMAs of both queries.  The 8 waves' columns share every staged tile.
//  * Packed schedule (with a workspace): the columns of a (prompt, head),
//    all non-anchor rows one after another, are cut into chunks of 32, one
//    per wave, whatever the row width, so no lane idles (52-wide rows would
//    leave 12 of every 64 idle otherwise).  Each column's three sums go to
//    the workspace and a second kernel adds them per row, x in order.
//    Row-aligned schedule (no workspace): a wave holds 32 columns of one
//    row, a group 4 / ceil(gw / 32) rows, and the workgroup adds its rows'
//    sums itself.
//  * K tiles (64 keys, 16 KB) are double-buffered in LDS and fetched
//    straight to LDS (buffer_load ... lds, no VGPR staging) by group 1 in its
//    vector phase: in phase 2t it fetches tile t + 1 into the slot tile t - 1
//    left, and waits for it at the end of its matrix phase 2t + 1, a phase
//    before group 0 reads it.  Rows past N lie outside the buffer range and
//    arrive as zeros; the vector phase masks their scores to -inf.  Matrix
//    phases issue no global-memory instruction.  (Tiles of 64 keys keep
//    both queries' scores in 64 VGPRs; 128-key tiles spill scalar registers
//    and measured 6% slower.)
//  * LDS rows are 256 B with 16-byte chunk c of row R at position
//    c ^ swz(R): conflict-free for the K reader (32 consecutive rows, one
//    chunk column).
//  * The 1-D grid is remapped so each XCD (own L2) walks a contiguous range
//    of (prompt, head, column block): workgroups on one XCD share their
//    head's key stream in its L2.
#include <hip/hip_runtime.h>

#include <math.h>

#include "bsattn_internal.h"
#include "cdna4_lds.h"

namespace bsattn {
namespace {

constexpr int RC_D = 128;
constexpr int RC_ROW = RC_D * 2;             // 256 bytes per key row
constexpr int RC_PF = 4;                     // MFMA operand read-ahead
constexpr int RC_NXCD = 8;
constexpr int RC_KB = 2;                     // 32-key blocks per staged tile
// tile sums of squares above this (or not finite): exact max for the tile
constexpr float RC_LIMIT = 18446744073709551616.0f;  // 2^64

// KB: 32-key blocks per staged tile (2 or 4); PACKED: the packed schedule
template <int KB, bool PACKED>
__global__ void __launch_bounds__(512, 1)
row_cos_bf16_d128(RowCosLaunch a) {
  constexpr int RC_KT = 32 * KB;              // keys per staged tile
  constexpr int RC_TILE = RC_KT * RC_ROW;     // 8 KB per block
  constexpr int BURSTS = KB / 2;              // 4 KB bursts per group-1 wave and tile
  // K slots [0, RC_TILE) and [RC_TILE, 2 RC_TILE) of an array aligned to
  // its size: one address bit picks the slot
  __shared__ __attribute__((aligned(2 * RC_TILE))) char kslots[2 * RC_TILE];
  __shared__ float red[8][3];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int wg = wave & 3;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  lds_char_t* const kl = uniform_lds((lds_char_t*)kslots);
  const uint32_t kl32 = (uint32_t)(uintptr_t)kl;

  // ---- workgroup -> (prompt, head, block of columns), XCD-contiguous
  const int wpr = (a.gw + 31) / 32;  // row-aligned: waves per row, 1..4
  const int rpg = 4 / wpr;           // row-aligned: rows per group
  const int nna = a.gh - (a.gh + a.stride - 1) / a.stride;
  const int rows_total = a.T * nna;
  const int cols = rows_total * a.gw;       // packed: columns per (prompt, head)
  const int chunks = (cols + 31) / 32;
  const int blocks = PACKED ? (chunks + 7) / 8 : (rows_total + 2 * rpg - 1) / (2 * rpg);
  uint32_t logical;
  {
    const uint32_t G = gridDim.x, hw = blockIdx.x;
    const uint32_t q8 = G / RC_NXCD, r8 = G % RC_NXCD, xcd = hw % RC_NXCD, slot = hw / RC_NXCD;
    const uint32_t lo = xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8;
    logical = lo + slot;
  }
  const int blk = (int)(logical % (uint32_t)blocks);
  const int bh = (int)(logical / (uint32_t)blocks);  // b * H + h
  const int h = bh % a.H, b = bh / a.H;

  // non-anchor row j: frame j / nna and the (j % nna)-th row of the frame
  // that is not a multiple of the stride
  auto row_of = [&](int j, int& fr, int& yr) INLINE {
    fr = j / nna;
    const int jj = j - fr * nna;
    yr = (jj / (a.stride - 1)) * a.stride + 1 + jj % (a.stride - 1);
  };
  // packed: wave -> chunk blk * 8 + 4 grp + wg, lane -> column chunk * 32 +
  // l32 = row j, position x; row-aligned: group g, row-in-group r -> row
  // (blk * 2 + g) * rpg + r, wave -> 32 of its columns
  const int rin = wg / wpr;
  const int chunk = blk * 8 + grp * 4 + wg;
  const int col = chunk * 32 + l32;
  const bool active = PACKED ? chunk < chunks
                             : (rin < rpg && (blk * 2 + grp) * rpg + rin < rows_total);
  int jrow, x;
  if constexpr (PACKED) {
    jrow = col / a.gw;
    x = col - jrow * a.gw;
  } else {
    jrow = (blk * 2 + grp) * rpg + rin;
    x = (wg - rin * wpr) * 32 + l32;
  }
  const bool col_ok = active && (PACKED ? col < cols : x < a.gw);
  int f = 0, y = 1;
  if (col_ok) row_of(jrow, f, y);
  const int ya = a.stride * (y / a.stride);
  const int N = a.N;
  const int P = a.gh * a.gw;
  const int64_t head_row = (int64_t)bh * N;

  bf16x8 q1[8], q2[8];
  {
    const __bf16* qb = reinterpret_cast<const __bf16*>(a.q);
    const int64_t r1 = (head_row + f * P + y * a.gw + x) * RC_D;
    const int64_t r2 = (head_row + f * P + ya * a.gw + x) * RC_D;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (col_ok) {
        q1[c] = *reinterpret_cast<const bf16x8*>(qb + r1 + c * 16 + half * 8);
        q2[c] = *reinterpret_cast<const bf16x8*>(qb + r2 + c * 16 + half * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          q1[c][e] = (__bf16)0.f;
          q2[c][e] = (__bf16)0.f;
        }
      }
    }
  }

  // ---- K fetches: load i (0 .. 4 BURSTS - 1) of group-1 wave wg fills
  // LDS bytes [(4 BURSTS wg + i) * 1024, +1024) of a slot, rows
  // 16 BURSTS wg + 4i + (0..3); lane l writes chunk position l % 16 of row
  // 16 BURSTS wg + 4i + l / 16 and so fetches global chunk
  // (l % 16) ^ swz(row) = (l % 16) ^ (4 (l / 16) + i % 4)
  const int T = (N + RC_KT - 1) / RC_KT;
  const i32x4 krs = raw_rsrc(reinterpret_cast<const char*>(a.k) + head_row * RC_ROW,
                             N * RC_ROW);
  uint32_t ld_off[4];
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const int r = 16 * BURSTS * wg + (lane >> 4);
    const int c = (lane & 15) ^ (((lane >> 4) << 2) | i4);
    ld_off[i4] = (uint32_t)r * RC_ROW + (uint32_t)(c * 16);
  }
  // burst p (4 KB) of this wave's share of tile t; skip is made wave-uniform
  auto fetch_burst = [&](int t, int p, uint32_t skip) INLINE {
    const uint32_t m0 = kl32 + (uint32_t)((t & 1) * RC_TILE) +
                        (uint32_t)((4 * BURSTS * wg + 4 * p) * 1024);
    dma_burst4(krs, m0, ld_off, (uint32_t)t * RC_TILE + (uint32_t)(p * 4096),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)skip));
  };
  auto fetch = [&](int t, uint32_t skip) INLINE {
#pragma unroll
    for (int p = 0; p < BURSTS; ++p) fetch_burst(t, p, skip);
  };

  // K reader: key row kb * 32 + l32, chunk 2c + half, slot 0; the slot bit
  // and c go in by XOR, kb by addition
  const int ks = swz(l32);
  const uint32_t kr = kl32 + (uint32_t)(l32 * RC_ROW + ((ks >> 1) << 5) + ((half ^ (ks & 1)) << 4));
  auto k_operand = [&](uint32_t slot, int kb, int c) INLINE {
    const uint32_t ad = ((kr | slot) ^ (uint32_t)(c << 5)) + (uint32_t)(kb * 32 * RC_ROW);
    return *(const lds_bf16x8_t*)(uintptr_t)ad;
  };

  f32x16 a1[KB], a2[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      a1[kb][e] = 0.f;
      a2[kb][e] = 0.f;
    }

  // matrix phase: S^T of tile t for both queries, 16 KB MFMAs in KB
  // interleaved chains per query (one per 32-key block), K operands read
  // RC_PF steps ahead
  auto matrix_phase = [&](int t) INLINE {
    __builtin_amdgcn_s_setprio(1);
    const uint32_t slot = (uint32_t)((t & 1) * RC_TILE);
    bf16x8 ring[RC_PF];
#pragma unroll
    for (int i = 0; i < RC_PF; ++i) ring[i] = k_operand(slot, i % KB, i / KB);
    __builtin_amdgcn_sched_group_barrier(0x100, RC_PF, 0);
#pragma unroll
    for (int k = 0; k < 8 * KB; ++k) {
      const int c = k / KB, kb = k % KB;
      const bf16x8 cur = ring[k % RC_PF];
      if (k + RC_PF < 8 * KB)
        ring[k % RC_PF] = k_operand(slot, (k + RC_PF) % KB, (k + RC_PF) / KB);
      if (c == 0) {
        const f32x16 zero = {};
        a1[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, q1[0], zero, 0, 0, 0);
        a2[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, q2[0], zero, 0, 0, 0);
      } else {
        a1[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, q1[c], a1[kb], 0, 0, 0);
        a2[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, q2[c], a2[kb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (k + RC_PF < 8 * KB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  const float c2 = a.scale_log2;
  // running state per lane (both halves of a column share m)
  float m1 = -INFINITY, m2 = -INFINITY;
  float z1 = 0.f, z2 = 0.f, s12 = 0.f, s11 = 0.f, s22 = 0.f;

  // exponentials and sums of the scores in a1/a2 against m1, m2; with a
  // fetch tile ft >= 0, the wave's bursts of it go out between blocks
  auto tile_sums = [&](float& t1, float& t2, float& t12, float& t11, float& t22, int ft,
                       uint32_t skip) INLINE {
    const float nm1 = -m1, nm2 = -m2;
    t1 = t2 = t12 = t11 = t22 = 0.f;
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (ft >= 0 && u % 2 == 0) {
        fetch_burst(ft, u / 2, skip);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(a1[u][e], c2, nm1));
        const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(a2[u][e], c2, nm2));
        t1 += e1;
        t2 += e2;
        t12 = __builtin_fmaf(e1, e2, t12);
        t11 = __builtin_fmaf(e1, e1, t11);
        t22 = __builtin_fmaf(e2, e2, t22);
      }
    }
  };

  // vector phase of tile t (and fetch of tile ft unless skip)
  auto vector_phase = [&](int t, int ft, uint32_t skip) INLINE {
    const int valid = N - t * RC_KT;
    if (valid < RC_KT) {  // keys past N -> -inf
      const int lim = valid - 4 * half;
#pragma unroll
      for (int u = 0; u < KB; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // an integer select: no per-element compare masks
            const uint32_t keep = (uint32_t)(((u * 32 + 8 * i + e) - lim) >> 31);
            a1[u][4 * i + e] = __uint_as_float((__float_as_uint(a1[u][4 * i + e]) & keep) |
                                               (0xff800000u & ~keep));
            a2[u][4 * i + e] = __uint_as_float((__float_as_uint(a2[u][4 * i + e]) & keep) |
                                               (0xff800000u & ~keep));
          }
    }
    float t1, t2, t12, t11, t22;
    tile_sums(t1, t2, t12, t11, t22, ft, skip);
    // (t1 + t2 + t12 in the test only keeps every sum ahead of the branch,
    // so the exponentials need not stay live across it)
    const bool bad = !(t11 <= RC_LIMIT) || !(t22 <= RC_LIMIT) || !(t1 + t2 + t12 >= 0.f);
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {
      // exact tile max per query over both halves of the column
      float mx1 = -INFINITY, mx2 = -INFINITY;
#pragma unroll
      for (int u = 0; u < KB; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          mx1 = fmaxf(mx1, a1[u][e]);
          mx2 = fmaxf(mx2, a2[u][e]);
        }
      mx1 = max_across_halves(mx1) * c2;
      mx2 = max_across_halves(mx2) * c2;
      const float n1 = fmaxf(m1, mx1), n2 = fmaxf(m2, mx2);
      // m = -inf (nothing summed yet) gives factor 0
      const float al1 = __builtin_amdgcn_exp2f(m1 - n1), al2 = __builtin_amdgcn_exp2f(m2 - n2);
      z1 *= al1;
      z2 *= al2;
      s12 *= al1 * al2;
      s11 *= al1 * al1;
      s22 *= al2 * al2;
      m1 = n1;
      m2 = n2;
      tile_sums(t1, t2, t12, t11, t22, -1, 1u);
    }
    z1 += t1;
    z2 += t2;
    s12 += t12;
    s11 += t11;
    s22 += t22;
  };

  // ---- prologue: tile 0 into slot 0 by group 1
  fetch(0, grp == 1 ? 0u : 1u);
  __builtin_amdgcn_s_waitcnt(WAIT_VM0);
  BARRIER();

  if (grp == 0) {
    for (int t = 0; t < T; ++t) {
      if (active) matrix_phase(t);
      BARRIER();
      if (active) vector_phase(t, -1, 1u);
      BARRIER();
    }
  } else {
    // phase 0: fetch tile 1
    fetch(1, T > 1 ? 0u : 1u);
    BARRIER();
    for (int t = 0; t < T; ++t) {
      if (active) matrix_phase(t);
      // tile t + 1 (fetched in the previous vector phase) has landed
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      BARRIER();
      const uint32_t skip = t + 2 < T ? 0u : 1u;
      if (active) {
        vector_phase(t, t + 2, skip);
      } else {
        fetch(t + 2, skip);
      }
      if (t + 1 < T) BARRIER();
    }
  }

  // both halves of a column (same m), then the probability-row sums
  z1 += __shfl_xor(z1, 32);
  z2 += __shfl_xor(z2, 32);
  s12 += __shfl_xor(s12, 32);
  s11 += __shfl_xor(s11, 32);
  s22 += __shfl_xor(s22, 32);
  float d12 = s12 / (z1 * z2), d11 = s11 / (z1 * z1), d22 = s22 / (z2 * z2);
  if constexpr (PACKED) {
    // this column's sums; the per-row additions follow in row_cos_finish
    if (col_ok && half == 0) {
      float* w = a.ws + ((int64_t)bh * cols + col) * 3;
      w[0] = d12;
      w[1] = d11;
      w[2] = d22;
    }
    return;
  }
  if (!col_ok) d12 = d11 = d22 = 0.f;
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) {
    d12 += __shfl_xor(d12, off);
    d11 += __shfl_xor(d11, off);
    d22 += __shfl_xor(d22, off);
  }
  if (lane == 0) {
    red[wave][0] = d12;
    red[wave][1] = d11;
    red[wave][2] = d22;
  }
  __syncthreads();
  // one thread per row of the workgroup
  if (tid < 2 * rpg) {
    const int g = tid / rpg, r = tid - g * rpg;
    const int j = (blk * 2 + g) * rpg + r;
    if (j < rows_total) {
      int fr, yr;
      row_of(j, fr, yr);
      float t12 = 0.f, t11 = 0.f, t22 = 0.f;
      for (int w = 4 * g + r * wpr; w < 4 * g + (r + 1) * wpr; ++w) {
        t12 += red[w][0];
        t11 += red[w][1];
        t22 += red[w][2];
      }
      a.cos[((int64_t)bh * a.T + fr) * a.gh + yr] = t12 / sqrtf(t11 * t22);
    }
  }
}

// packed schedule, second step: one thread per (prompt, head, non-anchor
// row) adds its columns' sums, x in order, and writes the cosine
__global__ void __launch_bounds__(256)
row_cos_finish(RowCosLaunch a, int64_t rows) {
  const int nna = a.gh - (a.gh + a.stride - 1) / a.stride;
  const int rows_total = a.T * nna;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bh = i / rows_total;
    const int j = (int)(i - bh * rows_total);
    const float* w = a.ws + (bh * rows_total + j) * (int64_t)a.gw * 3;
    float t12 = 0.f, t11 = 0.f, t22 = 0.f;
    for (int x = 0; x < a.gw; ++x) {
      t12 += w[3 * x];
      t11 += w[3 * x + 1];
      t22 += w[3 * x + 2];
    }
    const int fr = j / nna, jj = j - fr * nna;
    const int yr = (jj / (a.stride - 1)) * a.stride + 1 + jj % (a.stride - 1);
    a.cos[(bh * a.T + fr) * a.gh + yr] = t12 / sqrtf(t11 * t22);
  }
}

}  // namespace

int64_t row_cos_workspace_bytes(int64_t B, int64_t H, int64_t T, int32_t gh, int32_t gw,
                                int32_t stride) {
  const int64_t nna = gh - (gh + stride - 1) / stride;
  return 12 * B * H * T * nna * gw;
}

bool row_cos_tuned_fits(const RowCosLaunch& a) {
  const int nna = a.gh - (a.gh + a.stride - 1) / a.stride;
  return a.d == RC_D && a.dtype == 0 && (a.ws != nullptr || a.gw <= 128) && nna > 0 &&
         (int64_t)a.N * RC_ROW < (int64_t)1 << 31 &&
         (int64_t)a.T * nna * a.gw < (int64_t)1 << 30;
}

int launch_row_cos_tuned(const RowCosLaunch& a, void* stream) {
  const hipStream_t s = (hipStream_t)stream;
  const int nna = a.gh - (a.gh + a.stride - 1) / a.stride;
  const int64_t rows_total = (int64_t)a.T * nna;
  int64_t blocks;
  if (a.ws != nullptr) {
    blocks = ((rows_total * a.gw + 31) / 32 + 7) / 8;
  } else {
    const int rpg = 4 / ((a.gw + 31) / 32);
    blocks = (rows_total + 2 * rpg - 1) / (2 * rpg);
  }
  const int64_t grid = blocks * a.H * a.B;
  if (grid == 0) return hipSuccess;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (a.ws == nullptr) {
    hipLaunchKernelGGL((row_cos_bf16_d128<RC_KB, false>), dim3((unsigned)grid), dim3(512), 0, s,
                       a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((row_cos_bf16_d128<RC_KB, true>), dim3((unsigned)grid), dim3(512), 0, s, a);
  const int64_t rows = rows_total * a.H * a.B;
  int64_t fgrid = (rows + 255) / 256;
  if (fgrid > 1 << 16) fgrid = 1 << 16;
  hipLaunchKernelGGL(row_cos_finish, dim3((unsigned)fgrid), dim3(256), 0, s, a, rows);
  return hipGetLastError();
}

}  // namespace bsattn
