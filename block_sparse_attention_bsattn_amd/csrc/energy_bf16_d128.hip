// Block energies of full softmax attention, tuned instance: bf16 Q and K,
// head dim 128, 128 x 128 blocks (CalibAtt page, "A. Fase di Calibrazione"
// step 1).  E[b, h, i, j] = sum over the query rows of tile i and the keys of
// tile j of the softmax probabilities over all N keys.  In the exp2 domain
// x = s * scale * log2(e), with l = sum_k 2^(x_k - m) a row's normaliser
// relative to m, a row contributes 2^(x - m) / l to E.
//
// One sweep (with a workspace): per row and key tile, b_j = sum of
// 2^(x - m) over the tile's keys goes to the workspace as the sweep passes
// (the row's l accumulates alongside); after the sweep the workgroup
// divides each row's b_j by its l and adds them per tile: E[i, j] =
// sum_rows b_j / l.  Workgroups are persistent, at most EN_SLOTS of them,
// each with its slot of the workspace (2 x 128 rows x T floats).
// Two sweeps (no workspace): sweep 1 computes L = m + log2(l) per row,
// sweep 2 sums p = 2^(x - L) per tile (each wave over its 32 rows, the
// group's four waves' sums added in LDS), twice the matrix and exponential
// work.
//
// Lazy max: a tile's exponentials are taken against the current m; only
// when a lane's tile sum exceeds 2^64 or is not finite (the first tile, m =
// -inf) does the wave take the tile's exact max (over both lane halves of
// each row), rescale l (and, in one sweep, the row's b_j stored so far) and
// redo the tile.  No max is taken per score.
//
// Mapping onto CDNA4 (gfx950)
// ---------------------------
//  * Workgroup = 8 waves in two groups of 4 (waves w and w + 4 share a
//    SIMD); group g owns query tile 2p + g (4 waves x 32 rows).  Both groups
//    walk the same key tiles, so each staged K tile serves 256 query rows.
//    Ping-pong: in phase 2t group 0 computes the scores of step t (matrix
//    phase: S^T = K Q^T, 32 MFMAs v_mfma_f32_32x32x16_bf16, A = K rows from
//    LDS, B = Q^T in VGPRs; lane l holds row l % 32 and 64 keys of the tile)
//    while group 1 runs the exponentials of step t - 1 (vector phase); in
//    phase 2t + 1 the roles swap.  Per score the vector work (argument,
//    exponential, sum) and the matrix work are about equal, so the two
//    overlap.  128 VGPRs: two workgroups share a CU (4 waves a SIMD).
//  * K tiles (128 keys, 32 KB) are double-buffered in LDS and fetched
//    straight to LDS (buffer_load ... lds) by group 1 in its vector phase:
//    in phase 2t it fetches step t + 1's tile into the slot step t - 1
//    used, and waits for it at the end of its matrix phase 2t + 1, a phase
//    before group 0 reads it.  Rows past N lie outside the buffer range and
//    arrive as zeros; the vector phase masks their scores to -inf.
//  * LDS rows are 256 B with 16-byte chunk c of row R at position
//    c ^ swz(R): conflict-free for the K reader.
//  * The grid is remapped so each XCD (own L2) walks contiguous ranges of
//    (prompt, head, query-tile pair): workgroups on one XCD share their
//    head's key stream in its L2.
#include <hip/hip_runtime.h>

#include <math.h>

#include <type_traits>

#include "bsattn_internal.h"
#include "cdna4_lds.h"

namespace bsattn {
namespace {

constexpr int EN_D = 128;
constexpr int EN_BT = 128;                   // tile: query rows and keys
constexpr int EN_ROW = EN_D * 2;             // 256 bytes per key row
constexpr int EN_TILE = EN_BT * EN_ROW;      // 32 KB
constexpr int EN_PF = 4;                     // MFMA operand read-ahead
constexpr int EN_NXCD = 8;
constexpr int EN_SLOTS = 512;                // one sweep: persistent workgroups at most
// tile sums above this (or not finite): exact max for the tile (sweep 1)
constexpr float EN_LIMIT = 18446744073709551616.0f;  // 2^64

// ONE: one sweep with the workspace; otherwise two sweeps
template <bool ONE>
__global__ void __launch_bounds__(512, 4)
energy_bf16_d128(EnergyLaunch a) {
  // K slots [0, 32K) and [32K, 64K) of a 64 KB-aligned array: bit 15 of an
  // address picks the slot
  __shared__ __attribute__((aligned(65536))) char kslots[2 * EN_TILE];
  __shared__ float wsum[2][2][4];  // two sweeps: [group][step parity][wave] tile sums
  __shared__ float invl[2][128];   // one sweep: [group][row] 1 / l

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int wg = wave & 3;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  lds_char_t* const kl = uniform_lds((lds_char_t*)kslots);
  const uint32_t kl32 = (uint32_t)(uintptr_t)kl;

  // ---- workgroups -> items (prompt, head, query-tile pair), XCD-contiguous
  const int T = a.tiles;
  const int pairs = (T + 1) / 2;
  const uint32_t items = (uint32_t)pairs * (uint32_t)(a.B * a.H);
  const uint32_t G = gridDim.x;
  uint32_t logical;
  {
    const uint32_t hw = blockIdx.x;
    const uint32_t q8 = G / EN_NXCD, r8 = G % EN_NXCD, xcd = hw % EN_NXCD, slot = hw / EN_NXCD;
    const uint32_t lo = xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8;
    logical = lo + slot;
  }
  const int N = a.N;
  // one sweep: this workgroup's workspace slot, [group][row][tile]
  float* const wslot = ONE ? a.ws + (int64_t)logical * 2 * 128 * T : nullptr;
  for (uint32_t item = logical; item < items; item += G) {
  const int pr = (int)(item % (uint32_t)pairs);
  const int bh = (int)(item / (uint32_t)pairs);  // b * H + h
  const int qt = 2 * pr + grp;
  const bool active = qt < T;  // wave-uniform
  const int64_t head_row = (int64_t)bh * N;
  const int qrow = qt * EN_BT + wg * 32 + l32;
  const bool row_ok = active && qrow < N;

  bf16x8 qf[8];
  {
    const __bf16* qb = reinterpret_cast<const __bf16*>(a.q) + (head_row + qrow) * EN_D;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (row_ok) {
        qf[c] = *reinterpret_cast<const bf16x8*>(qb + c * 16 + half * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[c][e] = (__bf16)0.f;
      }
    }
  }

  // ---- K fetches: load i (0..7) of group-1 wave wg fills LDS bytes
  // [(8 wg + i) * 1024, +1024) of a slot, rows 32 wg + 4i + (0..3); lane l
  // writes chunk position l % 16 of row 32 wg + 4i + l / 16 and so fetches
  // global chunk (l % 16) ^ swz(row) = (l % 16) ^ (4 (l / 16) + i % 4)
  const int steps = ONE ? T : 2 * T;  // two sweeps: tiles 0 .. T-1, then again
  const i32x4 krs = raw_rsrc(reinterpret_cast<const char*>(a.k) + head_row * EN_ROW,
                             N * EN_ROW);
  uint32_t ld_off[4];
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const int r = 32 * wg + (lane >> 4);
    const int c = (lane & 15) ^ (((lane >> 4) << 2) | i4);
    ld_off[i4] = (uint32_t)r * EN_ROW + (uint32_t)(c * 16);
  }
  // burst p (0, 1) of this wave's share of step st's tile into slot st & 1
  auto fetch_burst = [&](int st, int p, uint32_t skip) INLINE {
    const int tile = st < T ? st : st - T;
    const uint32_t m0 = kl32 + (uint32_t)((st & 1) * EN_TILE) + (uint32_t)((8 * wg + 4 * p) * 1024);
    dma_burst4(krs, m0, ld_off, (uint32_t)tile * EN_TILE + (uint32_t)(p * 4096),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)skip));
  };

  // K reader: key row kb * 32 + l32, chunk 2c + half, slot 0
  const int ks = swz(l32);
  const uint32_t kr = kl32 + (uint32_t)(l32 * EN_ROW + ((ks >> 1) << 5) + ((half ^ (ks & 1)) << 4));
  auto k_operand = [&](uint32_t slot, int kb, int c) INLINE {
    const uint32_t ad = ((kr | slot) ^ (uint32_t)(c << 5)) + (uint32_t)(kb * 32 * EN_ROW);
    return *(const lds_bf16x8_t*)(uintptr_t)ad;
  };

  f32x16 s[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;

  // matrix phase: S^T of step st's tile, 32 MFMAs in four interleaved
  // chains (one per 32-key block), K operands read EN_PF steps ahead
  auto matrix_phase = [&](int st) INLINE {
    __builtin_amdgcn_s_setprio(1);
    const uint32_t slot = (uint32_t)((st & 1) * EN_TILE);
    bf16x8 ring[EN_PF];
#pragma unroll
    for (int i = 0; i < EN_PF; ++i) ring[i] = k_operand(slot, i & 3, i >> 2);
    __builtin_amdgcn_sched_group_barrier(0x100, EN_PF, 0);
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int c = k >> 2, kb = k & 3;
      const bf16x8 cur = ring[k % EN_PF];
      if (k + EN_PF < 32) ring[k % EN_PF] = k_operand(slot, (k + EN_PF) & 3, (k + EN_PF) >> 2);
      if (c == 0) {
        const f32x16 zero = {};
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[0], zero, 0, 0, 0);
      } else {
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[c], s[kb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (k + EN_PF < 32) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  const float c2 = a.scale_log2;
  float m = -INFINITY;  // sweep 1: running max (shared by both lane halves)
  float l = 0.f;        // sweep 1: this lane's share of sum 2^(x - m)
  float L = 0.f;        // sweep 2: log2 of the row's normaliser
  float* const ebase = a.energy + ((int64_t)bh * T + qt) * T;
  // one sweep: the workspace slot as a buffer resource, this lane's row at
  // byte offset wrow, tile j at + 4 j
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      ONE ? (void*)wslot : (void*)a.energy, (short)0, ONE ? 2 * 128 * T * 4 : 0, 0x00020000);
  const int wrow = (grp * 128 + wg * 32 + l32) * T * 4;

  // sum of 2^(x * c2 - ref) over the lane's 64 scores; fetch of step ft's
  // tile (unless ft < 0) in two bursts between blocks
  auto tile_sum = [&](float ref, int ft, uint32_t skip) INLINE {
    const float nref = -ref;
    float t = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (ft >= 0 && (kb == 0 || kb == 2)) {
        fetch_burst(ft, kb >> 1, skip);
        __builtin_amdgcn_sched_barrier(0);
      }
      float tk = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        tk += __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], c2, nref));
      t += tk;
    }
    return t;
  };

  // vector phase of step st of sweep SW (and fetch of step ft unless skip)
  auto vector_phase = [&](auto sweep, int st, int ft, uint32_t skip) INLINE {
    constexpr int SW = decltype(sweep)::value;
    const int tile = SW == 1 ? st : st - T;
    const int valid = N - tile * EN_BT;
    if (valid < EN_BT) {  // keys past N -> -inf
      const int lim = valid - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // an integer select: no per-element compare masks
            const uint32_t keep = (uint32_t)(((kb * 32 + 8 * i + e) - lim) >> 31);
            s[kb][4 * i + e] = __uint_as_float((__float_as_uint(s[kb][4 * i + e]) & keep) |
                                               (0xff800000u & ~keep));
          }
    }
    if constexpr (SW == 1) {
      // normaliser, lazy max
      float t = tile_sum(m, ft, skip);
      if (__builtin_amdgcn_ballot_w64(!(t <= EN_LIMIT)) != 0) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
        const float n = fmaxf(m, max_across_halves(mx) * c2);
        const float al = __builtin_amdgcn_exp2f(m - n);  // m = -inf: nothing summed yet
        l *= al;
        if constexpr (ONE) {
          // the row's tile sums stored so far move to the new max (this
          // wave's own stores: wait for them first)
          if (tile > 0) {
            __builtin_amdgcn_s_waitcnt(WAIT_VM0);
            if (half == 0)
              for (int j = 0; j < tile; ++j) {
                const float v = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(wrs, wrow, 4 * j, 0));
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v * al), wrs,
                                                      wrow, 4 * j, 0);
              }
          }
        }
        m = n;
        t = tile_sum(m, -1, 1u);
      }
      l += t;
      if constexpr (ONE) {
        const float b = sum_across_halves(t);  // the row's sum over the tile
        if (half == 0)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, b), wrs, wrow,
                                                4 * tile, 0);
      }
    } else {
      // the previous tile's energy (its four sums are in LDS since the
      // barrier before this phase), then this tile's sums
      if (wg == 0 && lane == 0 && tile > 0) {
        const float* w = wsum[grp][(tile - 1) & 1];
        ebase[tile - 1] = (w[0] + w[1]) + (w[2] + w[3]);
      }
      float ps = tile_sum(L, ft, skip);
      if (!row_ok) ps = 0.f;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off);
      if (lane == 0) wsum[grp][tile & 1][wg] = ps;
    }
  };
  // after sweep 1: both halves of the row, then L
  auto finish_sweep1 = [&]() INLINE {
    const float lt = sum_across_halves(l);
    L = m + log2f(lt);
  };
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;

  // ---- prologue: step 0's tile into slot 0 by all 8 waves (group g: burst g)
  fetch_burst(0, grp, 0u);
  __builtin_amdgcn_s_waitcnt(WAIT_VM0);
  BARRIER();

  if (grp == 0) {
    for (int st = 0; st < T; ++st) {
      if (active) matrix_phase(st);
      BARRIER();
      if (active) vector_phase(S1(), st, -1, 1u);
      BARRIER();
    }
    if constexpr (!ONE) {
      finish_sweep1();
      for (int st = T; st < steps; ++st) {
        if (active) matrix_phase(st);
        BARRIER();
        if (active) vector_phase(S2(), st, -1, 1u);
        BARRIER();
      }
    }
  } else {
    // phase 0: fetch step 1's tile
    fetch_burst(1, 0, steps > 1 ? 0u : 1u);
    fetch_burst(1, 1, steps > 1 ? 0u : 1u);
    BARRIER();
    // matrix phase of step st, wait for step st + 1's tile (fetched in the
    // previous vector phase), barrier, vector phase with the fetch of step
    // st + 2's tile
    auto step = [&](auto sweep, int st) INLINE {
      if (active) matrix_phase(st);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      BARRIER();
      const uint32_t skip = st + 2 < steps ? 0u : 1u;
      if (active) {
        vector_phase(sweep, st, st + 2, skip);
      } else {
        fetch_burst(st + 2, 0, skip);
        fetch_burst(st + 2, 1, skip);
      }
    };
    for (int st = 0; st < T; ++st) {
      step(S1(), st);
      if (ONE ? st + 1 < T : true) BARRIER();
    }
    if constexpr (!ONE) {
      finish_sweep1();
      for (int st = T; st < steps; ++st) {
        step(S2(), st);
        if (st + 1 < steps) BARRIER();
      }
    }
  }
  if constexpr (ONE) {
    // E[qt, j] = sum over the group's rows of b_j / l: 1 / l per row to
    // LDS, then thread r of the group (r = 0 .. 255) adds tile j = r, r +
    // 256, ... over the 128 rows, the rows' stores visible after the
    // barrier (same workgroup, same CU)
    const float lt = sum_across_halves(l);
    if (half == 0) invl[grp][wg * 32 + l32] = row_ok ? 1.0f / lt : 0.0f;
    __syncthreads();
    if (active) {
      const float* const wg0 = wslot + (int64_t)grp * 128 * T;
      for (int j = wg * 64 + lane; j < T; j += 256) {
        float e0 = 0.f, e1 = 0.f;
#pragma unroll 8
        for (int r = 0; r < 128; r += 2) {
          e0 = __builtin_fmaf(wg0[(int64_t)r * T + j], invl[grp][r], e0);
          e1 = __builtin_fmaf(wg0[(int64_t)(r + 1) * T + j], invl[grp][r + 1], e1);
        }
        ebase[j] = e0 + e1;
      }
    }
  } else {
    // the last tile's energy
    __syncthreads();
    if (active && wg == 0 && lane == 0) {
      const float* w = wsum[grp][(T - 1) & 1];
      ebase[T - 1] = (w[0] + w[1]) + (w[2] + w[3]);
    }
  }
  // the next item's prologue refills K slot 0 and, in one sweep, the
  // workspace slot and invl
  __syncthreads();
  }  // items
}

}  // namespace

int64_t energy_workspace_bytes(int64_t B, int64_t H, int64_t N, int32_t tile) {
  if (tile != EN_BT) return 0;
  const int64_t T = (N + EN_BT - 1) / EN_BT;
  int64_t slots = (T + 1) / 2 * B * H;
  if (slots > EN_SLOTS) slots = EN_SLOTS;
  return slots * 2 * 128 * T * (int64_t)sizeof(float);
}

bool energy_tuned_fits(const EnergyLaunch& a) {
  return a.d == EN_D && a.tile == EN_BT && a.dtype == 0 &&
         (int64_t)a.N * EN_ROW < (int64_t)1 << 31;
}

int launch_energy_tuned(const EnergyLaunch& a, void* stream) {
  const int64_t items = (int64_t)((a.tiles + 1) / 2) * a.H * a.B;
  if (items == 0) return hipSuccess;
  if (items > INT32_MAX) return hipErrorInvalidValue;
  if (a.ws == nullptr) {
    hipLaunchKernelGGL(energy_bf16_d128<false>, dim3((unsigned)items), dim3(512), 0,
                       (hipStream_t)stream, a);
  } else {
    const int64_t grid = items < EN_SLOTS ? items : EN_SLOTS;
    hipLaunchKernelGGL(energy_bf16_d128<true>, dim3((unsigned)grid), dim3(512), 0,
                       (hipStream_t)stream, a);
  }
  return hipGetLastError();
}

}  // namespace bsattn
