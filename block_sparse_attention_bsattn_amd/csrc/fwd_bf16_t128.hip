// Block-sparse attention forward, tuned instance: bf16 Q/K/V/O, head dim 128,
// 128x128 tiles (the video workloads' block size: CalibAtt page, "A. Fase di
// Calibrazione"; attention only over each query tile's listed key tiles:
// CalibAtt page, "B. Fase di Inferenza", and LVSA page, "Meccanismo Core").
//
// Math per query row (online softmax, Milakov and Gimelshein 2018), in the
// exp2 domain x = s * scale * log2(e):
//   m' = max(m, max_j x_j);  P = 2^(x - m');  l = l 2^(m - m') + sum P;
//   O  = O 2^(m - m') + P V;   finally O / l.
// The running max is only moved when a tile's max exceeds it by more than
// TAU (then every value is rescaled); otherwise P may exceed 1 by at most
// 2^TAU, which is harmless in fp32 and bf16, and the result is unchanged.
//
// Mapping onto CDNA4 (gfx950)
// ---------------------------
// On a SIMD, matrix-core work of one wave overlaps the vector-ALU work of
// another wave almost perfectly, while inside one wave the two mostly
// serialise.  The kernel is therefore a two-group ping-pong:
//   * workgroup = 8 waves = two groups of 4; group g owns query tile
//     2p + g (128 rows, 32 per wave).  Waves w and w + 4 share a SIMD.
//   * time is cut into phases separated by workgroup barriers.  In every
//     phase one group runs its matrix phase (O += P_{t-1} V_{t-1}, then
//     S_t = K_t Q^T: 64 MFMAs per wave) while the other runs its vector phase
//     (the online softmax of S_t); the roles swap at each barrier, so every
//     SIMD always has one MFMA wave and one VALU wave.
//   * each group owns one K and one V buffer in LDS (4 x 32 KB = 128 KB).
//     At the start of its vector phase a group fetches K_{t+1} and V_t with
//     buffer_load ... lds (16 B per lane, no VGPR staging; rows past the
//     sequence end are outside the buffer range and arrive as zeros), and
//     waits for them at the end of that phase.
//   * LDS layout: row-major, 256 B per row, 16-byte chunk c of row R at chunk
//     position c ^ S(R), S(R) = 4*(R % 4) + (R / 4) % 4: conflict-free for the
//     K reader (16 consecutive rows, one chunk column) and for the
//     transposing V reader (4 consecutive rows x 4 chunks).
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T
//     held in VGPRs).  Lane l holds query l % 32 and, per 32-key block, keys
//     8i + 4(l/32) + e, so a row max needs one swap between lane halves
//     (v_permlane32_swap).
//   * O^T += V^T P^T on the same MFMA, P straight from the score registers
//     with the reduction index permuted to the keys the lane holds.  The V^T
//     operand comes from row-major V via ds_read_b64_tr_b16 (lane i of each
//     16-lane group receives element i % 4 of source lane 4e + i / 4).
//   * Row sums use v_dot2 on the bf16-rounded P, the values PV consumes.
//   * Workgroups are remapped so each XCD (own L2) walks a contiguous range
//     of (head, query-tile pair); neighbouring query tiles share most of
//     their key tiles.
#include <hip/hip_runtime.h>

#include <math.h>

#include "bsattn_internal.h"

namespace bsattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;
typedef __attribute__((address_space(3))) char lds_char_t;
// Read-only, wave-uniform data (the active lists) goes through the constant
// address space, i.e. the scalar path, and never waits on the vector-memory
// counter that the K/V fetches use.
typedef const __attribute__((address_space(4))) int32_t* sconst_i32;

constexpr int BT = 128;                     // tile rows / columns
constexpr int D = 128;                      // head dim
constexpr int ROW_BYTES = D * 2;            // 256
constexpr int TILE_BYTES = BT * ROW_BYTES;  // 32 KB
constexpr float TAU = 8.0f;                 // lazy-rescale threshold (log2 units)
constexpr int NXCD = 8;

// Workgroup barrier that first drains this wave's LDS reads: a buffer that a
// barrier releases for refilling must have no read of it still queued.
#define BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")
#define WAIT_VM0() asm volatile("s_waitcnt vmcnt(0)" ::: "memory")

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// max over the two lanes (l, l ^ 32) that hold the same query row
__device__ __forceinline__ float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ int list_len(sconst_i32 row_ptr, int64_t cap, int mrow, int& begin) {
  int64_t b0 = row_ptr[mrow], e0 = row_ptr[mrow + 1];
  if (b0 < 0) b0 = 0;
  if (e0 > cap) e0 = cap;
  begin = (int)b0;
  return e0 > b0 ? (int)(e0 - b0) : 0;
}

__global__ void __launch_bounds__(512, 1)
fwd_bf16_t128_d128(FwdLaunch a) {
  // per group one K tile and one V tile; four distinct LDS objects, so the
  // compiler never mistakes a pending fetch into one for a read of another
  __shared__ __attribute__((aligned(1024))) char kbuf0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char kbuf1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf1[TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index via readfirstlane: the compiler then knows it (and all that
  // derives from it: group, list bounds, tile indices) is wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  const int grp = wave >> 2;  // 0 or 1
  const int wg = wave & 3;    // wave within the group
  const int half = lane >> 5;
  const int l32 = lane & 31;
  // Wave-uniform LDS bases, kept in the LDS address space throughout (the
  // LDS-DMA destination M0 is scalar; offset 0 is a valid LDS address, so
  // these must never pass through a generic pointer, where 0 means null).
  lds_char_t* const kbuf = (lds_char_t*)(uintptr_t)__builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(grp ? (lds_char_t*)kbuf1 : (lds_char_t*)kbuf0));
  lds_char_t* const vbuf = (lds_char_t*)(uintptr_t)__builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(grp ? (lds_char_t*)vbuf1 : (lds_char_t*)vbuf0));

  // ---- XCD-aware remap of the 1-D grid onto (batch*head, query-tile pair)
  const uint32_t G = gridDim.x, hw = blockIdx.x;
  const uint32_t q8 = G / NXCD, r8 = G % NXCD, xcd = hw % NXCD, slot = hw / NXCD;
  const uint32_t logical =
      (xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8) + slot;
  const uint32_t pairs = (uint32_t)(a.tiles + 1) >> 1;
  const int bh = (int)(logical / pairs);
  const int qt0 = 2 * (int)(logical % pairs);
  const int qt = qt0 + grp;
  const int h = bh % a.H;
  const int N = a.N;
  const int64_t head_row = (int64_t)bh * N;

  // ---- active lists of both groups (both are needed to agree on the
  // number of phases)
  const sconst_i32 row_ptr = (sconst_i32)(uintptr_t)a.row_ptr;
  const sconst_i32 col_idx = (sconst_i32)(uintptr_t)a.col_idx;
  const int hrow = (a.mask_heads == 1 ? 0 : h) * a.tiles;
  int jb0 = 0, jb1 = 0;
  const int nA = list_len(row_ptr, a.col_cap, hrow + qt0, jb0);
  const int nB = qt0 + 1 < a.tiles ? list_len(row_ptr, a.col_cap, hrow + qt0 + 1, jb1) : 0;
  const int n = grp ? nB : nA;
  const int jb = grp ? jb1 : jb0;
  // group 0 has matrix phases at even indices 0..2nA, group 1 at odd
  // indices 1..2nB+1
  const int phases = max(2 * nA, 2 * nB + 1) + 1;

  // ---- Q^T operand: lane holds q[row l%32][8 d values], 8 chunks of 16 d
  const bool q_tile_real = qt < a.tiles;
  const int qrow = qt * BT + wg * 32 + l32;
  bf16x8 qf[8];
  {
    const __bf16* qptr =
        reinterpret_cast<const __bf16*>(a.q) + (head_row + qrow) * D + half * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (q_tile_real && qrow < N) {
        qf[c] = *reinterpret_cast<const bf16x8*>(qptr + c * 16);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[c][e] = (__bf16)0.f;
      }
    }
  }

  // ---- buffer resources for this head's K and V rows
  const char* kbase = reinterpret_cast<const char*>(a.k) + head_row * ROW_BYTES;
  const char* vbase = reinterpret_cast<const char*>(a.v) + head_row * ROW_BYTES;
  const int nbytes = N * ROW_BYTES;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, nbytes, 0x00020000);

  // Direct-load offsets.  Load i (0..7) of wave wg fills LDS bytes
  // [(8 wg + i) * 1024, +1024): rows 32 wg + 4i + (0..3).  Lane l writes
  // chunk position l % 16 of row 32 wg + 4i + l / 16, so it fetches global
  // chunk (l % 16) ^ S(row), S(row) = 4 (l / 16) + i % 4.
  uint32_t ld_off[4];
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const int r = 32 * wg + (lane >> 4);
    const int c = (lane & 15) ^ (((lane >> 4) << 2) | i4);
    ld_off[i4] = (uint32_t)(r * ROW_BYTES + c * 16);
  }
  // key tile of list entry t; an index outside [0, Tk) is fetched from past
  // the buffer end (zeros) and all its scores are discarded, i.e. skipped
  auto tile_of = [&](int t) { return col_idx[jb + t]; };
  auto fetch_tile = [&](const __amdgpu_buffer_rsrc_t& rs, lds_char_t* buf, int j) {
    const uint32_t toff =
        (j >= 0 && j < a.tiles) ? (uint32_t)j * TILE_BYTES : 0x80000000u;
    // load i = 4 ih + il: the immediate offset 1024 il applies to both the
    // global and the LDS address, so only two M0 / soffset values are needed
#define BSATTN_FETCH4(ih)                                                        \
  do {                                                                           \
    lds_void_t* dst = (lds_void_t*)(buf + (8 * wg + 4 * (ih)) * 1024);           \
    const uint32_t so = toff + 4096 * (ih);                                      \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, ld_off[0], so, 0, 0);    \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, ld_off[1], so, 1024, 0); \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, ld_off[2], so, 2048, 0); \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, ld_off[3], so, 3072, 0); \
  } while (0)
    BSATTN_FETCH4(0);
    BSATTN_FETCH4(1);
#undef BSATTN_FETCH4
  };

  // K reader: lane reads key row kb*32 + l%32, chunk 2c + half.
  // Per-lane LDS addresses (base folded in once), so every read is one VGPR
  // plus an immediate offset.
  const int ks = swz(l32);
  lds_char_t* const kl = kbuf;
  lds_char_t* const vl = vbuf;
  lds_char_t* kr_addr[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
    kr_addr[c] = kl + (l32 * ROW_BYTES + (((2 * c + half) ^ ks) << 4));

  // V^T reader (ds_read_b64_tr_b16): source lane s (= l % 16) of 16-lane
  // group g16 (= l / 16) points at key row R0 + s/4, d = 32 db + 16 (g16%2) +
  // 4 (s%4); R0 = kb*32 + 8 i0 + 8 sec + 4 half.
  const int s16 = lane & 15;
  const int g16 = lane >> 4;
  lds_char_t* vr_addr[2][4];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int rrel = 8 * sec + 4 * half + (s16 >> 2);
      const int chunk = 4 * db + 2 * (g16 & 1) + ((s16 & 3) >> 1);
      const int sw = ((s16 >> 2) << 2) | ((2 * sec + half) & 3);
      vr_addr[sec][db] = vl + (rrel * ROW_BYTES + ((chunk ^ sw) << 4) + 8 * (s16 & 1));
    }

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  // S_t^T scores; after the softmax the same registers hold P_t as packed
  // bf16 pairs: P for keys of chunk kc = 2 kb + hh sits in s[kb][4 hh .. 4 hh + 3]
  f32x16 s[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
  float m = -INFINITY;
  float l = 0.f;
  const float c2 = a.scale_log2;
  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};

  auto v_operand = [&](int kc, int db) {
    const int rows = (kc >> 1) * 32 * ROW_BYTES + (kc & 1) * 16 * ROW_BYTES;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vr_addr[0][db] + rows));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vr_addr[1][db] + rows));
    const bf16x4 lob = __builtin_bit_cast(bf16x4, lo);
    const bf16x4 hib = __builtin_bit_cast(bf16x4, hi);
    bf16x8 va;
    va[0] = lob[0]; va[1] = lob[1]; va[2] = lob[2]; va[3] = lob[3];
    va[4] = hib[0]; va[5] = hib[1]; va[6] = hib[2]; va[7] = hib[3];
    return va;
  };
  auto k_operand = [&](int kb, int c) {
    return *(const lds_bf16x8_t*)(kr_addr[c] + kb * 32 * ROW_BYTES);
  };
  auto p_operand = [&](int kc) {
    const f32x16& v = s[kc >> 1];
    const int o = (kc & 1) * 4;
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    const f32x4_t w = {v[o], v[o + 1], v[o + 2], v[o + 3]};
    return __builtin_bit_cast(bf16x8, w);
  };

  // matrix phase t: O += P_{t-1} V_{t-1} (if any), then S_t = K_t Q^T (if
  // any): two streams of 32 MFMAs.  Each MFMA's LDS operand is read PF steps
  // ahead from a rotating buffer, and the interleave (one MFMA, then the
  // reads for step + PF) is pinned with scheduling-group barriers, so the
  // matrix core does not wait for an LDS round trip.  The streams are kept
  // apart (P and the new scores share registers).
  constexpr int PF = 4;
  auto matrix_phase = [&](int t) {
    const bool do_pv = t >= 1 && t - 1 < n;
    const bool do_qk = t < n;
    // step k: 0..31 PV (kc = k / 4, db = k % 4), 32..63 QK (c = (k-32) / 4,
    // kb = (k-32) % 4)
    auto load = [&](int k) -> bf16x8 {
      return k < 32 ? v_operand(k >> 2, k & 3) : k_operand((k - 32) & 3, (k - 32) >> 2);
    };
    auto step = [&](int k, const bf16x8& opnd) {
      if (k < 32) {
        const int kc = k >> 2, db = k & 3;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd, p_operand(kc), oacc[db], 0, 0, 0);
      } else {
        const int c = (k - 32) >> 2, kb = (k - 32) & 3;
        if (c == 0) {
          const f32x16 zero = {};
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd, qf[0], zero, 0, 0, 0);
        } else {
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd, qf[c], s[kb], 0, 0, 0);
        }
      }
    };
#define BSATTN_MATRIX_STREAM(K0, K1)                                                  \
  do {                                                                                \
    bf16x8 ring[PF];                                                                  \
    _Pragma("unroll") for (int i = 0; i < PF; ++i) ring[i] = load((K0) + i);          \
    __builtin_amdgcn_sched_group_barrier(0x100, (K0) < 32 ? 2 * PF : PF, 0);          \
    _Pragma("unroll") for (int k = (K0); k < (K1); ++k) {                              \
      const bf16x8 cur = ring[(k - (K0)) % PF];                                       \
      if (k + PF < (K1)) ring[(k - (K0)) % PF] = load(k + PF);                        \
      step(k, cur);                                                                   \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                              \
      if (k + PF < (K1)) {                                                            \
        if (k + PF < 32) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);          \
        else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                      \
      }                                                                               \
    }                                                                                 \
  } while (0)
    if (do_pv) {
      BSATTN_MATRIX_STREAM(0, 32);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (do_qk) {
      BSATTN_MATRIX_STREAM(32, 64);
    }
#undef BSATTN_MATRIX_STREAM
  };

  // vector phase t: fetch K_{t+1} and V_t, then the online softmax of S_t
  auto vector_phase = [&](int t) {
    if (t + 1 < n) fetch_tile(krs, kbuf, tile_of(t + 1));
    if (t >= 0 && t < n) {
      const int j = tile_of(t);
      fetch_tile(vrs, vbuf, j);
      // keys past the end of the sequence never enter the softmax
      const int valid = (j >= 0 && j < a.tiles) ? N - j * BT : 0;
      if (valid < BT) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (kb * 32 + 8 * i + 4 * half + e >= valid) s[kb][4 * i + e] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
      mx = max_across_halves(mx) * c2;
      if (__any(mx > m + TAU)) {
        const float m_new = fmaxf(m, mx);
        // m_new = -inf only while every tile so far was skipped
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
      }
      const float msub = m == -INFINITY ? 0.f : m;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          // raw v_exp_f32: results below 2^-126 flush to zero, negligible
          // next to the row's largest weight (about 1)
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], c2, -msub));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e + 1], c2, -msub));
          bf16x2 pk;
          pk[0] = (__bf16)p0;
          pk[1] = (__bf16)p1;
          l = __builtin_amdgcn_fdot2_f32_bf16(pk, ones2, l, false);
          // packed pair e/2 of this block; position e/2 <= e was already read
          s[kb][e >> 1] = __builtin_bit_cast(float, pk);
        }
    }
    WAIT_VM0();  // this wave's share of K_{t+1} and V_t has landed
  };

  // ---- prologue: group 0 fetches its first K tile (group 1 does so in its
  // first vector phase)
  if (grp == 0 && n > 0) fetch_tile(krs, kbuf, tile_of(0));
  WAIT_VM0();
  BARRIER();

  // group 0: matrix phases at even phase indices; group 1 starts with a
  // vector phase and is one phase behind.  Both pass `phases` barriers.
  int ph = 0;
  if (grp == 1) {
    vector_phase(-1);
    BARRIER();
    ph = 1;
  }
  for (int t = 0; ph < phases; ++t) {
    matrix_phase(t);
    BARRIER();
    if (++ph >= phases) break;
    vector_phase(t);
    BARRIER();
    ++ph;
  }

  // ---- epilogue: O = O^T / l, rows past N (or of a missing tile) not written
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l),
                                                    false, false);
    l = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if (q_tile_real && qrow < N) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    __bf16* op = reinterpret_cast<__bf16*>(a.o) + (head_row + qrow) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 v;
        v[0] = (__bf16)(oacc[db][4 * i] * inv);
        v[1] = (__bf16)(oacc[db][4 * i + 1] * inv);
        v[2] = (__bf16)(oacc[db][4 * i + 2] * inv);
        v[3] = (__bf16)(oacc[db][4 * i + 3] * inv);
        *reinterpret_cast<bf16x4*>(op + db * 32 + 8 * i + 4 * half) = v;
      }
    if (a.lse != nullptr && half == 0)
      a.lse[head_row + qrow] =
          l > 0.f ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
  }
}

}  // namespace

int launch_fwd_bf16_t128_d128(const FwdLaunch& a, void* stream) {
  const int64_t blocks = (int64_t)a.B * a.H * ((a.tiles + 1) / 2);
  hipLaunchKernelGGL(fwd_bf16_t128_d128, dim3((unsigned)blocks), dim3(512), 0,
                     (hipStream_t)stream, a);
  return hipGetLastError();
}

}  // namespace bsattn
