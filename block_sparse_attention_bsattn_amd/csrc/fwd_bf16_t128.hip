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
// Mapping onto CDNA4 (gfx950):
//   * workgroup = 4 waves = one 128-row query tile; 2 workgroups per CU
//     (64 KB LDS each: one K tile + one V tile, both 128 x 128 bf16).
//   * K and V tiles travel HBM/L2 -> LDS with buffer_load ... lds (16 B per
//     lane, no VGPR staging); rows past the sequence end fall outside the
//     buffer range and arrive as zeros.  The next K tile is fetched while the
//     softmax runs, the next V tile while the next S = K Q^T runs.
//   * LDS layout: row-major, 256 B per row, 16-byte chunk c of row R stored at
//     chunk position c ^ S(R), S(R) = 4*(R % 4) + (R / 4) % 4.  Both readers
//     are then free of bank conflicts: the K reader (16 consecutive rows, one
//     chunk column) and the transposing V reader (4 consecutive rows x 4
//     chunks).
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T
//     held in VGPRs for the whole kernel).  Lane l holds query l % 32 and,
//     per 32-key block, keys 8i + 4(l/32) + e.
//   * O^T += V^T P^T on the same MFMA.  P comes straight from the score
//     registers; the MFMA's reduction index is permuted to the keys the lane
//     holds.  The V^T operand is read from row-major V with
//     ds_read_b64_tr_b16, which hands lane i of each 16-lane group element
//     (i % 4) of source lane 4e + i / 4: source lanes point at 4 consecutive
//     d values of 4 consecutive keys, so lane i receives 4 keys of d = i.
//   * Row sums use v_dot2 on the bf16-rounded P, the same values the PV
//     product consumes.
//   * Workgroups are remapped so that each XCD (its own L2) works through a
//     contiguous range of (head, query tile) pairs; neighbouring query tiles
//     read mostly the same key tiles.
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
// Read-only, wave-uniform data (the active lists) is read through the
// constant address space so that it goes down the scalar path and never
// waits on the vector-memory counter the K/V prefetch uses.
typedef const __attribute__((address_space(4))) int32_t* sconst_i32;

constexpr int BT = 128;          // tile rows / columns
constexpr int D = 128;           // head dim
constexpr int ROW_BYTES = D * 2; // 256
constexpr int TILE_BYTES = BT * ROW_BYTES;  // 32 KB
constexpr float TAU = 8.0f;      // lazy-rescale threshold (log2 units)
constexpr int NXCD = 8;

constexpr uint32_t waitcnt_vm(int n) {
  // gfx9 s_waitcnt encoding: vmcnt[3:0] + vmcnt[5:4] at [15:14],
  // expcnt [6:4] and lgkmcnt [11:8] left at their maxima (no wait).
  return (uint32_t)((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

#define WAIT_VM(n) __builtin_amdgcn_s_waitcnt(waitcnt_vm(n))
// Workgroup barrier that first drains this wave's LDS reads: a buffer that a
// barrier releases for refilling must have no read of it still queued.
#define BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

__global__ void __launch_bounds__(256, 2)
fwd_bf16_t128_d128(FwdLaunch a) {
  // two distinct LDS objects, so the compiler can tell a pending K fetch from
  // a V read (and vice versa) and does not serialise them
  __shared__ __attribute__((aligned(1024))) char kbuf[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf[TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // ---- XCD-aware remap of the 1-D grid onto (batch, head, query tile)
  const uint32_t G = gridDim.x, hw = blockIdx.x;
  const uint32_t q8 = G / NXCD, r8 = G % NXCD, xcd = hw % NXCD, slot = hw / NXCD;
  const uint32_t logical =
      (xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8) + slot;
  const int qt = (int)(logical % (uint32_t)a.tiles);
  const int bh = (int)(logical / (uint32_t)a.tiles);
  const int h = bh % a.H;
  const int N = a.N;
  const int64_t head_row = (int64_t)bh * N;

  // ---- Q^T operand: lane holds q[row l%32][8 d values], 8 chunks of 16 d
  const int qrow = qt * BT + wave * 32 + l32;
  const __bf16* qptr = reinterpret_cast<const __bf16*>(a.q) + (head_row + qrow) * D + half * 8;
  bf16x8 qf[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if (qrow < N) {
      qf[c] = *reinterpret_cast<const bf16x8*>(qptr + c * 16);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[c][e] = (__bf16)0.f;
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

  // Direct-load offsets.  Load i (0..7) of wave w fills LDS bytes
  // [(8w + i) * 1024, +1024): rows 32w + 4i + (0..3).  Lane l writes LDS
  // chunk position l % 16 of row 32w + 4i + l / 16, so it fetches global
  // chunk (l % 16) ^ S(row); S(row) = 4 (l / 16) + i % 4.
  uint32_t ld_off[4];
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const int r = 32 * wave + (lane >> 4);
    const int c = (lane & 15) ^ (((lane >> 4) << 2) | i4);
    ld_off[i4] = (uint32_t)(r * ROW_BYTES + c * 16);
  }
  auto issue_tile = [&](const __amdgpu_buffer_rsrc_t& rs, char* buf, int j) {
    const uint32_t toff = (uint32_t)j * TILE_BYTES;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (lds_void_t*)(buf + (8 * wave + i) * 1024), 16, ld_off[i & 3],
          toff + 1024 * i, 0, 0);
    }
  };

  // K reader: lane reads key row kb*32 + l%32, chunk 2c + half.
  const int krow = l32;
  const int ks = swz(krow);
  uint32_t kr_off[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
    kr_off[c] = (uint32_t)(krow * ROW_BYTES + (((2 * c + half) ^ ks) << 4));

  // V^T reader (ds_read_b64_tr_b16): source lane s (= l % 16) of group g
  // (= l / 16) points at key row R0 + s/4, d = 32 db + 16 (g%2) + 4 (s%4);
  // R0 = kb*32 + 8 i0 + 8 sec + 4 half.
  const int s16 = lane & 15;
  const int g = lane >> 4;
  uint32_t vr_off[2][4];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int rrel = 8 * sec + 4 * half + (s16 >> 2);
      const int chunk = 4 * db + 2 * (g & 1) + ((s16 & 3) >> 1);
      const int sw = ((s16 >> 2) << 2) | ((2 * sec + half) & 3);
      vr_off[sec][db] = (uint32_t)(rrel * ROW_BYTES + ((chunk ^ sw) << 4) + 8 * (s16 & 1));
    }

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m = -INFINITY;
  float l = 0.f;
  const float c2 = a.scale_log2;
  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};

  const sconst_i32 row_ptr = (sconst_i32)(uintptr_t)a.row_ptr;
  const sconst_i32 col_idx = (sconst_i32)(uintptr_t)a.col_idx;
  const int mrow = (a.mask_heads == 1 ? 0 : h) * a.tiles + qt;
  int jj = row_ptr[mrow];
  int64_t je = row_ptr[mrow + 1];
  if (jj < 0) jj = 0;
  if (je > a.col_cap) je = a.col_cap;
  auto next_valid = [&](int x) {
    while (x < je) {
      const int j = col_idx[x];
      if (j >= 0 && j < a.tiles) break;
      ++x;
    }
    return x;
  };

  jj = next_valid(jj);
  if (jj < je) {
    const int j0 = col_idx[jj];
    issue_tile(krs, kbuf, j0);
    issue_tile(vrs, vbuf, j0);
  }

  while (jj < je) {
    const int j = col_idx[jj];
    const int jn = next_valid(jj + 1);
    const bool has_next = jn < je;
    const int j_next = has_next ? col_idx[jn] : 0;

    // ---- S^T = K_j Q^T
    WAIT_VM(8);  // this wave's K_j chunks landed (V_j's 8 may be in flight)
    BARRIER();   // ... and every other wave's
    f32x16 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(kbuf + kb * 32 * ROW_BYTES + kr_off[c]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[kb], 0, 0, 0);
      }
    }
    BARRIER();  // all waves are done with K_j
    if (has_next) issue_tile(krs, kbuf, j_next);

    // ---- online softmax
    const int valid = N - j * BT;
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
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
    if (__any(mx > m + TAU)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // m = -inf -> 0
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    }
    bf16x8 pb[8];
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const int kb = kc >> 1;
      const int i0 = (kc & 1) * 8;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        // raw v_exp_f32: results below 2^-126 flush to zero, which is
        // negligible next to the row's largest weight (about 1)
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i0 + e], c2, -m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i0 + e + 1], c2, -m));
        bf16x2 pk;
        pk[0] = (__bf16)p0;
        pk[1] = (__bf16)p1;
        l = __builtin_amdgcn_fdot2_f32_bf16(pk, ones2, l, false);
        pb[kc][e] = pk[0];
        pb[kc][e + 1] = pk[1];
      }
    }

    // ---- O^T += V_j^T P^T
    if (has_next) {
      WAIT_VM(8);  // V_j landed (K_{j+1}'s 8 may be in flight)
    } else {
      WAIT_VM(0);
    }
    BARRIER();
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const int kb = kc >> 1;
      const int i0 = (kc & 1) * 2;
      const char* vt = vbuf + (kb * 32 + 8 * i0) * ROW_BYTES;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(vt + vr_off[0][db]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(vt + vr_off[1][db]));
        bf16x8 va;
        const bf16x4 lob = __builtin_bit_cast(bf16x4, lo);
        const bf16x4 hib = __builtin_bit_cast(bf16x4, hi);
        va[0] = lob[0]; va[1] = lob[1]; va[2] = lob[2]; va[3] = lob[3];
        va[4] = hib[0]; va[5] = hib[1]; va[6] = hib[2]; va[7] = hib[3];
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kc], oacc[db], 0, 0, 0);
      }
    }
    BARRIER();  // all waves are done with V_j
    if (has_next) issue_tile(vrs, vbuf, j_next);
    jj = jn;
  }

  // ---- epilogue: O = O^T / l, rows past N are not written
  l += __shfl_xor(l, 32);
  if (qrow < N) {
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
  const int64_t blocks = (int64_t)a.B * a.H * a.tiles;
  hipLaunchKernelGGL(fwd_bf16_t128_d128, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, a);
  return hipGetLastError();
}

}  // namespace bsattn
