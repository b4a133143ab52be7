// Block-sparse attention forward, tuned instance for bf16 Q/K/V/O, head dim
// 64, 64 x 64 tiles (LVSA page, "Meccanismo Core"; CalibAtt page, "B. Fase
// di Inferenza": attention only over each query tile's listed key tiles).
// The math is the tuned d = 128 instance's: online softmax in the exp2
// domain x = s * scale * log2(e), Q multiplied by scale * log2(e) as it is
// loaded (rounded back to bf16), the score MFMAs starting from -m, and the
// running max moved only when a tile's max exceeds it by more than TAU.
//
// Mapping onto CDNA4 (gfx950)
// ---------------------------
//  * Workgroup = 8 waves in two groups of 4 (waves w and w + 4 share a
//    SIMD) over four consecutive query tiles 4p .. 4p+3: wave (g, w) holds
//    rows 32 (w % 2) .. +32 of tile 4p + 2g + w / 2.  All four tiles walk
//    the union of their four lists (key tiles ascending, built once per
//    workgroup in LDS from the CSR); an entry carries one bit per tile, and
//    a wave whose tile does not list the key tile skips its work on it.
//    Neighbouring tiles of a window mask list nearly the same key tiles, so
//    each staged K/V tile serves up to 256 query rows.
//  * Ping-pong: in phase 2w group 0 runs its matrix phase (O += P V of
//    entry w - 1, then S = K Q^T of entry w: 16 MFMAs per wave) while group
//    1 runs the softmax of entry w - 1; in phase 2w + 1 the roles swap.
//  * K and V tiles (64 rows x 128 B = 8 KB each) are double-buffered in LDS
//    and fetched straight to LDS (buffer_load ... lds) by group 1 in its
//    vector phase 2w (waves 0-1 of the group K of entry w + 1, waves 2-3 V
//    of entry w), waited for at the end of its matrix phase 2w + 1, a phase
//    before first use.  Rows past N lie outside the buffer range and arrive
//    as zeros; their scores are masked to -inf.
//  * LDS rows are 128 B, so two rows share each 256 B line of the 64 banks.
//    16-byte chunk c of K row R sits at position c ^ gK(R), gK(R) =
//    (R / 2) % 8: the K reader's 16 lanes a cycle (16 consecutive rows, one
//    chunk column) meet 16 distinct (line half, position) pairs.  V row R
//    puts chunk c at c ^ gV(R), gV(R) = 4 ((R / 2) % 2): the transposing V
//    reader's 32 lanes a cycle (4 rows x 4 chunks x 8 B) meet 64 distinct
//    banks.  (c ^ (R % 8) for both measured 2-way conflicts and no faster
//    than the phases' MFMAs allowed.)
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T
//    in VGPRs): lane l holds query l % 32 and, per 32-key block, keys
//    8i + 4(l/32) + e.  O^T += V^T P^T on the same MFMA, P straight from the
//    score registers (packed to bf16 in place), the reduction index permuted
//    to the keys the lane holds; the V^T operand comes from row-major V via
//    ds_read_b64_tr_b16 (lane i of each 16-lane group receives element
//    i % 4 of source lane 4e + i / 4).
//  * The grid is remapped so each XCD (own L2) walks a contiguous range of
//    (head, query-tile quad).
#include <hip/hip_runtime.h>

#include <math.h>

#include "bsattn_internal.h"
#include "cdna4_lds.h"

namespace bsattn {
namespace {

typedef const __attribute__((address_space(4))) int32_t* sconst_i32_d64;

constexpr int Q_BT = 64;                    // tile rows / columns
constexpr int Q_D = 64;                     // head dim
constexpr int Q_ROW = Q_D * 2;              // 128 bytes
constexpr int Q_TILE = Q_BT * Q_ROW;        // 8 KB
constexpr float Q_TAU = 8.0f;               // lazy-rescale threshold (log2 units)
constexpr int Q_NXCD = 8;
constexpr int Q_PF = 4;                     // MFMA operand read-ahead (steps)
constexpr int Q_MAXT = 4096;                // key tiles at most (union list in LDS)

// One entry of the union list of the four tiles: key tile index in bits
// 0..26, bit 30 - i set when tile i of the quad lists it; Q_NONE past the
// end.
constexpr int Q_NONE = -1;
__device__ __forceinline__ int q_tile(int e) { return e < 0 ? -1 : (e & 0x07FFFFFF); }
__device__ __forceinline__ bool q_in(int e, int sub) { return e >= 0 && ((e >> (30 - sub)) & 1); }

__device__ __forceinline__ int q_list_len(sconst_i32_d64 row_ptr, int64_t cap, int mrow,
                                          int& begin) {
  int64_t b0 = row_ptr[mrow], e0 = row_ptr[mrow + 1];
  if (b0 < 0) b0 = 0;
  if (e0 > cap) e0 = cap;
  begin = (int)b0;
  return e0 > b0 ? (int)(e0 - b0) : 0;
}

__global__ void __launch_bounds__(512, 1)
fwd_bf16_d64_t64(FwdLaunch a) {
  // K slots [0, 8K) and [8K, 16K) of a 16 KB-aligned array, so one XOR of
  // bit 13 moves a read address to the other slot; V likewise
  __shared__ __attribute__((aligned(16384))) char kslots[2 * Q_TILE];
  __shared__ __attribute__((aligned(16384))) char vslots[2 * Q_TILE];
  __shared__ uint32_t ulist[Q_MAXT];           // union list: tile | need bits << 27
  __shared__ uint32_t bmap[4 * (Q_MAXT / 32)];  // the four lists as bitmaps
  __shared__ int wcount[8];
  __shared__ uint32_t okeys[32];
  __shared__ int oitem[32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int wg = wave & 3;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const uint32_t kl32 = (uint32_t)(uintptr_t)uniform_lds((lds_char_t*)kslots);
  const uint32_t vl32 = (uint32_t)(uintptr_t)uniform_lds((lds_char_t*)vslots);

  // ---- workgroup -> (batch * head, quad of query tiles), XCD-contiguous.
  // Each XCD's range is cut into chunks of 32 quads (about one per compute
  // unit of the XCD), and the k-th workgroup of a chunk to be dispatched
  // takes its k-th longest quad (by the four lists' summed length, ties by
  // position), so long quads start first and short ones fill the end.
  const int quads = (a.tiles + 3) >> 2;
  uint32_t logical;
  {
    const uint32_t G = gridDim.x, hw = blockIdx.x;
    const uint32_t q8 = G / Q_NXCD, r8 = G % Q_NXCD, xcd = hw % Q_NXCD, slot = hw / Q_NXCD;
    const uint32_t lo = xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8;
    const uint32_t len = q8 + (xcd < r8 ? 1u : 0u);
    const uint32_t c0 = lo + (slot & ~31u);
    const int nchunk = (int)min(32u, lo + len - c0);
    if (tid < 32) {
      uint32_t key = 0;
      if (tid < nchunk) {
        const uint32_t it = c0 + (uint32_t)tid;
        const int qd = (int)(it % (uint32_t)quads);
        const int hh = (int)(it / (uint32_t)quads) % a.H;
        const int r0 = (a.mask_heads == 1 ? 0 : hh) * a.tiles + 4 * qd;
        const int r1 = min(r0 + 4, (a.mask_heads == 1 ? 0 : hh) * a.tiles + a.tiles);
        const int64_t n = (int64_t)a.row_ptr[r1] - a.row_ptr[r0];
        key = ((uint32_t)min(max(n, (int64_t)0), (int64_t)0xFFFFFF) << 8 | (uint32_t)(31 - tid)) + 1;
      }
      okeys[tid] = key;
    }
    __syncthreads();
    if (tid < nchunk) {
      const uint32_t mine = okeys[tid];
      int rank = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) rank += okeys[j] > mine ? 1 : 0;
      oitem[rank] = tid;
    }
    __syncthreads();
    logical = c0 + (uint32_t)oitem[slot & 31u];
  }
  const int quad = (int)(logical % (uint32_t)quads);
  const int bh = (int)(logical / (uint32_t)quads);
  const int h = bh % a.H;
  const int N = a.N;
  const int64_t head_row = (int64_t)bh * N;
  const int sub = 2 * grp + (wg >> 1);        // this wave's tile within the quad
  const int qt = 4 * quad + sub;
  const int qr = qt * Q_BT + (wg & 1) * 32 + l32;
  const bool row_ok = qt < a.tiles && qr < N;

  // ---- Q, multiplied by scale * log2(e) (rounded to bf16)
  bf16x8 qf[4];
  {
    const __bf16* qptr = reinterpret_cast<const __bf16*>(a.q) + (head_row + qr) * Q_D + half * 8;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (row_ok) {
        const bf16x8 raw = *reinterpret_cast<const bf16x8*>(qptr + c * 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[c][e] = (__bf16)((float)raw[e] * a.scale_log2);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[c][e] = (__bf16)0.f;
      }
    }
  }

  // ---- the union of the four lists, built once in LDS: each list's key
  // tiles set bits of its bitmap, then every key tile with a bit set is
  // written in ascending order with its four bits (a key tile listed twice
  // counts once; indices outside [0, Tk) are dropped)
  int ulen;
  {
    const sconst_i32_d64 row_ptr = (sconst_i32_d64)(uintptr_t)a.row_ptr;
    const int hrow = (a.mask_heads == 1 ? 0 : h) * a.tiles;
    const int words = (a.tiles + 31) >> 5;
    for (int i = tid; i < 4 * words; i += 512) bmap[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int jb = 0, n = 0;
      if (4 * quad + i < a.tiles) n = q_list_len(row_ptr, a.col_cap, hrow + 4 * quad + i, jb);
      for (int x = tid; x < n; x += 512) {
        const int t = a.col_idx[jb + x];
        if (t >= 0 && t < a.tiles) atomicOr(&bmap[i * words + (t >> 5)], 1u << (t & 31));
      }
    }
    __syncthreads();
    int base = 0;
    for (int c0 = 0; c0 < a.tiles; c0 += 512) {
      const int t = c0 + tid;
      uint32_t nb = 0;
      if (t < a.tiles) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          nb |= ((bmap[i * words + (t >> 5)] >> (t & 31)) & 1u) << (3 - i);
      }
      const uint64_t bal = __ballot(nb != 0);
      const int below = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wcount[wave] = __popcll(bal);
      __syncthreads();
      int before = 0, total = 0;
#pragma unroll
      for (int w8 = 0; w8 < 8; ++w8) {
        const int c = wcount[w8];
        before += w8 < wave ? c : 0;
        total += c;
      }
      if (nb != 0) ulist[base + before + below] = (uint32_t)t | (nb << 27);
      base += total;
      __syncthreads();
    }
    ulen = base;
  }
  int uidx = 0;
  auto next_entry = [&]() INLINE {
    const int e = uidx < ulen ? (int)ulist[uidx] : Q_NONE;
    ++uidx;
    return __builtin_amdgcn_readfirstlane(e);
  };

  // ---- fetches: group-1 waves 0-1 fetch K rows 32 (w % 2) .. +32 of a
  // tile, waves 2-3 the same rows of V, one burst of four 1 KB loads (8 rows
  // each).  Lane l writes chunk position l % 8 of row R = 32 (w % 2) + 8i +
  // l / 8, so it fetches global chunk (l % 8) ^ gK(R) = (l % 8) ^ ((4i +
  // l / 16) % 8) for K and (l % 8) ^ gV(R) = (l % 8) ^ 4 ((l / 16) % 2) for
  // V.
  const int nbytes = N * Q_ROW;
  const i32x4 krs = raw_rsrc(reinterpret_cast<const char*>(a.k) + head_row * Q_ROW, nbytes);
  const i32x4 vrs = raw_rsrc(reinterpret_cast<const char*>(a.v) + head_row * Q_ROW, nbytes);
  const int frow = 32 * (wg & 1);
  uint32_t ld_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = wg >= 2 ? 4 * ((lane >> 4) & 1) : ((4 * i + (lane >> 4)) & 7);
    ld_off[i] = (uint32_t)((frow + (lane >> 3)) * Q_ROW + (((lane & 7) ^ g) << 4));
  }
  auto tile_off = [&](int t) INLINE {
    return (t >= 0 && t < a.tiles) ? (uint32_t)t * Q_TILE : 0x80000000u;
  };
  // K tile tk into K slot base kbuf (waves 0-1) or V tile tv into V slot
  // base vbuf (waves 2-3); skip: nothing
  auto fetch = [&](int tk, int tv, uint32_t kbuf, uint32_t vbuf, uint32_t skip) INLINE {
    const bool isv = wg >= 2;
    const uint32_t m0 = (isv ? vbuf : kbuf) + (uint32_t)(frow * Q_ROW);
    const uint32_t so = tile_off(isv ? tv : tk);
    const uint32_t sk = (uint32_t)__builtin_amdgcn_readfirstlane((int)(skip | ((isv ? tv : tk) < 0)));
    dma_burst4(isv ? vrs : krs, m0, ld_off, so, sk);
  };

  // ---- LDS read addresses (slot 0; the slot bit goes in by XOR)
  // K reader: key row R = kb*32 + l32, logical chunk 2c + half at position
  // (2c + half) ^ gK(R) = (c << 1) ^ (half ^ (l32 / 2) % 8).
  uint32_t kr = kl32 + (uint32_t)(l32 * Q_ROW + ((half ^ ((l32 >> 1) & 7)) << 4));
  // V^T reader (ds_read_b64_tr_b16): source lane s (= l % 16) of 16-lane
  // group g16 (= l / 16) points at key row R0 + Y, Y = 4 (g16 / 2) + s / 4,
  // d = 32 db + 16 (g16 % 2) + 4 (s % 4); with R0 % 8 = 0 the chunk
  // position is (4 db + X) ^ gV(Y), X = 2 (g16 % 2) + (s % 4) / 2.
  uint32_t vr;
  {
    const int s16 = lane & 15, g16 = lane >> 4;
    const int X = 2 * (g16 & 1) + ((s16 & 3) >> 1);
    const int Y = 4 * (g16 >> 1) + (s16 >> 2);
    const int gv = 4 * ((Y >> 1) & 1);
    vr = vl32 + (uint32_t)(Y * Q_ROW + ((X ^ gv) << 4) + 8 * (s16 & 1)) + (uint32_t)Q_TILE;
  }
  auto flip_slots = [&]() INLINE {
    kr ^= (uint32_t)Q_TILE;
    vr ^= (uint32_t)Q_TILE;
  };
  auto k_operand = [&](int kb, int c) INLINE {
    const uint32_t ad = (kr ^ (uint32_t)(c << 5)) + (uint32_t)(kb * 32 * Q_ROW);
    return *(const lds_bf16x8_t*)(uintptr_t)ad;
  };
  // keys of MFMA step kc: rows kb*32 + 16 (kc % 2) + 8 sec + ..., kb = kc / 2
  auto v_operand = [&](int kc, int db) INLINE {
    const uint32_t rows = (uint32_t)(((kc >> 1) * 32 + (kc & 1) * 16) * Q_ROW);
    const uint32_t a0 = (vr ^ (uint32_t)(db << 6)) + rows;
    const uint32_t a1 = a0 + (uint32_t)(8 * Q_ROW);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)a0);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)a1);
    const bf16x4 lob = __builtin_bit_cast(bf16x4, lo);
    const bf16x4 hib = __builtin_bit_cast(bf16x4, hi);
    bf16x8 va;
    va[0] = lob[0]; va[1] = lob[1]; va[2] = lob[2]; va[3] = lob[3];
    va[4] = hib[0]; va[5] = hib[1]; va[6] = hib[2]; va[7] = hib[3];
    return va;
  };

  f32x16 oacc[2];
  f32x16 s[2];
  f32x16 nm;  // -m in every element (0 while m = -inf)
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    oacc[0][e] = 0.f;
    oacc[1][e] = 0.f;
    s[0][e] = 0.f;
    s[1][e] = 0.f;
    nm[e] = 0.f;
  }
  float m = -INFINITY;
  float l = 0.f;
  auto p_operand = [&](int kc) INLINE {
    const f32x16& v = s[kc >> 1];
    const int o = (kc & 1) * 4;
    const f32x4 w4 = {v[o], v[o + 1], v[o + 2], v[o + 3]};
    return __builtin_bit_cast(bf16x8, w4);
  };

  // matrix phase: O += P V (if do_pv; 8 MFMAs), then S = K Q^T (if do_qk;
  // 8 MFMAs); operands read Q_PF steps ahead
  auto matrix_phase = [&](bool do_pv, bool do_qk) INLINE {
    __builtin_amdgcn_s_setprio(1);
    if (do_pv) {
      bf16x8 ring[Q_PF];
#pragma unroll
      for (int i = 0; i < Q_PF; ++i) ring[i] = v_operand(i >> 1, i & 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * Q_PF, 0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bf16x8 cur = ring[k % Q_PF];
        if (k + Q_PF < 8) ring[k % Q_PF] = v_operand((k + Q_PF) >> 1, (k + Q_PF) & 1);
        const int kc = k >> 1, db = k & 1;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, p_operand(kc), oacc[db], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (k + Q_PF < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (do_qk) {
      bf16x8 ring[Q_PF];
#pragma unroll
      for (int i = 0; i < Q_PF; ++i) ring[i] = k_operand(i & 1, i >> 1);
      __builtin_amdgcn_sched_group_barrier(0x100, Q_PF, 0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bf16x8 cur = ring[k % Q_PF];
        if (k + Q_PF < 8) ring[k % Q_PF] = k_operand((k + Q_PF) & 1, (k + Q_PF) >> 1);
        const int c = k >> 1, kb = k & 1;
        if (c == 0)
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[0], nm, 0, 0, 0);
        else
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[c], s[kb], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (k + Q_PF < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // online softmax of S for key tile j (tail mask for the last tile); P
  // replaces S in the same registers, packed as bf16 pairs
  auto softmax = [&](int j) INLINE {
    const int valid = (j >= 0 && j < a.tiles) ? N - j * Q_BT : 0;
    if (valid < Q_BT) {
      const int lim = valid - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t keep = (uint32_t)(((kb * 32 + 8 * i + e) - lim) >> 31);
            s[kb][4 * i + e] =
                __uint_as_float((__float_as_uint(s[kb][4 * i + e]) & keep) | (0xff800000u & ~keep));
          }
    }
    float mx0 = s[0][0], mx1 = s[1][0];
#pragma unroll
    for (int e = 1; e < 16; ++e) {
      mx0 = fmaxf(mx0, s[0][e]);
      mx1 = fmaxf(mx1, s[1][e]);
    }
    // the tile's max relative to the bias the scores carry (-m, or 0 while
    // m = -inf)
    const float mx = max_across_halves(fmaxf(mx0, mx1));
    if (__any(m == -INFINITY ? mx != -INFINITY : mx > Q_TAU)) {
      const float msub = m == -INFINITY ? 0.f : m;
      const float m_new = fmaxf(m, msub + mx);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
      const float shift = m_new == -INFINITY ? 0.f : m_new - msub;
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        oacc[0][e] *= alpha;
        oacc[1][e] *= alpha;
        s[0][e] -= shift;
        s[1][e] -= shift;
      }
      const float nb = m == -INFINITY ? 0.f : -m;
#pragma unroll
      for (int e = 0; e < 16; ++e) nm[e] = nb;
    }
    float lp0 = 0.f, lp1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(s[kb][e]);
        const float p1 = __builtin_amdgcn_exp2f(s[kb][e + 1]);
        bf16x2 pk;
        pk[0] = (__bf16)p0;
        pk[1] = (__bf16)p1;
        if (kb == 0) lp0 += p0 + p1; else lp1 += p0 + p1;
        s[kb][e >> 1] = __builtin_bit_cast(float, pk);
      }
    }
    l += lp0 + lp1;
  };

  // ---- merged-list window: entries w-1, w, w+1, w+2 at phase pair w
  int e_m1 = Q_NONE;
  int e_0 = next_entry();
  int e_1 = next_entry();
  int e_2 = next_entry();
  int w = 0;

  // ---- prologue: K of entry 0 into K slot 0 (group 1, waves 0-1)
  fetch(q_tile(e_0), -1, kl32, vl32, (grp == 1 && wg < 2) ? 0u : 1u);
  __builtin_amdgcn_s_waitcnt(WAIT_VM0);
  BARRIER();

  // Pair w = phases 2w (group 0 matrix: P V of entry w-1, S of entry w;
  // group 1 vector: softmax of entry w-1, fetches K of entry w+1 into K
  // slot (w+1)%2 and V of entry w into V slot w%2) and 2w+1 (group 0
  // vector: softmax of entry w; group 1 matrix).  Both slots a fetch fills
  // were last read in phase 2w-1.
  auto advance = [&]() INLINE {
    e_m1 = e_0;
    e_0 = e_1;
    e_1 = e_2;
    e_2 = next_entry();
    flip_slots();
  };
  const uint32_t gskip = grp != 1 ? 1u : 0u;
  auto run_vector_phase = [&](bool in_loop) INLINE {
    const int es = in_loop ? e_0 : Q_NONE;
    const int tk = q_tile(in_loop ? e_2 : e_1);
    const int tv = q_tile(in_loop ? e_1 : e_0);
    if (in_loop) {
      advance();
      ++w;
    }
    fetch(tk, tv, kl32 + (uint32_t)(((w + 1) & 1) * Q_TILE), vl32 + (uint32_t)((w & 1) * Q_TILE),
          gskip);
    __builtin_amdgcn_sched_barrier(0);
    if (q_in(es, sub)) softmax(q_tile(es));
  };
  if (grp == 1 && e_0 != Q_NONE) {
    run_vector_phase(false);
    BARRIER();
  }
  while (e_0 != Q_NONE || e_m1 != Q_NONE) {
    matrix_phase(q_in(e_m1, sub), q_in(e_0, sub));
    if (grp == 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    BARRIER();
    if (grp == 1 && !(e_1 != Q_NONE || e_0 != Q_NONE)) break;
    run_vector_phase(true);
    BARRIER();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: O = O^T / l, LSE
  l = sum_across_halves(l);
  if (row_ok) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    __bf16* op = reinterpret_cast<__bf16*>(a.o) + (head_row + qr) * Q_D;
#pragma unroll
    for (int db = 0; db < 2; ++db)
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
      a.lse[head_row + qr] = l > 0.f ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
  }
}

}  // namespace

bool fwd_d64_t64_fits(const FwdLaunch& a) {
  return a.tile == Q_BT && a.d == Q_D && a.dtype == 0 && a.window == 0 &&
         a.plan == nullptr && a.tiles <= Q_MAXT && (int64_t)a.N * Q_ROW < ((int64_t)1 << 31);
}

int launch_fwd_d64_t64(const FwdLaunch& a, void* stream) {
  const int64_t grid = (int64_t)((a.tiles + 3) / 4) * a.H * a.B;
  if (grid == 0) return hipSuccess;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fwd_bf16_d64_t64, dim3((unsigned)grid), dim3(512), 0, (hipStream_t)stream,
                     a);
  return hipGetLastError();
}

}  // namespace bsattn
