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
// Q is multiplied by scale * log2(e) once, as it is loaded (rounded back to
// bf16), and the score MFMAs start from an accumulator holding -m, so they
// deliver x - m directly: the softmax spends no instruction per score on the
// scale or the shift, only the exponential, the pack and the row sum.
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
//   * the two groups share their K/V tiles: they walk the union of their
//     two active lists (key tiles ascending; a tile only one group needs is
//     skipped by the other), so each staged tile serves 256 query rows.
//     Neighbouring query tiles of a window mask need nearly the same key
//     tiles, and L2 -> LDS staging traffic per flop halves.
//   * K and V tiles are double-buffered in LDS (2 x 2 x 32 KB).  Entry w's
//     K is read in phases 2w (group 0) and 2w+1 (group 1), its V in phases
//     2w+2 and 2w+3.  Both slots that K_{w+1} and V_w go to are free from
//     phase 2w, so group 1 fetches both in its vector phase 2w (each wave 8
//     KB of each tile, in bursts spread over its exponentials) and waits for
//     them at the end of its matrix phase 2w+1, a phase before first use.
//     Matrix phases issue no global-memory instruction, so the MFMA stream
//     never stalls on the memory-address queue.  Loads are buffer_load ...
//     lds (16 B per lane, no VGPR staging; rows past the sequence end are
//     outside the buffer range and arrive as zeros).
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
//     16-lane group receives element i % 4 of source lane 4e + i / 4).  MFMA
//     operands are read from LDS four MFMAs ahead of use.
//   * Row sums add the fp32 P values with plain VALU adds.  Dot instructions
//     (v_dot2_*) issue only when the matrix core is idle, so next to the
//     other group's MFMA stream they would stall the softmax.
//   * Workgroups are remapped so each XCD (own L2) walks a contiguous range
//     of (head, query-tile pair); neighbouring query tiles share most of
//     their key tiles.  Inside a range the longest pairs go first (per chunk
//     of 32); per-head masks with uneven heads are instead dealt over the
//     XCDs globally, longest first.
//   * A second instance reads and writes through the grouped view of the
//     tokens (SQuad's global pass: the position-major order of windows of w
//     tokens) instead of contiguous rows; only the addresses differ.
#include <hip/hip_runtime.h>

#include <math.h>

#include "bsattn_internal.h"
#include "cdna4_lds.h"

namespace bsattn {
namespace {

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
constexpr int PF = 4;                       // MFMA operand read-ahead (steps)
constexpr int LPT_CHUNK = 32;               // workgroups ordered longest-first together
constexpr int DEAL_MAX = 4096;              // per-head masks: items ranked globally (LDS keys)
constexpr int DEAL_TILES = 4095;            // ... and key bins 0 .. 2 * tiles in 32 KB of LDS

__device__ __forceinline__ int list_len(sconst_i32 row_ptr, int64_t cap, int mrow, int& begin) {
  int64_t b0 = row_ptr[mrow], e0 = row_ptr[mrow + 1];
  if (b0 < 0) b0 = 0;
  if (e0 > cap) e0 = cap;
  begin = (int)b0;
  return e0 > b0 ? (int)(e0 - b0) : 0;
}

// Load i (0..3) of the first half of a tile fetch: 1 KB of the tile (rows
// 4i .. 4i+3 of the wave's 16) into LDS.  The immediate offset 1024 i
// applies to both the global and the LDS address; `step` adds to the global
// one what rows 4i lie further apart than 1024 bytes (0 for contiguous rows).
template <int I>
__device__ __forceinline__ void fetch_load(__amdgpu_buffer_rsrc_t rs, lds_char_t* buf, int wg,
                                           uint32_t voff, uint32_t toff, uint32_t step) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(buf + 8 * wg * 1024), 16, voff,
                                           toff + I * step, 1024 * I, 0);
}
__device__ __forceinline__ void fetch_load_i(int i, __amdgpu_buffer_rsrc_t rs, lds_char_t* buf,
                                             int wg, const uint32_t* ld_off, uint32_t toff,
                                             uint32_t step) {
  switch (i) {  // resolved at compile time: every caller's loop is unrolled
    case 0: fetch_load<0>(rs, buf, wg, ld_off[0], toff, step); break;
    case 1: fetch_load<1>(rs, buf, wg, ld_off[1], toff, step); break;
    case 2: fetch_load<2>(rs, buf, wg, ld_off[2], toff, step); break;
    default: fetch_load<3>(rs, buf, wg, ld_off[3], toff, step); break;
  }
}

// One entry of the merged list of the two groups: key tile index in bits
// 0..28 (BAD_TILE for an index outside [0, Tk)), bit 30 set when group 0
// needs it, bit 29 when group 1 does; NONE past the end of both lists.
constexpr int NONE = -1;
constexpr int BAD_TILE = 0x0FFFFFFE;  // sorts after every real tile
constexpr int LIST_END = 0x0FFFFFFF;  // head of an exhausted list
__device__ __forceinline__ int ent_tile(int e) { return e < 0 ? -1 : (e & 0x1FFFFFFF); }
__device__ __forceinline__ bool ent_in(int e, int grp) {
  return e >= 0 && ((e >> (30 - grp)) & 1);
}

// GRP: the grouped view (a.window = w > 0, G = N / w a multiple of 128):
// attention runs over the position-major order of the windows of w tokens,
// position p = r * G + c standing for buffer row c * w + r, so tile t is the
// 128 buffer rows from row0(t) = (128 t mod G) * w + 128 t / G on at stride
// w.  Every address below goes through that map; the arithmetic is the same.
// PLANNED: one persistent workgroup per worker of a work plan (see the
// pipelined stream below) instead of one workgroup per query-tile pair.
template <bool GRP, bool PLANNED>
__global__ void __launch_bounds__(512, 1)
fwd_bf16_t128_d128(FwdLaunch a) {
  // K slots [0, 32K) and [32K, 64K) of a 64 KB-aligned array, so one XOR of
  // bit 15 moves a read address to the other slot; V likewise
  __shared__ __attribute__((aligned(65536))) char kslots[2 * TILE_BYTES];
  __shared__ __attribute__((aligned(65536))) char vslots[2 * TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index via readfirstlane: the compiler then knows it (and all that
  // derives from it: group, list bounds, tile indices) is wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  const int grp = wave >> 2;  // 0 or 1
  const int wg = wave & 3;    // wave within the group
  const int half = lane >> 5;
  const int l32 = lane & 31;
  // Wave-uniform LDS bases, kept in the LDS address space throughout (offset
  // 0 is a valid LDS address; through a generic pointer it would read as
  // null).
  lds_char_t* const kl = uniform_lds((lds_char_t*)kslots);
  lds_char_t* const vl = uniform_lds((lds_char_t*)vslots);

  // one workgroup per query-tile pair (qt0, qt0 + 1)
  const uint32_t pairs = (uint32_t)(a.tiles + 1) >> 1;
  uint32_t logical = 0;
  if constexpr (!PLANNED) {
  // ---- XCD-aware remap of the 1-D grid onto (batch*head, query-tile pair)
  const uint32_t G = gridDim.x, hw = blockIdx.x;
  const uint32_t q8 = G / NXCD, r8 = G % NXCD, xcd = hw % NXCD, slot = hw / NXCD;
  const uint32_t lo = xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8;
  const uint32_t cnt = q8 + (xcd < r8 ? 1u : 0u);
  // Longest first: the XCD's range is cut into chunks of LPT_CHUNK
  // workgroups, and inside a chunk the workgroup dispatched k-th takes the
  // pair with the k-th longest pair of lists (ties by position).  Pair
  // lengths vary with how a tile pair meets the frames; walked in position
  // order the last long pairs would run alone at the end of the launch.
  // A chunk of about one workgroup per CU of the XCD keeps the pairs in
  // flight together close in position, so they share key tiles in the L2
  // (larger chunks spread them: more L2 misses, measured slower).
  // Each workgroup ranks its chunk itself (row_ptr differences, one item
  // per thread, ranks by broadcast LDS reads); a malformed row_ptr only
  // changes the order, which stays a permutation.
  // Per-head masks (Hm = H) differ from head to head, so the contiguous XCD
  // ranges carry unequal work and a long pair late in a range ends the
  // launch alone.  There every workgroup ranks all items instead (counting
  // sort on the list length, ties by position) and the ranks are dealt to
  // the XCDs round by round in snake order (round s: ranks 8s .. 8s+7 to
  // XCDs 0..7, reversed on odd rounds; the last, partial round in order),
  // so every XCD gets an even share, longest first.
  bool deal = a.mask_heads > 1 && G <= (uint32_t)DEAL_MAX && a.tiles <= DEAL_TILES;
  int* const keys_d = reinterpret_cast<int*>(kslots);  // G list lengths
  int* const misc = keys_d + DEAL_MAX;                 // scan partials and results
  int* const cnt_b = reinterpret_cast<int*>(vslots);   // items per length
  if (deal) {
    // dealt only when the heads' masks differ in size by over an eighth:
    // with even heads (a random static mask) the contiguous ranges' shared
    // key tiles in the L2 are worth more than the balance
    if (tid < 2) misc[540 + tid] = tid == 0 ? 0x7FFFFFFF : 0;
    __syncthreads();
    int hmin = 0x7FFFFFFF, hmax = 0;
    for (int h = tid; h < a.H; h += 512) {
      const int64_t nnz = (int64_t)a.row_ptr[(h + 1) * a.tiles] - a.row_ptr[h * a.tiles];
      const int v = (int)min(max(nnz, (int64_t)0), (int64_t)0x3FFFFFFF);
      hmin = min(hmin, v);
      hmax = max(hmax, v);
    }
    atomicMin(&misc[540], hmin);
    atomicMax(&misc[541], hmax);
    __syncthreads();
    deal = 8 * (int64_t)misc[541] > 9 * (int64_t)misc[540];
  }
  if (deal) {
    const int nb = 2 * a.tiles + 1;
    for (int b = tid; b < nb; b += 512) cnt_b[b] = 0;
    __syncthreads();
    for (uint32_t i = (uint32_t)tid; i < G; i += 512) {
      const uint32_t bhi = i / pairs;
      const int qt = 2 * (int)(i % pairs);
      const int hr = (int)(bhi % (uint32_t)a.H) * a.tiles;
      const int64_t len = (int64_t)a.row_ptr[hr + min(qt + 2, a.tiles)] - a.row_ptr[hr + qt];
      const int key = (int)min(max(len, (int64_t)0), (int64_t)2 * a.tiles);
      keys_d[i] = key;
      atomicAdd(&cnt_b[key], 1);
    }
    __syncthreads();
    int* const keys = keys_d;
    int* const start_b = cnt_b + 8192;                 // items longer than each length
    // start_b[b] = items with a length above b: thread t sums its run of
    // bins taken from the top, the runs' sums are scanned, then spread
    const int per = (nb + 511) / 512;
    const int q0 = min(tid * per, nb), q1 = min(q0 + per, nb);
    int sum = 0;
    for (int qq = q0; qq < q1; ++qq) sum += cnt_b[nb - 1 - qq];
    misc[tid] = sum;
    __syncthreads();
    for (int dd = 1; dd < 512; dd <<= 1) {
      const int add = tid >= dd ? misc[tid - dd] : 0;
      __syncthreads();
      misc[tid] += add;
      __syncthreads();
    }
    int run = tid > 0 ? misc[tid - 1] : 0;
    for (int qq = q0; qq < q1; ++qq) {
      const int b = nb - 1 - qq;
      start_b[b] = run;
      run += cnt_b[b];
    }
    __syncthreads();
    const uint32_t rounds = G / NXCD;
    const int rho = (int)(slot < rounds ? slot * NXCD + ((slot & 1) ? NXCD - 1 - xcd : xcd) : hw);
    for (int b = tid; b < nb; b += 512) {
      const int c = cnt_b[b], st = start_b[b];
      if (c > 0 && rho >= st && rho < st + c) {
        misc[512] = b;
        misc[513] = rho - st;
      }
    }
    __syncthreads();
    const int kstar = misc[512], ostar = misc[513];
    // the ostar-th item in index order among those of length kstar
    const uint64_t below = (1ull << lane) - 1;
    int base = 0;
    for (uint32_t i0 = 0; i0 < G; i0 += 512) {
      const uint32_t i = i0 + (uint32_t)tid;
      const bool f = i < G && keys[i] == kstar;
      const uint64_t bal = __ballot(f);
      if (lane == 0) misc[520 + wave] = __popcll(bal);
      __syncthreads();
      int wpre = 0, tot = 0;
      for (int wv = 0; wv < 8; ++wv) {
        const int c = misc[520 + wv];
        wpre += wv < wave ? c : 0;
        tot += c;
      }
      if (f && base + wpre + __popcll(bal & below) == ostar) misc[530] = (int)i;
      base += tot;
      __syncthreads();  // the wave counts are rewritten by the next block
      if (base > ostar) break;
    }
    logical = (uint32_t)__builtin_amdgcn_readfirstlane(misc[530]);
    __syncthreads();  // the LDS is refilled by tile fetches below
  } else {
    int* const keys = reinterpret_cast<int*>(kslots);
    int* const pick = keys + LPT_CHUNK;
    const uint32_t c0 = (slot / LPT_CHUNK) * LPT_CHUNK;
    const int cn = (int)min(cnt - c0, (uint32_t)LPT_CHUNK);
    if (tid < LPT_CHUNK) {
      int key = -1;  // past the chunk: never counted below
      if (tid < cn) {
        const uint32_t item = lo + c0 + (uint32_t)tid;
        const int bhi = (int)(item / pairs);
        const int qt = 2 * (int)(item % pairs);
        const int hr = (a.mask_heads == 1 ? 0 : bhi % a.H) * a.tiles;
        const int64_t len = (int64_t)a.row_ptr[hr + min(qt + 2, a.tiles)] - a.row_ptr[hr + qt];
        key = (int)min(max(len, (int64_t)0), (int64_t)2 * a.tiles);
      }
      keys[tid] = key;
    }
    __syncthreads();
    if (tid < cn) {
      const int mine = keys[tid];
      int rank = 0;
      const i32x4* const k4 = reinterpret_cast<const i32x4*>(keys);
#pragma unroll
      for (int u4 = 0; u4 < LPT_CHUNK / 4; ++u4) {
        const i32x4 kv = k4[u4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          rank += (kv[e] > mine || (kv[e] == mine && 4 * u4 + e < tid)) ? 1 : 0;
      }
      if (rank == (int)(slot - c0)) *pick = (int)(lo + c0) + tid;
    }
    __syncthreads();
    logical = (uint32_t)__builtin_amdgcn_readfirstlane(*pick);
    __syncthreads();  // the LDS is refilled by tile fetches below
  }
  }  // !PLANNED
  // the work item: (batch*head, query-tile pair); the planned stream moves
  // from item to item
  int bh = (int)(logical / pairs);
  int qt0 = 2 * (int)(logical % pairs);
  int h = bh % a.H;
  const int N = a.N;
  int64_t head_row = (int64_t)bh * N;
  const int gw = GRP ? a.window : 1;
  const int gG = GRP ? N / a.window : 1;
  // buffer row of the first row of position-major tile t; rows of a tile are
  // RS bytes apart
  auto row0 = [&](int t) INLINE { return GRP ? ((t * BT) % gG) * gw + (t * BT) / gG : t * BT; };
  const uint32_t RS = (uint32_t)gw * ROW_BYTES;

  // ---- active lists of both groups, merged on the fly (scalar, identical
  // in every wave)
  const sconst_i32 row_ptr = (sconst_i32)(uintptr_t)a.row_ptr;
  const sconst_i32 col_idx = (sconst_i32)(uintptr_t)a.col_idx;
  int jb0 = 0, jb1 = 0, n0 = 0, n1 = 0;
  // the two lists of query tiles qt0 and qt0 + 1 of head h
  auto item_lists = [&]() INLINE {
    const int hrow = (a.mask_heads == 1 ? 0 : h) * a.tiles;
    n0 = list_len(row_ptr, a.col_cap, hrow + qt0, jb0);
    n1 = qt0 + 1 < a.tiles ? list_len(row_ptr, a.col_cap, hrow + qt0 + 1, jb1) : 0;
  };
  if constexpr (!PLANNED) item_lists();
  // Each list keeps its validated head c (index i) and the raw entry at
  // index i + 1, loaded one step ahead: a value is validated only when it
  // becomes the head, by which time its scalar load has long completed.
  // Branch-free (selects only), so the scalar work interleaves with the
  // vector work around it: the look-ahead is reloaded on every step from a
  // clamped index (the same entry again when its list did not move; a
  // row_ptr entry when the list is empty).
  auto valid = [&](int r) INLINE { return (r >= 0 && r < a.tiles) ? r : BAD_TILE; };
  sconst_i32 la0, la1;
  int m0n, m1n, last0, last1, i0, i1, c0, c1, r0, r1;
  // (re)start the iterator on lists A = (jbA, nA) and B = (jbB, nB)
  auto init_lists = [&](int jbA, int nA, int jbB, int nB) INLINE {
    m0n = nA;
    m1n = nB;
    la0 = nA > 0 ? col_idx + jbA : row_ptr;
    la1 = nB > 0 ? col_idx + jbB : row_ptr;
    last0 = nA > 0 ? nA - 1 : 0;
    last1 = nB > 0 ? nB - 1 : 0;
    i0 = 0;
    i1 = 0;
    c0 = nA > 0 ? valid(la0[0]) : LIST_END;
    c1 = nB > 0 ? valid(la1[0]) : LIST_END;
    r0 = la0[min(1, last0)];
    r1 = la1[min(1, last1)];
  };
  auto next_entry = [&]() INLINE {
    const bool done = c0 == LIST_END && c1 == LIST_END;
    const int j = min(c0, c1);
    const int f0 = !done && c0 == j, f1 = !done && c1 == j;
    // new heads first, from values loaded earlier; then the new look-aheads
    i0 += f0;
    i1 += f1;
    const int h0 = i0 < m0n ? valid(r0) : LIST_END;
    const int h1 = i1 < m1n ? valid(r1) : LIST_END;
    c0 = f0 ? h0 : c0;
    c1 = f1 ? h1 : c1;
    r0 = la0[min(i0 + 1, last0)];
    r1 = la1[min(i1 + 1, last1)];
    return done ? NONE : (j | (f0 << 30) | (f1 << 29));
  };

  // ---- mode of this workgroup.  Pair mode (both groups walk the union of
  // their two lists, each staged tile serving both query tiles) wins when
  // the lists largely coincide, as for window masks.  When they do not (a
  // random static mask), each group would sit idle through the entries
  // only the other needs; split mode instead runs the two query tiles one
  // after the other, both groups on the same tile, taking alternate list
  // entries.  A split phase costs about 1.6 pair phases (each staged tile
  // serves half the rows, and a fetch has one phase to land instead of
  // two).  With I entries common to both lists, pair mode runs
  // n0 + n1 - I phases and split mode about 0.8 (n0 + n1) pair-phase
  // equivalents, so split mode is taken when 5 I < n0 + n1, and always when
  // one list is empty.  I is counted exactly, all threads at once: list B's
  // tiles set bits of a bitmap in the (still unused) V slots, then list A's
  // entries test them.  The choice affects speed only.
  bool split = false;
  if constexpr (!PLANNED) {
    uint32_t* const bits = reinterpret_cast<uint32_t*>(vslots);
    constexpr int BW = 2 * TILE_BYTES / 4 - 1;  // bitmap words; the last one counts
    uint32_t* const common = bits + BW;
    const int nw = (a.tiles + 31) >> 5;
    const int nthr = (int)blockDim.x;
    if (n0 > 0 && n1 > 0 && nw <= BW) {
      for (int c = tid; c < nw; c += nthr) bits[c] = 0u;
      if (tid == 0) *common = 0u;
      __syncthreads();
      for (int i = tid; i < n1; i += nthr) {
        const int t = col_idx[jb1 + i];
        if (t >= 0 && t < a.tiles) atomicOr(&bits[t >> 5], 1u << (t & 31));
      }
      __syncthreads();
      int hits = 0;
      for (int i = tid; i < n0; i += nthr) {
        const int t = col_idx[jb0 + i];
        hits += (t >= 0 && t < a.tiles && ((bits[t >> 5] >> (t & 31)) & 1u)) ? 1 : 0;
      }
      // sum over the wave, then one LDS add per wave
      for (int o = 32; o > 0; o >>= 1) hits += __shfl_xor(hits, o, 64);
      if (lane == 0 && hits > 0) atomicAdd(common, (uint32_t)hits);
      __syncthreads();
      const int shared_n = __builtin_amdgcn_readfirstlane((int)*common);
      split = 5 * shared_n < n0 + n1;
      __syncthreads();  // the V slots are refilled by tile fetches below
    } else {
      split = n0 == 0 || n1 == 0;
    }
  }

  // ---- Q^T operand: lane holds q[row l%32][8 d values], 8 chunks of 16 d
  // (hr = the head's first row, b*H*N + h*N), scaled by scale*log2(e) and
  // rounded to bf16
  bf16x8 qf[8];
  auto load_q = [&](int64_t hr, int tq) INLINE {
    const int qr = tq * BT + wg * 32 + l32;
    const int64_t qb = GRP ? (int64_t)row0(tq) + (int64_t)(wg * 32 + l32) * gw : qr;
    const __bf16* qptr = reinterpret_cast<const __bf16*>(a.q) + (hr + qb) * D + half * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (tq < a.tiles && qr < N) {
        const bf16x8 raw = *reinterpret_cast<const bf16x8*>(qptr + c * 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[c][e] = (__bf16)((float)raw[e] * a.scale_log2);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[c][e] = (__bf16)0.f;
      }
    }
  };

  // ---- buffer resources for a head's K and V rows (hr = its first row)
  const int nbytes = N * ROW_BYTES;
  auto k_rsrc = [&](int64_t hr) INLINE {
    return raw_rsrc(reinterpret_cast<const char*>(a.k) + hr * ROW_BYTES, nbytes);
  };
  auto v_rsrc = [&](int64_t hr) INLINE {
    return raw_rsrc(reinterpret_cast<const char*>(a.v) + hr * ROW_BYTES, nbytes);
  };
  auto k_brsrc = [&](int64_t hr) INLINE {
    return __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.k) + hr * ROW_BYTES), (short)0, nbytes,
        0x00020000);
  };
  i32x4 krs4 = k_rsrc(head_row);
  i32x4 vrs4 = v_rsrc(head_row);

  // Direct-load offsets.  Load i (0..7) of wave wg fills LDS bytes
  // [(8 wg + i) * 1024, +1024) of a slot: rows 32 wg + 4i + (0..3).  Lane l
  // writes chunk position l % 16 of row 32 wg + 4i + l / 16, so it fetches
  // global chunk (l % 16) ^ S(row), S(row) = 4 (l / 16) + i % 4.
  uint32_t ld_off[4];
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const int r = 32 * wg + (lane >> 4);
    const int c = (lane & 15) ^ (((lane >> 4) << 2) | i4);
    ld_off[i4] = (uint32_t)r * RS + (uint32_t)(c * 16);
  }
  auto tile_off = [&](int j) INLINE {
    return (j >= 0 && j < a.tiles) ? (uint32_t)row0(j) * ROW_BYTES : 0x80000000u;
  };

  // Per-lane LDS read addresses of slot 0 (K) and slot 1 (V) (base folded in
  // once), so every read is one VGPR plus an immediate offset; bit 15 flips
  // the slot.  K reader: key row kb*32 + l%32, chunk 2c + half.  V^T reader
  // (ds_read_b64_tr_b16): source lane s (= l % 16) of 16-lane group g16
  // (= l / 16) points at key row R0 + s/4, d = 32 db + 16 (g16%2) + 4 (s%4);
  // R0 = kb*32 + 8 i0 + 8 sec + 4 half.
  const int ks = swz(l32);
  uint32_t kr = (uint32_t)(uintptr_t)kl +
                (uint32_t)(l32 * ROW_BYTES + ((ks >> 1) << 5) + ((half ^ (ks & 1)) << 4));
  const int s16 = lane & 15;
  const int g16 = lane >> 4;
  uint32_t vr[2];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec) {
    const int q4 = s16 >> 2;
    const int rrel = 8 * sec + 4 * half + q4;
    const int low = (2 * (g16 & 1) + ((s16 & 3) >> 1)) ^ ((2 * sec + half) & 3);
    vr[sec] = (uint32_t)(uintptr_t)vl +
              (uint32_t)(TILE_BYTES + rrel * ROW_BYTES + (q4 << 6) + (low << 4) + 8 * (s16 & 1));
  }
  auto flip_slots = [&]() INLINE {
    kr ^= (uint32_t)TILE_BYTES;
    vr[0] ^= (uint32_t)TILE_BYTES;
    vr[1] ^= (uint32_t)TILE_BYTES;
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  // S^T scores; after the softmax the same registers hold P as packed bf16
  // pairs: P for keys of chunk kc = 2 kb + hh sits in s[kb][4 hh .. 4 hh + 3]
  f32x16 s[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
  float m = -INFINITY;
  float l = 0.f;
  // -m in every element (0 while m = -inf): the accumulator the first MFMA
  // of each score chain starts from, so S arrives as x - m
  f32x16 nm;
#pragma unroll
  for (int e = 0; e < 16; ++e) nm[e] = 0.f;

  auto v_operand = [&](int kc, int db) INLINE {
    const int rows = (kc >> 1) * 32 * ROW_BYTES + (kc & 1) * 16 * ROW_BYTES;
    const uint32_t a0 = (vr[0] ^ (uint32_t)(db << 6)) + (uint32_t)rows;
    const uint32_t a1 = (vr[1] ^ (uint32_t)(db << 6)) + (uint32_t)rows;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)a0);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)a1);
    const bf16x4 lob = __builtin_bit_cast(bf16x4, lo);
    const bf16x4 hib = __builtin_bit_cast(bf16x4, hi);
    bf16x8 va;
    va[0] = lob[0]; va[1] = lob[1]; va[2] = lob[2]; va[3] = lob[3];
    va[4] = hib[0]; va[5] = hib[1]; va[6] = hib[2]; va[7] = hib[3];
    return va;
  };
  auto k_operand = [&](int kb, int c) INLINE {
    const uint32_t ad = (kr ^ (uint32_t)(c << 5)) + (uint32_t)(kb * 32 * ROW_BYTES);
    return *(const lds_bf16x8_t*)(uintptr_t)ad;
  };
  auto p_operand = [&](int kc) INLINE {
    const f32x16& v = s[kc >> 1];
    const int o = (kc & 1) * 4;
    const f32x4 w = {v[o], v[o + 1], v[o + 2], v[o + 3]};
    return __builtin_bit_cast(bf16x8, w);
  };

  // matrix phase: O += P V (if do_pv), then S = K Q^T (if do_qk): two
  // streams of 32 MFMAs.  Each MFMA's LDS operand is read PF steps ahead
  // from a rotating buffer; the interleave is pinned with scheduling-group
  // barriers.  No global-memory instruction is issued here, so the MFMA
  // stream never waits on the memory-address queue.
  auto matrix_phase = [&](bool do_pv, bool do_qk) INLINE {
    // the MFMA stream wins issue ties against the other group's VALU work
    __builtin_amdgcn_s_setprio(1);
    // S stream order: chunk-outer, four interleaved accumulation chains
    // (one per key block), which hides the MFMA result latency
    auto qk_kb = [](int k) { return (k - 32) & 3; };
    auto qk_c = [](int k) { return (k - 32) >> 2; };
    auto load = [&](int k) INLINE -> bf16x8 {
      return k < 32 ? v_operand(k >> 2, k & 3) : k_operand(qk_kb(k), qk_c(k));
    };
    auto step = [&](int k, const bf16x8& opnd) INLINE {
      if (k < 32) {
        const int kc = k >> 2, db = k & 3;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd, p_operand(kc), oacc[db], 0, 0, 0);
      } else {
        const int c = qk_c(k), kb = qk_kb(k);
        if (c == 0) {
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd, qf[0], nm, 0, 0, 0);
        } else {
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd, qf[c], s[kb], 0, 0, 0);
        }
      }
    };
    if (do_pv) {
      bf16x8 ring[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i) ring[i] = load(i);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const bf16x8 cur = ring[k % PF];
        if (k + PF < 32) ring[k % PF] = load(k + PF);
        step(k, cur);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (k + PF < 32) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (do_qk) {
      bf16x8 ring[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i) ring[i] = load(32 + i);
      __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
      for (int k = 32; k < 64; ++k) {
        const bf16x8 cur = ring[(k - 32) % PF];
        if (k + PF < 64) ring[(k - 32) % PF] = load(k + PF);
        step(k, cur);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (k + PF < 64) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // online softmax of S for key tile j (tail mask for the last tile); P
  // replaces S in the same registers, packed as bf16 pairs
  auto softmax = [&](int j, auto&& fetch_part) INLINE {
    // keys past the end of the sequence never enter the softmax; integer
    // select (no per-element compare masks) for this rare tile
    const int valid = (j >= 0 && j < a.tiles) ? N - j * BT : 0;
    if (valid < BT) {
      const int lim = valid - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int keep = ((kb * 32 + 8 * i + e) - lim) >> 31;  // -1: keep
            const uint32_t bits = __float_as_uint(s[kb][4 * i + e]);
            s[kb][4 * i + e] =
                __uint_as_float((bits & (uint32_t)keep) | (0xff800000u & ~(uint32_t)keep));
          }
    }
    float mxp[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      mxp[kb] = s[kb][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mxp[kb] = fmaxf(mxp[kb], s[kb][e]);
    }
    float mx = fmaxf(fmaxf(mxp[0], mxp[1]), fmaxf(mxp[2], mxp[3]));
    // the tile's max relative to the bias the scores carry (-m, or 0 while
    // m = -inf)
    mx = max_across_halves(mx);
    if (__any(m == -INFINITY ? mx != -INFINITY : mx > TAU)) {
      const float msub = m == -INFINITY ? 0.f : m;
      const float m_new = fmaxf(m, msub + mx);
      // m_new = -inf only while every tile so far was skipped
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
      const float shift = m_new == -INFINITY ? 0.f : m_new - msub;
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kb][e] -= shift;
      const float nb = m == -INFINITY ? 0.f : -m;
#pragma unroll
      for (int e = 0; e < 16; ++e) nm[e] = nb;
    }
    float lp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      fetch_part(kb);
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        // raw v_exp_f32: results below 2^-126 flush to zero, negligible
        // next to the row's largest weight (about 1)
        const float p0 = __builtin_amdgcn_exp2f(s[kb][e]);
        const float p1 = __builtin_amdgcn_exp2f(s[kb][e + 1]);
        bf16x2 pk;
        pk[0] = (__bf16)p0;
        pk[1] = (__bf16)p1;
        // plain fp32 adds: a v_dot2 here would wait for the matrix core,
        // which the other wave on this SIMD keeps busy
        lp[kb] += p0 + p1;
        // packed pair e/2 of this block; position e/2 <= e was already read
        s[kb][e >> 1] = __builtin_bit_cast(float, pk);
      }
    }
    l += (lp[0] + lp[1]) + (lp[2] + lp[3]);
  };

  // vector phase: the online softmax of S (if do_sm; key tile j for the
  // tail mask) and, unless skip, this wave's share of two tile fetches (8
  // loads each: K tile tk into LDS slot kbuf, V tile tv into slot vbuf) in
  // four bursts spread over the exponentials: the direct-to-LDS path drains
  // about 64 B per clock per CU, and issuing all 16 loads at once would
  // stall the wave until the queue had room.
  auto vector_phase = [&](bool do_sm, int j, int tk, int tv, uint32_t kbuf, uint32_t vbuf,
                          uint32_t skip, const i32x4& rsk, const i32x4& rsv) INLINE {
    const uint32_t tko = tile_off(tk), tvo = tile_off(tv);
    // part 0: K loads 0-3; 1: K loads 4-7; 2: V loads 0-3; 3: V loads 4-7
    // (part is a constant after unrolling)
    auto fetch_part = [&](int part) INLINE {
      const i32x4& rs = part < 2 ? rsk : rsv;
      const uint32_t buf = (part < 2 ? kbuf : vbuf) + (uint32_t)(8 * wg * 1024);
      const uint32_t to = part < 2 ? tko : tvo;
      // loads 4(part%2) .. +3: rows 16(part%2) .. of this wave's 32-row share
      if constexpr (GRP)
        dma_burst4_strided(rs, buf + (part & 1) * 4096, ld_off, to + (part & 1) * 16 * RS,
                           4 * RS - 1024, skip);
      else
        dma_burst4(rs, buf + (part & 1) * 4096, ld_off, to + (part & 1) * 4096, skip);
      __builtin_amdgcn_sched_barrier(0);
    };
    if (do_sm) {
      softmax(j, fetch_part);
    } else {
#pragma unroll
      for (int part = 0; part < 4; ++part) fetch_part(part);
    }
  };

  const uint32_t kl32 = (uint32_t)(uintptr_t)kl, vl32 = (uint32_t)(uintptr_t)vl;
  const uint32_t kr_slot0 = kr, vr0_slot0 = vr[0] ^ (uint32_t)TILE_BYTES,
                 vr1_slot0 = vr[1] ^ (uint32_t)TILE_BYTES;

  // K of entry e (a key tile) into K slot 0, loaded by all 8 waves (4 KB
  // each), then a full wait and a barrier
  auto load_first_k = [&](int e, const __amdgpu_buffer_rsrc_t& krs) INLINE {
    if (e != NONE) {
      const uint32_t t0 = tile_off(ent_tile(e));
      lds_char_t* dst = kl + (grp * 4) * 1024;  // group g loads rows 16g.. of each 64-row half
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fetch_load_i(i, krs, dst, wg, ld_off, t0 + grp * 16 * RS, GRP ? 4 * RS - 1024 : 0);
    }
    // as a builtin, so the compiler knows every load before the loop is done
    // and inserts no wait of its own inside it
    __builtin_amdgcn_s_waitcnt(WAIT_VM0);
    BARRIER();
  };

  // O = O^T / l for this wave's rows of query tile tq (rows past N not
  // written); db0 .. db0 + ndb - 1 are the 32-wide d blocks written
  auto store_o = [&](int64_t hr, int tq, float inv, int db0, int ndb) INLINE {
    const int qr = tq * BT + wg * 32 + l32;
    if (tq < a.tiles && qr < N) {
      const int64_t qb = GRP ? (int64_t)row0(tq) + (int64_t)(wg * 32 + l32) * gw : qr;
      __bf16* op = reinterpret_cast<__bf16*>(a.o) + (hr + qb) * D;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        if (db < db0 || db >= db0 + ndb) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x4 v;
          v[0] = (__bf16)(oacc[db][4 * i] * inv);
          v[1] = (__bf16)(oacc[db][4 * i + 1] * inv);
          v[2] = (__bf16)(oacc[db][4 * i + 2] * inv);
          v[3] = (__bf16)(oacc[db][4 * i + 3] * inv);
          *reinterpret_cast<bf16x4*>(op + db * 32 + 8 * i + 4 * half) = v;
        }
      }
    }
  };
  auto store_lse = [&](int64_t hr, int tq, float mm, float ll) INLINE {
    const int qr = tq * BT + wg * 32 + l32;
    const int64_t qb = GRP ? (int64_t)row0(tq) + (int64_t)(wg * 32 + l32) * gw : qr;
    if (tq < a.tiles && qr < N && a.lse != nullptr && half == 0)
      a.lse[hr + qb] = ll > 0.f ? (mm + log2f(ll)) * 0.69314718055994531f : -INFINITY;
  };
  auto l_over_halves = [&]() INLINE {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l),
                                                    false, false);
    l = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  };

  int e_m1, e_0, e_1, e_2;
  auto reset_state = [&]() INLINE {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) nm[e] = 0.f;
  };

  if constexpr (!PLANNED) {
  if (!split) {
    // ================= pair mode =================
    const int qt = qt0 + grp;
    load_q(head_row, qt);
    init_lists(jb0, n0, jb1, n1);
    kr = kr_slot0;
    vr[0] = vr0_slot0 ^ (uint32_t)TILE_BYTES;
    vr[1] = vr1_slot0 ^ (uint32_t)TILE_BYTES;
    int w = 0;  // phase pair index (counted per group)

    // ---- merged-list window: entries w-1, w, w+1, w+2 at phase pair w
    e_m1 = NONE;
    e_0 = next_entry();
    e_1 = next_entry();
    e_2 = next_entry();

    // ---- prologue: K_0 into slot 0
    load_first_k(e_0, k_brsrc(head_row));

    // Every wave alternates matrix and vector phases; group 1 starts with a
    // vector phase (phase 0) and so is one phase behind.  Pair w = phases
    // 2w (group 0 matrix: P V of entry w-1, S of entry w; group 1 vector:
    // softmax of entry w-1) and 2w+1 (group 0 vector: softmax of entry w;
    // group 1 matrix: P V of entry w-1, S of entry w).  In its vector phase
    // 2w, group 1 sees the window (e_m1, e_0, e_1, e_2) = entries
    // (w-1, w, w+1, w+2) and fetches K_{w+1} into K slot (w+1)%2 (last read
    // in phase 2w-1) and V_w into V slot w%2 (last read in phase 2w-1).  It
    // waits for both fetches at the end of its matrix phase 2w+1; both tiles
    // are first read in phase 2w+2.
    auto advance = [&]() INLINE {
      e_m1 = e_0;
      e_0 = e_1;
      e_1 = e_2;
      e_2 = next_entry();
      flip_slots();
    };
    // One call site for both groups (arguments selected by group), so the
    // softmax is instantiated once per mode.  The window advances at the
    // start of a vector phase: its scalar loads of the next list entries
    // then complete under the softmax (a vector phase reads no LDS), not at
    // a barrier.  In the loop both groups run the softmax of entry e_0
    // (before the advance) and group 1 fetches K of e_2 and V of e_1 (also
    // before the advance); in phase 0 group 1 does not advance (softmax of
    // nothing, fetches K of e_1 and V of e_0).
    const uint32_t skip = __builtin_amdgcn_readfirstlane(grp != 1 ? 1u : 0u);
    auto run_vector_phase = [&](bool in_loop) INLINE {
      const int es = in_loop ? e_0 : NONE;
      const int tk = ent_tile(in_loop ? e_2 : e_1);
      const int tv = ent_tile(in_loop ? e_1 : e_0);
      if (in_loop) {
        advance();
        ++w;
      }
      vector_phase(ent_in(es, grp), ent_tile(es), tk, tv,
                   kl32 + (uint32_t)(((w + 1) & 1) * TILE_BYTES),
                   vl32 + (uint32_t)((w & 1) * TILE_BYTES), skip, krs4, vrs4);
    };
    if (grp == 1 && e_0 != NONE) {
      // phase 0 (with no entry at all there is none: group 0 runs no
      // iteration either)
      run_vector_phase(false);
      BARRIER();
    }
    while (e_0 != NONE || e_m1 != NONE) {
      matrix_phase(ent_in(e_m1, grp), ent_in(e_0, grp));
      if (grp == 1) {
        // the tiles fetched in the previous vector phase have landed
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      BARRIER();
      // group 1's window after its next advance would be (e_0, e_1, ...)
      if (grp == 1 && !(e_1 != NONE || e_0 != NONE)) break;
      run_vector_phase(true);
      BARRIER();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue: O = O^T / l
    l_over_halves();
    store_o(head_row, qt, l > 0.f ? 1.f / l : 0.f, 0, 4);
    store_lse(head_row, qt, m, l);
  }
  } else {
    // ================= planned: one persistent workgroup per worker =================
    // The worker's pair-mode items form one stream of steps (each item's
    // union list, item after item), walked exactly as one item's list in
    // pair mode above, with no drain between items: when the next entry
    // begins a new item, the vector phase ends by loading and scaling that
    // item's Q rows (Q is free once the old item's last S is done) and
    // clearing the -m bias; when the current entry begins a new item, the
    // vector phase first writes the old item's O and LSE (its last P V ran
    // in the matrix phase just ended) and clears O, m and l.  K and V tiles
    // are fetched from the head of the item each entry belongs to.  Then
    // the worker's split-mode items run one after the other as above.
    const sconst_i32 hdr = (sconst_i32)(uintptr_t)a.plan;
    const int wk = (int)blockIdx.x;
    const int BH = a.B * a.H;
    if (hdr[0] != kPlanMagic || hdr[1] != a.B || hdr[2] != a.H || hdr[3] != N ||
        hdr[4] != a.tiles || hdr[5] != a.mask_heads || hdr[6] != (int)gridDim.x ||
        hdr[7] != (int)pairs)
      return;  // a plan made for other arguments (uniform: nothing ran yet)
    // this worker's streams: [w0, w1) pair-mode steps, [w1, w2) group 0's
    // single-tile steps, [w2, w3) group 1's (clamped into the step array)
    const int cap = (int)min(a.pl.step_cap, (int64_t)0x7FFFFFFF);
    const sconst_i32 wstep = (sconst_i32)(uintptr_t)(a.plan + a.pl.off_wstep);
    const int w0 = min(max(wstep[4 * wk], 0), cap);
    const int w1 = min(max(wstep[4 * wk + 1], w0), cap);
    const int w2 = min(max(wstep[4 * wk + 2], w1), cap);
    const int w3 = min(max(wstep[4 * wk + 3], w2), cap);
    const int sb = w0, se = w1;
    // For the XCD feedback table: the workgroup's start and the load its
    // plan gave it (the plan's cost units: 5 per pair-mode step and per
    // item, 4 per single-tile step), kept in VGPRs (scalar registers are
    // scarce in the stream loop).
    uint64_t t_start = __builtin_amdgcn_s_memrealtime();
    int fb_load = 5 * (w1 - w0) + 4 * (w3 - w1) +
                  5 * max(((sconst_i32)(uintptr_t)(a.plan + a.pl.off_witem))[2 * wk + 1], 0);
    asm volatile("" : "+v"(t_start), "+v"(fb_load));
    typedef const __attribute__((address_space(4))) uint64_t* sconst_u64;
    const sconst_u64 steps = (sconst_u64)(uintptr_t)(a.plan + a.pl.off_steps);
    // item word -> the head's first row, and this group's query tile
    auto item_hr = [&](int iw) INLINE {
      return (int64_t)min((int)((uint32_t)iw >> kPlanPairBits), BH - 1) * N;
    };
    auto item_qt = [&](int iw) INLINE {
      return 2 * min(iw & ((1 << kPlanPairBits) - 1), (int)pairs - 1) + grp;
    };
    int i_m1 = -1, i_0 = -1, i_1 = -1, i_2 = -1;  // item words of the window
    if (sb < se) {
      int sidx = sb;
      const int slast = se - 1;
      uint64_t look = steps[sb];  // the next step, loaded one call ahead
      auto next_step = [&](int& iw) INLINE {
        const bool have = sidx < se;
        const uint64_t cur = look;
        ++sidx;
        look = steps[min(sidx, slast)];
        iw = have ? (int)(uint32_t)(cur >> 32) : -1;
        return have ? (int)((uint32_t)cur & 0x7FFFFFFFu) : NONE;
      };
      e_m1 = NONE;
      e_0 = next_step(i_0);
      e_1 = next_step(i_1);
      e_2 = next_step(i_2);
      int cur = i_0;  // the item whose O this group accumulates
      int64_t cur_hr = item_hr(cur);
      int cur_qt = item_qt(cur);
      load_q(cur_hr, cur_qt);
      kr = kr_slot0;
      vr[0] = vr0_slot0 ^ (uint32_t)TILE_BYTES;
      vr[1] = vr1_slot0 ^ (uint32_t)TILE_BYTES;
      int w = 0;
      load_first_k(e_0, k_brsrc(item_hr(i_0)));
      auto advance = [&]() INLINE {
        e_m1 = e_0;
        i_m1 = i_0;
        e_0 = e_1;
        i_0 = i_1;
        e_1 = e_2;
        i_1 = i_2;
        e_2 = next_step(i_2);
        flip_slots();
      };
      const uint32_t skip = __builtin_amdgcn_readfirstlane(grp != 1 ? 1u : 0u);
      auto run_vector_phase = [&](bool in_loop) INLINE {
        const int es = in_loop ? e_0 : NONE;
        const int tk = ent_tile(in_loop ? e_2 : e_1);
        const int ik = in_loop ? i_2 : i_1;
        const int tv = ent_tile(in_loop ? e_1 : e_0);
        const int iv = in_loop ? i_1 : i_0;
        bool bnd = false, nxt = false;
        int ncur = 0, nq = 0;
        if (in_loop) {
          bnd = e_0 != NONE && e_m1 != NONE && i_0 != i_m1;
          nxt = e_1 != NONE && i_1 != i_0;
          ncur = i_0;
          nq = i_1;
          advance();
          ++w;
        }
        if (bnd) {
          l_over_halves();
          store_o(cur_hr, cur_qt, l > 0.f ? 1.f / l : 0.f, 0, 4);
          store_lse(cur_hr, cur_qt, m, l);
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
          m = -INFINITY;
          l = 0.f;
          cur = ncur;
          cur_hr = item_hr(cur);
          cur_qt = item_qt(cur);
        }
        vector_phase(ent_in(es, grp), ent_tile(es), tk, tv,
                     kl32 + (uint32_t)(((w + 1) & 1) * TILE_BYTES),
                     vl32 + (uint32_t)((w & 1) * TILE_BYTES), skip, k_rsrc(item_hr(ik)),
                     v_rsrc(item_hr(iv)));
        if (nxt) {
          // the new item's Q, loaded and scaled here so that no load of it
          // is pending in the matrix phases (group 1 also waits here for
          // this phase's tile fetches, once per item)
          load_q(item_hr(nq), item_qt(nq));
#pragma unroll
          for (int e = 0; e < 16; ++e) nm[e] = 0.f;
        }
      };
      if (grp == 1) {
        run_vector_phase(false);  // phase 0
        BARRIER();
      }
      while (e_0 != NONE || e_m1 != NONE) {
        matrix_phase(ent_in(e_m1, grp), ent_in(e_0, grp));
        if (grp == 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        BARRIER();
        if (grp == 1 && !(e_1 != NONE || e_0 != NONE)) break;
        run_vector_phase(true);
        BARRIER();
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      l_over_halves();
      store_o(cur_hr, cur_qt, l > 0.f ? 1.f / l : 0.f, 0, 4);
      store_lse(cur_hr, cur_qt, m, l);
    }

    // ---- the split-mode items: each group walks its own stream of single
    // query tiles (tile 2p of an item in group 0's, 2p + 1 in group 1's),
    // with its own K slot and V slot, item after item with no drain.  As in
    // split mode, group g's matrix phase i runs P V of its entry i-1 and S
    // of entry i; its vector phase i the softmax of entry i and the fetches
    // of K of entry i+1 and V of entry i, awaited before the phase ends.
    // Both groups run n = 1 + (the longer stream's length) matrix phases
    // and pass the same barriers; a group whose stream is done idles.
    if (w3 > w1) {
      reset_state();
      const int gb = grp ? w2 : w1, ge = grp ? w3 : w2;
      const int niter = max(w2 - w1, w3 - w2) + 1;
      auto tile_hr = [&](int iw) INLINE {
        return (int64_t)min((int)((uint32_t)iw >> kPlanTileBits), BH - 1) * N;
      };
      auto tile_qt = [&](int iw) INLINE {
        return min(iw & ((1 << kPlanTileBits) - 1), a.tiles - 1);
      };
      int sidx = gb;
      const int slast = max(ge - 1, gb);
      uint64_t look = gb < ge ? steps[gb] : 0;
      auto next_step = [&](int& iw) INLINE {
        const bool have = sidx < ge;
        const uint64_t cur = look;
        ++sidx;
        look = steps[min(sidx, slast)];
        iw = have ? (int)(uint32_t)(cur >> 32) : -1;
        return have ? (int)((uint32_t)cur & 0x1FFFFFFFu) : NONE;
      };
      e_m1 = NONE;
      i_m1 = -1;
      e_0 = next_step(i_0);
      e_1 = next_step(i_1);
      int cur = i_0;  // -1: this group's stream is empty
      int64_t cur_hr = cur >= 0 ? tile_hr(cur) : 0;
      int cur_qt = cur >= 0 ? tile_qt(cur) : 0;
      if (cur >= 0) load_q(cur_hr, cur_qt);
      kr = kr_slot0 ^ (uint32_t)(grp * TILE_BYTES);
      vr[0] = vr0_slot0 ^ (uint32_t)(grp * TILE_BYTES);
      vr[1] = vr1_slot0 ^ (uint32_t)(grp * TILE_BYTES);
      const uint32_t kown = kl32 + (uint32_t)(grp * TILE_BYTES);
      const uint32_t vown = vl32 + (uint32_t)(grp * TILE_BYTES);
      // prologue: each group fetches the K tile of its first entry
      vector_phase(false, -1, ent_tile(e_0), -1, kown, vown, 0u,
                   k_rsrc(cur >= 0 ? cur_hr : 0), v_rsrc(0));
      __builtin_amdgcn_s_waitcnt(WAIT_VM0);
      BARRIER();
      auto ind_vector = [&]() INLINE {
        const bool bnd = e_0 != NONE && e_m1 != NONE && i_0 != i_m1;
        const bool nxt = e_1 != NONE && i_1 != i_0;
        if (bnd) {
          l_over_halves();
          store_o(cur_hr, cur_qt, l > 0.f ? 1.f / l : 0.f, 0, 4);
          store_lse(cur_hr, cur_qt, m, l);
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
          m = -INFINITY;
          l = 0.f;
          cur = i_0;
          cur_hr = tile_hr(cur);
          cur_qt = tile_qt(cur);
        }
        // (the softmax always runs: with no entry every score is masked, so
        // P = 0 and m, l and O stay as they are)
        vector_phase(true, ent_tile(e_0), ent_tile(e_1), ent_tile(e_0), kown, vown, 0u,
                     k_rsrc(e_1 != NONE ? tile_hr(i_1) : 0),
                     v_rsrc(e_0 != NONE ? tile_hr(i_0) : 0));
        if (nxt) {
          load_q(tile_hr(i_1), tile_qt(i_1));
#pragma unroll
          for (int e = 0; e < 16; ++e) nm[e] = 0.f;
        }
        // this phase's fetches (and the new Q) have landed; as a builtin, so
        // the compiler keeps no wait of its own in the matrix phases
        __builtin_amdgcn_s_waitcnt(WAIT_VM0);
        BARRIER();
        e_m1 = e_0;
        i_m1 = i_0;
        e_0 = e_1;
        i_0 = i_1;
        e_1 = next_step(i_1);
      };
      if (grp == 1) BARRIER();  // phase 0: group 0's first matrix phase
#pragma unroll 1
      for (int it = 0; it < niter; ++it) {
        matrix_phase(e_m1 != NONE, e_0 != NONE);
        BARRIER();
        if (grp == 1 && it + 1 == niter) break;
        ind_vector();
      }
      if (cur >= 0) {
        l_over_halves();
        store_o(cur_hr, cur_qt, l > 0.f ? 1.f / l : 0.f, 0, 4);
        store_lse(cur_hr, cur_qt, m, l);
      }
    }
    // XCD feedback: how long this workgroup ran and its load, read by the
    // next plan on this device
    if (tid == 0) {
      const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
      reinterpret_cast<int2*>(a.xfb)[wk] =
          make_int2((int)min(t_end - t_start, (uint64_t)0x7FFFFFFF), fb_load);
    }
  }

  // ================= split-mode items =================
  // Not planned: this workgroup's pair, when its mode is split.  Planned:
  // the worker's split-mode items, one after the other (both groups have
  // passed the same barriers in the stream, and no LDS read or tile fetch
  // is in flight).
  const int ic = PLANNED ? 0 : (split ? 1 : 0);
#pragma unroll 1
  for (int t = 0; t < ic; ++t) {
    // ================= split mode =================
    // Both groups work on one query tile (the same 128 rows, the same Q),
    // entry e of its list going to group e % 2.  Phase p: group p % 2 runs
    // its matrix phase (P V of entry p-2, S of entry p) from its own K and
    // V slots (slot g of group g); the other group runs the softmax of
    // entry p-1 and fetches K of entry p+1 and V of entry p-1 into its own
    // slots (last read in phase p-1), awaited before the barrier that ends
    // phase p.  Each group thus holds partial (m, l, O) over its entries;
    // they are combined at the end.
    float* const xo = reinterpret_cast<float*>(kslots);  // exchange area
    float* const xml = reinterpret_cast<float*>(vslots);
#pragma unroll 1
    for (int tt = 0; tt < 2; ++tt) {
      const int tq = qt0 + tt;
      if (tq >= a.tiles) break;
      if (tt > 0) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
        m = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) nm[e] = 0.f;
      }
      load_q(head_row, tq);
      init_lists(tt == 0 ? jb0 : jb1, tt == 0 ? n0 : n1, 0, 0);
      kr = kr_slot0 ^ (uint32_t)(grp * TILE_BYTES);
      vr[0] = vr0_slot0 ^ (uint32_t)(grp * TILE_BYTES);
      vr[1] = vr1_slot0 ^ (uint32_t)(grp * TILE_BYTES);
      // window: entries p-2, p-1, p, p+1 in phase p
      e_2 = NONE;  // entry p-2
      e_m1 = NONE;
      e_0 = next_entry();
      e_1 = next_entry();
      load_first_k(e_0, k_brsrc(head_row));
      const uint32_t kown = kl32 + (uint32_t)(grp * TILE_BYTES);
      const uint32_t vown = vl32 + (uint32_t)(grp * TILE_BYTES);
      // n + 2 phases (p = 0 .. n+1); group g runs its matrix phases at
      // p = g, g+2, ... and its vector phases in between, so both groups
      // pass the same n + 2 barriers
      const int nphase = (tt == 0 ? n0 : n1) + 2;
      auto split_advance = [&]() INLINE {
        e_2 = e_m1;
        e_m1 = e_0;
        e_0 = e_1;
        e_1 = next_entry();
      };
      auto split_vector = [&]() INLINE {
        // the softmax always runs: with no entry (j = -1) every score is
        // masked to -inf, so P = 0 and m, l and O stay as they are (a
        // runtime choice here costs the register allocator dearly)
        vector_phase(true, ent_tile(e_m1), ent_tile(e_1), ent_tile(e_m1), kown, vown, 0u, krs4,
                     vrs4);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        BARRIER();
        split_advance();
      };
      if (grp == 1) split_vector();  // phase 0
      // (an exit rather than a conditional vector phase: the matrix and
      // vector phases then never sit on alternative paths, which costs the
      // register allocator dearly)
#pragma unroll 1
      for (int p = grp; p < nphase; p += 2) {
        matrix_phase(e_2 != NONE, e_0 != NONE);
        BARRIER();
        split_advance();
        if (p + 1 >= nphase) break;
        split_vector();
      }
      // ---- combine the two groups' (m, l, O): group 0 finishes d blocks 0
      // and 1, group 1 blocks 2 and 3; each hands the other half over
      // through LDS (the K slots, free now)
      l_over_halves();
      // (d-block indices are compile-time constants in every access: a
      // runtime index would move the accumulators to scratch memory)
      auto give_half = [&](int base) INLINE {
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
          for (int f4 = 0; f4 < 4; ++f4) {
            f32x4 v;
            v[0] = oacc[base + d2][4 * f4];
            v[1] = oacc[base + d2][4 * f4 + 1];
            v[2] = oacc[base + d2][4 * f4 + 2];
            v[3] = oacc[base + d2][4 * f4 + 3];
            *reinterpret_cast<f32x4*>(xo + ((wave * 8 + d2 * 4 + f4) * 64 + lane) * 4) = v;
          }
      };
      if (grp == 0) give_half(2); else give_half(0);
      xml[(wave * 64 + lane) * 2] = m;
      xml[(wave * 64 + lane) * 2 + 1] = l;
      BARRIER();
      const int pw = wave ^ 4;  // the other group's wave with the same rows
      const float mp = xml[(pw * 64 + lane) * 2];
      const float lpn = xml[(pw * 64 + lane) * 2 + 1];
      const float mt = fmaxf(m, mp);
      const float a0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mt);
      const float a1 = mp == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mp - mt);
      auto keep_half = [&](int base) INLINE {
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
          for (int f4 = 0; f4 < 4; ++f4) {
            const f32x4 v =
                *reinterpret_cast<const f32x4*>(xo + ((pw * 8 + d2 * 4 + f4) * 64 + lane) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              oacc[base + d2][4 * f4 + e] = oacc[base + d2][4 * f4 + e] * a0 + v[e] * a1;
          }
      };
      if (grp == 0) keep_half(0); else keep_half(2);
      const float lt = l * a0 + lpn * a1;
      if (grp == 0)
        store_o(head_row, tq, lt > 0.f ? 1.f / lt : 0.f, 0, 2);
      else
        store_o(head_row, tq, lt > 0.f ? 1.f / lt : 0.f, 2, 2);
      if (grp == 0) store_lse(head_row, tq, mt, lt);
      // the exchange area is the next tile's K slot 0
      BARRIER();
    }
  }
}

}  // namespace

int launch_fwd_bf16_t128_d128(const FwdLaunch& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.plan != nullptr) {
    // one persistent workgroup per worker of the plan
    const dim3 grid((unsigned)a.pl.workers);
    FwdLaunch b = a;
    const int fe = xcd_feedback(&b.xfb);
    if (fe != hipSuccess) return fe;
    if (a.window > 0)
      hipLaunchKernelGGL((fwd_bf16_t128_d128<true, true>), grid, dim3(512), 0, s, b);
    else
      hipLaunchKernelGGL((fwd_bf16_t128_d128<false, true>), grid, dim3(512), 0, s, b);
    return hipGetLastError();
  }
  // one workgroup per (batch*head, query-tile pair), in either mode
  const int64_t blocks = (int64_t)a.B * a.H * ((a.tiles + 1) / 2);
  if (a.window > 0)
    hipLaunchKernelGGL((fwd_bf16_t128_d128<true, false>), dim3((unsigned)blocks), dim3(512), 0,
                       s, a);
  else
    hipLaunchKernelGGL((fwd_bf16_t128_d128<false, false>), dim3((unsigned)blocks), dim3(512), 0,
                       s, a);
  return hipGetLastError();
}

}  // namespace bsattn
