// Work plan of the planned block-sparse forward (bf16, d 128, 128x128 tiles).
//
// The active lists are static inputs of the forward (CalibAtt page, "B. Fase
// di Inferenza": the kernel follows precomputed per-block lists and takes no
// decision itself), so everything the forward's workgroups would otherwise
// work out for themselves at every launch is worked out once per list set:
// which query-tile pairs go to which worker (one persistent workgroup per
// compute unit), in which order, and the merged key-tile list of every pair.
//
// A work item is one (batch, head, query-tile pair p) -- query tiles 2p and
// 2p + 1.  When the two active lists largely coincide (pair mode), the
// worker's two groups of four waves own one query tile each and walk the
// union of the two lists, so every staged key tile serves both.  When they
// have little in common (split mode: 5 I < n0 + n1, I common tiles of lists
// of n0 and n1 entries, and always when one list is empty), tile 2p goes to
// group 0 and tile 2p + 1 to group 1, each walking its own list.  A worker
// thus has three streams of steps: its pair-mode items (one step per union
// tile) and one single-tile stream per group.
//
// Three launches:
//   1. pairs:  one wave per (mask slice, pair): the two lists become bitmaps
//              in LDS; the union and common tile counts are popcounts.
//   2. assign: one workgroup per XCD.  Items are cut into eight contiguous ranges
//              of equal estimated cost (neighbouring pairs of a head share
//              key tiles, which the XCD's L2 then serves), and each range is
//              spread over the XCD's workers (worker w runs on XCD w % 8):
//              256 items at a time (a whole range at most shapes) are ranked
//              by cost, longest first, and dealt in rounds of half the
//              XCD's workers, the longest of a round to the least-loaded
//              worker.  Ranges of up to 1024 items are then refined: in
//              rounds, the k-th most loaded worker and the k-th least loaded
//              exchange the item (or pair of items) that best evens them
//              out, and each worker runs its items in item order.  Records
//              each item's worker, its place in the worker's order and the
//              offsets of its steps in the worker's streams.
//   3. steps:  one wave per item: the worker's item list; for a pair-mode
//              item its union list in ascending key-tile order, one step per
//              tile, (tile | group 0 needs it << 30 | group 1 needs it << 29,
//              item word); for a split-mode item each tile's own list into
//              its group's stream, (tile, tile's item word).  An empty list
//              is one step with no tile (its rows are still written).
//
// Outputs depend only on the lists: the forward computes every item the same
// way whichever worker runs it.  Every read of the CSR is clamped to its
// capacity and every write to the plan's own capacity.
#include <hip/hip_runtime.h>

#include <mutex>

#include "bsattn_internal.h"

namespace bsattn {
namespace {

constexpr int kWave = 64;
constexpr int kWords = kPlanMaxTiles / 32;  // bitmap words per list
constexpr int kBadTile = 0x0FFFFFFE;        // a step with no key tile

struct PlanArgs {
  PlanLayout L;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int64_t col_cap;
  char* plan;
  const int32_t* xfb;  // the device's XCD feedback table (int32 pairs)
};

__device__ __forceinline__ int32_t* P32(const PlanArgs& a, int64_t off) {
  return reinterpret_cast<int32_t*>(a.plan + off);
}

// list of CSR row r: first entry and length, clamped to the capacity
__device__ __forceinline__ int list_of(const PlanArgs& a, int r, int64_t& begin) {
  int64_t b0 = a.row_ptr[r], e0 = a.row_ptr[r + 1];
  if (b0 < 0) b0 = 0;
  if (e0 > a.col_cap) e0 = a.col_cap;
  begin = b0;
  return e0 > b0 ? (int)(e0 - b0) : 0;
}

// The two lists of pair p in mask slice s as bitmaps in this wave's LDS
// words (bm[0..kWords) for tile 2p, bm[kWords..2 kWords) for tile 2p + 1);
// entries outside [0, tiles) are left out.  Returns the raw list lengths.
// Called by every wave of the workgroup (it holds workgroup barriers); a
// wave with use == false builds empty bitmaps.
__device__ void lists_to_bitmaps(const PlanArgs& a, bool use, int s, int p, uint32_t* bm,
                                 int lane, int& n0, int& n1) {
  const int tiles = a.L.tiles;
  for (int wd = lane; wd < 2 * kWords; wd += kWave) bm[wd] = 0u;
  __syncthreads();
  n0 = n1 = 0;
  int64_t b0 = 0, b1 = 0;
  if (use) {
    const int r0 = s * tiles + 2 * p;
    n0 = list_of(a, r0, b0);
    n1 = 2 * p + 1 < tiles ? list_of(a, r0 + 1, b1) : 0;
  }
  for (int e = lane; e < n0; e += kWave) {
    const int t = a.col_idx[b0 + e];
    if (t >= 0 && t < tiles) atomicOr(&bm[t >> 5], 1u << (t & 31));
  }
  for (int e = lane; e < n1; e += kWave) {
    const int t = a.col_idx[b1 + e];
    if (t >= 0 && t < tiles) atomicOr(&bm[kWords + (t >> 5)], 1u << (t & 31));
  }
  __syncthreads();
}

// the 64 tiles 64 lane .. 64 lane + 63 of both bitmaps
__device__ __forceinline__ void lane_words(const uint32_t* bm, int lane, uint64_t& wa,
                                           uint64_t& wb) {
  const int w0 = 2 * lane;
  wa = (uint64_t)bm[w0] | ((uint64_t)bm[w0 + 1] << 32);
  wb = (uint64_t)bm[kWords + w0] | ((uint64_t)bm[kWords + w0 + 1] << 32);
}

__device__ __forceinline__ int wave_sum(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// The XCDs of one GPU run at different speeds (up to a tenth apart, in the
// same order whatever the work), and a launch lasts as long as its slowest
// XCD.  Every planned forward leaves, per worker, how long its workgroup
// ran (s_memrealtime ticks) and the load the plan gave it (the cost units
// of item_cost_sp); worker w ran on XCD w mod 8.  Each XCD's speed is its
// summed load over its summed time, and the XCD ranges of the next plan
// are cut in proportion to the speeds, relative to their mean and clamped
// to [0.9, 1.1].  Only long launches are trusted: when the loaded
// workgroups ran under 400 us on average (short lists, such as SQuad's
// passes, where fetch latency and the launch's own start and end dominate)
// the speeds mislead (measured: 8 % slower than equal weights there), and
// every weight is 1, as with no record at all.  The weights go
// into the plan, so that the eight workgroups of the assign kernel cut by
// the same ones even while another launch writes the table.  Workers with
// no load are left out.  Run by one workgroup of 256 threads.
__device__ void xcd_weights(const PlanArgs& a) {
  __shared__ int64_t xs[4][3 * kPlanXcds];
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  int64_t ld = 0, bz = 0, nw = 0;  // this thread's workers: tid, tid + 256 (XCD tid % 8)
  for (int w = tid; w < a.L.workers; w += 256) {
    const int2 r = reinterpret_cast<const int2*>(a.xfb)[w];
    if (r.x > 0 && r.y > 0) {
      bz += r.x;
      ld += r.y;
      nw += 1;
    }
  }
  // lanes l, l + 8, ..., l + 56 share an XCD
  for (int o = 8; o < kWave; o <<= 1) {
    ld += __shfl_xor(ld, o, kWave);
    bz += __shfl_xor(bz, o, kWave);
    nw += __shfl_xor(nw, o, kWave);
  }
  if (lane < kPlanXcds) {
    xs[wv][lane] = ld;
    xs[wv][kPlanXcds + lane] = bz;
    xs[wv][2 * kPlanXcds + lane] = nw;
  }
  __syncthreads();
  if (tid == 0) {
    double sp[kPlanXcds], mean = 0.0;
    int64_t btot = 0, ntot = 0;
    bool ok = true;
    for (int x = 0; x < kPlanXcds; ++x) {
      const int64_t l = xs[0][x] + xs[1][x] + xs[2][x] + xs[3][x];
      const int64_t b = xs[0][kPlanXcds + x] + xs[1][kPlanXcds + x] + xs[2][kPlanXcds + x] +
                        xs[3][kPlanXcds + x];
      const int64_t n = xs[0][2 * kPlanXcds + x] + xs[1][2 * kPlanXcds + x] +
                        xs[2][2 * kPlanXcds + x] + xs[3][2 * kPlanXcds + x];
      ok = ok && l > 0 && b > 0;
      sp[x] = ok ? (double)l / (double)b : 0.0;
      mean += sp[x];
      btot += b;
      ntot += n;
    }
    // 400 us (100 MHz ticks) per loaded workgroup on average
    ok = ok && ntot > 0 && btot >= 40000 * ntot;
    mean /= kPlanXcds;
    int32_t* xw = P32(a, a.L.off_xw);
    for (int x = 0; x < kPlanXcds; ++x) {
      const double r = ok && mean > 0.0 ? fmin(fmax(sp[x] / mean, 0.9), 1.1) : 1.0;
      xw[x] = (int32_t)(r * kPlanWeightOne + 0.5);
    }
  }
}

// ---- 1. per (mask slice, pair): union and common tile counts
__global__ void __launch_bounds__(256) plan_pairs_kernel(PlanArgs a) {
  __shared__ uint32_t bms[4][2 * kWords];
  const int lane = threadIdx.x % kWave;
  const int wv = threadIdx.x / kWave;
  const int64_t sp = (int64_t)blockIdx.x * 4 + wv;
  const PlanLayout& L = a.L;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    int32_t* h = P32(a, 0);
    h[0] = kPlanMagic;
    h[1] = L.B;
    h[2] = L.H;
    h[3] = L.N;
    h[4] = L.tiles;
    h[5] = L.mask_heads;
    h[6] = L.workers;
    h[7] = L.pairs;
    // the sections, in units of 16 bytes, and the step capacity (for readers
    // of the plan other than the forward)
    h[8] = (int32_t)(L.off_wstep / 16);
    h[9] = (int32_t)(L.off_witem / 16);
    h[10] = (int32_t)(L.off_wcnt / 16);
    h[11] = (int32_t)(L.off_witems / 16);
    h[12] = (int32_t)(L.off_pinfo / 16);
    h[13] = (int32_t)(L.off_itmp / 16);
    h[14] = (int32_t)(L.off_steps / 16);
    h[15] = (int32_t)min(L.step_cap, (int64_t)0x7FFFFFFF);
  }
  if (blockIdx.x == 0) xcd_weights(a);
  const bool use = sp < (int64_t)L.mask_heads * L.pairs;
  const int s = use ? (int)(sp / L.pairs) : 0, p = use ? (int)(sp % L.pairs) : 0;
  int n0, n1;
  lists_to_bitmaps(a, use, s, p, bms[wv], lane, n0, n1);
  uint64_t wa, wb;
  lane_words(bms[wv], lane, wa, wb);
  const int u = wave_sum(__popcll(wa | wb));
  const int common = wave_sum(__popcll(wa & wb));
  const int va = wave_sum(__popcll(wa));
  const int vb = wave_sum(__popcll(wb));
  if (use && lane == 0) {
    int32_t* pi = P32(a, L.off_pinfo) + 8 * sp;
    pi[0] = u;
    pi[1] = common;
    pi[2] = n0;
    pi[3] = n1;
    pi[4] = va;
    pi[5] = vb;
  }
}

struct ItemCost {
  int cost;   // estimated work, in fifths of a pair-mode step
  int steps;  // steps in the worker's pair-mode stream (0 in split mode)
  int sa, sb; // steps in the groups' single-tile streams (0 in pair mode)
  int split;
};

// cost of the item of (mask slice s, pair p)
__device__ __forceinline__ ItemCost item_cost_sp(const PlanArgs& a, int s, int p) {
  const PlanLayout& L = a.L;
  const int32_t* pi = P32(a, L.off_pinfo) + 8 * ((int64_t)s * L.pairs + p);
  const int u = pi[0], common = pi[1], n0 = pi[2], n1 = pi[3], va = pi[4], vb = pi[5];
  ItemCost c;
  // the rule of bsattn_fwd: split mode unless the lists largely coincide
  c.split = (n0 == 0 || n1 == 0 || 5 * common < n0 + n1) ? 1 : 0;
  c.steps = c.split ? 0 : max(u, 1);
  c.sa = c.split ? max(va, 1) : 0;
  c.sb = c.split && 2 * p + 1 < L.tiles ? max(vb, 1) : 0;
  // a single-tile step serves half the rows of a pair-mode step and its
  // fetch has one phase to land instead of two: about 0.8 of a pair-mode
  // step each (two run side by side); every item also pays a hand-over
  c.cost = c.split ? 4 * (c.sa + c.sb) + 5 : 5 * (c.steps + 1);
  return c;
}

// The assign kernel keeps every (mask slice, pair)'s cost in LDS when they
// fit (cost, and steps | split << 30), else reads them from the plan.
constexpr int kLdsPairs = 4096;

struct CostTable {
  const int* cost;   // LDS, or null
  const int* steps;  // steps | split << 30, or sa | sb << 15 | split << 30
  __device__ __forceinline__ ItemCost get(const PlanArgs& a, int s, int p) const {
    if (cost == nullptr) return item_cost_sp(a, s, p);
    const int sp = s * a.L.pairs + p;
    ItemCost c;
    const int st = steps[sp];
    c.cost = cost[sp];
    c.split = st >> 30;
    c.steps = c.split ? 0 : st & 0x3FFFFFFF;
    c.sa = c.split ? st & 0x7FFF : 0;
    c.sb = c.split ? (st >> 15) & 0x7FFF : 0;
    return c;
  }
  __device__ __forceinline__ ItemCost item(const PlanArgs& a, int i) const {
    const int bh = i / a.L.pairs;
    return get(a, a.L.mask_heads == 1 ? 0 : bh % a.L.H, i - bh * a.L.pairs);
  }
};

// ---- 2. per XCD: the item range and its deal over the XCD's workers
constexpr int kAssignThreads = 256;
// items ranked together: the deal balances the workers only as well as the
// longest items of a range are seen before the short ones, and ranges of a
// few hundred lumpy items (lists of 12 to 180 tiles in one calibrated mask)
// need the whole range at once
constexpr int kBatch = kAssignThreads;
// XCD ranges of at most this many items are refined after the deal (below)
constexpr int kRefineItems = 1024;
constexpr int kRefineWords = kRefineItems / 32;
constexpr int kRefineRounds = 8;
constexpr int kListCap = 32;  // items per worker the refinement searches

__global__ void __launch_bounds__(kAssignThreads) plan_assign_kernel(PlanArgs a) {
  __shared__ int64_t part[kAssignThreads];
  __shared__ __attribute__((aligned(16))) uint32_t keys[kBatch];
  __shared__ int sorted[kBatch];
  __shared__ int s_cost[kBatch], s_steps[kBatch];
  // each dealt item's record, kept here until its batch is dealt: a global
  // store before every round's barrier would make each barrier wait for it
  __shared__ __attribute__((aligned(16))) int s_it[kBatch][4];
  __shared__ __attribute__((aligned(16))) int64_t s_load[kPlanMaxWorkersPerXcd];
  __shared__ int t_cost[kLdsPairs], t_steps[kLdsPairs];
  // refinement: each item's cost and steps, each worker's items as a bitmap
  // (for the records) and as a list (for the search), the workers by load,
  // whether a round moved anything, and whether a list overflowed
  __shared__ int s_ic[kRefineItems], s_ist[kRefineItems];
  __shared__ uint32_t s_wbm[kPlanMaxWorkersPerXcd][kRefineWords];
  __shared__ int16_t s_list[kPlanMaxWorkersPerXcd][kListCap];
  __shared__ __attribute__((aligned(16))) int s_lc[kPlanMaxWorkersPerXcd][kListCap];
  __shared__ int s_lcnt[kPlanMaxWorkersPerXcd];
  __shared__ int s_order[kPlanMaxWorkersPerXcd];
  __shared__ int s_lover;
  const int tid = threadIdx.x;
  const int x = blockIdx.x;  // XCD
  const PlanLayout& L = a.L;
  const int G = (int)L.items;
  const int R = L.workers / kPlanXcds;  // workers of this XCD: w = x + 8 j
  const int nsp = L.mask_heads * L.pairs;
  CostTable tab;
  tab.cost = nullptr;
  tab.steps = nullptr;
  if (nsp <= kLdsPairs) {
    for (int sp = tid; sp < nsp; sp += kAssignThreads) {
      const ItemCost c = item_cost_sp(a, sp / L.pairs, sp % L.pairs);
      t_cost[sp] = c.cost;
      t_steps[sp] = (c.split ? c.sa | (c.sb << 15) : c.steps) | (c.split << 30);
    }
    __syncthreads();
    tab.cost = t_cost;
    tab.steps = t_steps;
  }

  // item i goes to XCD floor(8 (2 prefix(i) + cost(i)) / (2 C)): contiguous
  // ranges of about equal cost.  Thread t sums a contiguous chunk, walking
  // (head, pair) incrementally.
  const int per = (G + kAssignThreads - 1) / kAssignThreads;
  const int c0 = min(tid * per, G), c1 = min(c0 + per, G);
  const int bh0 = c0 / L.pairs;
  const int p0 = c0 - bh0 * L.pairs;
  const int h0 = bh0 % L.H;
  int64_t sum = 0;
  {
    int p = p0, h = h0;
    for (int i = c0; i < c1; ++i) {
      sum += tab.get(a, L.mask_heads == 1 ? 0 : h, p).cost;
      if (++p == L.pairs) {
        p = 0;
        if (++h == L.H) h = 0;
      }
    }
  }
  // prefix of the chunk sums over the threads: within each wave by
  // shuffles, then across the four waves
  const int lane = tid & (kWave - 1), wv = tid / kWave;
  int64_t incl = sum;
  for (int o = 1; o < kWave; o <<= 1) {
    const int64_t t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) part[wv] = incl;
  __syncthreads();
  int64_t total = 0, before = 0;
  for (int w2 = 0; w2 < kAssignThreads / kWave; ++w2) {
    const int64_t t = part[w2];
    before += w2 < wv ? t : 0;
    total += t;
  }
  int64_t run = before + incl - sum;
  // XCD x takes the items whose cost midpoint falls in its share of the
  // total, shares in proportion to the weights wt (XCD speeds, from the
  // pairs kernel): item i lies below x when A < B C(x), A = (2 prefix(i) +
  // cost(i)) C(8), B = 2 total, C(x) = wt(0) + ... + wt(x - 1); at most x
  // when A < B C(x + 1) or x = 7
  //
  // The weights are used only when the items' costs vary (coefficient of
  // variation at least 0.1, as on window masks): a range then takes a
  // slightly larger or smaller share and the refinement spreads the
  // difference over its workers by exchanging items of different cost.
  // With items of one cost (a dense mask: six per worker) a few per cent
  // more work on an XCD is a seventh item on some of its workers, 17 %
  // more for them, and nothing can even that out (measured: 6 % slower
  // than equal weights).  Integer sums over the cost table, so every
  // workgroup decides the same.
  int64_t cs = 0, cs2 = 0;
  for (int sp = tid; sp < nsp; sp += kAssignThreads) {
    const int64_t c = tab.get(a, sp / L.pairs, sp % L.pairs).cost;
    cs += c;
    cs2 += c * c;
  }
  for (int o = kWave / 2; o > 0; o >>= 1) {
    cs += __shfl_xor(cs, o, kWave);
    cs2 += __shfl_xor(cs2, o, kWave);
  }
  __syncthreads();  // every wave has read part[] above
  if (lane == 0) {
    part[wv] = cs;
    part[kAssignThreads / kWave + wv] = cs2;
  }
  __syncthreads();
  cs = 0;
  cs2 = 0;
  for (int w2 = 0; w2 < kAssignThreads / kWave; ++w2) {
    cs += part[w2];
    cs2 += part[kAssignThreads / kWave + w2];
  }
  const double csd = (double)cs;
  const bool use_w = cs > 0 && 100.0 * ((double)nsp * (double)cs2 - csd * csd) >= csd * csd;
  int64_t cw_lo = 0, cw_hi = 0, cw_all = 0;
  {
    const int32_t* xw = P32(a, L.off_xw);
    for (int x2 = 0; x2 < kPlanXcds; ++x2) {
      const int64_t wt = use_w ? min(max(xw[x2], 1), 4 * kPlanWeightOne) : kPlanWeightOne;
      cw_lo += x2 < x ? wt : 0;
      cw_hi += x2 <= x ? wt : 0;
      cw_all += wt;
    }
  }
  int below = 0, upto = 0;  // items of this chunk on XCDs < x, <= x
  {
    const int64_t B2 = 2 * total;
    int p = p0, h = h0;
    for (int i = c0; i < c1; ++i) {
      const int c = tab.get(a, L.mask_heads == 1 ? 0 : h, p).cost;
      const int64_t A = cw_all * (2 * run + c);
      below += (total > 0 ? A < cw_lo * B2 : x > 0) ? 1 : 0;
      upto += (total <= 0 || x == kPlanXcds - 1 || A < cw_hi * B2) ? 1 : 0;
      run += c;
      if (++p == L.pairs) {
        p = 0;
        if (++h == L.H) h = 0;
      }
    }
  }
  // the counts summed over the workgroup: within each wave, then across
  int64_t bu = ((int64_t)below << 32) | (uint32_t)upto;
  for (int o = kWave / 2; o > 0; o >>= 1) bu += __shfl_xor(bu, o, kWave);
  __syncthreads();  // every wave has read part[] above
  if (lane == 0) part[wv] = bu;
  __syncthreads();
  bu = 0;
  for (int w2 = 0; w2 < kAssignThreads / kWave; ++w2) bu += part[w2];
  const int lo = (int)(bu >> 32), hi = (int)(bu & 0xFFFFFFFF);
  // worker j's key: its load * 512 + j, so one comparison orders by load
  // and then by index; slots past R hold 2^62 and never come first (loads
  // stay far below 2^53)
  if (tid < kPlanMaxWorkersPerXcd) s_load[tid] = tid < R ? (int64_t)tid : ((int64_t)1 << 62);

  // deal [lo, hi) over the R workers, kBatch items at a time; thread j < R
  // keeps worker j's item count and the lengths of its three streams (its
  // load in LDS)
  // Ranges of at most kRefineItems items keep only each item's worker in
  // the deal; the refinement below then evens the workers out and writes
  // the records.
  const bool refine = hi - lo <= kRefineItems && R >= 2;
  if (refine) {
    for (int k = tid; k < kPlanMaxWorkersPerXcd * kRefineWords; k += kAssignThreads)
      s_wbm[k / kRefineWords][k % kRefineWords] = 0u;
    if (tid == 0) s_lover = 0;
  }
  int cnt = 0, nsteps = 0, na = 0, nb = 0;
  for (int b0 = lo; b0 < hi; b0 += kBatch) {
    const int nvalid = min(kBatch, hi - b0);
    uint32_t key = 0;
    if (tid < nvalid) {
      const ItemCost ic = tab.item(a, b0 + tid);
      // longest first, ties by position; 0 marks an empty slot
      key = ((uint32_t)min(ic.cost, (1 << 23) - 1) << 8 | (uint32_t)(kBatch - 1 - tid)) + 1;
      s_cost[tid] = ic.cost;
      s_steps[tid] = (ic.split ? ic.sa | (ic.sb << 15) : ic.steps) | (ic.split << 30);
      if (refine) {
        s_ic[b0 - lo + tid] = ic.cost;
        s_ist[b0 - lo + tid] = s_steps[tid];
      }
    }
    keys[tid] = key;
    __syncthreads();
    if (tid < nvalid) {
      int rank = 0;
      const uint4* k4 = reinterpret_cast<const uint4*>(keys);
#pragma unroll
      for (int j = 0; j < kBatch / 4; ++j) {
        const uint4 kv = k4[j];
        rank += (kv.x > key) + (kv.y > key) + (kv.z > key) + (kv.w > key);
      }
      sorted[rank] = tid;
    }
    __syncthreads();
    // A round hands one item to each of its least-loaded workers.  When the
    // batch's items are uneven (its longest more than twice the median),
    // rounds of half the workers let a worker already holding some of the
    // longest sit rounds out instead of taking one item every round; when
    // they are even, rounds of all the workers deal the same way in half
    // the rounds.
    const int c_max = s_cost[sorted[0]], c_mid = s_cost[sorted[nvalid / 2]];
    const bool even = c_max <= 2 * c_mid;
    // an item of the refined path: its worker's bitmap bit, list entry and
    // cost (list overflow switches the refinement off)
    auto note = [&](int src, int n) {
      const int j = b0 - lo + src;
      s_wbm[tid][j >> 5] |= 1u << (j & 31);
      if (n < kListCap) {
        s_list[tid][n] = (int16_t)j;
        s_lc[tid][n] = s_cost[src];
      } else {
        s_lover = 1;
      }
    };
    if (refine && even) {
      // Even batches of a refined range are dealt in a snake, with no
      // ranking of the workers: rank r goes to worker r mod R on even
      // sweeps and R - 1 - (r mod R) on odd ones (the refinement evens out
      // what is left).
      if (tid < R) {
        int64_t ld = s_load[tid];
        bool odd = false;
        for (int r0 = 0; r0 < nvalid; r0 += R, odd = !odd) {
          const int r = r0 + (odd ? R - 1 - tid : tid);
          if (r < nvalid) {
            const int src = sorted[r];
            note(src, cnt);
            ld += (int64_t)s_cost[src] << 9;
            cnt += 1;
          }
        }
        s_load[tid] = ld;
      }
      __syncthreads();
    } else {
    const int per_round = even ? R : max(1, R / 2);
    for (int r0 = 0; r0 < nvalid; r0 += per_round) {
      const int k = min(per_round, nvalid - r0);
      int wr = R;
      int64_t mine = 0;
      if (tid < R) {
        // rank of worker tid by load (ties by index): the keys below mine,
        // counted by the sign of the difference over every slot, so the
        // reads issue back to back with no compare per slot
        mine = s_load[tid];
        wr = 0;
        if (R <= 32) {
#pragma unroll
          for (int j2 = 0; j2 < 32; ++j2) wr += (int)((uint64_t)(s_load[j2] - mine) >> 63);
        } else {
#pragma unroll
          for (int j2 = 0; j2 < kPlanMaxWorkersPerXcd; ++j2)
            wr += (int)((uint64_t)(s_load[j2] - mine) >> 63);
        }
      }
      __syncthreads();
      if (tid < R && wr < k) {
        const int src = sorted[r0 + wr];
        const int st = s_steps[src];
        const int split = st >> 30;
        int* it = s_it[src];
        it[0] = x + kPlanXcds * tid;
        it[1] = cnt;
        s_load[tid] = mine + ((int64_t)s_cost[src] << 9);
        if (refine) {
          note(src, cnt);
        } else if (split) {
          // the two tiles go to the two groups' streams, the longer list to
          // the shorter stream (orient 1: tile 2p + 1 to group 0's)
          const int sa = st & 0x7FFF, sb = (st >> 15) & 0x7FFF;
          const int orient = max(na + sb, nb + sa) < max(na + sa, nb + sb) ? 1 : 0;
          it[2] = na;
          it[3] = nb | (orient << 30);
          na += orient ? sb : sa;
          nb += orient ? sa : sb;
        } else {
          it[2] = nsteps;
          it[3] = 0;
          nsteps += st & 0x3FFFFFFF;
        }
        cnt += 1;
      }
      __syncthreads();
    }
    }
    if (!refine)
      for (int i = tid; i < nvalid; i += kAssignThreads)
        *reinterpret_cast<int4*>(P32(a, L.off_itmp) + 4 * (int64_t)(b0 + i)) =
            *reinterpret_cast<const int4*>(s_it[i]);
  }
  if (refine) {
    // With a few items per worker the deal leaves some workers an item more
    // than others (a range of 194 items on 32 workers: two hold seven), up
    // to 8 % above the mean load.  Each round ranks the workers by load and
    // pairs the k-th least loaded with the k-th most loaded; every pair
    // makes its best single move (an item of the heavier to the lighter)
    // or swap (an item each way), the one that brings their difference d
    // closest to zero, if it lowers the heavier's load.  Both new loads lie
    // between the old two, so no worker ever exceeds the old maximum.
    // Sixteen lanes search a pair, each taking every sixteenth word of the
    // heavier worker's bitmap; pairs are disjoint, so they move at once.
    const int nwd = (hi - lo + 31) >> 5;
    if (tid < R) s_lcnt[tid] = cnt;
    // (also when the range is empty and the deal passed no barrier: every
    // thread must read the same s_lover)
    __syncthreads();
    const int rounds = s_lover ? 0 : kRefineRounds;
    int64_t prev_max = INT64_MAX;
    for (int round = 0; round < rounds; ++round) {
      if (tid < R) {
        const int64_t mine = s_load[tid];
        int wr = 0;
        if (R <= 32) {
#pragma unroll
          for (int j2 = 0; j2 < 32; ++j2) wr += (int)((uint64_t)(s_load[j2] - mine) >> 63);
        } else {
#pragma unroll
          for (int j2 = 0; j2 < kPlanMaxWorkersPerXcd; ++j2)
            wr += (int)((uint64_t)(s_load[j2] - mine) >> 63);
        }
        s_order[wr] = tid;
      }
      __syncthreads();
      // stop once a round has not lowered the heaviest load
      const int64_t cur_max = s_load[s_order[R - 1]] >> 9;
      if (cur_max >= prev_max) break;
      prev_max = cur_max;
      const int grp16 = tid >> 4, gl = tid & 15;
      for (int k = grp16; k < R / 2; k += kAssignThreads / 16) {
        const int lw = s_order[k], hw = s_order[R - 1 - k];
        const int gap = (int)min((s_load[hw] >> 9) - (s_load[lw] >> 9), (int64_t)(1 << 24));
        const int nh = s_lcnt[hw], nl = s_lcnt[lw];
        // Lane gl tries the items at positions gl, gl + 16 of the heavier
        // list against every item of the lighter one and against none (a
        // move, while the lighter list has room); a candidate with
        // difference d, 0 < d < gap, scores |gap - 2 d|.  Key: score << 12 |
        // position of a << 6 | position of b (nl: a move).
        int64_t best = INT64_MAX;
        if (gap > 0) {
          const int nb1 = nl < kListCap ? nl + 1 : nl;
          for (int ai = gl; ai < nh; ai += 16) {
            const int ca = s_lc[hw][ai];
            int bl = INT32_MAX;  // score << 6 | b
            for (int b4 = 0; b4 < nb1; b4 += 4) {
              const int4 c4 = *reinterpret_cast<const int4*>(&s_lc[lw][b4]);
              const int cb[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int bi = b4 + e;
                const int d = ca - (bi < nl ? cb[e] : 0);
                const int v = abs(gap - 2 * d);
                if (bi < nb1 && d > 0 && d < gap) bl = min(bl, (v << 6) | bi);
              }
            }
            if (bl != INT32_MAX)
              best = min(best, ((int64_t)(bl >> 6) << 12) | (ai << 6) | (bl & 63));
          }
        }
        for (int o = 8; o > 0; o >>= 1) best = min(best, (int64_t)__shfl_xor(best, o, 16));
        if (gl == 0 && best != INT64_MAX) {
          const int ai = (int)((best >> 6) & 63), bi = (int)(best & 63);
          const int ia = s_list[hw][ai];
          int64_t d = s_lc[hw][ai];
          s_wbm[hw][ia >> 5] &= ~(1u << (ia & 31));
          s_wbm[lw][ia >> 5] |= 1u << (ia & 31);
          if (bi < nl) {
            const int ib = s_list[lw][bi];
            const int cb = s_lc[lw][bi];
            d -= cb;
            s_wbm[lw][ib >> 5] &= ~(1u << (ib & 31));
            s_wbm[hw][ib >> 5] |= 1u << (ib & 31);
            s_lc[lw][bi] = s_lc[hw][ai];
            s_list[lw][bi] = (int16_t)ia;
            s_list[hw][ai] = (int16_t)ib;
            s_lc[hw][ai] = cb;
          } else {
            s_list[lw][nl] = (int16_t)ia;
            s_lc[lw][nl] = s_lc[hw][ai];
            s_lcnt[lw] = nl + 1;
            s_list[hw][ai] = s_list[hw][nh - 1];
            s_lc[hw][ai] = s_lc[hw][nh - 1];
            s_lcnt[hw] = nh - 1;
          }
          s_load[hw] -= d << 9;
          s_load[lw] += d << 9;
        }
      }
      __syncthreads();
    }
    // each worker's records, its items in item order: its place, and the
    // offsets of its steps in its three streams
    cnt = nsteps = na = nb = 0;
    if (tid < R) {
      for (int wd = 0; wd < nwd; ++wd) {
        uint32_t bits = s_wbm[tid][wd];
        while (bits != 0u) {
          const int j = 32 * wd + __ffs(bits) - 1;
          bits &= bits - 1u;
          const int st = s_ist[j];
          int4 rec;
          rec.x = x + kPlanXcds * tid;
          rec.y = cnt;
          if (st >> 30) {
            // the longer list to the shorter stream, as in the deal
            const int sa = st & 0x7FFF, sb = (st >> 15) & 0x7FFF;
            const int orient = max(na + sb, nb + sa) < max(na + sa, nb + sb) ? 1 : 0;
            rec.z = na;
            rec.w = nb | (orient << 30);
            na += orient ? sb : sa;
            nb += orient ? sa : sb;
          } else {
            rec.z = nsteps;
            rec.w = 0;
            nsteps += st & 0x3FFFFFFF;
          }
          *reinterpret_cast<int4*>(P32(a, L.off_itmp) + 4 * (int64_t)(lo + j)) = rec;
          cnt += 1;
        }
      }
    }
  }
  // worker j's items take witems[lo + (items of workers < j), ...)
  if (tid < kWave) {
    int pc = tid < R ? cnt : 0;
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_up(pc, o, kWave);
      if (tid >= o) pc += t;
    }
    if (tid < R) {
      const int w = x + kPlanXcds * tid;
      P32(a, L.off_witem)[2 * w] = lo + pc - cnt;
      P32(a, L.off_witem)[2 * w + 1] = cnt;
      P32(a, L.off_wcnt)[3 * w] = nsteps;
      P32(a, L.off_wcnt)[3 * w + 1] = na;
      P32(a, L.off_wcnt)[3 * w + 2] = nb;
    }
  }
}

// The tiles set in list A's bitmap (and, with B, in either list's) in
// ascending order into the steps at `base`, item word `word`: 64 tiles at a
// time, each lane testing one and a ballot giving its place, so the whole
// wave stores at once.  With B each step carries the group flags (tile |
// group 0 needs it << 30 | group 1 needs it << 29).  An empty result is one
// step with no tile.
__device__ void write_tiles(int2* steps, int64_t cap, int64_t base, const uint32_t* bma,
                            const uint32_t* bmb, int tiles, int lane, int word) {
  int n = 0;
  for (int c0 = 0; c0 < tiles; c0 += kWave) {
    const int t = c0 + lane;
    uint32_t fa = 0, fb = 0;
    if (t < tiles) {
      fa = (bma[t >> 5] >> (t & 31)) & 1u;
      if (bmb != nullptr) fb = (bmb[t >> 5] >> (t & 31)) & 1u;
    }
    const bool on = (fa | fb) != 0u;
    const uint64_t m = __ballot(on);
    if (on) {
      const int64_t at = base + n + __popcll(m & ((1ull << lane) - 1ull));
      const int e = bmb != nullptr ? (t | (int)(fa << 30) | (int)(fb << 29)) : t;
      if (at < cap) steps[at] = make_int2(e, word);
    }
    n += __popcll(m);
  }
  if (n == 0 && lane == 0 && base < cap) steps[base] = make_int2(kBadTile, word);
}

// ---- 3. per item: the worker's item list and the item's steps
__global__ void __launch_bounds__(256) plan_steps_kernel(PlanArgs a) {
  __shared__ uint32_t bms[4][2 * kWords];
  __shared__ int64_t wbase[kPlanXcds * kPlanMaxWorkersPerXcd + 1];
  __shared__ int64_t part[256];
  const PlanLayout& L = a.L;
  const int W = L.workers;  // at most 512: two per thread
  const int tid = threadIdx.x;
  const int32_t* wc = P32(a, L.off_wcnt);
  // every workgroup scans the workers' total stream lengths
  {
    const int64_t v0 = 2 * tid < W
                           ? (int64_t)wc[6 * tid] + wc[6 * tid + 1] + wc[6 * tid + 2]
                           : 0;
    const int64_t v1 = 2 * tid + 1 < W
                           ? (int64_t)wc[6 * tid + 3] + wc[6 * tid + 4] + wc[6 * tid + 5]
                           : 0;
    part[tid] = v0 + v1;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int64_t t = tid >= o ? part[tid - o] : 0;
      __syncthreads();
      part[tid] += t;
      __syncthreads();
    }
    const int64_t ex = part[tid] - v0 - v1;
    if (2 * tid < W) wbase[2 * tid] = ex;
    if (2 * tid + 1 < W) wbase[2 * tid + 1] = ex + v0;
    if (tid == 255) wbase[W] = part[255];
    __syncthreads();
  }
  if (blockIdx.x == 0) {
    for (int w = tid; w < W; w += blockDim.x) {
      int32_t* ws = P32(a, L.off_wstep) + 4 * w;
      const int64_t b = wbase[w];
      ws[0] = (int32_t)min(b, L.step_cap);
      ws[1] = (int32_t)min(b + wc[3 * w], L.step_cap);
      ws[2] = (int32_t)min(b + wc[3 * w] + wc[3 * w + 1], L.step_cap);
      ws[3] = (int32_t)min(wbase[w + 1], L.step_cap);
    }
  }
  const int lane = tid % kWave;
  const int wv = tid / kWave;
  int2* steps = reinterpret_cast<int2*>(a.plan + L.off_steps);
  for (int64_t i0 = (int64_t)blockIdx.x * 4; i0 < L.items; i0 += (int64_t)gridDim.x * 4) {
    const int64_t i = i0 + wv;
    bool use = i < L.items;
    int w = 0, seq = 0, offa = 0, offb = 0, orient = 0;
    if (use) {
      const int32_t* it = P32(a, L.off_itmp) + 4 * i;
      w = it[0];
      seq = it[1];
      offa = it[2];
      offb = it[3] & 0x3FFFFFFF;
      orient = (it[3] >> 30) & 1;
      use = w >= 0 && w < W;  // every item is dealt; kept as a guard
    }
    const int64_t bh = use ? i / L.pairs : 0;
    const int p = use ? (int)(i - bh * L.pairs) : 0;
    const int s = L.mask_heads == 1 ? 0 : (int)(bh % L.H);
    const ItemCost ic = item_cost_sp(a, s, p);
    const int word = (int)((bh << kPlanPairBits) | p);
    if (use && lane == 0) {
      const int32_t* wi = P32(a, L.off_witem) + 2 * w;
      if (seq < wi[1]) P32(a, L.off_witems)[wi[0] + seq] = word | (ic.split << 31);
    }
    int n0, n1;
    lists_to_bitmaps(a, use, s, p, bms[wv], lane, n0, n1);
    if (!use) continue;  // (no barrier below)
    const int64_t b = wbase[w];
    if (ic.split) {
      const int64_t ba = b + wc[3 * w] + offa;                   // group 0's stream
      const int64_t bb = b + wc[3 * w] + wc[3 * w + 1] + offb;   // group 1's stream
      const int wda = (int)((bh << kPlanTileBits) | (2 * p));
      write_tiles(steps, L.step_cap, orient ? bb : ba, bms[wv], nullptr, L.tiles, lane, wda);
      if (2 * p + 1 < L.tiles)
        write_tiles(steps, L.step_cap, orient ? ba : bb, bms[wv] + kWords, nullptr, L.tiles,
                    lane, wda + 1);
      continue;
    }
    write_tiles(steps, L.step_cap, b + offa, bms[wv], bms[wv] + kWords, L.tiles, lane, word);
  }
}

}  // namespace

PlanLayout plan_layout(int32_t B, int32_t H, int32_t N, int32_t tile, int32_t mask_heads,
                       int64_t nnz_bound, int32_t workers) {
  PlanLayout L;
  L.B = B;
  L.H = H;
  L.N = N;
  L.tiles = (int32_t)(((int64_t)N + tile - 1) / tile);
  L.mask_heads = mask_heads;
  L.workers = workers;
  L.pairs = (L.tiles + 1) / 2;
  L.items = (int64_t)B * H * L.pairs;
  // An item's steps number at most n0 + n1 + 2 (an empty list is one
  // step).  A pair-mode item has at most Tk; a split-mode one a + b = union
  // + common < Tk + (n0 + n1) / 5 + 2, under 7 Tk / 5 + 2 for lists of
  // distinct tiles.  Per head, the lists of a mask slice are used once per
  // batch entry and per head that shares the slice.
  const int64_t share = mask_heads > 0 ? (int64_t)H / mask_heads : 0;
  const int64_t by_lists =
      (int64_t)B * share * (nnz_bound + 2 * (int64_t)mask_heads * L.pairs);
  const int64_t tk = L.tiles > 1 ? L.tiles : 1;
  const int64_t by_tiles = L.items * ((7 * tk + 4) / 5 + 2);
  L.step_cap = by_lists < by_tiles ? by_lists : by_tiles;
  auto up16 = [](int64_t v) { return (v + 15) & ~(int64_t)15; };
  int64_t off = up16(kPlanHeaderInts * 4);
  L.off_xw = off;
  off = up16(off + 4 * kPlanXcds);
  L.off_wstep = off;
  off = up16(off + 16 * (int64_t)workers);
  L.off_witem = off;
  off = up16(off + 8 * (int64_t)workers);
  L.off_wcnt = off;
  off = up16(off + 12 * (int64_t)workers);
  L.off_witems = off;
  off = up16(off + 4 * L.items);
  L.off_pinfo = off;
  off = up16(off + 32 * (int64_t)mask_heads * L.pairs);
  L.off_itmp = off;
  off = up16(off + 16 * L.items);
  L.off_steps = off;
  off = up16(off + 8 * L.step_cap);
  L.bytes = off;
  return L;
}

// ---- the allocation-free forward: the plan lives in this file-scope
// device array (one per GPU, held until the process ends) instead of a
// caller's buffer.  Host code never uses the array's name as an address:
// each device's address comes from hipGetSymbolAddress, taken once per
// device with that device current, on the first call there.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

// The XCD feedback table (one per GPU, zero until a planned forward runs):
// (busy ticks, planned load) per worker.
static __device__ __align__(16) int2 xcd_table[kPlanXcds * kPlanMaxWorkersPerXcd];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
char* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

int noalloc_scratch(char** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = static_cast<char*>(p);
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {
std::once_flag g_xfb_once[kMaxDevices];
int32_t* g_xfb_ptr[kMaxDevices];
hipError_t g_xfb_err[kMaxDevices];
}  // namespace

int xcd_feedback(int32_t** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_xfb_once[dev], [dev]() {
    void* p = nullptr;
    g_xfb_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(xcd_table));
    g_xfb_ptr[dev] = static_cast<int32_t*>(p);
  });
  if (g_xfb_err[dev] != hipSuccess) return g_xfb_err[dev];
  *ptr = g_xfb_ptr[dev];
  return hipSuccess;
}

int device_compute_units() {
  int dev = 0, cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  return cu;
}

int launch_fwd_plan(const PlanLayout& L, const int32_t* row_ptr, const int32_t* col_idx,
                    int64_t col_cap, char* plan, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  PlanArgs a;
  a.L = L;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.col_cap = col_cap;
  a.plan = plan;
  int32_t* xfb = nullptr;
  const int fe = xcd_feedback(&xfb);
  if (fe != hipSuccess) return fe;
  a.xfb = xfb;
  const int64_t sp = (int64_t)L.mask_heads * L.pairs;
  hipLaunchKernelGGL(plan_pairs_kernel, dim3((unsigned)((sp + 3) / 4 > 0 ? (sp + 3) / 4 : 1)),
                     dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(plan_assign_kernel, dim3(kPlanXcds), dim3(kAssignThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t blocks = (L.items + 3) / 4;
  const unsigned grid = (unsigned)(blocks < 1 ? 1 : (blocks > 65536 ? 65536 : blocks));
  hipLaunchKernelGGL(plan_steps_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bsattn
