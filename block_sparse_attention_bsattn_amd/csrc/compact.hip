// Tile mask -> per-query-tile lists of active key tiles (CSR).
//
// CalibAtt page, "B. Fase di Inferenza": the kernel is driven by precomputed
// per-block lists, so no decision is taken inside the attention kernel.  This
// file turns a [rows, Tk] byte mask into row_ptr / col_idx with no workspace.
// A mask of up to 128 KiB (256 x 256 tiles at 32 760 tokens) takes one
// launch: each workgroup of 16 rows also counts the active cells of every
// row before its own (16 bytes a load, the nonzero bytes of each word
// counted at once), so no workgroup waits for another.  Larger masks take three small
// launches:
//   1. count:  one wave per row; a 64-column chunk at a time, the active
//              columns are counted with a wavefront ballot + popcount and the
//              count is written to row_ptr[r + 1] (row_ptr[0] = 0);
//   2. scan:   one workgroup turns row_ptr[1..rows] into its inclusive prefix
//              sum in place;
//   3. fill:   one wave per row; each active lane's slot is the popcount of
//              the ballot bits below it, so columns land in ascending order.
#include <hip/hip_runtime.h>

#include "bsattn_internal.h"

namespace bsattn {
namespace {

constexpr int kWave = 64;
constexpr int kRowsPerBlock = 4;  // waves per 256-thread workgroup
constexpr int kScanThreads = 1024;

__global__ void __launch_bounds__(256)
count_rows_kernel(const uint8_t* __restrict__ mask, int rows, int tk,
                  int* __restrict__ row_ptr) {
  const int lane = threadIdx.x % kWave;
  const int row = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (blockIdx.x == 0 && threadIdx.x == 0) row_ptr[0] = 0;
  if (row >= rows) return;
  const uint8_t* m = mask + (int64_t)row * tk;
  int count = 0;
  for (int c0 = 0; c0 < tk; c0 += kWave) {
    const int c = c0 + lane;
    const bool on = c < tk && m[c] != 0;
    count += __popcll(__ballot(on));
  }
  if (lane == 0) row_ptr[row + 1] = count;
}

__global__ void __launch_bounds__(kScanThreads)
scan_rows_kernel(int* __restrict__ row_ptr, int rows) {
  __shared__ int part[kScanThreads];
  const int t = threadIdx.x;
  const int per = (rows + kScanThreads - 1) / kScanThreads;
  const int begin = min(t * per, rows);
  const int end = min(begin + per, rows);
  int sum = 0;
  for (int i = begin; i < end; ++i) sum += row_ptr[1 + i];
  part[t] = sum;
  __syncthreads();
  // Hillis-Steele inclusive scan over the per-thread sums.
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int add = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  int run = t > 0 ? part[t - 1] : 0;
  for (int i = begin; i < end; ++i) {
    run += row_ptr[1 + i];
    row_ptr[1 + i] = run;
  }
}

__global__ void __launch_bounds__(256)
fill_rows_kernel(const uint8_t* __restrict__ mask, int rows, int tk,
                 const int* __restrict__ row_ptr, int* __restrict__ col_idx) {
  const int lane = threadIdx.x % kWave;
  const int row = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (row >= rows) return;
  const uint8_t* m = mask + (int64_t)row * tk;
  int base = row_ptr[row];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int c0 = 0; c0 < tk; c0 += kWave) {
    const int c = c0 + lane;
    const bool on = c < tk && m[c] != 0;
    const uint64_t bal = __ballot(on);
    if (on) col_idx[base + __popcll(bal & below)] = c;
    base += __popcll(bal);
  }
}

// nonzero bytes of a 32-bit word: bit 7 of each byte is set when the byte
// is nonzero (its low seven bits plus 0x7F carry into bit 7, or bit 7 was
// set), and no sum carries into the next byte
__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
  return __popc((((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w) & 0x80808080u);
}

constexpr int kOneThreads = 1024;
constexpr int kOneRows = kOneThreads / kWave;  // one wave per row
constexpr int64_t kOneMaxCells = 1 << 17;
constexpr int kHeldChunks = 8;                 // ballots of the first 512 columns kept

__device__ __forceinline__ int nonzero_bytes16(const uint4& x) {
  return nonzero_bytes(x.x) + nonzero_bytes(x.y) + nonzero_bytes(x.z) + nonzero_bytes(x.w);
}

__global__ void __launch_bounds__(kOneThreads)
compact_small_kernel(const uint8_t* __restrict__ mask, int rows, int tk,
                     int* __restrict__ row_ptr, int* __restrict__ col_idx) {
  __shared__ int part[kOneRows];
  __shared__ int rowcnt[kOneRows];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int r0 = blockIdx.x * kOneRows;
  const int row = r0 + wave;
  const uint8_t* m = mask + (int64_t)row * tk;
  // the wave's row: ballots of its first 512 columns, all loads issued at once
  uint64_t bals[kHeldChunks];
  int count = 0;
#pragma unroll
  for (int k = 0; k < kHeldChunks; ++k) {
    const int c = k * kWave + lane;
    bals[k] = __ballot(row < rows && c < tk && m[c] != 0);
    count += __popcll(bals[k]);
  }
  for (int c0 = kHeldChunks * kWave; c0 < tk; c0 += kWave) {
    const int c = c0 + lane;
    count += __popcll(__ballot(row < rows && c < tk && m[c] != 0));
  }
  // active cells of rows [0, r0), counted by the whole workgroup (16 bytes,
  // then single bytes when the mask is not 16-byte aligned and for the tail)
  const int64_t nb = (int64_t)r0 * tk;
  int before = 0;
  int64_t done = 0;
  if ((reinterpret_cast<uintptr_t>(mask) & 15) == 0) {
    const uint4* w16 = reinterpret_cast<const uint4*>(mask);
    const int64_t nv = nb / 16;
#pragma unroll 4
    for (int64_t i = tid; i < nv; i += kOneThreads) before += nonzero_bytes16(w16[i]);
    done = nv * 16;
  }
  for (int64_t i = done + tid; i < nb; i += kOneThreads) before += mask[i] != 0;
  for (int off = kWave / 2; off > 0; off >>= 1) before += __shfl_xor(before, off);
  if (lane == 0) {
    part[wave] = before;
    rowcnt[wave] = count;
  }
  __syncthreads();
  int base = 0;
  for (int w = 0; w < kOneRows; ++w) base += part[w] + (w < wave ? rowcnt[w] : 0);
  if (row >= rows) return;
  // the row's entries, ascending, and its end in row_ptr
  if (blockIdx.x == 0 && tid == 0) row_ptr[0] = 0;
  if (lane == 0) row_ptr[row + 1] = base + count;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
  for (int k = 0; k < kHeldChunks; ++k) {
    if ((bals[k] >> lane) & 1) col_idx[base + __popcll(bals[k] & below)] = k * kWave + lane;
    base += __popcll(bals[k]);
  }
  for (int c0 = kHeldChunks * kWave; c0 < tk; c0 += kWave) {
    const int c = c0 + lane;
    const bool on = c < tk && m[c] != 0;
    const uint64_t bal = __ballot(on);
    if (on) col_idx[base + __popcll(bal & below)] = c;
    base += __popcll(bal);
  }
}

}  // namespace

int launch_compact(int32_t rows, int32_t tk, const uint8_t* mask,
                   int32_t* row_ptr, int32_t* col_idx, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (rows > 0 && (int64_t)rows * tk <= kOneMaxCells) {
    hipLaunchKernelGGL(compact_small_kernel, dim3((rows + kOneRows - 1) / kOneRows),
                       dim3(kOneThreads), 0, s, mask, rows, tk, row_ptr, col_idx);
    return hipGetLastError();
  }
  const int grid = rows > 0 ? (rows + kRowsPerBlock - 1) / kRowsPerBlock : 1;
  hipLaunchKernelGGL(count_rows_kernel, dim3(grid), dim3(256), 0, s, mask, rows,
                     tk, row_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || rows == 0) return e;
  hipLaunchKernelGGL(scan_rows_kernel, dim3(1), dim3(kScanThreads), 0, s,
                     row_ptr, rows);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fill_rows_kernel, dim3(grid), dim3(256), 0, s, mask, rows,
                     tk, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace bsattn
