// Tile mask -> per-query-tile lists of active key tiles (CSR).
//
// CalibAtt page, "B. Fase di Inferenza": the kernel is driven by precomputed
// per-block lists, so no decision is taken inside the attention kernel.  This
// file turns a [rows, Tk] byte mask into row_ptr / col_idx with three small
// launches and no workspace:
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

}  // namespace

int launch_compact(int32_t rows, int32_t tk, const uint8_t* mask,
                   int32_t* row_ptr, int32_t* col_idx, void* stream) {
  hipStream_t s = (hipStream_t)stream;
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
