// Token reorder between window-major and position-major order (SQuad page,
// "1. Operatore di Attenzione SQuad": the global pass mixes the tokens at the
// same position inside every window).  With G = N / w windows of w tokens,
// the forward reorder moves token a*w + r to r*G + a, so every position
// group becomes a contiguous run of G tokens and the global pass is plain
// block-diagonal attention; the inverse moves the results back.
//
// A pure copy, bound by HBM bandwidth: one 16-byte chunk per thread, the
// destination row decides the source row, so consecutive threads write
// consecutive bytes and each source row is read as one contiguous run.
#include <hip/hip_runtime.h>

#include "bsattn_internal.h"

namespace bsattn {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256)
window_reorder_kernel(int64_t rows_total, int32_t N, int32_t cpr, int32_t w, int32_t G,
                      const i32x4* __restrict__ src, i32x4* __restrict__ dst, int inverse) {
  const int64_t total = rows_total * cpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += stride) {
    const int64_t row = idx / cpr;
    const int c = (int)(idx - row * cpr);
    const int64_t bh = row / N;
    const int n = (int)(row - bh * N);
    int sn;
    if (!inverse) {
      const int r = n / G, a = n - r * G;  // destination r*G + a
      sn = a * w + r;
    } else {
      const int a = n / w, r = n - a * w;  // destination a*w + r
      sn = r * G + a;
    }
    dst[idx] = src[(bh * N + sn) * cpr + c];
  }
}

}  // namespace

int launch_window_reorder(int64_t BH, int32_t N, int32_t row_bytes, int32_t w, const void* src,
                          void* dst, int inverse, void* stream) {
  const int64_t rows = BH * N;
  const int32_t cpr = row_bytes / 16;
  const int64_t total = rows * cpr;
  if (total == 0) return hipSuccess;
  const int block = 256;
  int64_t grid = (total + block - 1) / block;
  if (grid > 1 << 20) grid = 1 << 20;
  hipLaunchKernelGGL(window_reorder_kernel, dim3((unsigned)grid), dim3(block), 0,
                     (hipStream_t)stream, rows, N, cpr, w, N / w,
                     reinterpret_cast<const i32x4*>(src), reinterpret_cast<i32x4*>(dst), inverse);
  return hipGetLastError();
}

}  // namespace bsattn
