// Achievable bf16 matrix-core rate on this device: back-to-back
// v_mfma_f32_32x32x16_bf16 with register operands only (no memory traffic),
// four independent accumulator chains per wave so the MFMA latency is hidden.
// The attention forward issues the same instruction, so this is the ceiling
// its roofline fraction is read against, next to the vendor's dense peak.
#include <hip/hip_runtime.h>

#include "bsattn_internal.h"

namespace bsattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int CHAINS = 4;
constexpr int UNROLL = 4;  // MFMAs per chain per loop trip

__global__ void __launch_bounds__(512) mfma_ceiling_kernel(int iters, float* sink) {
  const int tid = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // small values: the sums stay finite for any iteration count
    a[e] = (__bf16)((float)((tid + e) & 7) * (1.0f / 1024.0f));
    b[e] = (__bf16)((float)((tid * 3 + e) & 7) * (1.0f / 1024.0f));
  }
  f32x16 acc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int c = 0; c < CHAINS; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CHAINS; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  // one value per workgroup keeps the chains live
  if (tid == 0) sink[blockIdx.x] = s;
}

}  // namespace

int64_t mfma_ceiling_flops(int blocks, int iters) {
  // 8 waves per workgroup; each MFMA is 32 x 32 x 16 multiply-adds
  return (int64_t)blocks * 8 * iters * UNROLL * CHAINS * (2LL * 32 * 32 * 16);
}

int launch_mfma_ceiling(int blocks, int iters, float* sink, void* stream) {
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3((unsigned)blocks), dim3(512), 0,
                     (hipStream_t)stream, iters, sink);
  return hipGetLastError();
}

}  // namespace bsattn
