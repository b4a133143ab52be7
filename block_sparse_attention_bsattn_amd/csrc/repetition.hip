// Spatial repetition (CalibAtt page, "A. Fase di Calibrazione" step 3 and
// "B. Fase di Inferenza"): in a repetitive head the spatial rows of a frame
// attend alike, so attention is computed for the anchor rows only and
// copied to the rows between them.
//
// Tokens are frame-major, n = f*P + y*gw + x (P = gh*gw); the anchor of row
// y is a(y) = s*floor(y/s) for the stride s.
//
// row_cosine_kernel: one wave per 32 columns x of a non-anchor spatial row
// (f, y), as many consecutive non-anchor rows per workgroup as 8 waves
// hold, so each staged K tile serves several rows (anchor rows get 1 from a
// small kernel of their own).  Lane (x, half) holds two queries, q1 = (f, y, x) and its
// anchor q2 = (f, a(y), x), and 64 keys of each 128-key tile, as in the
// forward's S^T = K Q^T mapping; each K operand read from LDS feeds the
// MFMAs of both queries, 64 keys at a time.  One sweep over the keys keeps,
// per query, an online max m and, relative to it, the normaliser
// z = sum_k e (e = 2^(s log2(e) scale - m)) and, per column, the raw sums
// sum_k e1 e2, sum_k e1^2 and sum_k e2^2, all rescaled when a max grows;
// dividing by z1 z2, z1^2 and z2^2 at the end gives sum_k p1 p2,
// sum_k p1^2 and sum_k p2^2 of the probability rows.
// The workgroup adds its columns (shuffles, then LDS) and writes
//   cos(y) = sum_x <p1, p2> / sqrt(sum_x |p1|^2 * sum_x |p2|^2);
// anchor rows get exactly 1.  No N x N matrix is ever stored.
//
// repetitive_heads_kernel: one thread per head adds the non-anchor rows'
// cosines in float64 in (prompt, frame, row) order and compares the mean
// with gamma, the same arithmetic the oracle uses, so equal cosines give the
// same decision.
//
// anchor_rows_kernel: an HBM-bound row copy.  Gather packs the anchor rows'
// tokens (frame by frame, row by row) into Na rows of a buffer; broadcast
// gives every token its anchor row's value from such a buffer.  With
// per-head flags, only the heads whose flag is set are gathered or
// broadcast; the others are copied row for row (CalibAtt's inference runs
// repetitive and other heads in one layer).  The packed
// index a sits at buffer row a, or, spread in blocks of block_rows rows, at
// row floor(g * Pg / Rg) * block_rows + a mod block_rows with g = a /
// block_rows, Rg = ceil(Na / block_rows) and Pg = ceil(N / block_rows).  With
// Rg < Pg no block reaches the last (possibly partial) slot; with Rg == Pg
// the layout is the packed one; so every row written lies below N.
#include <hip/hip_runtime.h>

#include <math.h>

#include "bsattn_internal.h"

namespace bsattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int KT = 128;  // keys staged per step

template <bool F32IN>
__device__ __forceinline__ bf16x8 load8(const void* base, int64_t off) {
  if constexpr (F32IN) {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + off);
    const f32x4 x = p[0], y = p[1];
    bf16x8 r;
    r[0] = (__bf16)x[0]; r[1] = (__bf16)x[1]; r[2] = (__bf16)x[2]; r[3] = (__bf16)x[3];
    r[4] = (__bf16)y[0]; r[5] = (__bf16)y[1]; r[6] = (__bf16)y[2]; r[7] = (__bf16)y[3];
    return r;
  } else {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(base) + off);
  }
}

template <int D, bool F32IN>
__global__ void __launch_bounds__(512)
row_cosine_kernel(RowCosLaunch a) {
  constexpr int DC = D / 16;
  constexpr int KP = D + 8;
  constexpr int KB = KT / 32;
  __shared__ __bf16 Ks[KT * KP];
  __shared__ float red[8][3];

  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  // rows_per_wg consecutive non-anchor rows share each staged K tile; wpr
  // waves per row.  Non-anchor row j of the head: frame j / nna, and the
  // (j % nna)-th row of the frame that is not a multiple of the stride.
  const int wpr = (a.gw + 31) / 32;
  const int rows_per_wg = (nthreads / 64) / wpr;
  const int nna = a.gh - (a.gh + a.stride - 1) / a.stride;  // non-anchor rows per frame
  const int rows_total = a.T * nna;
  const int rsub = wave / wpr;
  auto row_of = [&](int j, int& fr, int& yr) {
    fr = j / nna;
    const int jj = j - fr * nna;
    yr = (jj / (a.stride - 1)) * a.stride + 1 + jj % (a.stride - 1);
  };
  const int jrow = blockIdx.x * rows_per_wg + rsub;
  const int h = blockIdx.y, b = blockIdx.z;
  int f = 0, y = 1;
  if (jrow < rows_total) row_of(jrow, f, y);
  const int ya = a.stride * (y / a.stride);
  // wave-uniform: this wave has a row
  const bool active = jrow < rows_total;
  float* const cos_base = a.cos + ((int64_t)b * a.H + h) * a.T * a.gh;
  const int N = a.N;
  const int P = a.gh * a.gw;
  const int64_t head_row = ((int64_t)b * a.H + h) * N;
  const int x = (wave - rsub * wpr) * 32 + l32;
  const bool col_ok = active && x < a.gw;
  const int n1 = f * P + y * a.gw + x;
  const int n2 = f * P + ya * a.gw + x;

  bf16x8 q1[DC], q2[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    if (col_ok) {
      q1[c] = load8<F32IN>(a.q, (head_row + n1) * D + c * 16 + half * 8);
      q2[c] = load8<F32IN>(a.q, (head_row + n2) * D + c * 16 + half * 8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        q1[c][e] = (__bf16)0.f;
        q2[c][e] = (__bf16)0.f;
      }
    }
  }

  const int tiles = (N + KT - 1) / KT;
  auto stage = [&](int j) {
    __syncthreads();  // the previous tile's operand reads are done
    for (int c = tid; c < KT * D / 8; c += nthreads) {
      const int r = c / (D / 8);
      const int cc = (c % (D / 8)) * 8;
      const int tok = j * KT + r;
      bf16x8 kv;
      if (tok < N) {
        kv = load8<F32IN>(a.k, (head_row + tok) * D + cc);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kv[e] = (__bf16)0.f;
      }
      *reinterpret_cast<bf16x8*>(&Ks[r * KP + cc]) = kv;
    }
    __syncthreads();
  };
  // S^T of key blocks kb0, kb0 + 1 of the staged tile for both queries (one
  // K operand read feeds two MFMAs); keys past N -> -inf
  auto scores2 = [&](f32x16* a1, f32x16* a2, int j, int kb0) {
#pragma unroll
    for (int c = 0; c < DC; ++c)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
            &Ks[((kb0 + u) * 32 + l32) * KP + c * 16 + half * 8]);
        if (c == 0) {
          const f32x16 zero = {};
          a1[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, q1[0], zero, 0, 0, 0);
          a2[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, q2[0], zero, 0, 0, 0);
        } else {
          a1[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, q1[c], a1[u], 0, 0, 0);
          a2[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, q2[c], a2[u], 0, 0, 0);
        }
      }
    const int valid = N - j * KT;
    if (valid < KT) {
      const int lim = valid - 4 * half;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int keep = (((kb0 + u) * 32 + 8 * i + e) - lim) >> 31;  // -1: keep
            const uint32_t sel = (uint32_t)keep;
            a1[u][4 * i + e] = __uint_as_float((__float_as_uint(a1[u][4 * i + e]) & sel) |
                                               (0xff800000u & ~sel));
            a2[u][4 * i + e] = __uint_as_float((__float_as_uint(a2[u][4 * i + e]) & sel) |
                                               (0xff800000u & ~sel));
          }
    }
  };
  const float c2 = a.scale_log2;
  // per lane (one query column, one half of the keys): max m, normaliser z
  // and the raw sums, relative to m; both halves share m
  f32x16 a1[2], a2[2];
  float m1 = -INFINITY, z1 = 0.f, m2 = -INFINITY, z2 = 0.f;
  float s12 = 0.f, s11 = 0.f, s22 = 0.f;
  for (int j = 0; j < tiles; ++j) {
    stage(j);
    if (!active) continue;
#pragma unroll
    for (int kb0 = 0; kb0 < KB; kb0 += 2) {
      scores2(a1, a2, j, kb0);
      float mx1 = -INFINITY, mx2 = -INFINITY;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          mx1 = fmaxf(mx1, a1[u][e]);
          mx2 = fmaxf(mx2, a2[u][e]);
        }
      mx1 = fmaxf(mx1, __shfl_xor(mx1, 32)) * c2;
      mx2 = fmaxf(mx2, __shfl_xor(mx2, 32)) * c2;
      // key 0 is in the first step, so m is finite from then on
      const float n1 = fmaxf(m1, mx1), n2 = fmaxf(m2, mx2);
      const float al1 = (n1 == m1) ? 1.f : __builtin_amdgcn_exp2f(m1 - n1);
      const float al2 = (n2 == m2) ? 1.f : __builtin_amdgcn_exp2f(m2 - n2);
      m1 = n1;
      m2 = n2;
      z1 *= al1;
      z2 *= al2;
      s12 *= al1 * al2;
      s11 *= al1 * al1;
      s22 *= al2 * al2;
      float t1 = 0.f, t2 = 0.f, t12 = 0.f, t11 = 0.f, t22 = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(a1[u][e], c2, -m1));
          const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(a2[u][e], c2, -m2));
          t1 += e1;
          t2 += e2;
          t12 = __builtin_fmaf(e1, e2, t12);
          t11 = __builtin_fmaf(e1, e1, t11);
          t22 = __builtin_fmaf(e2, e2, t22);
        }
      z1 += t1;
      z2 += t2;
      s12 += t12;
      s11 += t11;
      s22 += t22;
    }
  }
  // both halves of a column (same m), then the probability-row sums
  z1 += __shfl_xor(z1, 32);
  z2 += __shfl_xor(z2, 32);
  s12 += __shfl_xor(s12, 32);
  s11 += __shfl_xor(s11, 32);
  s22 += __shfl_xor(s22, 32);
  float d12 = s12 / (z1 * z2), d11 = s11 / (z1 * z1), d22 = s22 / (z2 * z2);
  // then the wave's 32 columns, then the waves
  if (!col_ok) d12 = d11 = d22 = 0.f;
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) {
    d12 += __shfl_xor(d12, off);
    d11 += __shfl_xor(d11, off);
    d22 += __shfl_xor(d22, off);
  }
  if (lane == 0) {
    red[wave][0] = d12;
    red[wave][1] = d11;
    red[wave][2] = d22;
  }
  __syncthreads();
  // one thread per row of this workgroup
  if (tid < rows_per_wg) {
    const int j = blockIdx.x * rows_per_wg + tid;
    if (j < rows_total) {
      int fr, yr;
      row_of(j, fr, yr);
      float t12 = 0.f, t11 = 0.f, t22 = 0.f;
      for (int w = tid * wpr; w < (tid + 1) * wpr; ++w) {
        t12 += red[w][0];
        t11 += red[w][1];
        t22 += red[w][2];
      }
      cos_base[fr * a.gh + yr] = t12 / sqrtf(t11 * t22);
    }
  }
}

// anchor rows: cosine 1 by definition
__global__ void anchor_cos_kernel(int64_t rows, int32_t gh, int32_t stride, float* cos) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int y = (int)(i % gh);
    if (stride * (y / stride) == y) cos[i] = 1.0f;
  }
}

__global__ void repetitive_heads_kernel(int32_t B, int32_t H, int32_t T, int32_t gh,
                                        int32_t stride, const float* __restrict__ cos,
                                        double gamma, uint8_t* __restrict__ flags) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  double total = 0.0;
  int64_t n = 0;
  for (int b = 0; b < B; ++b)
    for (int f = 0; f < T; ++f)
      for (int y = 0; y < gh; ++y) {
        if (stride * (y / stride) == y) continue;
        total += (double)cos[(((int64_t)b * H + h) * T + f) * gh + y];
        ++n;
      }
  flags[h] = (n == 0 || total / (double)n >= gamma) ? 1 : 0;
}

__global__ void __launch_bounds__(256)
anchor_rows_kernel(int64_t BH, int32_t N, int32_t cpr, int32_t gh, int32_t gw, int32_t stride,
                   int32_t na, int broadcast, int32_t block_rows, int32_t rg, int32_t pg,
                   const i32x4* __restrict__ src, i32x4* __restrict__ dst,
                   const uint8_t* __restrict__ flags, int32_t H) {
  // buffer row of packed index p
  auto place = [&](int p) {
    if (block_rows == 0) return p;
    const int g = p / block_rows;
    return (int)(((int64_t)g * pg) / rg) * block_rows + (p - g * block_rows);
  };
  const int P = gh * gw;
  const int T = N / P;
  const int per_frame_a = na * gw;
  const int packed = T * per_frame_a;
  // destination rows per head: with per-head flags every row (a head whose
  // flag is 0 is copied row for row)
  const int rows = (broadcast || flags != nullptr) ? N : packed;
  const int64_t total = BH * rows * cpr;
  const int64_t stride_g = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += stride_g) {
    const int64_t r = idx / cpr;
    const int c = (int)(idx - r * cpr);
    const int64_t bh = r / rows;
    const int dn = (int)(r - bh * rows);
    if (flags != nullptr && flags[bh % H] == 0) {
      dst[(bh * N + dn) * cpr + c] = src[(bh * N + dn) * cpr + c];
      continue;
    }
    if (!broadcast && dn >= packed) continue;  // not an anchor token's row
    int sn;
    if (!broadcast) {  // dst row dn = compact index: (frame, anchor number, x)
      const int f = dn / per_frame_a, rem = dn - f * per_frame_a;
      const int ai = rem / gw, x = rem - ai * gw;
      sn = f * P + ai * stride * gw + x;
    } else {           // dst row dn = token (f, y, x) <- compact (f, y / s, x)
      const int f = dn / P, rem = dn - f * P;
      const int y = rem / gw, x = rem - y * gw;
      sn = f * per_frame_a + (y / stride) * gw + x;
    }
    const int drow = broadcast ? dn : place(dn);
    const int srow = broadcast ? place(sn) : sn;
    dst[(bh * N + drow) * cpr + c] = src[(bh * N + srow) * cpr + c];
  }
}

template <int D, bool F32IN>
int launch_cos(const RowCosLaunch& a, hipStream_t s) {
  const int64_t all_rows = (int64_t)a.B * a.H * a.T * a.gh;
  int64_t cgrid = (all_rows + 255) / 256;
  if (cgrid > 1 << 16) cgrid = 1 << 16;
  hipLaunchKernelGGL(anchor_cos_kernel, dim3((unsigned)cgrid), dim3(256), 0, s, all_rows, a.gh,
                     a.stride, a.cos);
  const int nna = a.gh - (a.gh + a.stride - 1) / a.stride;
  if (nna == 0) return hipGetLastError();
  if (row_cos_tuned_fits(a)) {
    const int e = hipGetLastError();
    return e != hipSuccess ? e : launch_row_cos_tuned(a, s);
  }
  const int wpr = (a.gw + 31) / 32;      // waves per row, <= 8
  const int rows_per_wg = 8 / wpr;       // up to 8 waves per workgroup
  const int rows = a.T * nna;
  dim3 grid((rows + rows_per_wg - 1) / rows_per_wg, a.H, a.B);
  hipLaunchKernelGGL((row_cosine_kernel<D, F32IN>), grid, dim3(64 * wpr * rows_per_wg), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int launch_row_cosines(const RowCosLaunch& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.d == 64) return a.dtype == 1 ? launch_cos<64, true>(a, s) : launch_cos<64, false>(a, s);
  return a.dtype == 1 ? launch_cos<128, true>(a, s) : launch_cos<128, false>(a, s);
}

int launch_repetitive_heads(int32_t B, int32_t H, int32_t T, int32_t gh, int32_t stride,
                            const float* cos, double gamma, uint8_t* flags, void* stream) {
  hipLaunchKernelGGL(repetitive_heads_kernel, dim3((H + 63) / 64), dim3(64), 0,
                     (hipStream_t)stream, B, H, T, gh, stride, cos, gamma, flags);
  return hipGetLastError();
}

int launch_anchor_rows(int64_t BH, int32_t N, int32_t row_bytes, int32_t gh, int32_t gw,
                       int32_t stride, int broadcast, int32_t block_rows, const void* src,
                       void* dst, const uint8_t* flags, int32_t H, void* stream) {
  const int32_t cpr = row_bytes / 16;
  const int32_t na = (gh + stride - 1) / stride;
  const int32_t T = N / (gh * gw);
  const int32_t packed = T * na * gw;
  const int32_t rg = block_rows > 0 ? (packed + block_rows - 1) / block_rows : 1;
  const int32_t pg = block_rows > 0 ? (N + block_rows - 1) / block_rows : 1;
  const int64_t rows = (broadcast || flags != nullptr) ? (int64_t)N : (int64_t)T * na * gw;
  const int64_t total = BH * rows * cpr;
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  if (grid > 1 << 20) grid = 1 << 20;
  hipLaunchKernelGGL(anchor_rows_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                     BH, N, cpr, gh, gw, stride, na, broadcast, block_rows, rg, pg,
                     reinterpret_cast<const i32x4*>(src), reinterpret_cast<i32x4*>(dst), flags,
                     H > 0 ? H : 1);
  return hipGetLastError();
}

}  // namespace bsattn
