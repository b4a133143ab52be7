// Static-mask calibration kernels (CalibAtt page, "A. Fase di Calibrazione").
//
// Step 1, block energies: for every (batch, head) the attention matrix of
// full softmax attention is cut into tile x tile blocks, and E[i, j] is the
// sum of the softmax probabilities inside block (i, j).  Every query row
// contributes 1 in total, so row i of E sums to the rows of query tile i.
//
//   block_energy_kernel: one workgroup per (batch, head, query tile), one
//   wave per 32 query rows.  Two sweeps over all key tiles:
//     sweep 1  S^T = K_j Q^T on v_mfma_f32_32x32x16_bf16 (the forward's
//              mapping: lane l holds query l % 32 and 64 keys of each tile),
//              online row max and row sum -> L = m + log2(l) per row, in the
//              exp2 domain x = s * scale * log2(e);
//     sweep 2  S^T again, p = 2^(x - L) is the exact softmax probability;
//              each wave sums its p over the tile (its 32 rows x all keys),
//              the waves' sums are added in LDS and one thread writes E.
//   K tiles are staged in LDS (row pitch d + 8 bf16, conflict-free for the
//   operand reads); the next tile's rows are loaded into registers while the
//   current one is multiplied.  Rows past N contribute nothing; keys past N
//   never enter a softmax.  The exponentials are the raw v_exp_f32: results
//   below 2^-126 flush to zero, probabilities far below anything a block sum
//   can register.
//
// Step 1, selection: per query block, the fewest key blocks whose cumulative
// energy reaches eps of the row's total.  Blocks are ordered by decreasing
// energy, the lower index first on ties (a bitonic sort of 64-bit keys
// (~energy bits, index) in LDS: for non-negative floats the bit patterns
// order as the values).  The sums that decide how many are kept are float64
// and taken one at a time in that order by one thread, so the decision is
// reproducible bit for bit.
//
// Step 2, aggregation over prompts: a block is kept when the number of
// prompt masks selecting it is >= rho * P (float64).
#include <hip/hip_runtime.h>

#include <math.h>

#include "bsattn_internal.h"

namespace bsattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// Two workgroups per CU (two waves per SIMD), so one wave's exponentials
// overlap the other's matrix products.
template <int BT, int D, bool F32IN>
__global__ void __launch_bounds__(BT * 2, 2)
block_energy_kernel(EnergyLaunch a) {
  constexpr int NT = BT * 2;           // threads: BT / 32 waves
  constexpr int NW = BT / 32;          // waves
  constexpr int KB = BT / 32;          // 32-key blocks per tile
  constexpr int DC = D / 16;           // 16-wide reduction chunks over d
  constexpr int KP = D + 8;            // K row pitch in LDS (bf16)
  constexpr int PER = BT * D / 8 / NT; // 8-element chunks of a tile per thread
  __shared__ __bf16 Ks[BT * KP];
  __shared__ float wsum[2][NW];  // per-wave tile sums, by tile parity

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int N = a.N;
  const int T = a.tiles;
  const int64_t head_row = ((int64_t)b * a.H + h) * N;
  const int qrow = qt * BT + wave * 32 + l32;
  const bool row_ok = qrow < N;

  bf16x8 qf[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    if (row_ok) {
      qf[c] = load8<F32IN>(a.q, (head_row + qrow) * D + c * 16 + half * 8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[c][e] = (__bf16)0.f;
    }
  }

  // K tile j: rows into registers (prefetch), then into LDS
  bf16x8 kreg[PER];
  auto fetch = [&](int j) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + u * NT;
      const int r = c / (D / 8);
      const int cc = (c % (D / 8)) * 8;
      const int tok = j * BT + r;
      if (j < T && tok < N) {
        kreg[u] = load8<F32IN>(a.k, (head_row + tok) * D + cc);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kreg[u][e] = (__bf16)0.f;
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + u * NT;
      const int r = c / (D / 8);
      const int cc = (c % (D / 8)) * 8;
      *reinterpret_cast<bf16x8*>(&Ks[r * KP + cc]) = kreg[u];
    }
  };
  // S^T of the staged tile; keys past N set to -inf
  f32x16 s[KB];
  auto scores = [&](int j) {
    // chunk-outer over the key blocks: KB independent accumulation chains;
    // the first product of each starts from the constant 0
#pragma unroll
    for (int c = 0; c < DC; ++c)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 ka =
            *reinterpret_cast<const bf16x8*>(&Ks[(kb * 32 + l32) * KP + c * 16 + half * 8]);
        if (c == 0) {
          const f32x16 zero = {};
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[0], zero, 0, 0, 0);
        } else {
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[c], s[kb], 0, 0, 0);
        }
      }
    // an integer select (no per-element compare masks) for the ragged tile
    const int valid = N - j * BT;
    if (valid < BT) {
      const int lim = valid - 4 * half;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
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
  };

  const float c2 = a.scale_log2;
  float m = -INFINITY;  // running max of x = s * scale * log2(e)
  float l = 0.f;        // this lane's share of the running sum

  // ---- sweep 1: row max and row sum over every key tile
  fetch(0);
  for (int j = 0; j < T; ++j) {
    __syncthreads();  // the previous tile's operand reads are done
    stage();
    __syncthreads();
    fetch(j + 1);
    scores(j);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
    const float m_new = fmaxf(m, mx);
    const float alpha = (m_new == m) ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    // the tile's share first, then into the running sum: thousands of
    // terms added one by one into a single float would lose ~1e-4 of it
    float lt = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float lk = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) lk += __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], c2, -m));
      lt += lk;
    }
    l = l * alpha + lt;
  }
  l += __shfl_xor(l, 32);
  const float L = m + log2f(l);  // log2 of the row's normaliser (in x units)

  // ---- sweep 2: probabilities summed per key tile.  The waves' sums of
  // tile j are added (and E written) by thread 0 after the next tile's
  // first barrier, so no barrier of its own is needed.
  float* const erow = a.energy + (((int64_t)b * a.H + h) * T + qt) * T;
  auto write_tile = [&](int j) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += wsum[j & 1][w];
    erow[j] = t;
  };
  fetch(0);
  for (int j = 0; j < T; ++j) {
    __syncthreads();
    if (tid == 0 && j > 0) write_tile(j - 1);
    stage();
    __syncthreads();
    fetch(j + 1);
    scores(j);
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float pk = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) pk += __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], c2, -L));
      ps += pk;
    }
    if (!row_ok) ps = 0.f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off);
    if (lane == 0) wsum[j & 1][wave] = ps;
  }
  __syncthreads();
  if (tid == 0 && T > 0) write_tile(T - 1);
}

template <int BT, int D, bool F32IN>
int launch_t(const EnergyLaunch& a, hipStream_t s) {
  dim3 grid(a.tiles, a.H, a.B);
  hipLaunchKernelGGL((block_energy_kernel<BT, D, F32IN>), grid, dim3(BT * 2), 0, s, a);
  return hipGetLastError();
}

template <int BT, int D>
int launch_dtype(const EnergyLaunch& a, hipStream_t s) {
  return a.dtype == 1 ? launch_t<BT, D, true>(a, s) : launch_t<BT, D, false>(a, s);
}

template <int BT>
int launch_d(const EnergyLaunch& a, hipStream_t s) {
  return a.d == 64 ? launch_dtype<BT, 64>(a, s) : launch_dtype<BT, 128>(a, s);
}

// ---------------------------------------------------------------- selection
constexpr int SEL_THREADS = 256;

__global__ void __launch_bounds__(SEL_THREADS)
select_blocks_kernel(int32_t tk, int32_t pow2, const float* __restrict__ energy, double eps,
                     uint8_t* __restrict__ mask) {
  extern __shared__ uint64_t keys[];  // pow2 entries
  __shared__ int keep_n;
  const int64_t row = blockIdx.x;
  const float* e = energy + row * tk;
  uint8_t* out = mask + row * tk;
  for (int j = threadIdx.x; j < pow2; j += SEL_THREADS) {
    if (j < tk) {
      const uint32_t bits = __float_as_uint(e[j]);
      keys[j] = ((uint64_t)(~bits) << 32) | (uint32_t)j;
    } else {
      keys[j] = ~(uint64_t)0;  // after every real entry
    }
  }
  __syncthreads();
  // bitonic sort, ascending
  for (int k = 2; k <= pow2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = threadIdx.x; i < pow2; i += SEL_THREADS) {
        const int p = i ^ jj;
        if (p > i) {
          const uint64_t x = keys[i], y = keys[p];
          const bool up = (i & k) == 0;
          if ((x > y) == up) {
            keys[i] = y;
            keys[p] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) {
    double total = 0.0;
    for (int r = 0; r < tk; ++r) total += (double)e[(uint32_t)keys[r]];
    const double target = eps * total;
    double cum = 0.0;
    int n = 0;
    while (n < tk && cum < target) {
      cum += (double)e[(uint32_t)keys[n]];
      ++n;
    }
    keep_n = n;
  }
  __syncthreads();
  const int n = keep_n;
  for (int r = threadIdx.x; r < tk; r += SEL_THREADS)
    out[(uint32_t)keys[r]] = r < n ? 1 : 0;
}

__global__ void aggregate_kernel(int32_t P, int64_t cells, const uint8_t* __restrict__ masks,
                                 double rho, uint8_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const double need = rho * (double)P;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < cells; c += stride) {
    int count = 0;
    for (int p = 0; p < P; ++p) count += masks[(int64_t)p * cells + c] != 0;
    out[c] = (double)count >= need ? 1 : 0;
  }
}

}  // namespace

int launch_block_energy(const EnergyLaunch& a, void* stream) {
  if (energy_tuned_fits(a)) return launch_energy_tuned(a, stream);
  hipStream_t s = (hipStream_t)stream;
  return a.tile == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

int launch_select_blocks(int32_t rows, int32_t tk, const float* energy, double eps,
                         uint8_t* mask, void* stream) {
  if (rows == 0 || tk == 0) return hipSuccess;
  int pow2 = 1;
  while (pow2 < tk) pow2 <<= 1;
  hipLaunchKernelGGL(select_blocks_kernel, dim3((unsigned)rows), dim3(SEL_THREADS),
                     (size_t)pow2 * sizeof(uint64_t), (hipStream_t)stream, tk, pow2, energy, eps,
                     mask);
  return hipGetLastError();
}

int launch_aggregate(int32_t P, int64_t cells, const uint8_t* masks, double rho, uint8_t* out,
                     void* stream) {
  if (cells == 0) return hipSuccess;
  const int block = 256;
  int64_t grid = (cells + block - 1) / block;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(aggregate_kernel, dim3((unsigned)grid), dim3(block), 0, (hipStream_t)stream,
                     P, cells, masks, rho, out);
  return hipGetLastError();
}

}  // namespace bsattn
