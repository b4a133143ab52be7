// Fused block-sparse attention forward for CDNA4 (gfx950).
//
// LVSA page ("Meccanismo Core") and CalibAtt page ("B. Fase di Inferenza"):
// attention is computed only over the key tiles each query tile's active list
// names; skipped tiles are never loaded.  Inside an active tile the math is
// ordinary softmax attention, accumulated over the tiles with the online
// (running max / running sum) softmax of Milakov and Gimelshein (2018).
//
// Work decomposition: one workgroup per (batch, head, query tile) with
// tile/32 waves; each wave owns 32 query rows.
//
// Staging: K/V tiles are double-buffered in LDS.  While the waves compute on
// the tile in one buffer, the next listed tile's rows are already loading
// into registers (issued before the tile's matrix products); after the
// tile's last LDS read they are written into the other buffer, and one
// barrier per tile separates the two uses of each buffer.
//
// Per active key tile j:
//   * K_j is staged in LDS row-major and V_j transposed (V^T, keys
//     contiguous; each thread writes two consecutive keys at once), so both
//     matrix products read MFMA operands as short runs.
//   * S^T = K_j Q^T on v_mfma_f32_32x32x16_bf16: A = K rows (32 keys x 16 d),
//     B = Q^T (16 d x 32 queries).  Lane l then holds query (l % 32) and, per
//     32-key block, keys 8*i + 4*(l/32) + e (i, e in 0..3), so every lane sees
//     one query row and the softmax needs one cross-lane step (l <-> l ^ 32).
//   * Online softmax in the exp2 domain: x = s * scale * log2(e).
//   * O^T += V_j^T P^T on the same MFMA, P taken straight from the score
//     registers (rounded to bf16).  The MFMA's reduction index is permuted to
//     the keys the lane already holds; V^T's operand is read in that order.
//   * Epilogue: O = acc / l, rows >= N are not stored.
#include <hip/hip_runtime.h>

#include <math.h>
#include <type_traits>

#include "bsattn_internal.h"

namespace bsattn {
namespace {

#define INLINE_FN __attribute__((always_inline))

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 8 consecutive elements of a row as loaded from memory: bf16, or fp32
// rounded to bf16 only when written to LDS (so the load stays in flight).
template <bool F32IN> struct Raw8;
template <> struct Raw8<false> { bf16x8 v; };
template <> struct Raw8<true> { f32x4 lo, hi; };

template <bool F32IN>
__device__ __forceinline__ void load_raw(Raw8<F32IN>& r, const void* base, int64_t off) {
  if constexpr (F32IN) {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + off);
    r.lo = p[0];
    r.hi = p[1];
  } else {
    r.v = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(base) + off);
  }
}

template <bool F32IN>
__device__ __forceinline__ void zero_raw(Raw8<F32IN>& r) {
  if constexpr (F32IN) {
#pragma unroll
    for (int e = 0; e < 4; ++e) r.lo[e] = r.hi[e] = 0.f;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) r.v[e] = (__bf16)0.f;
  }
}

template <bool F32IN>
__device__ __forceinline__ bf16x8 to_bf16(const Raw8<F32IN>& r) {
  if constexpr (F32IN) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = (__bf16)r.lo[e];
      o[e + 4] = (__bf16)r.hi[e];
    }
    return o;
  } else {
    return r.v;
  }
}

template <bool F32IN>
__device__ __forceinline__ bf16x8 load8(const void* base, int64_t off) {
  Raw8<F32IN> r;
  load_raw<F32IN>(r, base, off);
  return to_bf16<F32IN>(r);
}

template <bool F32IN>
__device__ __forceinline__ void store4(void* base, int64_t off, float a, float b,
                                       float c, float d) {
  if constexpr (F32IN) {
    f32x4 v = {a, b, c, d};
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + off) = v;
  } else {
    bf16x4 v;
    v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
    *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(base) + off) = v;
  }
}

// Waves per SIMD the register allocation must leave room for: at d = 64 the
// tile is small enough that more resident workgroups hide latency better
// than a deeper prefetch would.
template <int BT, int D>
constexpr int kMinWaves = D == 64 ? (BT == 64 ? 3 : 2) : 1;

template <int BT, int D, bool F32IN>
__global__ void __launch_bounds__(BT * 2)
__attribute__((amdgpu_waves_per_eu(kMinWaves<BT, D>, 8)))
fwd_kernel(FwdLaunch a) {
  constexpr int NT = BT * 2;         // threads: BT/32 waves of 64
  constexpr int KB = BT / 32;        // 32-key blocks per tile
  constexpr int DC = D / 16;         // 16-wide reduction chunks over d
  constexpr int DB = D / 32;         // 32-row blocks of O^T
  constexpr int KP = D + 8;          // K row pitch in LDS (bf16 elements)
  constexpr int VP = BT + 8;         // V^T row pitch in LDS
  constexpr int CPR = D / 8;         // 8-element chunks per row
  // staging items per thread: (pair of consecutive rows, chunk) of K and V
  constexpr int ITEMS = (BT / 2) * CPR / NT;
  static_assert((BT / 2) * CPR == ITEMS * NT, "tile rows must split evenly over the threads");
  __shared__ __bf16 Ks[2][BT * KP];
  __shared__ __bf16 Vt[2][D * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int N = a.N;
  const int64_t head_row = ((int64_t)b * a.H + h) * N;
  const int qrow = qt * BT + wave * 32 + l32;

  bf16x8 qf[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    if (qrow < N) {
      qf[c] = load8<F32IN>(a.q, (head_row + qrow) * D + c * 16 + half * 8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[c][e] = (__bf16)0.f;
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m = -INFINITY;  // running max of x = s * scale * log2(e)
  float l = 0.f;        // this lane's share of the running sum

  const int mrow = (a.mask_heads == 1 ? 0 : h) * a.tiles + qt;
  int jb = a.row_ptr[mrow];
  int64_t je64 = a.row_ptr[mrow + 1];
  if (jb < 0) jb = 0;
  if (je64 > a.col_cap) je64 = a.col_cap;
  const int je = (int)je64;  // row_ptr entries are int32

  // first entry at or after jj naming a key tile in [0, tiles); je if none.
  // Every thread reads the same list entries, so the result is uniform.
  auto next_valid = [&](int jj) INLINE_FN {
    for (; jj < je; ++jj) {
      const int j = a.col_idx[jj];
      if (j >= 0 && j < a.tiles) break;
    }
    return jj;
  };

  // the next tile's rows, held in registers while the current one is computed
  Raw8<F32IN> kr[ITEMS][2], vr[ITEMS][2];
  auto fetch = [&](int j) INLINE_FN {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int c = tid + it * NT;
      const int r = 2 * (c / CPR);
      const int cc = (c % CPR) * 8;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int tok = j * BT + r + e;
        if (tok < N) {
          load_raw<F32IN>(kr[it][e], a.k, (head_row + tok) * D + cc);
          load_raw<F32IN>(vr[it][e], a.v, (head_row + tok) * D + cc);
        } else {
          zero_raw<F32IN>(kr[it][e]);
          zero_raw<F32IN>(vr[it][e]);
        }
      }
    }
  };
  auto stage = [&](int st) INLINE_FN {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int c = tid + it * NT;
      const int r = 2 * (c / CPR);
      const int cc = (c % CPR) * 8;
      *reinterpret_cast<bf16x8*>(&Ks[st][r * KP + cc]) = to_bf16<F32IN>(kr[it][0]);
      *reinterpret_cast<bf16x8*>(&Ks[st][(r + 1) * KP + cc]) = to_bf16<F32IN>(kr[it][1]);
      const bf16x8 v0 = to_bf16<F32IN>(vr[it][0]), v1 = to_bf16<F32IN>(vr[it][1]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x2 pr;
        pr[0] = v0[e];
        pr[1] = v1[e];
        *reinterpret_cast<bf16x2*>(&Vt[st][(cc + e) * VP + r]) = pr;
      }
    }
  };

  int jj = next_valid(jb);
  if (jj < je) {
    fetch(a.col_idx[jj]);
    stage(0);
  }
  __syncthreads();
  int st = 0;
  while (jj < je) {
    const int j = a.col_idx[jj];
    const int jn = next_valid(jj + 1);
    const bool more = jn < je;  // uniform
    if (more) fetch(a.col_idx[jn]);

    // S^T = K_j Q^T
    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
            &Ks[st][(kb * 32 + l32) * KP + c * 16 + half * 8]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[c], s[kb], 0, 0, 0);
      }
    }

    // keys past the end of the sequence never enter the softmax
    const int valid = N - j * BT;
    if (valid < BT) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (kb * 32 + 8 * i + 4 * half + e >= valid) s[kb][4 * i + e] = -INFINITY;
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx * a.scale_log2);
    const float alpha = (m_new == m) ? 1.f : exp2f(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    const float ms = (m == -INFINITY) ? 0.f : m;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2f(s[kb][e] * a.scale_log2 - ms);
        s[kb][e] = p;
        l += p;
      }

    // O^T += V_j^T P^T
#pragma unroll
    for (int kc = 0; kc < BT / 16; ++kc) {
      const int kb = kc >> 1;
      const int i0 = (kc & 1) * 2;
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[kb][i0 * 4 + e];
      const int key0 = kb * 32 + 8 * i0 + 4 * half;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int dd = db * 32 + l32;
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(&Vt[st][dd * VP + key0]);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(&Vt[st][dd * VP + key0 + 8]);
        bf16x8 va;
        va[0] = lo[0]; va[1] = lo[1]; va[2] = lo[2]; va[3] = lo[3];
        va[4] = hi[0]; va[5] = hi[1]; va[6] = hi[2]; va[7] = hi[3];
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[db], 0, 0, 0);
      }
    }

    // buffer st ^ 1 was last read before the previous barrier
    if (more) stage(st ^ 1);
    __syncthreads();
    st ^= 1;
    jj = jn;
  }

  l += __shfl_xor(l, 32);
  if (qrow < N) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * half;
        store4<F32IN>(a.o, (head_row + qrow) * D + d0, oacc[db][4 * i] * inv,
                      oacc[db][4 * i + 1] * inv, oacc[db][4 * i + 2] * inv,
                      oacc[db][4 * i + 3] * inv);
      }
    if (a.lse != nullptr && half == 0)
      a.lse[head_row + qrow] = l > 0.f ? (m + log2f(l)) * 0.69314718055994531f
                                       : -INFINITY;
  }
}

template <int BT, int D, bool F32IN>
int launch_t(const FwdLaunch& a, hipStream_t s) {
  dim3 grid(a.tiles, a.H, a.B);
  hipLaunchKernelGGL((fwd_kernel<BT, D, F32IN>), grid, dim3(BT * 2), 0, s, a);
  return hipGetLastError();
}

template <int BT, int D>
int launch_dtype(const FwdLaunch& a, hipStream_t s) {
  return a.dtype == 1 ? launch_t<BT, D, true>(a, s) : launch_t<BT, D, false>(a, s);
}

template <int BT>
int launch_d(const FwdLaunch& a, hipStream_t s) {
  return a.d == 64 ? launch_dtype<BT, 64>(a, s) : launch_dtype<BT, 128>(a, s);
}

}  // namespace

int launch_fwd(const FwdLaunch& a, void* stream) {
  if (a.tile == 128 && a.d == 128 && a.dtype == 0 &&
      (int64_t)a.N * 256 < ((int64_t)1 << 31))
    return launch_fwd_bf16_t128_d128(a, stream);
  if (fwd_d64_t64_fits(a)) return launch_fwd_d64_t64(a, stream);
  hipStream_t s = (hipStream_t)stream;
  return a.tile == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace bsattn
