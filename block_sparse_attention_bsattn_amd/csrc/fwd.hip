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
// Per active key tile j:
//   * K_j is staged in LDS row-major and V_j transposed (V^T, keys
//     contiguous), so both matrix products read MFMA operands as short runs.
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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool F32IN>
__device__ __forceinline__ bf16x8 load8(const void* base, int64_t off) {
  if constexpr (F32IN) {
    const f32x4* p = reinterpret_cast<const f32x4*>(
        reinterpret_cast<const float*>(base) + off);
    const f32x4 x = p[0], y = p[1];
    bf16x8 r;
    r[0] = (__bf16)x[0]; r[1] = (__bf16)x[1]; r[2] = (__bf16)x[2]; r[3] = (__bf16)x[3];
    r[4] = (__bf16)y[0]; r[5] = (__bf16)y[1]; r[6] = (__bf16)y[2]; r[7] = (__bf16)y[3];
    return r;
  } else {
    return *reinterpret_cast<const bf16x8*>(
        reinterpret_cast<const __bf16*>(base) + off);
  }
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

template <int BT, int D, bool F32IN>
__global__ void __launch_bounds__(BT * 2)
fwd_kernel(FwdLaunch a) {
  constexpr int NT = BT * 2;         // threads: BT/32 waves of 64
  constexpr int KB = BT / 32;        // 32-key blocks per tile
  constexpr int DC = D / 16;         // 16-wide reduction chunks over d
  constexpr int DB = D / 32;         // 32-row blocks of O^T
  constexpr int KP = D + 8;          // K row pitch in LDS (bf16 elements)
  constexpr int VP = BT + 8;         // V^T row pitch in LDS
  __shared__ __bf16 Ks[BT * KP];
  __shared__ __bf16 Vt[D * VP];

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
  int64_t je = a.row_ptr[mrow + 1];
  if (jb < 0) jb = 0;
  if (je > a.col_cap) je = a.col_cap;

  for (int jj = jb; jj < je; ++jj) {
    const int j = a.col_idx[jj];
    if (j < 0 || j >= a.tiles) continue;  // uniform across the workgroup
    __syncthreads();                      // previous tile's LDS reads done
    for (int c = tid; c < BT * D / 8; c += NT) {
      const int r = c / (D / 8);
      const int cc = (c % (D / 8)) * 8;
      const int tok = j * BT + r;
      bf16x8 kv, vv;
      if (tok < N) {
        kv = load8<F32IN>(a.k, (head_row + tok) * D + cc);
        vv = load8<F32IN>(a.v, (head_row + tok) * D + cc);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { kv[e] = (__bf16)0.f; vv[e] = (__bf16)0.f; }
      }
      *reinterpret_cast<bf16x8*>(&Ks[r * KP + cc]) = kv;
#pragma unroll
      for (int e = 0; e < 8; ++e) Vt[(cc + e) * VP + r] = vv[e];
    }
    __syncthreads();

    // S^T = K_j Q^T
    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
            &Ks[(kb * 32 + l32) * KP + c * 16 + half * 8]);
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
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(&Vt[dd * VP + key0]);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(&Vt[dd * VP + key0 + 8]);
        bf16x8 va;
        va[0] = lo[0]; va[1] = lo[1]; va[2] = lo[2]; va[3] = lo[3];
        va[4] = hi[0]; va[5] = hi[1]; va[6] = hi[2]; va[7] = hi[3];
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[db], 0, 0, 0);
      }
    }
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
