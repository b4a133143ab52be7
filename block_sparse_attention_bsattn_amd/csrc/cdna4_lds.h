// CDNA4 (gfx950) building blocks shared by the tuned kernels: vector
// types, LDS address-space views, the workgroup barrier with its waits, the
// XOR swizzle of 256-byte LDS rows, and direct-to-LDS tile fetches
// (buffer_load ... lds).  Device-only; included by .hip sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;
typedef __attribute__((address_space(3))) char lds_char_t;

// Lambdas are forced inline: an outlined lambda would reach its captures
// through memory and turn every buffer resource into a waterfall loop.
#define INLINE __attribute__((always_inline))

// Workgroup barrier that first drains this wave's LDS reads (a buffer a
// barrier releases for refilling must have no read of it still queued) and
// scalar loads.
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt fields at their maximum)
constexpr int WAIT_VM0 = 0x0F70;
// s_waitcnt lgkmcnt(0) (vmcnt and expcnt fields at their maximum)
constexpr int WAIT_LGKM0 = 0xC07F;
// The wait is the builtin, so the compiler knows no scalar load is pending
// after a barrier.
#define BARRIER()                              \
  do {                                         \
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);    \
    asm volatile("s_barrier" ::: "memory");    \
  } while (0)

// Swizzle of 16-byte chunk positions in a 256-byte LDS row: chunk c of row
// R sits at position c ^ swz(R).
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// max over the two lanes (l, l ^ 32) that hold the same query row
__device__ __forceinline__ float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// sum over the two lanes (l, l ^ 32); both lanes get the same value
__device__ __forceinline__ float sum_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Direct-to-LDS tile fetches written as inline asm.  buffer_load_dwordx4
// ... lds moves 16 bytes per lane from global memory to LDS address
// M0 + immediate offset + 16 * lane, with no VGPR staging; the immediate
// offset applies to the global address as well.  The compiler's wait-count
// pass cannot tell LDS slots apart, and would wait for an in-flight fetch
// into one slot before any LDS read of another; it does not see these, and
// the kernel's own s_waitcnt + barrier pairs order them.  They have no
// register results, and their operands are read at issue.  One wait state
// separates the M0 write from the load.
//
// Four loads (1 KB each, at immediate offsets 0, 1024, 2048, 3072, one M0)
// as one statement that the wave skips as a whole when `skip` is nonzero:
// no branch is visible to the compiler, so the statement can be pinned
// between blocks of other work.  voff[i] is load i's per-lane byte offset,
// soff the scalar one.
__device__ __forceinline__ void dma_burst4(const i32x4& rs, uint32_t m0, const uint32_t* voff,
                                           uint32_t soff, uint32_t skip) {
  asm volatile(
      "s_cmp_eq_u32 %0, 0\n\t"
      "s_cbranch_scc0 .Lbsattn_skip_%=\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %5, %6 offen offset:0 lds\n\t"
      "buffer_load_dwordx4 %2, %5, %6 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %3, %5, %6 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %4, %5, %6 offen offset:3072 lds\n"
      ".Lbsattn_skip_%=:"
      :
      : "s"(skip), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(rs), "s"(soff),
        "{m0}"(m0)
      : "memory", "scc");
}
// The same four loads when consecutive rows of a tile lie `row stride`
// bytes apart in memory (the grouped view): load k takes the scalar offset
// soff + k * step, step = 4 * row stride - 1024, so that with the immediate
// 1024 k it reaches rows 4k further on while the LDS address still advances
// by 1024 k from the one M0.
__device__ __forceinline__ void dma_burst4_strided(const i32x4& rs, uint32_t m0,
                                                   const uint32_t* voff, uint32_t soff,
                                                   uint32_t step, uint32_t skip) {
  const uint32_t s1 = soff + step, s2 = soff + 2 * step, s3 = soff + 3 * step;
  asm volatile(
      "s_cmp_eq_u32 %0, 0\n\t"
      "s_cbranch_scc0 .Lbsattn_skips_%=\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %5, %6 offen offset:0 lds\n\t"
      "buffer_load_dwordx4 %2, %5, %7 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %3, %5, %8 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %4, %5, %9 offen offset:3072 lds\n"
      ".Lbsattn_skips_%=:"
      :
      : "s"(skip), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(rs), "s"(soff),
        "s"(s1), "s"(s2), "s"(s3), "{m0}"(m0)
      : "memory", "scc");
}
__device__ __forceinline__ i32x4 raw_rsrc(const void* base, int nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)((uint32_t)(a >> 32) & 0xFFFFu);  // stride 0
  r[2] = nbytes;                                  // range, in bytes
  r[3] = 0x00020000;                              // as the builtin's flags
  return r;
}

__device__ __forceinline__ lds_char_t* uniform_lds(lds_char_t* p) {
  return (lds_char_t*)(uintptr_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}


}  // namespace
}  // namespace bsattn
