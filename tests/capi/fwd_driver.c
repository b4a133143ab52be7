/*
 * A plain C program that uses libbsattn through include/bsattn.h only: no
 * PyTorch, no Python.  It reads a problem from a binary file, copies it to
 * the device with the HIP runtime's C API, runs the three calls of the path
 * (bsattn_build_mask -> bsattn_compact -> bsattn_fwd) on a stream of its
 * own, and writes the mask, the lists, O and the LSE back to a file.
 *
 * Input (little-endian): int32 B, H, N, d, tile, dtype, frames, grid_h,
 * grid_w, window, num_anchors, rotation; then Q, K, V, each B*H*N*d elements
 * of 2 (bf16) or 4 (fp32) bytes.
 * Output: int32 Tq, nnz; uint8 mask[Tq*Tq]; int32 row_ptr[Tq+1];
 * int32 col_idx[nnz]; O (as Q); float LSE[B*H*N].
 * Exit status 0 on success; a message on stderr otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "bsattn.h"

#define HIP_OK(call)                                                        \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));    \
      return 2;                                                             \
    }                                                                       \
  } while (0)

#define BS_OK(call)                                                         \
  do {                                                                      \
    int s_ = (call);                                                        \
    if (s_ != BSATTN_OK) {                                                  \
      fprintf(stderr, "%s: %s (%s)\n", #call, bsattn_status_string(s_),     \
              bsattn_last_error());                                         \
      return 3;                                                             \
    }                                                                       \
  } while (0)

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }
static int write_all(FILE* f, const void* p, size_t n) { return fwrite(p, 1, n, f) == n; }

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s input output\n", argv[0]);
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    perror(argv[1]);
    return 1;
  }
  int32_t hdr[12];
  if (!read_all(in, hdr, sizeof hdr)) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  const int32_t B = hdr[0], H = hdr[1], N = hdr[2], d = hdr[3], tile = hdr[4],
                dtype = hdr[5];
  bsattn_layout layout = {hdr[6], hdr[7], hdr[8], tile};
  bsattn_mask_params mp;
  memset(&mp, 0, sizeof mp);
  mp.kind = BSATTN_MASK_WINDOW_ANCHOR;
  mp.window = hdr[9];
  mp.num_anchors = hdr[10];
  mp.rotation = hdr[11];
  mp.mask_heads = 1;

  const int32_t Tq = bsattn_num_tiles(N, tile);
  const size_t elt = dtype == BSATTN_DTYPE_F32 ? 4 : 2;
  const size_t nel = (size_t)B * H * N * d, bytes = nel * elt;
  void* host[3];
  for (int t = 0; t < 3; ++t) {
    host[t] = malloc(bytes);
    if (!host[t] || !read_all(in, host[t], bytes)) {
      fprintf(stderr, "short input\n");
      return 1;
    }
  }
  fclose(in);

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  void *q, *k, *v, *o;
  float* lse;
  uint8_t* mask;
  int32_t *row_ptr, *col_idx;
  HIP_OK(hipMalloc(&q, bytes));
  HIP_OK(hipMalloc(&k, bytes));
  HIP_OK(hipMalloc(&v, bytes));
  HIP_OK(hipMalloc(&o, bytes));
  HIP_OK(hipMalloc((void**)&lse, (size_t)B * H * N * sizeof(float)));
  HIP_OK(hipMalloc((void**)&mask, (size_t)Tq * Tq));
  HIP_OK(hipMalloc((void**)&row_ptr, (size_t)(Tq + 1) * sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&col_idx, (size_t)Tq * Tq * sizeof(int32_t)));
  HIP_OK(hipMemcpy(q, host[0], bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, host[1], bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, host[2], bytes, hipMemcpyHostToDevice));

  BS_OK(bsattn_build_mask(&layout, &mp, mask, stream));
  BS_OK(bsattn_compact(Tq, Tq, mask, row_ptr, col_idx, stream));
  BS_OK(bsattn_fwd(B, H, N, d, tile, dtype, q, k, v, o, lse, 1, row_ptr, col_idx, 0.0f,
                   stream));
  HIP_OK(hipStreamSynchronize(stream));

  uint8_t* hmask = malloc((size_t)Tq * Tq);
  int32_t* hrp = malloc((size_t)(Tq + 1) * sizeof(int32_t));
  float* hlse = malloc((size_t)B * H * N * sizeof(float));
  if (!hmask || !hrp || !hlse) return 1;
  HIP_OK(hipMemcpy(hmask, mask, (size_t)Tq * Tq, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hrp, row_ptr, (size_t)(Tq + 1) * sizeof(int32_t), hipMemcpyDeviceToHost));
  const int32_t nnz = hrp[Tq];
  int32_t* hci = malloc((size_t)(nnz > 0 ? nnz : 1) * sizeof(int32_t));
  if (!hci) return 1;
  if (nnz > 0)
    HIP_OK(hipMemcpy(hci, col_idx, (size_t)nnz * sizeof(int32_t), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(host[0], o, bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hlse, lse, (size_t)B * H * N * sizeof(float), hipMemcpyDeviceToHost));

  FILE* out = fopen(argv[2], "wb");
  if (!out) {
    perror(argv[2]);
    return 1;
  }
  const int32_t counts[2] = {Tq, nnz};
  if (!write_all(out, counts, sizeof counts) || !write_all(out, hmask, (size_t)Tq * Tq) ||
      !write_all(out, hrp, (size_t)(Tq + 1) * sizeof(int32_t)) ||
      !write_all(out, hci, (size_t)nnz * sizeof(int32_t)) || !write_all(out, host[0], bytes) ||
      !write_all(out, hlse, (size_t)B * H * N * sizeof(float))) {
    fprintf(stderr, "short write\n");
    return 1;
  }
  fclose(out);
  hipFree(q);
  hipFree(k);
  hipFree(v);
  hipFree(o);
  hipFree(lse);
  hipFree(mask);
  hipFree(row_ptr);
  hipFree(col_idx);
  hipStreamDestroy(stream);
  printf("ok: Tq %d nnz %d\n", Tq, nnz);
  return 0;
}
