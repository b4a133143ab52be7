// Host-only check of the C ABI's argument validation under AddressSanitizer
// and UndefinedBehaviorSanitizer: every entry point is called with invalid
// arguments (and with empty problems, which are no-ops) and must return the
// documented status with a message, never reaching a launch.  Device
// pointers are stand-in addresses: no call here may dereference or launch
// on them.  Built and run by tests/test_asan_api.py.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "bsattn.h"

static int g_failures = 0;

static void expect(int got, int want, const char* what, int line) {
  const char* msg = bsattn_last_error();
  if (got != want) {
    printf("FAIL line %d: %s returned %d, expected %d (%s)\n", line, what, got, want, msg);
    ++g_failures;
    return;
  }
  // errors carry a message; successes clear it
  if ((want != BSATTN_OK) != (msg != nullptr && msg[0] != 0)) {
    printf("FAIL line %d: %s: message '%s' for status %d\n", line, what, msg, got);
    ++g_failures;
  }
}
#define EXPECT(call, want) expect((int)(call), (want), #call, __LINE__)

int main() {
  void* p = (void*)64;          // aligned stand-ins, never dereferenced
  void* p2 = (void*)128;
  void* odd = (void*)65;
  const int32_t* ip = (const int32_t*)64;
  const uint8_t* bp = (const uint8_t*)64;
  uint8_t* bo = (uint8_t*)128;
  float* fp = (float*)64;
  const float nanf_ = nanf("");
  const int INV = BSATTN_ERR_INVALID_ARG, UNS = BSATTN_ERR_UNSUPPORTED, OK = BSATTN_OK;

  // strings
  for (int s = -5; s <= 5; ++s)
    if (bsattn_status_string(s) == nullptr || strlen(bsattn_status_string(s)) == 0) {
      printf("FAIL: empty status string for %d\n", s);
      ++g_failures;
    }
  if (bsattn_num_tiles(32760, 128) != 256 || bsattn_num_tiles(10, 0) != -1) {
    printf("FAIL: num_tiles\n");
    ++g_failures;
  }

  // masks and lists
  bsattn_layout lay = {4, 8, 8, 64};
  bsattn_mask_params mp;
  memset(&mp, 0, sizeof mp);
  mp.kind = 0; mp.window = 1; mp.num_anchors = 1; mp.mask_heads = 1;
  EXPECT(bsattn_build_mask(nullptr, &mp, bo, nullptr), INV);
  EXPECT(bsattn_build_mask(&lay, nullptr, bo, nullptr), INV);
  EXPECT(bsattn_build_mask(&lay, &mp, nullptr, nullptr), INV);
  bsattn_layout bad = {0, 8, 8, 64};
  EXPECT(bsattn_build_mask(&bad, &mp, bo, nullptr), INV);
  bsattn_layout huge = {1 << 20, 64, 64, 64};
  EXPECT(bsattn_build_mask(&huge, &mp, bo, nullptr), INV);
  bsattn_mask_params mp2 = mp;
  mp2.kind = -1;
  EXPECT(bsattn_build_mask(&lay, &mp2, bo, nullptr), INV);
  mp2 = mp; mp2.num_anchors = 5;
  EXPECT(bsattn_build_mask(&lay, &mp2, bo, nullptr), INV);
  mp2 = mp; mp2.kind = 1; mp2.thresh24 = (1u << 24) + 1;
  EXPECT(bsattn_build_mask(&lay, &mp2, bo, nullptr), INV);
  mp2 = mp; mp2.kind = 4; mp2.block_tiles = 0;
  EXPECT(bsattn_build_mask(&lay, &mp2, bo, nullptr), INV);
  mp2 = mp; mp2.kind = 6; mp2.block_tiles = 2; mp2.query_tiles = 1 << 20;
  EXPECT(bsattn_build_mask(&lay, &mp2, bo, nullptr), INV);
  EXPECT(bsattn_compact(-1, 4, bp, (int32_t*)p, (int32_t*)p, nullptr), INV);
  EXPECT(bsattn_compact(4, 4, bp, nullptr, (int32_t*)p, nullptr), INV);
  EXPECT(bsattn_compact(1 << 16, 1 << 16, bp, (int32_t*)p, (int32_t*)p, nullptr), INV);

  // forward
  EXPECT(bsattn_fwd(1, 2, 100, 96, 64, 0, p, p, p, p2, nullptr, 1, ip, ip, 0.f, nullptr), UNS);
  EXPECT(bsattn_fwd(1, 2, 100, 64, 32, 0, p, p, p, p2, nullptr, 1, ip, ip, 0.f, nullptr), UNS);
  EXPECT(bsattn_fwd(1, 2, 100, 64, 64, 5, p, p, p, p2, nullptr, 1, ip, ip, 0.f, nullptr), UNS);
  EXPECT(bsattn_fwd(1, 2, -1, 64, 64, 0, p, p, p, p2, nullptr, 1, ip, ip, 0.f, nullptr), INV);
  EXPECT(bsattn_fwd(1, 2, 100, 64, 64, 0, p, p, p, p2, nullptr, 3, ip, ip, 0.f, nullptr), INV);
  EXPECT(bsattn_fwd(1, 2, 100, 64, 64, 0, nullptr, p, p, p2, nullptr, 1, ip, ip, 0.f, nullptr),
         INV);
  EXPECT(bsattn_fwd(1, 2, 100, 64, 64, 0, odd, p, p, p2, nullptr, 1, ip, ip, 0.f, nullptr), INV);
  EXPECT(bsattn_fwd(1, 2, 100, 64, 64, 0, p, p, p, p2, nullptr, 1, ip, ip, nanf_, nullptr), INV);
  EXPECT(bsattn_fwd(1, 70000, 100, 64, 64, 0, p, p, p, p2, nullptr, 1, ip, ip, 0.f, nullptr),
         INV);
  EXPECT(bsattn_fwd(0, 2, 100, 64, 64, 0, nullptr, nullptr, nullptr, nullptr, nullptr, 1, ip, ip,
                    0.f, nullptr),
         OK);
  EXPECT(bsattn_fwd_grouped(1, 2, 32768, 64, 128, 0, p, p, p, p2, nullptr, 1, ip, ip, 256, 0.f,
                            nullptr),
         UNS);
  EXPECT(bsattn_fwd_grouped(1, 2, 32760, 128, 128, 0, p, p, p, p2, nullptr, 1, ip, ip, 256, 0.f,
                            nullptr),
         INV);
  EXPECT(bsattn_fwd_grouped(1, 2, 1000, 128, 128, 0, p, p, p, p2, nullptr, 1, ip, ip, 10, 0.f,
                            nullptr),
         INV);
  EXPECT(bsattn_fwd_noalloc(1, 2, 100, 96, 64, 0, p, p, p, p2, nullptr, 1, ip, ip, 0.f, nullptr),
         UNS);
  EXPECT(bsattn_fwd_noalloc(1, 2, 100, 64, 64, 0, odd, p, p, p2, nullptr, 1, ip, ip, 0.f,
                            nullptr),
         INV);

  // plans
  if (bsattn_fwd_plan_bytes(1, 12, 32760, 128, 1, -1, 256) <= 0) {
    printf("FAIL: plan bytes\n");
    ++g_failures;
  }
  if (bsattn_fwd_plan_bytes(1, 12, 32760, 64, 1, -1, 256) >= 0 ||
      bsattn_fwd_plan_bytes(-1, 12, 32760, 128, 1, -1, 256) >= 0) {
    printf("FAIL: plan bytes accepted bad sizes\n");
    ++g_failures;
  }
  EXPECT(bsattn_fwd_plan(1, 12, 32760, 128, 1, ip, ip, 256, nullptr, 1 << 20, nullptr), INV);
  EXPECT(bsattn_fwd_plan(1, 12, 32760, 128, 1, ip, ip, 256, p, 16, nullptr), INV);
  EXPECT(bsattn_fwd_plan(1, 12, 32760, 128, 5, ip, ip, 256, p, 1 << 20, nullptr), INV);
  EXPECT(bsattn_fwd_planned(1, 12, 32760, 64, 128, 0, p, p, p, p2, nullptr, 1, ip, ip, p,
                            1 << 20, 256, 0, 0.f, nullptr),
         UNS);
  EXPECT(bsattn_fwd_planned(1, 12, 32760, 128, 128, 0, p, p, p, p2, nullptr, 1, ip, ip, nullptr,
                            1 << 20, 256, 0, 0.f, nullptr),
         INV);
  EXPECT(bsattn_window_reorder(1, 1, 100, 64, 0, 0, p, p2, 0, nullptr), INV);
  EXPECT(bsattn_window_reorder(1, 1, 100, 64, 7, 0, p, p2, 0, nullptr), INV);
  EXPECT(bsattn_window_reorder(1, 1, 100, 64, 10, 0, p, p, 0, nullptr), INV);

  // repetition
  EXPECT(bsattn_row_cosines(1, 1, 2, 4, 8, 128, 0, 0, p, p, fp, 0.f, nullptr, 0, nullptr), INV);
  EXPECT(bsattn_row_cosines(1, 1, 2, 4, 300, 128, 2, 0, p, p, fp, 0.f, nullptr, 0, nullptr), UNS);
  EXPECT(bsattn_row_cosines(1, 1, 2, 4, 8, 96, 2, 0, p, p, fp, 0.f, nullptr, 0, nullptr), UNS);
  EXPECT(bsattn_row_cosines(1, 1, 2, 4, 8, 128, 2, 0, p, p, fp, nanf_, nullptr, 0, nullptr), INV);
  const int64_t need = bsattn_row_cosines_workspace_bytes(1, 1, 2, 4, 8, 2);
  EXPECT(bsattn_row_cosines(1, 1, 2, 4, 8, 128, 2, 0, p, p, fp, 0.f, p2, need - 1, nullptr), INV);
  EXPECT(bsattn_row_cosines(0, 1, 2, 4, 8, 128, 2, 0, nullptr, nullptr, nullptr, 0.f, nullptr, 0,
                            nullptr),
         OK);
  EXPECT(bsattn_repetitive_heads(1, 2, 3, 4, 0, fp, 0.9, bo, nullptr), INV);
  EXPECT(bsattn_repetitive_heads(1, 2, 3, 4, 2, fp, INFINITY, bo, nullptr), INV);
  EXPECT(bsattn_anchor_rows(1, 1, 2, 4, 8, 128, 2, 0, p, p, 0, 0, nullptr), INV);
  EXPECT(bsattn_anchor_rows(1, 1, 2, 4, 8, 128, 2, 0, p, p2, 0, -1, nullptr), INV);
  EXPECT(bsattn_anchor_rows(1, 1, 2, 4, 8, 4, 2, 0, p, p2, 0, 0, nullptr), INV);
  EXPECT(bsattn_anchor_rows_heads(1, 1, 2, 4, 8, 128, 2, 0, p, p2, 1, 0, nullptr, nullptr), INV);
  EXPECT(bsattn_mask_select(2, 4, 4, bp, bp, 3, bp, 1, bo, nullptr), INV);
  EXPECT(bsattn_mask_select(2, 4, 4, nullptr, bp, 1, bp, 1, bo, nullptr), INV);
  EXPECT(bsattn_mask_select(0, 4, 4, nullptr, nullptr, 1, nullptr, 1, nullptr, nullptr), OK);

  // calibration
  EXPECT(bsattn_block_energy(1, 1, 256, 128, 128, 0, p, p, nullptr, 0.f, nullptr, 0, nullptr),
         INV);
  EXPECT(bsattn_block_energy(1, 1, 256, 96, 128, 0, p, p, fp, 0.f, nullptr, 0, nullptr), UNS);
  EXPECT(bsattn_block_energy(1, 1, 256, 128, 32, 0, p, p, fp, 0.f, nullptr, 0, nullptr), UNS);
  EXPECT(bsattn_block_energy(70000, 1, 256, 128, 128, 0, p, p, fp, 0.f, nullptr, 0, nullptr), INV);
  const int64_t eneed = bsattn_block_energy_workspace_bytes(1, 1, 256, 128);
  EXPECT(bsattn_block_energy(1, 1, 256, 128, 128, 0, p, p, fp, 0.f, p2, eneed - 1, nullptr), INV);
  EXPECT(bsattn_block_energy(1, 1, 256, 128, 128, 0, p, p, fp, 0.f, odd, eneed, nullptr), INV);
  EXPECT(bsattn_select_blocks(-1, 4, fp, 0.5, bo, nullptr), INV);
  EXPECT(bsattn_select_blocks(4, 4097, fp, 0.5, bo, nullptr), UNS);
  EXPECT(bsattn_select_blocks(4, 4, fp, nan(""), bo, nullptr), INV);
  EXPECT(bsattn_aggregate_masks(0, 4, bp, 0.5, bo, nullptr), INV);
  EXPECT(bsattn_aggregate_masks(2, 4, bp, nan(""), bo, nullptr), INV);
  if (bsattn_mfma_ceiling(0, 10, fp, nullptr) != INV || bsattn_mfma_ceiling(4, 10, nullptr,
                                                                            nullptr) != INV) {
    printf("FAIL: mfma_ceiling accepted bad arguments\n");
    ++g_failures;
  }

  printf("%s: %d failures\n", g_failures ? "FAILED" : "ok", g_failures);
  return g_failures ? 1 : 0;
}
