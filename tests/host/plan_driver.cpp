// Host-only driver of the plan code, built by the CPU test suite with
// AddressSanitizer and UndefinedBehaviorSanitizer: host-only plans (no HIP
// call is made) from 1x1 grids to 8K, ragged grids, both LR modes and radii
// up to 4, every host export, descriptor validation, and the hand-out order
// of the work-queue cursor slots.  Prints "ok" and exits 0 on success.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "ultragen.h"
#include "slot_ring.hpp"

namespace {

int failures = 0;

void expect(bool ok, const char* what, const char* ctx) {
  if (!ok) {
    std::fprintf(stderr, "FAIL %s (%s): %s\n", what, ctx, ug_last_error());
    ++failures;
  }
}

ug_desc desc(int hr_h, int hr_w, int lr_h, int lr_w, int text, int radius, int lr_mode, int heads = 24,
             int head_dim = 128, int batch = 1) {
  ug_desc d;
  std::memset(&d, 0, sizeof(d));
  d.batch = batch;
  d.heads = heads;
  d.head_dim = head_dim;
  d.hr_h = hr_h;
  d.hr_w = hr_w;
  d.lr_h = lr_h;
  d.lr_w = lr_w;
  d.n_text = text;
  d.window = 16;
  d.radius = radius;
  d.rho = 4;
  d.dtype = UG_BF16;
  d.flags = UG_PLAN_HOST_ONLY;
  d.lr_mode = lr_mode;
  d.rope_theta = 10000.0;
  return d;
}

void exercise(const ug_desc& d, const char* ctx) {
  ug_plan_t p = nullptr;
  if (ug_plan(&d, &p) != UG_OK) {
    expect(false, "ug_plan", ctx);
    return;
  }
  ug_info info;
  expect(ug_plan_info(p, &info) == UG_OK, "ug_plan_info", ctx);
  std::vector<int32_t> perm(info.n_hr + 1), win_off(info.n_windows + 1), nbr(info.n_neighbour_entries + 1),
      nbr_off(info.n_windows + 1), lr_perm(info.n_lr + 1), lr_win_off(info.n_windows + 2),
      attn_items(2 * info.attn_blocks + 1), bwd_items(2 * info.bwd_blocks + 1), q_tiles(4 * info.attn_tasks + 1),
      k_ranges(2 * info.attn_ranges + 1), k_tiles(4 * info.bwd_key_tasks + 1), q_ranges(2 * info.bwd_key_ranges + 1),
      mask_off(info.bwd_key_tasks + 1);
  std::vector<uint64_t> masks(info.bwd_mask_words + 1);
  expect(ug_plan_export(p, perm.data(), win_off.data(), nbr.data(), nbr_off.data()) == UG_OK, "export", ctx);
  expect(ug_plan_export_lr(p, lr_perm.data(), lr_win_off.data()) == UG_OK, "export_lr", ctx);
  expect(ug_plan_export_queues(p, attn_items.data(), bwd_items.data()) == UG_OK, "export_queues", ctx);
  expect(ug_plan_export_blocks(p, q_tiles.data(), k_ranges.data(), k_tiles.data(), q_ranges.data(), mask_off.data(),
                               masks.data()) == UG_OK,
         "export_blocks", ctx);
  // every query tile's key count adds up to the pair count
  int64_t pairs = 0;
  for (int64_t t = 0; t < info.attn_tasks; ++t) {
    int64_t keys = 0;
    for (int32_t r = q_tiles[4 * t + 2]; r < q_tiles[4 * t + 3]; ++r) keys += k_ranges[2 * r + 1] - k_ranges[2 * r];
    pairs += keys * (q_tiles[4 * t + 1] - q_tiles[4 * t]);
  }
  expect(pairs == info.pairs_per_head, "pair count of the query tiles", ctx);
  // the permutation is a bijection
  std::vector<char> seen(info.n_hr, 0);
  bool bij = true;
  for (int64_t j = 0; j < info.n_hr; ++j) {
    if (perm[j] < 0 || perm[j] >= info.n_hr || seen[perm[j]]) bij = false;
    else seen[perm[j]] = 1;
  }
  expect(bij, "perm is a bijection", ctx);
  expect(ug_plan_free(p) == UG_OK, "ug_plan_free", ctx);
}

void slot_ring() {
  ug::SlotRing<64> ring;
  for (int round = 0; round < 3; ++round)
    for (int s = 0; s < 64; ++s) {
      const auto t = ring.take();
      expect(t.slot == s, "slot order", "slot ring");
      expect(t.reused == (round > 0), "reuse flag", "slot ring");
    }
  expect(ring.handed_out() == 192, "hand-out count", "slot ring");
}

}  // namespace

int main() {
  exercise(desc(1, 1, 1, 1, 0, 1, 0, 1, 64), "1x1");
  exercise(desc(32, 32, 8, 8, 16, 1, 0, 2, 64), "tiny");
  exercise(desc(48, 48, 12, 12, 16, 1, 1, 2, 64), "tiny corr");
  exercise(desc(37, 45, 11, 13, 9, 1, 1, 2, 64), "overhanging corr");
  {
    ug_desc none = desc(40, 56, 0, 0, 0, 1, 0, 3);
    none.flags |= UG_PLAN_NO_LR;
    exercise(none, "no text, no LR");
  }
  exercise(desc(40, 56, 0, 0, 0, 1, 0, 3), "no text, default LR grid");
  exercise(desc(64, 64, 16, 16, 512, 1, 0), "1K");
  exercise(desc(256, 256, 64, 64, 512, 1, 0), "4K");
  exercise(desc(256, 256, 64, 64, 512, 1, 1), "4K corr");
  exercise(desc(256, 256, 64, 64, 512, 2, 0), "4K radius 2");
  exercise(desc(160, 160, 40, 40, 32, 4, 1), "radius 4 corr");
  exercise(desc(250, 380, 63, 95, 512, 1, 0), "ragged");
  exercise(desc(72, 88, 18, 22, 64, 1, 0, 8, 128, 2), "batch 2");
  exercise(desc(512, 512, 128, 128, 512, 1, 0), "8K");
  // invalid descriptors are rejected without touching anything
  ug_plan_t p = nullptr;
  ug_desc bad = desc(0, 16, 4, 4, 0, 1, 0);
  expect(ug_plan(&bad, &p) == UG_ERR_INVALID_ARGUMENT && p == nullptr, "zero grid rejected", "validation");
  bad = desc(16, 16, 4, 4, 0, 1, 0, 2, 6);
  expect(ug_plan(&bad, &p) == UG_ERR_INVALID_ARGUMENT && p == nullptr, "head_dim 6 rejected", "validation");
  bad = desc(16, 16, 4, 4, 0, 1, 0, 2, 96);
  bad.flags = 0;  // a device plan: refused by validation, before any HIP call
  expect(ug_plan(&bad, &p) == UG_ERR_UNSUPPORTED && p == nullptr, "device head_dim 96 refused", "validation");
  bad = desc(16, 16, 4, 4, 0, 1, 2);
  expect(ug_plan(&bad, &p) == UG_ERR_INVALID_ARGUMENT && p == nullptr, "lr_mode 2 rejected", "validation");
  expect(ug_plan(nullptr, &p) == UG_ERR_INVALID_ARGUMENT, "NULL descriptor rejected", "validation");
  bad = desc(16, 16, 0, 4, 0, 1, 0);
  expect(ug_plan(&bad, &p) == UG_ERR_INVALID_ARGUMENT && p == nullptr, "one zero LR side rejected", "validation");
  bad = desc(16, 16, 4, 4, 0, 1, 0);
  bad.flags |= UG_PLAN_NO_LR;
  expect(ug_plan(&bad, &p) == UG_ERR_INVALID_ARGUMENT && p == nullptr, "NO_LR with an LR grid rejected", "validation");
  {  // 0 x 0 without the flag: ceil(H/rho) x ceil(W/rho)
    ug_desc dflt = desc(37, 45, 0, 0, 8, 1, 0, 2, 64);
    ug_plan_t q = nullptr;
    ug_info info;
    expect(ug_plan(&dflt, &q) == UG_OK && ug_plan_info(q, &info) == UG_OK && info.n_lr == 10 * 12,
           "default LR grid", "resolution");
    ug_plan_free(q);
  }
  slot_ring();
  if (failures) return 1;
  std::printf("ok\n");
  return 0;
}
