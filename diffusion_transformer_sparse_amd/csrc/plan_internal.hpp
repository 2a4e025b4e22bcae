// Internal plan layout shared by the host plan builder (plan.cpp) and the
// kernel launchers (kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/ultragen.h"
#include "slot_ring.hpp"

namespace ug {

// One query tile of the attention: query rows [q0, q1) (at most 256 rows,
// all sharing one key set) and its key ranges ranges[r0 .. r1).  The
// backward's key-major tasks use the same record for a key tile: key rows
// [q0, q1) and the ranges of the queries that see them.
struct Task {
  int32_t q0, q1, r0, r1;
};
// A contiguous run of key rows [k0, k1) in the permuted sequence.
struct Range {
  int32_t k0, k1;
};
// What one workgroup of the attention launch does: query tile `task` of the
// flattened (batch, head) index `bh`; task < 0 marks an idle workgroup.
struct Block {
  int32_t task, bh;
};
// The attention forward's view of one work item (Block): its query rows, its
// key ranges (ranges[r0 .. r0 + nr)), (batch, head), its 64-key tile count
// and its first two tiles (start row, rows; a tile that does not exist has
// 0 rows), so that one record read is enough to start the item's loads.
// nr == 0 marks an idle item (Block::task < 0).
struct AttnItem {
  int32_t q0, q1, r0, nr, bh, ntiles, ks0, nv0, ks1, nv1, pad0, pad1;
};

constexpr int kAttnQueryTile = 256;  // query rows per workgroup (8 waves x 32)
constexpr int kAttnKeyTile = 64;     // key rows per LDS stage
constexpr int kXcds = 8;             // gfx950: workgroups round-robin over 8 XCDs
constexpr int kAttnMaxRanges = 64;   // key ranges one query tile may have (staged in LDS)
// Work-queue cursors of the persistent attention grid: each launch takes one
// slot of kQueueSlotInts int32 (one cursor per XCD queue, then the count of
// workgroups that have finished), round-robin over kQueueSlots slots, so that
// launches with one plan that run at the same time use different cursors; a
// launch that gets a slot back waits for the slot's previous launch (an event
// per slot), so two launches never share cursors.
constexpr int kQueueSlots = 64;
constexpr int kQueueSlotInts = 16;

}  // namespace ug

struct ug_plan_s {
  ug_desc d{};
  int64_t T = 0, N = 0, Nlr = 0, L = 0;
  int32_t gy = 0, gx = 0, nwin = 0;
  bool host_only = true;
  int device = -1;

  // host tables
  std::vector<int32_t> perm, inv, win_off, nbr, nbr_off;
  // LR window-first order (lr_mode 1; the identity otherwise) and window offsets
  std::vector<int32_t> lr_perm, lr_inv, lr_win_off;
  int32_t rope_P = 0;
  std::vector<float> rope_cs;  // [rope_P][D/4][2]: cos, sin of pos * omega_k
  std::vector<ug::Task> tasks;
  std::vector<ug::Range> ranges;
  std::vector<ug::Block> blocks;
  std::vector<ug::AttnItem> items;  // one per blocks[] entry
  int32_t queue_items[ug::kXcds] = {};  // items of each XCD queue before its padding
  int64_t pairs = 0;      // allowed (q, k) pairs per (batch, head)
  int64_t key_tiles = 0;  // 64-key tiles per (batch, head)
  int32_t max_nbr = 0;
  int32_t max_task_ranges = 0;  // most key ranges of any query tile
  // key-major view of the mask (backward dK/dV pass): key tiles with the
  // query ranges that see them, and their workgroup order
  std::vector<ug::Task> ktasks;
  std::vector<ug::Range> kranges;
  std::vector<ug::Block> kblocks;
  int32_t kmax_task_ranges = 0;
  // Key tiles that group several LR windows (lr_mode 1) see the union of
  // their windows' query ranges; bit r of kmasks[kmask_off[t] + j] says
  // whether key row ktasks[t].q0 + j sees the task's query range r.
  // kmask_off[t] < 0: every key of the tile sees every range.
  std::vector<int32_t> kmask_off;
  std::vector<uint64_t> kmasks;

  // Backward statistics (log2-scaled LSE and Delta per row) live in the
  // caller's workspace as two [batch*heads][stat_rows] float arrays; the rows
  // past L are padding (zeros), so a 64-row tile starting at any row < L can
  // be read whole.
  int64_t stat_rows() const { return (L + 64 + 63) / 64 * 64; }
  int64_t bwd_workspace_bytes() const { return 2 * int64_t(d.batch) * d.heads * stat_rows() * int64_t(sizeof(float)); }

  // device copies (owned)
  int32_t* d_perm = nullptr;
  int32_t* d_inv = nullptr;
  int32_t* d_lr_perm = nullptr;  // null unless lr_mode 1
  int32_t* d_lr_inv = nullptr;
  float* d_rope = nullptr;
  ug::Task* d_tasks = nullptr;
  ug::Range* d_ranges = nullptr;
  ug::Block* d_blocks = nullptr;
  ug::AttnItem* d_items = nullptr;
  ug::Task* d_ktasks = nullptr;
  ug::Range* d_kranges = nullptr;
  ug::Block* d_kblocks = nullptr;
  int32_t* d_kmask_off = nullptr;
  uint64_t* d_kmasks = nullptr;  // null when no key tile is masked

  // Persistent attention grid: one workgroup per compute unit, and the
  // zeroed work-queue cursor slots (each launch leaves its slot at zero),
  // handed out by `slots` under `launch_mu`, with the event recorded after
  // each slot's latest launch.
  int32_t cus = 0;
  int32_t* d_queue = nullptr;
  std::mutex launch_mu;
  ug::SlotRing<ug::kQueueSlots> slots;
  hipEvent_t slot_events[ug::kQueueSlots] = {};

  // The backward's second stream: its dK/dV pass runs there, beside the dQ
  // pass on the caller's stream, between a fork and a join event; `bwd_mu`
  // keeps each call's record / wait / launch sequence whole.
  std::mutex bwd_mu;
  hipStream_t bwd_aux = nullptr;
  hipEvent_t bwd_fork = nullptr;
  hipEvent_t bwd_join = nullptr;
};

namespace ug {
// thread-local last-error message helpers (plan.cpp)
ug_status fail(ug_status s, const std::string& msg);
void clear_error();

// Launch of a persistent grid with one of the plan's cursor slots: refuses
// stream capture (a captured launch would take its slot at capture time and
// share it with every replay), takes the next slot, makes the stream wait
// for the slot's previous launch, runs `launch(cursors)` and records the
// slot's event after it.  Returns UG_OK or a failure already reported.
// UG_OK unless `s` is capturing (refused: a captured persistent launch would
// take its cursor slot at capture time and share it with every replay).
inline ug_status refuse_capture(hipStream_t s, const char* fn) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return fail(UG_ERR_HIP, std::string(fn) + ": hipStreamIsCapturing failed");
  }
  if (cs != hipStreamCaptureStatusNone)
    return fail(UG_ERR_UNSUPPORTED, std::string(fn) + ": stream capture is not supported (each launch takes a "
                                                      "work-queue cursor slot at launch time)");
  return UG_OK;
}

template <typename F>
ug_status launch_with_slot(ug_plan_s* p, hipStream_t s, const char* fn, F&& launch) {
  const ug_status cap = refuse_capture(s, fn);
  if (cap != UG_OK) return cap;
  std::lock_guard<std::mutex> lock(p->launch_mu);
  const auto t = p->slots.take();
  if (t.reused && hipStreamWaitEvent(s, p->slot_events[t.slot], 0) != hipSuccess)
    return fail(UG_ERR_HIP, std::string(fn) + ": hipStreamWaitEvent failed: " + hipGetErrorString(hipGetLastError()));
  const ug_status st = launch(p->d_queue + size_t(t.slot) * kQueueSlotInts);
  if (st != UG_OK) return st;
  if (hipEventRecord(p->slot_events[t.slot], s) != hipSuccess)
    return fail(UG_ERR_HIP, std::string(fn) + ": hipEventRecord failed: " + hipGetErrorString(hipGetLastError()));
  return UG_OK;
}
}  // namespace ug
