// Host side of the library: descriptor validation, the plan's tables and
// their upload, info/export, status strings and the thread-local last error.
//
// The tables follow UltraGen's hierarchical local attention ("UltraGen:
// Efficient Ultra-High-Resolution Image Generation with Hierarchical Local
// Attention", papernotes.org notes, 关键设计 1 and 2):
//  - window-first order: HR tokens regrouped window by window, windows and
//    tokens row-major, partial windows at the right/bottom edge of a ragged
//    grid, compact (no padding);
//  - neighbourhood: the windows within Chebyshev distance `radius`;
//  - key ranges: after the window-first permutation every query tile's keys
//    are a union of contiguous row ranges (text, runs of neighbouring
//    windows, LR), so the kernel never evaluates a per-element mask;
//  - RoPE table: cos/sin of pos * theta^(-2k/(D/2)) for every integer
//    position an HR or scaled LR token can take.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <initializer_list>
#include <new>
#include <numeric>
#include <stdexcept>

#include "plan_internal.hpp"

namespace ug {

namespace {
thread_local std::string g_last_error;
}

ug_status fail(ug_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

void clear_error() { g_last_error.clear(); }

namespace {

constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1024;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

ug_status validate(const ug_desc* d) {
  if (!d) return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: desc is NULL");
  if (d->batch < 1 || d->heads < 1) return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: batch and heads must be >= 1");
  if (d->head_dim < 4 || d->head_dim % 4 != 0)
    return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: head_dim must be a positive multiple of 4");
  if (d->hr_h < 1 || d->hr_w < 1) return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: hr_h and hr_w must be >= 1");
  if (d->lr_h < 0 || d->lr_w < 0) return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: lr_h and lr_w must be >= 0");
  if ((d->lr_h == 0) != (d->lr_w == 0))
    return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: lr_h and lr_w must both be 0 (default or none) or both > 0");
  if ((d->flags & UG_PLAN_NO_LR) && d->lr_h != 0)
    return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: UG_PLAN_NO_LR needs lr_h = lr_w = 0");
  if (d->n_text < 0) return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: n_text must be >= 0");
  if (d->window < 1) return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: window must be >= 1");
  if (d->radius < 0) return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: radius must be >= 0");
  if (d->rho < 1) return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: rho must be >= 1");
  if (!(d->rope_theta > 0.0) || !std::isfinite(d->rope_theta))
    return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: rope_theta must be finite and > 0");
  if (d->dtype != UG_F32 && d->dtype != UG_BF16) return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: unknown dtype");
  if (d->flags & ~(UG_PLAN_HOST_ONLY | UG_PLAN_NO_LR)) return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: unknown flags");
  if (d->lr_mode != 0 && d->lr_mode != 1) return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: lr_mode must be 0 or 1");
  const int64_t N = int64_t(d->hr_h) * d->hr_w;
  const int64_t Nlr = int64_t(d->lr_h) * d->lr_w;
  const int64_t L = int64_t(d->n_text) + N + Nlr;
  if (L > kMaxRows) return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: sequence too long (rows must fit int32)");
  // largest RoPE position must fit an int32 table index
  const int64_t maxpos = std::max<int64_t>({int64_t(d->hr_h) - 1, int64_t(d->hr_w) - 1,
                                            int64_t(d->rho) * std::max(d->lr_h - 1, 0),
                                            int64_t(d->rho) * std::max(d->lr_w - 1, 0)});
  if (maxpos > (int64_t(1) << 24)) return fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: positions too large");
  if (!(d->flags & UG_PLAN_HOST_ONLY)) {
    if (d->head_dim != 64 && d->head_dim != 128)
      return fail(UG_ERR_UNSUPPORTED, "ug_plan: GPU kernels support head_dim 64 or 128");
    const int64_t rowbytes = int64_t(d->heads) * d->head_dim * (d->dtype == UG_BF16 ? 2 : 4);
    if (rowbytes % 16 != 0) return fail(UG_ERR_UNSUPPORTED, "ug_plan: heads*head_dim*elem must be a multiple of 16 B");
  }
  return UG_OK;
}

// Window-first order (关键设计 1): slot j of window w = (wy, wx) holds the
// token at row wy*l + j / hx, column wx*l + j % hx inside the window's hy x hx
// extent, windows numbered row-major.
void build_windows(ug_plan_s& p) {
  const int H = p.d.hr_h, W = p.d.hr_w, l = p.d.window;
  p.gy = int32_t(ceil_div(H, l));
  p.gx = int32_t(ceil_div(W, l));
  p.nwin = p.gy * p.gx;
  p.perm.resize(p.N);
  p.inv.resize(p.N);
  p.win_off.resize(p.nwin + 1);
  int64_t j = 0;
  for (int wy = 0; wy < p.gy; ++wy) {
    const int hy = std::min(l, H - wy * l);
    for (int wx = 0; wx < p.gx; ++wx) {
      const int hx = std::min(l, W - wx * l);
      p.win_off[wy * p.gx + wx] = int32_t(j);
      for (int ry = 0; ry < hy; ++ry)
        for (int rx = 0; rx < hx; ++rx) {
          const int64_t raster = int64_t(wy * l + ry) * W + (wx * l + rx);
          p.perm[j] = int32_t(raster);
          p.inv[raster] = int32_t(j);
          ++j;
        }
    }
  }
  p.win_off[p.nwin] = int32_t(j);
  // neighbourhoods: windows within Chebyshev distance `radius`, ascending
  const int R = p.d.radius;
  p.nbr.clear();
  p.nbr_off.assign(p.nwin + 1, 0);
  p.max_nbr = 0;
  for (int wy = 0; wy < p.gy; ++wy)
    for (int wx = 0; wx < p.gx; ++wx) {
      const int w = wy * p.gx + wx;
      p.nbr_off[w] = int32_t(p.nbr.size());
      for (int ay = std::max(0, wy - R); ay <= std::min(p.gy - 1, wy + R); ++ay)
        for (int ax = std::max(0, wx - R); ax <= std::min(p.gx - 1, wx + R); ++ax) p.nbr.push_back(ay * p.gx + ax);
      p.max_nbr = std::max<int32_t>(p.max_nbr, int32_t(p.nbr.size()) - p.nbr_off[w]);
    }
  p.nbr_off[p.nwin] = int32_t(p.nbr.size());
}

// LR anchors by window (关键设计 2, "corresponding" anchors): LR token
// (m, n) sits at (rho*m, rho*n) and belongs to the window containing that
// position.  Window-first order of the LR grid: windows row-major, tokens
// row-major inside; tokens outside the window grid last, in raster order.
// With lr_mode 0 the LR rows keep the raster order (identity).
void build_lr_windows(ug_plan_s& p) {
  const int lh = p.d.lr_h, lw = p.d.lr_w, l = p.d.window, rho = p.d.rho;
  const int64_t nl = p.Nlr;
  std::vector<int64_t> count(size_t(p.nwin) + 1, 0);  // last bucket: outside the grid
  auto win_of = [&](int m, int n) -> int64_t {
    const int64_t a = int64_t(rho) * m / l, b = int64_t(rho) * n / l;
    return (a < p.gy && b < p.gx) ? a * p.gx + b : int64_t(p.nwin);
  };
  for (int m = 0; m < lh; ++m)
    for (int n = 0; n < lw; ++n) ++count[size_t(win_of(m, n))];
  p.lr_win_off.assign(size_t(p.nwin) + 2, 0);
  for (int w = 0; w <= p.nwin; ++w) p.lr_win_off[w + 1] = p.lr_win_off[w] + int32_t(count[w]);
  p.lr_perm.resize(nl);
  p.lr_inv.resize(nl);
  if (p.d.lr_mode == 0) {
    for (int64_t i = 0; i < nl; ++i) p.lr_perm[i] = p.lr_inv[i] = int32_t(i);
    return;
  }
  std::vector<int32_t> fill(p.lr_win_off.begin(), p.lr_win_off.end() - 1);
  for (int m = 0; m < lh; ++m)
    for (int n = 0; n < lw; ++n) {
      const int32_t slot = fill[size_t(win_of(m, n))]++;
      p.lr_perm[slot] = m * lw + n;
      p.lr_inv[m * lw + n] = slot;
    }
}

// RoPE table, double precision rounded to float: cs[pos][k] = (cos, sin) of
// pos * theta^(-2k/(D/2)), k < D/4.
void build_rope(ug_plan_s& p) {
  const int D = p.d.head_dim, K4 = D / 4;
  int64_t maxpos = std::max(p.d.hr_h, p.d.hr_w) - 1;
  if (p.Nlr > 0) maxpos = std::max<int64_t>(maxpos, int64_t(p.d.rho) * (std::max(p.d.lr_h, p.d.lr_w) - 1));
  p.rope_P = int32_t(maxpos + 1);
  p.rope_cs.resize(size_t(p.rope_P) * K4 * 2);
  for (int k = 0; k < K4; ++k) {
    const double omega = std::pow(p.d.rope_theta, -2.0 * k / (D / 2));
    for (int pos = 0; pos < p.rope_P; ++pos) {
      const double a = pos * omega;
      p.rope_cs[(size_t(pos) * K4 + k) * 2 + 0] = float(std::cos(a));
      p.rope_cs[(size_t(pos) * K4 + k) * 2 + 1] = float(std::sin(a));
    }
  }
}

// Sort and merge key ranges that touch or overlap.
void push_merged(std::vector<ug::Range>& out, std::vector<ug::Range> rs) {
  std::sort(rs.begin(), rs.end(), [](const ug::Range& a, const ug::Range& b) { return a.k0 < b.k0; });
  const size_t base = out.size();
  for (const auto& r : rs) {
    if (r.k1 <= r.k0) continue;
    if (out.size() > base && out.back().k1 >= r.k0)
      out.back().k1 = std::max(out.back().k1, r.k1);
    else
      out.push_back(r);
  }
}

int64_t tiles_of(const std::vector<ug::Range>& ranges, const ug::Task& t) {
  int64_t n = 0;
  for (int r = t.r0; r < t.r1; ++r) n += ceil_div(ranges[r].k1 - ranges[r].k0, ug::kAttnKeyTile);
  return n;
}

// Tiles of rows [q0, q1) that share the row ranges `rs`, appended to a task
// list: one task per kAttnQueryTile rows.
void add_tasks(std::vector<ug::Task>& tasks, std::vector<ug::Range>& ranges, int32_t q0, int32_t q1,
               const std::vector<ug::Range>& rs) {
  if (q1 <= q0) return;
  const int32_t r0 = int32_t(ranges.size());
  push_merged(ranges, rs);
  const int32_t r1 = int32_t(ranges.size());
  for (int32_t q = q0; q < q1; q += ug::kAttnQueryTile) tasks.push_back({q, std::min(q1, q + ug::kAttnQueryTile), r0, r1});
}

// Allowed pairs, 64-row tiles and the most ranges of any task of a list.
void count_tasks(const std::vector<ug::Task>& tasks, const std::vector<ug::Range>& ranges, int64_t* pairs,
                 int64_t* tiles, int32_t* max_ranges) {
  *pairs = 0;
  *tiles = 0;
  *max_ranges = 0;
  for (const auto& t : tasks) {
    *max_ranges = std::max(*max_ranges, t.r1 - t.r0);
    int64_t n = 0;
    for (int r = t.r0; r < t.r1; ++r) n += ranges[r].k1 - ranges[r].k0;
    *pairs += int64_t(t.q1 - t.q0) * n;
    *tiles += tiles_of(ranges, t);
  }
}

// Query tiles and their key ranges (the composite mask of 关键设计 2):
//  text rows -> text + HR; LR rows -> text + LR;
//  HR rows of window w -> text + neighbouring windows + LR (all of it, or with
//  lr_mode 1 the LR anchors of the neighbouring windows).
void build_tasks(ug_plan_s& p) {
  const int32_t T = int32_t(p.T), N = int32_t(p.N), L = int32_t(p.L);
  p.tasks.clear();
  p.ranges.clear();
  auto add_rows = [&](int32_t q0, int32_t q1, const std::vector<ug::Range>& rs) {
    add_tasks(p.tasks, p.ranges, q0, q1, rs);
  };
  if (T > 0) add_rows(0, T, {{0, T + N}});
  if (p.Nlr > 0) add_rows(T + N, L, {{0, T}, {T + N, L}});
  for (int w = 0; w < p.nwin; ++w) {
    std::vector<ug::Range> rs;
    if (T > 0) rs.push_back({0, T});
    for (int e = p.nbr_off[w]; e < p.nbr_off[w + 1]; ++e) {
      const int v = p.nbr[e];
      rs.push_back({T + p.win_off[v], T + p.win_off[v + 1]});
    }
    if (p.Nlr > 0 && p.d.lr_mode == 0) rs.push_back({T + N, L});
    if (p.Nlr > 0 && p.d.lr_mode == 1)
      for (int e = p.nbr_off[w]; e < p.nbr_off[w + 1]; ++e) {
        const int v = p.nbr[e];
        rs.push_back({T + N + p.lr_win_off[v], T + N + p.lr_win_off[v + 1]});
      }
    add_rows(T + p.win_off[w], T + p.win_off[w + 1], rs);
  }
  count_tasks(p.tasks, p.ranges, &p.pairs, &p.key_tiles, &p.max_task_ranges);
}

// The same mask seen from the keys, for the dK/dV pass of the backward: key
// tiles (<= 256 rows of one key group) with the ranges of the queries that
// attend to them.  Text keys are seen by every query; keys of HR window v by
// the text queries and the HR queries of the windows around v (the
// neighbourhood relation is symmetric); LR keys by the HR queries (all of
// them, or with lr_mode 1 those of the windows around the anchor's window)
// and by every LR query.  The transposed pair count must equal the forward's.
// Corresponding-LR key tiles (lr_mode 1).  The anchors of LR window u are
// seen by the LR rows and by the HR rows of the windows around u.  One
// window holds only (l/rho)^2 anchors (16 at l = 16, rho = 4), so a key tile
// per window would leave most of a 256-key workgroup idle.  Consecutive
// windows are grouped instead (up to 256 keys, as long as 1 + the number of
// HR windows around any of them stays within kAttnMaxRanges): the tile's
// query ranges are the LR rows (range 0) and each HR window around the
// group (ranges 1..), unmerged, and each key carries the bit mask of the
// ranges it sees.
void add_lr_key_groups(ug_plan_s& p) {
  const int32_t T = int32_t(p.T), N = int32_t(p.N), L = int32_t(p.L);
  auto around = [&](int u) {  // sorted
    std::vector<int32_t> a(p.nbr.begin() + p.nbr_off[u], p.nbr.begin() + p.nbr_off[u + 1]);
    std::sort(a.begin(), a.end());
    return a;
  };
  auto united = [](std::vector<int32_t> a, const std::vector<int32_t>& b) {
    a.insert(a.end(), b.begin(), b.end());
    std::sort(a.begin(), a.end());
    a.erase(std::unique(a.begin(), a.end()), a.end());
    return a;
  };
  for (int w = 0; w < p.nwin;) {
    std::vector<int32_t> hr = around(w);
    int w1 = w + 1;
    int32_t keys = p.lr_win_off[w1] - p.lr_win_off[w];
    while (w1 < p.nwin) {
      const int32_t kw = p.lr_win_off[w1 + 1] - p.lr_win_off[w1];
      std::vector<int32_t> cand = united(hr, around(w1));
      if (keys + kw > kAttnQueryTile || 1 + int32_t(cand.size()) > kAttnMaxRanges) break;
      hr.swap(cand);
      keys += kw;
      ++w1;
    }
    const int32_t q0 = T + N + p.lr_win_off[w], q1 = T + N + p.lr_win_off[w1];
    if (q1 > q0 && 1 + int32_t(hr.size()) <= kAttnMaxRanges) {
      const int32_t r0 = int32_t(p.kranges.size());
      p.kranges.push_back({T + N, L});
      for (int32_t v : hr) p.kranges.push_back({T + p.win_off[v], T + p.win_off[v + 1]});
      const int32_t r1 = int32_t(p.kranges.size());
      const int32_t m0 = int32_t(p.kmasks.size());
      for (int u = w; u < w1; ++u) {
        const std::vector<int32_t> nu = around(u);
        uint64_t bits = 1;  // the LR rows
        for (size_t j = 0; j < hr.size(); ++j)
          if (std::binary_search(nu.begin(), nu.end(), hr[j])) bits |= uint64_t(1) << (j + 1);
        for (int32_t k = p.lr_win_off[u]; k < p.lr_win_off[u + 1]; ++k) p.kmasks.push_back(bits);
      }
      for (int32_t q = q0; q < q1; q += kAttnQueryTile) {
        p.ktasks.push_back({q, std::min(q1, q + kAttnQueryTile), r0, r1});
        p.kmask_off.push_back(m0 + (q - q0));
      }
    } else if (q1 > q0) {  // one window whose neighbourhood alone exceeds the range limit: plain tiles
      std::vector<ug::Range> rs{{T + N, L}};
      for (int32_t v : around(w)) rs.push_back({T + p.win_off[v], T + p.win_off[v + 1]});
      add_tasks(p.ktasks, p.kranges, q0, q1, rs);
      p.kmask_off.resize(p.ktasks.size(), -1);
    }
    w = w1;
  }
}

void build_key_tasks(ug_plan_s& p) {
  const int32_t T = int32_t(p.T), N = int32_t(p.N), L = int32_t(p.L);
  p.ktasks.clear();
  p.kranges.clear();
  p.kmasks.clear();
  auto hr_runs_around = [&](int w, std::vector<ug::Range>& rs) {
    for (int e = p.nbr_off[w]; e < p.nbr_off[w + 1]; ++e) {
      const int v = p.nbr[e];
      rs.push_back({T + p.win_off[v], T + p.win_off[v + 1]});
    }
  };
  add_tasks(p.ktasks, p.kranges, 0, T, {{0, L}});
  for (int w = 0; w < p.nwin; ++w) {
    std::vector<ug::Range> rs;
    if (T > 0) rs.push_back({0, T});
    hr_runs_around(w, rs);
    add_tasks(p.ktasks, p.kranges, T + p.win_off[w], T + p.win_off[w + 1], rs);
  }
  if (p.Nlr > 0 && p.d.lr_mode == 0) add_tasks(p.ktasks, p.kranges, T + N, L, {{T, L}});
  p.kmask_off.assign(p.ktasks.size(), -1);
  if (p.Nlr > 0 && p.d.lr_mode == 1) {
    add_lr_key_groups(p);
    add_tasks(p.ktasks, p.kranges, T + N + p.lr_win_off[p.nwin], L, {{T + N, L}});
    p.kmask_off.resize(p.ktasks.size(), -1);
  }
  // allowed pairs, honouring the key masks
  int64_t pairs = 0;
  p.kmax_task_ranges = 0;
  for (size_t t = 0; t < p.ktasks.size(); ++t) {
    const ug::Task& kt = p.ktasks[t];
    p.kmax_task_ranges = std::max(p.kmax_task_ranges, kt.r1 - kt.r0);
    for (int r = kt.r0; r < kt.r1; ++r) {
      const int64_t len = p.kranges[r].k1 - p.kranges[r].k0;
      if (p.kmask_off[t] < 0) {
        pairs += int64_t(kt.q1 - kt.q0) * len;
        continue;
      }
      for (int32_t j = 0; j < kt.q1 - kt.q0; ++j)
        if ((p.kmasks[p.kmask_off[t] + j] >> (r - kt.r0)) & 1) pairs += len;
    }
  }
  if (pairs != p.pairs) throw std::logic_error("transposed mask pair count differs from the forward's");
}

// Per-XCD work queues.  Each XCD has its own L2, so the order is built per
// XCD: every XCD gets a queue whose long items (query tiles with many more
// key tiles than the average, i.e. text rows) come first, longest first, then
// a contiguous slice of the remaining items in (batch, head, locality) order,
// so that tiles of one head that share neighbour windows and the LR keys run
// on the same L2 (locality: the attention's window tiles in Z-order).  Queues are balanced by key-tile count and interleaved (item
// k * 8 + x is the k-th of XCD x's queue); short queues are padded with idle
// items.  The attention forward's persistent workgroups take items from these
// queues dynamically; the backward launches one workgroup per item, which the
// hardware hands to XCD i % 8 in the same interleaved order.
std::vector<ug::Block> order_blocks(const std::vector<ug::Task>& tasks, const std::vector<ug::Range>& ranges,
                                    int64_t BH, const std::vector<int64_t>& locality, bool group_long) {
  const int X = ug::kXcds;
  std::vector<int64_t> cost(tasks.size());
  double mean = 0;
  for (size_t t = 0; t < tasks.size(); ++t) mean += double(cost[t] = tiles_of(ranges, tasks[t]));
  mean /= double(std::max<size_t>(1, tasks.size()));
  std::vector<int32_t> long_tasks, normal_tasks;
  for (size_t t = 0; t < tasks.size(); ++t)
    (double(cost[t]) > 2.0 * mean ? long_tasks : normal_tasks).push_back(int32_t(t));
  if (!locality.empty())
    std::stable_sort(normal_tasks.begin(), normal_tasks.end(),
                     [&](int32_t a, int32_t b) { return locality[a] < locality[b]; });

  std::vector<std::vector<ug::Block>> q(X);
  std::vector<int64_t> load(X, 0);
  std::vector<int32_t> by_cost = long_tasks;
  std::stable_sort(by_cost.begin(), by_cost.end(), [&](int32_t a, int32_t b) { return cost[a] > cost[b]; });
  if (group_long && BH >= X) {
    // One head's long items together on one XCD, longest first: they start
    // at about the same time and share the rows they all stream (every key
    // of the head) in that XCD's L2.
    int64_t group = 0;
    for (int32_t t : long_tasks) group += cost[t];
    for (int64_t bh = 0; bh < BH; ++bh) {
      const int x = int(std::min_element(load.begin(), load.end()) - load.begin());
      for (int32_t t : by_cost) q[x].push_back({t, int32_t(bh)});
      load[x] += group;
    }
  } else {
    std::vector<ug::Block> longs;
    for (int64_t bh = 0; bh < BH; ++bh)
      for (int32_t t : long_tasks) longs.push_back({t, int32_t(bh)});
    std::stable_sort(longs.begin(), longs.end(),
                     [&](const ug::Block& a, const ug::Block& b) { return cost[a.task] > cost[b.task]; });
    for (const auto& b : longs) {
      const int x = int(std::min_element(load.begin(), load.end()) - load.begin());
      q[x].push_back(b);
      load[x] += cost[b.task];
    }
  }
  int64_t total = std::accumulate(load.begin(), load.end(), int64_t(0));
  for (int64_t bh = 0; bh < BH; ++bh)
    for (int32_t t : normal_tasks) total += cost[t];
  const double target = double(total) / X;
  int x = 0;
  for (int64_t bh = 0; bh < BH; ++bh)
    for (int32_t t : normal_tasks) {
      while (x < X - 1 && double(load[x]) >= target) ++x;
      q[x].push_back({t, int32_t(bh)});
      load[x] += cost[t];
    }
  // The queues end with their shortest items (those under 80% of the median
  // normal item, e.g. the LR query tiles), so the last items the CUs take are
  // short and they run out of work closer together.
  if (!normal_tasks.empty()) {
    std::vector<int64_t> nc;
    for (int32_t t : normal_tasks) nc.push_back(cost[t]);
    std::nth_element(nc.begin(), nc.begin() + nc.size() / 2, nc.end());
    const double short_cost = 0.8 * double(nc[nc.size() / 2]);
    for (auto& qq : q) {
      const size_t first_normal = std::min(qq.size(), size_t(std::count_if(
          qq.begin(), qq.end(), [&](const ug::Block& b) { return double(cost[b.task]) > 2.0 * mean; })));
      std::stable_partition(qq.begin() + first_normal, qq.end(),
                            [&](const ug::Block& b) { return double(cost[b.task]) >= short_cost; });
    }
  }
  size_t len = 0;
  for (const auto& qq : q) len = std::max(len, qq.size());
  std::vector<ug::Block> blocks(len * X, ug::Block{-1, 0});
  for (int xx = 0; xx < X; ++xx)
    for (size_t k = 0; k < q[xx].size(); ++k) blocks[k * X + xx] = q[xx][k];
  return blocks;
}

// The forward's item records: each queue item's task fields, tile count
// and first two 64-key tiles, walked as the kernel walks the key ranges
// (range after range, a range's last tile holding its remaining rows).
std::vector<ug::AttnItem> attn_items(const std::vector<ug::Block>& blocks, const std::vector<ug::Task>& tasks,
                                     const std::vector<ug::Range>& ranges) {
  std::vector<ug::AttnItem> items(blocks.size(), ug::AttnItem{0, 0, 0, 0, -1, 0, 0, 0, 0, 0, 0, 0});
  for (size_t k = 0; k < blocks.size(); ++k) {
    if (blocks[k].task < 0) continue;
    const ug::Task& t = tasks[blocks[k].task];
    ug::AttnItem& it = items[k];
    it.q0 = t.q0;
    it.q1 = t.q1;
    it.r0 = t.r0;
    it.nr = t.r1 - t.r0;
    it.bh = blocks[k].bh;
    it.ntiles = int32_t(tiles_of(ranges, t));
    int32_t got = 0;
    for (int r = t.r0; r < t.r1 && got < 2; ++r)
      for (int32_t ks = ranges[r].k0; ks < ranges[r].k1 && got < 2; ks += ug::kAttnKeyTile, ++got) {
        const int32_t nv = std::min(ug::kAttnKeyTile, ranges[r].k1 - ks);
        (got == 0 ? it.ks0 : it.ks1) = ks;
        (got == 0 ? it.nv0 : it.nv1) = nv;
      }
    if (got < 2) it.ks1 = it.ks0;  // one tile only: the second load reads no rows
    if (it.nr < 1 || it.ntiles < 1 || it.nv0 < 1) throw std::logic_error("attention item without key tiles");
  }
  return items;
}

// Morton (Z-order) code of a window's (row, column): consecutive codes stay
// in compact 2D blocks, so the query tiles that run at the same time on one
// XCD share more of their neighbour windows' K/V tiles in its L2.
int64_t morton(int32_t y, int32_t x) {
  int64_t m = 0;
  for (int b = 0; b < 16; ++b)
    m |= (int64_t((y >> b) & 1) << (2 * b + 1)) | (int64_t((x >> b) & 1) << (2 * b));
  return m;
}

void build_blocks(ug_plan_s& p) {
  const int64_t BH = int64_t(p.d.batch) * p.d.heads;
  // Query tiles of HR windows in Z-order over the window grid (tiles of one
  // window in row order), then the LR tiles, text tiles first.
  std::vector<int64_t> locality(p.tasks.size());
  for (size_t t = 0; t < p.tasks.size(); ++t) {
    const int64_t q0 = p.tasks[t].q0;
    if (q0 < p.T) {
      locality[t] = -1;
    } else if (q0 < p.T + p.N) {
      const int32_t j = int32_t(q0 - p.T);
      const int32_t w = int32_t(std::upper_bound(p.win_off.begin(), p.win_off.end(), j) - p.win_off.begin()) - 1;
      locality[t] = morton(w / p.gx, w % p.gx) * (int64_t(1) << 20) + (j - p.win_off[w]);
    } else {
      locality[t] = (int64_t(1) << 62) + q0;
    }
  }
  p.blocks = order_blocks(p.tasks, p.ranges, BH, locality, true);
  p.items = attn_items(p.blocks, p.tasks, p.ranges);
  // Each XCD queue's items come first and its padding after them.
  const size_t len = p.blocks.size() / ug::kXcds;
  for (int x = 0; x < ug::kXcds; ++x) {
    int32_t n = 0;
    while (size_t(n) < len && p.blocks[size_t(n) * ug::kXcds + x].task >= 0) ++n;
    for (size_t k = size_t(n); k < len; ++k)
      if (p.blocks[k * ug::kXcds + x].task >= 0) throw std::logic_error("work-queue item after padding");
    p.queue_items[x] = n;
  }
  // The dK/dV pass's long items (key tiles every query sees) stay spread
  // over the XCDs: grouped, 18 of them stream the same rows at once and the
  // pass ran 2.5-3% slower although it fetched less than half as much.
  p.kblocks = order_blocks(p.ktasks, p.kranges, BH, {}, false);
}

template <typename T>
ug_status upload(const std::vector<T>& h, T** d) {
  *d = nullptr;
  if (h.empty()) return UG_OK;
  const size_t bytes = h.size() * sizeof(T);
  if (hipMalloc(reinterpret_cast<void**>(d), bytes) != hipSuccess) {
    *d = nullptr;
    (void)hipGetLastError();
    return fail(UG_ERR_OUT_OF_MEMORY, "ug_plan: hipMalloc of a plan table failed");
  }
  if (hipMemcpy(*d, h.data(), bytes, hipMemcpyHostToDevice) != hipSuccess)
    return fail(UG_ERR_HIP, std::string("ug_plan: hipMemcpy failed: ") + hipGetErrorString(hipGetLastError()));
  return UG_OK;
}

void free_device(ug_plan_s* p) {
  void* ptrs[] = {p->d_perm,    p->d_inv,     p->d_lr_perm, p->d_lr_inv,     p->d_rope,
                  p->d_tasks,   p->d_ranges,  p->d_blocks,  p->d_items,      p->d_ktasks,     p->d_kranges,
                  p->d_kblocks, p->d_kmasks, p->d_kmask_off, p->d_queue};
  for (void* q : ptrs)
    if (q) (void)hipFree(q);
  for (hipEvent_t& e : p->slot_events) {
    if (e) (void)hipEventDestroy(e);
    e = nullptr;
  }
  for (hipEvent_t* e : {&p->bwd_fork, &p->bwd_join}) {
    if (*e) (void)hipEventDestroy(*e);
    *e = nullptr;
  }
  if (p->bwd_aux) (void)hipStreamDestroy(p->bwd_aux);
  p->bwd_aux = nullptr;
  p->d_perm = p->d_inv = nullptr;
  p->d_lr_perm = p->d_lr_inv = nullptr;
  p->d_rope = nullptr;
  p->d_tasks = nullptr;
  p->d_ranges = nullptr;
  p->d_blocks = nullptr;
  p->d_items = nullptr;
  p->d_ktasks = nullptr;
  p->d_kranges = nullptr;
  p->d_kblocks = nullptr;
  p->d_kmasks = nullptr;
  p->d_kmask_off = nullptr;
  p->d_queue = nullptr;
}

ug_status check_device(ug_plan_s* p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(UG_ERR_HIP, "ug_plan: no HIP device is available");
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(UG_ERR_HIP, "ug_plan: hipGetDeviceProperties failed");
  }
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(UG_ERR_UNSUPPORTED, std::string("ug_plan: kernels are built for gfx950, device is ") + prop.gcnArchName);
  p->device = dev;
  p->cus = prop.multiProcessorCount;
  if (p->cus <= 0) return fail(UG_ERR_HIP, "ug_plan: the device reports no compute units");
  return UG_OK;
}

// Zeroed work-queue cursor slots of the persistent attention grid.
ug_status alloc_queue(ug_plan_s* p) {
  const size_t bytes = size_t(kQueueSlots) * kQueueSlotInts * sizeof(int32_t);
  if (hipMalloc(reinterpret_cast<void**>(&p->d_queue), bytes) != hipSuccess) {
    p->d_queue = nullptr;
    (void)hipGetLastError();
    return fail(UG_ERR_OUT_OF_MEMORY, "ug_plan: hipMalloc of the work-queue cursors failed");
  }
  if (hipMemset(p->d_queue, 0, bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
    return fail(UG_ERR_HIP, std::string("ug_plan: clearing the work-queue cursors failed: ") +
                                hipGetErrorString(hipGetLastError()));
  for (hipEvent_t& e : p->slot_events)
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
      e = nullptr;
      return fail(UG_ERR_HIP, std::string("ug_plan: hipEventCreateWithFlags failed: ") +
                                  hipGetErrorString(hipGetLastError()));
    }
  // the backward's second stream (default priority) and its fork / join events
  if (hipStreamCreateWithFlags(&p->bwd_aux, hipStreamNonBlocking) != hipSuccess) {
    p->bwd_aux = nullptr;
    return fail(UG_ERR_HIP, std::string("ug_plan: hipStreamCreateWithFlags failed: ") +
                                hipGetErrorString(hipGetLastError()));
  }
  for (hipEvent_t* e : {&p->bwd_fork, &p->bwd_join})
    if (hipEventCreateWithFlags(e, hipEventDisableTiming) != hipSuccess) {
      *e = nullptr;
      return fail(UG_ERR_HIP, std::string("ug_plan: hipEventCreateWithFlags failed: ") +
                                  hipGetErrorString(hipGetLastError()));
    }
  return UG_OK;
}

}  // namespace
}  // namespace ug

extern "C" {

ug_status ug_plan(const ug_desc* user_desc, ug_plan_t* out) {
  ug::clear_error();
  if (!out) return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: out is NULL");
  *out = nullptr;
  if (!user_desc) return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_plan: desc is NULL");
  // 0 x 0 LR grid: the one the coordinate scaling implies, unless NO_LR
  ug_desc resolved = *user_desc;
  if (resolved.lr_h == 0 && resolved.lr_w == 0 && !(resolved.flags & UG_PLAN_NO_LR) && resolved.rho >= 1) {
    resolved.lr_h = int32_t((int64_t(resolved.hr_h) + resolved.rho - 1) / resolved.rho);
    resolved.lr_w = int32_t((int64_t(resolved.hr_w) + resolved.rho - 1) / resolved.rho);
  }
  const ug_desc* desc = &resolved;
  ug_status s = ug::validate(desc);
  if (s != UG_OK) return s;
  ug_plan_s* p = new (std::nothrow) ug_plan_s;
  if (!p) return ug::fail(UG_ERR_OUT_OF_MEMORY, "ug_plan: host allocation failed");
  try {
    p->d = *desc;
    p->host_only = (desc->flags & UG_PLAN_HOST_ONLY) != 0;
    p->T = desc->n_text;
    p->N = int64_t(desc->hr_h) * desc->hr_w;
    p->Nlr = int64_t(desc->lr_h) * desc->lr_w;
    p->L = p->T + p->N + p->Nlr;
    ug::build_windows(*p);
    ug::build_lr_windows(*p);
    ug::build_rope(*p);
    ug::build_tasks(*p);
    ug::build_key_tasks(*p);
    ug::build_blocks(*p);
  } catch (const std::bad_alloc&) {
    delete p;
    return ug::fail(UG_ERR_OUT_OF_MEMORY, "ug_plan: host allocation failed");
  } catch (const std::logic_error& e) {
    delete p;
    return ug::fail(UG_ERR_INTERNAL, std::string("ug_plan: ") + e.what());
  } catch (...) {
    delete p;
    return ug::fail(UG_ERR_INTERNAL, "ug_plan: unexpected exception");
  }
  if (!p->host_only) {
    s = ug::check_device(p);
    if (s == UG_OK) s = ug::upload(p->perm, &p->d_perm);
    if (s == UG_OK) s = ug::upload(p->inv, &p->d_inv);
    if (s == UG_OK && p->d.lr_mode == 1) s = ug::upload(p->lr_perm, &p->d_lr_perm);
    if (s == UG_OK && p->d.lr_mode == 1) s = ug::upload(p->lr_inv, &p->d_lr_inv);
    if (s == UG_OK) s = ug::upload(p->rope_cs, &p->d_rope);
    if (s == UG_OK) s = ug::upload(p->tasks, &p->d_tasks);
    if (s == UG_OK) s = ug::upload(p->ranges, &p->d_ranges);
    if (s == UG_OK) s = ug::upload(p->blocks, &p->d_blocks);
    if (s == UG_OK) s = ug::upload(p->items, &p->d_items);
    if (s == UG_OK) s = ug::upload(p->ktasks, &p->d_ktasks);
    if (s == UG_OK) s = ug::upload(p->kranges, &p->d_kranges);
    if (s == UG_OK) s = ug::upload(p->kblocks, &p->d_kblocks);
    if (s == UG_OK) s = ug::upload(p->kmask_off, &p->d_kmask_off);
    if (s == UG_OK) s = ug::upload(p->kmasks, &p->d_kmasks);
    if (s == UG_OK) s = ug::alloc_queue(p);
    if (s != UG_OK) {
      ug::free_device(p);
      delete p;
      return s;
    }
  }
  *out = p;
  return UG_OK;
}

ug_status ug_plan_free(ug_plan_t p) {
  ug::clear_error();
  if (!p) return UG_OK;
  if (!p->host_only) ug::free_device(p);
  delete p;
  return UG_OK;
}

ug_status ug_plan_info(ug_plan_t p, ug_info* out) {
  ug::clear_error();
  if (!p || !out) return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_plan_info: NULL argument");
  std::memset(out, 0, sizeof(*out));
  out->seq_len = p->L;
  out->n_hr = p->N;
  out->n_lr = p->Nlr;
  out->n_text = p->T;
  out->grid_y = p->gy;
  out->grid_x = p->gx;
  out->n_windows = p->nwin;
  out->max_neighbours = p->max_nbr;
  out->n_neighbour_entries = int64_t(p->nbr.size());
  out->pairs_per_head = p->pairs;
  out->eff_flops = 4.0 * p->d.head_dim * double(p->pairs) * p->d.heads * p->d.batch;
  out->workspace_bytes = 0;
  out->attn_tasks = int64_t(p->tasks.size());
  out->attn_blocks = int64_t(p->blocks.size());
  out->attn_key_tiles = p->key_tiles;
  out->rope_positions = p->rope_P;
  out->bwd_workspace_bytes = p->bwd_workspace_bytes();
  out->bwd_key_tasks = int64_t(p->ktasks.size());
  out->bwd_blocks = int64_t(p->kblocks.size());
  out->attn_ranges = int64_t(p->ranges.size());
  out->bwd_key_ranges = int64_t(p->kranges.size());
  out->bwd_mask_words = int64_t(p->kmasks.size());
  return UG_OK;
}

ug_status ug_plan_export(ug_plan_t p, int32_t* perm, int32_t* win_off, int32_t* nbr, int32_t* nbr_off) {
  ug::clear_error();
  if (!p) return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_plan_export: plan is NULL");
  if (perm) std::memcpy(perm, p->perm.data(), p->perm.size() * sizeof(int32_t));
  if (win_off) std::memcpy(win_off, p->win_off.data(), p->win_off.size() * sizeof(int32_t));
  if (nbr && !p->nbr.empty()) std::memcpy(nbr, p->nbr.data(), p->nbr.size() * sizeof(int32_t));
  if (nbr_off) std::memcpy(nbr_off, p->nbr_off.data(), p->nbr_off.size() * sizeof(int32_t));
  return UG_OK;
}

ug_status ug_plan_export_lr(ug_plan_t p, int32_t* lr_perm, int32_t* lr_win_off) {
  ug::clear_error();
  if (!p) return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_plan_export_lr: plan is NULL");
  if (lr_perm && !p->lr_perm.empty()) std::memcpy(lr_perm, p->lr_perm.data(), p->lr_perm.size() * sizeof(int32_t));
  if (lr_win_off) std::memcpy(lr_win_off, p->lr_win_off.data(), p->lr_win_off.size() * sizeof(int32_t));
  return UG_OK;
}

ug_status ug_plan_export_queues(ug_plan_t p, int32_t* attn_items, int32_t* bwd_items) {
  ug::clear_error();
  if (!p) return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_plan_export_queues: plan is NULL");
  auto put = [](const std::vector<ug::Block>& b, int32_t* out) {
    for (size_t i = 0; i < b.size(); ++i) {
      out[2 * i] = b[i].task;
      out[2 * i + 1] = b[i].bh;
    }
  };
  if (attn_items) put(p->blocks, attn_items);
  if (bwd_items) put(p->kblocks, bwd_items);
  return UG_OK;
}

ug_status ug_plan_export_blocks(ug_plan_t p, int32_t* q_tiles, int32_t* k_ranges, int32_t* k_tiles,
                                int32_t* q_ranges, int32_t* mask_off, uint64_t* masks) {
  ug::clear_error();
  if (!p) return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_plan_export_blocks: plan is NULL");
  auto put_tasks = [](const std::vector<ug::Task>& t, int32_t* out) {
    for (size_t i = 0; i < t.size(); ++i) {
      out[4 * i] = t[i].q0;
      out[4 * i + 1] = t[i].q1;
      out[4 * i + 2] = t[i].r0;
      out[4 * i + 3] = t[i].r1;
    }
  };
  auto put_ranges = [](const std::vector<ug::Range>& r, int32_t* out) {
    for (size_t i = 0; i < r.size(); ++i) {
      out[2 * i] = r[i].k0;
      out[2 * i + 1] = r[i].k1;
    }
  };
  if (q_tiles) put_tasks(p->tasks, q_tiles);
  if (k_ranges) put_ranges(p->ranges, k_ranges);
  if (k_tiles) put_tasks(p->ktasks, k_tiles);
  if (q_ranges) put_ranges(p->kranges, q_ranges);
  if (mask_off && !p->kmask_off.empty())
    std::memcpy(mask_off, p->kmask_off.data(), p->kmask_off.size() * sizeof(int32_t));
  if (masks && !p->kmasks.empty()) std::memcpy(masks, p->kmasks.data(), p->kmasks.size() * sizeof(uint64_t));
  return UG_OK;
}

const char* ug_status_str(ug_status s) {
  switch (s) {
    case UG_OK: return "UG_OK";
    case UG_ERR_INVALID_ARGUMENT: return "UG_ERR_INVALID_ARGUMENT";
    case UG_ERR_UNSUPPORTED: return "UG_ERR_UNSUPPORTED";
    case UG_ERR_OUT_OF_MEMORY: return "UG_ERR_OUT_OF_MEMORY";
    case UG_ERR_HIP: return "UG_ERR_HIP";
    case UG_ERR_INTERNAL: return "UG_ERR_INTERNAL";
  }
  return "UG_ERR_UNKNOWN";
}

const char* ug_last_error(void) { return ug::g_last_error.c_str(); }

}  // extern "C"
