// gfx950 kernels of the attention backward (dQ, dK, dV of the composite-
// masked attention, given dO and the forward's log-sum-exp) and the C-ABI
// entry point ug_attn_bwd.
//
// Method: UltraGen fine-tunes its LR branch through the joint attention
// ("UltraGen: Efficient Ultra-High-Resolution Image Generation with
// Hierarchical Local Attention", papernotes.org notes, 关键设计 3 and the
// training section), so the loss is differentiated through it.  With
// S = Q K^T / sqrt(D) over the allowed keys and P = exp(S - lse):
//   Delta_i = dO_i . O_i,  dP = dO V^T,  dS = P * (dP - Delta),
//   dQ = dS K / sqrt(D),   dK = dS^T Q / sqrt(D),   dV = P^T dO.
// Three launches, no atomics, every sum taken in a fixed order, so the
// result is deterministic:
//   prep   per row and head, lse in log2 units and Delta (fp32) into the
//          caller's workspace;
//   dQ     query-major over the forward's query tiles: the keys stream
//          through LDS in 64-row tiles, as in the forward;
//   dK/dV  key-major over the plan's transposed tiles: a workgroup owns up
//          to 256 keys (8 waves x 32) and streams the queries that see
//          them (Q, dO and their statistics) through LDS.
// Operands are bf16, products on v_mfma_f32_32x32x16_bf16 with fp32
// accumulation; P and dS are rounded to bf16 as MFMA operands.
#include "common.hpp"

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>

namespace {

using namespace ug::dev;
using ug::host::aligned16;
using ug::host::check_plan;
using ug::host::current_device;
using ug::host::launch_status;
using ug::host::overlap_ranges;
using ug::host::tensor_bytes;

constexpr int kThreads = 512;            // 8 waves
constexpr int kRows = ug::kAttnKeyTile;  // rows per LDS tile
constexpr float kLog2e = 1.4426950408889634f;

// One 64-row x D bf16 tile in LDS.  Rows are unpadded; the 16-byte chunks of
// row r are XOR-swizzled so that both ways the kernels read a tile are free
// of bank conflicts:
//  - row reads (ds_read_b128, an MFMA operand with the row as the lane
//    index): 16 consecutive rows of one logical chunk hit 16 different
//    physical chunk positions;
//  - transpose reads (ds_read_b64_tr_b16, an operand with the row as the
//    packed index): an aligned group of 4 rows x 32 dims hits 4 different
//    64-byte bank groups.
// For 16-chunk rows the swizzle swaps the two 2-bit halves of r mod 16; for
// 8-chunk rows (two rows per bank sweep) it does the same on the row pair
// index.
template <int D>
struct Tile {
  static constexpr int kChunks = D / 8;
  static constexpr int RB = D * 2;  // bytes per row
  static constexpr int kBytes = kRows * RB;
  static constexpr int kLoads = kBytes / 16 / kThreads;  // 16-byte loads per thread and tile
  static_assert(kChunks == 8 || kChunks == 16, "head_dim must be 64 or 128");
  static_assert(kLoads >= 1 && kBytes % (16 * kThreads) == 0, "tile must split evenly over the workgroup");
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (kChunks == 16) {
      return ((r & 3) << 2) | ((r >> 2) & 3);
    } else {
      const int m = r >> 1;
      return ((m & 1) << 2) | ((m >> 1) & 3);
    }
  }
  // byte offset of logical chunk c of row r
  __device__ static __forceinline__ int off(int r, int c) { return r * RB + ((c ^ swz(r)) << 4); }
};

// Direct global->LDS loads (global_load_lds_dwordx4) of the 64 rows ks ..
// ks+63 of a [rows][row_stride] bf16 array: slot s = i*512 + tid of the tile
// holds row s / kChunks, physical chunk s % kChunks.  A ragged tile (nv < 64)
// repeats its last row, so no load leaves the range; the kernels mask those
// rows.
template <int D>
struct Loader {
  using L = Tile<D>;
  uint32_t off[L::kLoads];
  __device__ __forceinline__ static int row_of(int i, int tid) { return (i * kThreads + tid) / L::kChunks; }
  __device__ __forceinline__ static int lchunk_of(int i, int tid) {
    const int slot = i * kThreads + tid;
    return (slot % L::kChunks) ^ L::swz(slot / L::kChunks);
  }
  __device__ __forceinline__ void init(int64_t rs, int tid) {
#pragma unroll
    for (int i = 0; i < L::kLoads; ++i) off[i] = uint32_t(row_of(i, tid) * rs * 2 + lchunk_of(i, tid) * 16);
  }
  // Rows nv .. 63 of a ragged tile read as zeros (the buffer descriptor
  // covers the nv valid rows only).  A zero row contributes nothing: a zero
  // K row to dQ, a zero Q row to dK, a zero dO row to dV (and its dP is 0,
  // so dS = P * (0 - Delta) only meets zero rows), so no mask is needed.
  __device__ __forceinline__ void issue(const __bf16* src, int64_t rs, int32_t ks, int32_t nv, char* tile, int tid,
                                        int wave) const {
    const char* base = reinterpret_cast<const char*>(src + int64_t(ks) * rs);  // wave-uniform
    const int32_t nvs = __builtin_amdgcn_readfirstlane(nv);
    const int32_t bytes = (nvs > 0 ? nvs : 0) * int32_t(rs) * 2;
#pragma unroll
    for (int i = 0; i < L::kLoads; ++i)
      load_lds<16>(base, off[i], (lds_void*)(tile + (i * kThreads + wave * 64) * 16), bytes);
    (void)tid;
  }
};

// Per-lane LDS offsets of the two operand forms; the swizzle depends on the
// row modulo 16 only, so 32-row blocks and 16-row chunks are constant
// offsets on top of these.
//  row[i]:     row l%32, logical chunk 2i + g (dims 16i + 8g .. +7);
//  tr[t][hh]:  the transpose read of rows 8hh + 4g + (l&15)/4, dims
//              32t + 16*((l>>4)&1) + 4*(l&3) .. +3 (see tr_operand).
template <int D>
struct LaneOffsets {
  int row[D / 16];
  int tr[D / 32][2];
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) row[i] = Tile<D>::off(l32, 2 * i + g);
    const int vrow = 4 * g + ((lane & 15) >> 2);
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      const int dim = 32 * t + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) tr[t][hh] = Tile<D>::off(vrow + 8 * hh, dim / 8) + (dim % 8) * 2;
    }
  }
};

// c (32 tile rows 32mb .. 32mb+31 x 32 register columns) = sum over the D
// dims of tile[row][dim] * b[column][dim]; b[i] holds dims 16i + 8g .. +7 of
// the lane's column.  Output lane l: column l%32, rows 8*(j/4) + 4g + j%4.
template <int D>
__device__ __forceinline__ f32x16 rows_x_regs(const char* tile, int mb, const bf16x8 (&b)[D / 16],
                                              const LaneOffsets<D>& lo) {
  const char* t0 = tile + mb * 32 * Tile<D>::RB;
  f32x16 c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(t0 + lo.row[0]), b[0],
                                                     f32x16{}, 0, 0, 0);
#pragma unroll
  for (int i = 1; i < D / 16; ++i)
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(t0 + lo.row[i]), b[i], c, 0, 0, 0);
  return c;
}

// Transposed operand: lane l gets dim 32t + l%32 of the 8 tile rows
// {4g .. 4g+3, 8+4g .. 8+4g+3} of 16-row chunk c, the same rows (in the same
// order) that a 32x32 MFMA output holds in registers 8*(c&1) .. +7 of block
// c>>1.  Within each 16-lane group the transpose read gives lane j dim j of
// the four rows the group addresses.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const char* tile, int t, int c, const LaneOffsets<D>& lo) {
  const char* t0 = tile + 16 * c * Tile<D>::RB;
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(t0 + lo.tr[t][0]));
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(t0 + lo.tr[t][1]));
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Writes a wave's 32 x D accumulator block (lane l: row l%32; registers j of
// 32-dim tile t: dims 32t + 8*(j/4) + 4g + j%4), times `scale`, as bf16 to
// rows row0 .. row0+31 (those < rend) of `out`, through the wave's own
// 32-row LDS area so that every row is written with 16-byte stores.  The
// wave reads back only what it wrote: one wave's LDS operations complete in
// order, so no barrier is needed.
template <int D>
__device__ __forceinline__ void store_block(const f32x16 (&acc)[D / 32], float scale, char* ost, __bf16* out,
                                            int64_t rs, int32_t row0, int32_t rend, int lane) {
  using L = Tile<D>;
  const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * t + 8 * q4 + 4 * g;
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = __bf16(acc[t][4 * q4 + e] * scale);
      *reinterpret_cast<bf16x4*>(ost + L::off(l32, d0 / 8) + (d0 % 8) * 2) = w;
    }
  constexpr int rows_per_pass = 64 / L::kChunks;
#pragma unroll
  for (int pass = 0; pass < 32 / rows_per_pass; ++pass) {
    const int r = pass * rows_per_pass + lane / L::kChunks;
    const int cc = lane % L::kChunks;
    const uint4 val = *reinterpret_cast<const uint4*>(ost + L::off(r, cc));
    if (row0 + r < rend) *reinterpret_cast<uint4*>(out + int64_t(row0 + r) * rs + cc * 8) = val;
  }
}

// ---------------------------------------------------------------------------
// prep: lse2[bh][row] = lse * log2(e) and delta[bh][row] = sum_d dO * O, in
// fp32, for rows < L; rows L .. stat_rows-1 are written as zeros.  A
// workgroup takes kRows rows of up to kPrepHeads heads (grid z covers the
// head groups): each thread owns one 16-byte column chunk and has four rows
// of O and dO in flight at once; the D/8 chunks of one head are consecutive
// lanes and are summed with shuffles.  The sums are collected in LDS, so each
// head's statistics leave as one contiguous run of kRows floats.  A
// workgroup walks its rows four at a time, one memory latency each, so small
// layers (fewer than two 64-row workgroups per compute unit) take 16-row
// workgroups: four times as many, each a quarter as long.
// ---------------------------------------------------------------------------
constexpr int kPrepRows = 64;       // rows per workgroup
constexpr int kPrepRowsSmall = 16;  // rows per workgroup of small layers
constexpr int kPrepHeads = 64;
constexpr int kPrepInFlight = 4;

template <int D, int kRows>
__global__ __launch_bounds__(1024) void bwd_prep_kernel(const __bf16* __restrict__ o, const __bf16* __restrict__ d_o,
                                                        const float* __restrict__ lse, float* __restrict__ lse2,
                                                        float* __restrict__ delta, int32_t L, int32_t Lp,
                                                        int32_t heads) {
  static_assert(kRows % kPrepInFlight == 0, "rows in whole batches");
  constexpr int C = D / 8;  // chunks per head
  __shared__ float s_sum[kPrepHeads * kRows];  // [head of the group][row]
  const int32_t h0 = blockIdx.z * kPrepHeads;
  const int32_t gh = min(kPrepHeads, heads - h0);  // heads of this group
  const int32_t units = gh * C;
  const int32_t b = blockIdx.y;
  const int32_t row0 = blockIdx.x * kRows;
  const int64_t boff = int64_t(b) * L * heads * D + int64_t(h0) * D;
  for (int32_t c0 = 0; c0 < units; c0 += blockDim.x) {  // uniform trip count: every lane shuffles
    const int32_t c = c0 + int32_t(threadIdx.x);
    for (int32_t rb = 0; rb < kRows; rb += kPrepInFlight) {
      bf16x8 x[kPrepInFlight], y[kPrepInFlight];
#pragma unroll
      for (int r = 0; r < kPrepInFlight; ++r) {
        const int32_t row = row0 + rb + r;
        if (c < units && row < L) {
          const int64_t e = boff + int64_t(row) * heads * D + int64_t(c) * 8;
          x[r] = *reinterpret_cast<const bf16x8*>(o + e);
          y[r] = *reinterpret_cast<const bf16x8*>(d_o + e);
        }
      }
#pragma unroll
      for (int r = 0; r < kPrepInFlight; ++r) {
        const int32_t row = row0 + rb + r;
        float sum = 0.f;
        if (c < units && row < L) {
#pragma unroll
          for (int k = 0; k < 8; ++k) sum = fmaf(float(x[r][k]), float(y[r][k]), sum);
        }
#pragma unroll
        for (int m = C / 2; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, C);
        if (c < units && c % C == 0) s_sum[(c / C) * kRows + rb + r] = sum;
      }
    }
  }
  __syncthreads();
  for (int32_t i = threadIdx.x; i < gh * kRows; i += blockDim.x) {
    const int32_t h = h0 + i / kRows, row = row0 + i % kRows;
    if (row >= Lp) continue;
    const int64_t s = (int64_t(b) * heads + h) * Lp + row;
    const bool in = row < L;
    delta[s] = in ? s_sum[i] : 0.f;
    lse2[s] = in ? lse[(int64_t(b) * heads + h) * L + row] * kLog2e : 0.f;
  }
}

struct BwdParams {
  const __bf16* q;    // permuted, rotated
  const __bf16* k;    // permuted, rotated
  const __bf16* v;
  const __bf16* d_o;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  const float* lse2;   // [batch*heads][Lp], log2 units
  const float* delta;  // [batch*heads][Lp]
  int64_t row_stride;    // elements between rows (heads * D)
  int64_t batch_stride;  // elements between batches (L * heads * D)
  int32_t heads;
  int32_t Lp;
  const ug::Task* tasks;
  const ug::Range* ranges;
  const ug::Block* blocks;
  const int32_t* mask_off;  // dK/dV pass: per key tile, offset of its key masks, or < 0
  const uint64_t* masks;    // bit r: the key row sees the tile's query range r
  float scale_log2;  // log2(e) / sqrt(D)
  float scale;       // 1 / sqrt(D)
  int32_t* queue;     // this launch's cursor slot: 8 per-XCD queue cursors, then the finished-workgroup count
  int32_t queue_len;  // items per XCD queue (blocks / 8)
  int32_t L, n_tasks, n_bh;  // rows, tasks of the current pass and batch*heads (index checks of the debug build)
};
typedef __attribute__((address_space(4))) const BwdParams* BArgs;
__device__ __forceinline__ BArgs bwd_args() { return opaque_args<BwdParams>(); }

// Persistent grid of the dQ pass: one workgroup per CU takes query tiles from
// the plan's per-XCD queues until they are empty, as the attention forward
// does.  The dK/dV pass keeps one workgroup per key tile: inside an item loop
// the addresses of its two LDS rings no longer fold into one base plus
// immediate offsets (twice the address arithmetic per step), which cost more
// than the dynamic schedule gained.
template <int kSmem, typename Item>
__device__ __forceinline__ void run_queue(Item item_fn) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];
  __shared__ ug::Range s_rng[ug::kAttnMaxRanges];
  __shared__ int32_t s_item;
  for (;;) {
    if (threadIdx.x == 0) {
      BArgs kp = bwd_args();
      s_item = queue_grab(kp->queue, kp->queue_len, kp->blocks, xcc_id());
    }
    __syncthreads();
    const int32_t item = s_item;
    if (item < 0) break;
    item_fn(bwd_args(), item, smem, s_rng);
    __syncthreads();  // the next item reuses the LDS and s_item
  }
  if (threadIdx.x == 0) queue_finish(bwd_args()->queue);
}

// ---------------------------------------------------------------------------
// dQ: per query tile (the forward's tasks, taken from the queues), 8 waves x 32
// queries.  Per wave, 32-key block u (half of a 64-key tile; K and V tiles
// in three-slot LDS rings):
//   A(u): S^T  = K Q^T     (A: K rows from LDS, B: the wave's Q in registers)
//         dP^T = V dO^T    (A: V rows from LDS, B: the wave's dO in registers)
//   B(u): dS^T = exp2(S^T * scale_log2 - lse2) * (dP^T - Delta)   lane = query
//   C(u): dQ^T += K^T dS^T (A: K transposed from LDS, B: dS^T from registers)
// Software pipeline over blocks: step u runs A(u+1) as one MFMA per slot with
// one (or two) dS elements of B(u) beside each, then C(u).  The slots are
// fenced so the compiler keeps the interleave; operand reads run kLead slots
// ahead.  Ring protocol (one barrier per tile, after its first block): the
// loads of tile i+2 are issued right after that barrier of tile i, into the
// slots of tile i-1, whose last reads (C of its second block, and A of its
// second block for V) come before it, and they must land by the barrier of
// tile i+1, which the block that first reads them (A of tile i+2's first
// block) follows.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void dq_item(BArgs kp, int32_t item, char* smem, ug::Range* s_rng) {
  using L = Tile<D>;
  constexpr int TB = L::kBytes;
  constexpr int RB = L::RB;
  constexpr int kQRegs = D / 16;           // k-steps of one 32-key block's S^T (and dP^T)
  constexpr int kASlots = 2 * kQRegs;      // A: S^T and dP^T MFMAs, alternating
  constexpr int kCSlots = 2 * (D / 32);    // C: two 16-key chunks x D/32 dim tiles
  constexpr int kSlots = kASlots + kCSlots;
  constexpr int kElPerSlot = 16 / kASlots;  // dS elements of B(u) per A slot
  constexpr int kLead = 4;
  static_assert(kElPerSlot * kASlots == 16, "16 dS elements per lane and block");

  UG_CHECK(item >= 0 && item < kp->queue_len * ug::kXcds, 0);
  const ug::Block blk = kp->blocks[item];
  UG_CHECK(blk.task >= 0 && blk.task < kp->n_tasks && blk.bh >= 0 && blk.bh < kp->n_bh, 0);
  const ug::Task task = kp->tasks[blk.task];
  UG_CHECK(task.q0 >= 0 && task.q0 < task.q1 && task.q1 <= kp->L && task.q1 - task.q0 <= ug::kAttnQueryTile, 1);
  const int32_t b = blk.bh / kp->heads, h = blk.bh - b * kp->heads;
  const int64_t hoff = int64_t(b) * kp->batch_stride + int64_t(h) * D;
  const int64_t rs = kp->row_stride;
  // wave index in a scalar register, masked so that alias analysis keeps its range
  const int tid = opaque_tid<kThreads>(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (kThreads / 64 - 1);
  const int l32 = lane & 31, g = lane >> 5;
  const int32_t qrow = task.q0 + wave * 32 + l32;
  const int32_t qload = min(qrow, task.q1 - 1);

  const int32_t nr = task.r1 - task.r0;
  UG_CHECK(nr >= 1 && nr <= ug::kAttnMaxRanges, 1);
  if (tid < nr) {
    const ug::Range r = kp->ranges[task.r0 + tid];
    UG_CHECK(r.k0 >= 0 && r.k0 < r.k1 && r.k1 <= kp->L, 1);
    s_rng[tid] = r;
  }

  bf16x8 qf[kQRegs], df[kQRegs];
#pragma unroll
  for (int i = 0; i < kQRegs; ++i) {
    qf[i] = *reinterpret_cast<const bf16x8*>(kp->q + hoff + qload * rs + 16 * i + 8 * g);
    df[i] = *reinterpret_cast<const bf16x8*>(kp->d_o + hoff + qload * rs + 16 * i + 8 * g);
  }
  UG_CHECK(qload < kp->Lp, 3);
  const int64_t srow = int64_t(blk.bh) * kp->Lp + qload;
  const float lse2 = kp->lse2[srow];
  const float dlt = kp->delta[srow];
  const float c2 = kp->scale_log2;
  __syncthreads();  // s_rng is filled

  int32_t ntiles = 0;
  for (int32_t r = 0; r < nr; ++r) ntiles += (s_rng[r].k1 - s_rng[r].k0 + kRows - 1) / kRows;
  ntiles = __builtin_amdgcn_readfirstlane(ntiles);

  const __bf16* kg = kp->k + hoff;
  const __bf16* vg = kp->v + hoff;
  Loader<D> ld;
  ld.init(rs, tid);
  LaneOffsets<D> lo;
  lo.init(lane);
  // Opaque offsets: with their known bits the compiler would fold the
  // constant part of every (offset, chunk) pair into its own register and
  // hold them all across the loop; opaque, the constant parts stay in the
  // LDS instructions' immediate offsets.
#pragma unroll
  for (int i = 0; i < D / 16; ++i) asm volatile("" : "+v"(lo.row[i]));
#pragma unroll
  for (int t = 0; t < D / 32; ++t) asm volatile("" : "+v"(lo.tr[t][0]), "+v"(lo.tr[t][1]));
  TileCursor cur;
  cur.init(s_rng, 0, nr);
  // K ring: slots 0..2 at [0, 3TB); V ring: slots 0..2 at [3TB, 6TB).  Tile
  // i uses slot i % 3, known at compile time in the unrolled loop below.
  auto issue_tile = [&](int slot) {  // the cursor's next tile into `slot`
    const int32_t nv = cur.nv();
    ld.issue(kg, rs, cur.ks, nv, smem + slot * TB, tid, wave);
    ld.issue(vg, rs, cur.ks, nv, smem + (3 + slot) * TB, tid, wave);
    cur.advance(s_rng);
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};

  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  float e_hold = 0.f;
  // dS element j (0..15) of a block: register j of S^T and dP^T; elements
  // 2m and 2m+1 form one packed pair of chunk j / 8.  The volatile asm pins
  // the work to its slot.
  auto ds_elem = [&](const f32x16& s, const f32x16& dp, bf16x8 (&ds)[2], int j) {
    // P <= 1 for every allowed key; the clamp (free on v_exp) keeps the zero
    // rows of a ragged tile finite whatever the row's LSE.
    const float pv = __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(fmaf(s[j], c2, -lse2)), 0.f, 1.f);
    const float d = pv * (dp[j] - dlt);
    if ((j & 1) == 0) {
      e_hold = d;
      asm volatile("" : "+v"(e_hold));
    } else {
      bf16x2 pr = {__bf16(e_hold), __bf16(d)};
      asm volatile("" : "+v"(pr));
      ds[j >> 3][(j & 7) - 1] = pr[0];
      ds[j >> 3][j & 7] = pr[1];
    }
  };

  // One block step: A of the next block (rows 32 mbA .. of the K and V tiles
  // at ka, va) into s_out / dp_out beside B of the current block (s_in,
  // dp_in -> ds), then C of the current block (the K tile at kc, chunks
  // 2 mbC and 2 mbC + 1).
  auto block_step = [&](const char* ka, const char* va, int mbA, const f32x16& s_in, const f32x16& dp_in,
                        f32x16& s_out, f32x16& dp_out, const char* kc, int mbC) {
    bf16x8 opnd[kLead + 1];
    bf16x8 ds[2];
    auto fetch = [&](int k) {
      if (k < kASlots) {  // even: K rows of k-step k/2; odd: V rows
        const char* base = ((k & 1) ? va : ka) + mbA * 32 * RB;
        opnd[k % (kLead + 1)] = *reinterpret_cast<const bf16x8*>(base + lo.row[k >> 1]);
      } else {  // C: chunk 2 mbC + c / (D/32), dim tile c % (D/32)
        const int c = k - kASlots;
        opnd[k % (kLead + 1)] = tr_operand<D>(kc, c % (D / 32), 2 * mbC + c / (D / 32), lo);
      }
    };
#pragma unroll
    for (int k = 0; k < kLead; ++k) fetch(k);
#pragma unroll
    for (int k = 0; k < kSlots; ++k) {
      if (k + kLead < kSlots) fetch(k + kLead);
      if (k < kASlots) {
        const int ks = k >> 1;
        if ((k & 1) == 0)
          s_out = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[k % (kLead + 1)], qf[ks], ks == 0 ? f32x16{} : s_out,
                                                          0, 0, 0);
        else
          dp_out = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[k % (kLead + 1)], df[ks],
                                                           ks == 0 ? f32x16{} : dp_out, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < kElPerSlot; ++e) ds_elem(s_in, dp_in, ds, k * kElPerSlot + e);
      } else {
        const int c = k - kASlots;
        acc[c % (D / 32)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[k % (kLead + 1)], ds[c / (D / 32)],
                                                                    acc[c % (D / 32)], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // prologue: tiles 0 and 1 into their slots, then A of block (0, 0)
  issue_tile(0);
  if (ntiles > 1) issue_tile(1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 sa, dpa, sb, dpb;
  sa = rows_x_regs<D>(smem, 0, qf, lo);
  dpa = rows_x_regs<D>(smem + 3 * TB, 0, df, lo);

  // Tile i (in slot S = i % 3): block (i, 0) is A(i, 1) || B(i, 0), C(i, 0);
  // then the barrier, the loads of tile i+2 into slot (S + 2) % 3, and block
  // (i, 1): A(i+1, 0) || B(i, 1), C(i, 1).  Past the last tile, A reads a
  // stale slot and its result is unused.
  auto tile = [&](int32_t i, auto slot) {
    constexpr int S = decltype(slot)::value;
    const char* kt = smem + S * TB;
    block_step(kt, smem + (3 + S) * TB, 1, sa, dpa, sb, dpb, kt, 0);
    __builtin_amdgcn_s_waitcnt(0);  // tile i+1 has landed (issued two blocks ago)
    __syncthreads();                // and every wave is past tile i-1's slots
    if (i + 2 < ntiles) issue_tile((S + 2) % 3);
    block_step(smem + ((S + 1) % 3) * TB, smem + (3 + (S + 1) % 3) * TB, 0, sb, dpb, sa, dpa, kt, 1);
  };
  // groups of three tiles, so that every slot is a compile-time offset; the
  // loop has no exit inside a group
  int32_t i = 0;
  for (; i + 3 <= ntiles; i += 3) {
    tile(i, std::integral_constant<int, 0>{});
    tile(i + 1, std::integral_constant<int, 1>{});
    tile(i + 2, std::integral_constant<int, 2>{});
  }
  if (i < ntiles) tile(i, std::integral_constant<int, 0>{});
  if (i + 1 < ntiles) tile(i + 1, std::integral_constant<int, 1>{});
  __syncthreads();  // every wave is done with the rings before the output staging
  kp = bwd_args();  // the epilogue's arguments are loaded here, not kept across the loop
  store_block<D>(acc, kp->scale, smem + wave * 32 * L::RB, kp->dq + hoff, rs, task.q0 + wave * 32, task.q1, lane);
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_bwd_dq_kernel(BwdParams p) {
  (void)p;  // read through bwd_args()
  run_queue<6 * Tile<D>::kBytes>([](BArgs kp, int32_t item, char* smem, ug::Range* s_rng) {  // K ring, V ring
    dq_item<D>(kp, item, smem, s_rng);
  });
}

// ---------------------------------------------------------------------------
// dK/dV: one workgroup per key tile (the plan's transposed tasks), 8 waves x
// 32 keys.  Per wave and 64-query tile (Q, dO and the rows' lse2 / Delta in
// two-slot LDS rings), one 32-query block mb at a time:
//   S  = Q K^T    (A: Q rows from LDS, B: the wave's K in registers)
//   dP = dO V^T   (A: dO rows from LDS, B: the wave's V rows, kept in LDS:
//                  K, V and the two accumulators would not fit in registers)
//   P  = exp2(S * scale_log2 - lse2), dS = P * (dP - Delta)   lane = key
//   dV^T += dO^T P, dK^T += Q^T dS   (A: dO / Q transposed from LDS)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void attn_bwd_dkdv_kernel(BwdParams p) {
  using L = Tile<D>;
  constexpr int TB = L::kBytes;
  constexpr int SB = 2 * kRows * int(sizeof(float));  // lse2 then Delta of 64 rows
  constexpr int VB = 32 * L::RB;                       // one wave's 32 V rows
  // Q ring [0, 2TB), dO ring [2TB, 4TB), statistics ring [4TB, 4TB + 2SB),
  // then the waves' V blocks
  __shared__ __attribute__((aligned(1024))) char smem[4 * TB + 2 * SB + 8 * VB];
  __shared__ ug::Range s_rng[ug::kAttnMaxRanges];

  const ug::Block blk = p.blocks[blockIdx.x];
  if (blk.task < 0) return;  // idle workgroup (uniform)
  UG_CHECK(blk.task < p.n_tasks && blk.bh >= 0 && blk.bh < p.n_bh, 0);
  const ug::Task task = p.tasks[blk.task];
  UG_CHECK(task.q0 >= 0 && task.q0 < task.q1 && task.q1 <= p.L && task.q1 - task.q0 <= ug::kAttnQueryTile, 1);
  const int32_t b = blk.bh / p.heads, h = blk.bh - b * p.heads;
  const int64_t hoff = int64_t(b) * p.batch_stride + int64_t(h) * D;
  const int64_t rs = p.row_stride;
  // wave index in a scalar register, masked so that alias analysis keeps its range
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (kThreads / 64 - 1);
  const int l32 = lane & 31, g = lane >> 5;
  const int32_t krow = task.q0 + wave * 32 + l32;
  const int32_t kload = min(krow, task.q1 - 1);

  const int32_t nr = task.r1 - task.r0;
  UG_CHECK(nr >= 1 && nr <= ug::kAttnMaxRanges, 1);
  if (tid < nr) {
    const ug::Range r = p.ranges[task.r0 + tid];
    UG_CHECK(r.k0 >= 0 && r.k0 < r.k1 && r.k1 <= p.L, 1);
    s_rng[tid] = r;
  }
  // Which of the tile's query ranges this lane's key sees (all of them
  // unless the tile groups corresponding-LR windows).
  const int32_t moff = p.mask_off ? p.mask_off[blk.task] : -1;  // uniform
  const uint64_t kmask = moff >= 0 ? p.masks[moff + (kload - task.q0)] : ~uint64_t(0);

  bf16x8 kf[D / 16];
  char* const vblk = smem + 4 * TB + 2 * SB + wave * VB;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    kf[i] = *reinterpret_cast<const bf16x8*>(p.k + hoff + kload * rs + 16 * i + 8 * g);
    *reinterpret_cast<bf16x8*>(vblk + L::off(l32, 2 * i + g)) =
        *reinterpret_cast<const bf16x8*>(p.v + hoff + kload * rs + 16 * i + 8 * g);
  }
  const float c2 = p.scale_log2;
  __syncthreads();  // s_rng is filled

  int32_t ntiles = 0;
  for (int32_t r = 0; r < nr; ++r) ntiles += (s_rng[r].k1 - s_rng[r].k0 + kRows - 1) / kRows;

  const __bf16* qg = p.q + hoff;
  const __bf16* dog = p.d_o + hoff;
  const int64_t sbase = int64_t(blk.bh) * p.Lp;
  Loader<D> ld;
  ld.init(rs, tid);
  LaneOffsets<D> lo;
  lo.init(lane);
  TileCursor cur;
  cur.init(s_rng, 0, nr);
  // rows ks .. ks+63 of the statistics (the workspace is padded past L, so a
  // whole tile can always be read): wave 0 loads lse2, wave 1 Delta
  auto issue_stats = [&](int32_t ks, char* dst) {
    if (wave < 2) {
      const float* src = (wave == 0 ? p.lse2 : p.delta) + sbase + ks + lane;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void*)(dst + wave * kRows * 4), 4, 0, 0);
    }
  };

  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) dka[t] = dva[t] = f32x16{};

  int32_t nv = cur.nv();
  int32_t rcur = cur.ri;  // query range (index into the tile's ranges) of the tile being processed
  ld.issue(qg, rs, cur.ks, nv, smem, tid, wave);
  ld.issue(dog, rs, cur.ks, nv, smem + 2 * TB, tid, wave);
  issue_stats(cur.ks, smem + 4 * TB);
  cur.advance(s_rng);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int32_t i = 0; i < ntiles; ++i) {
    const int slot = i & 1;
    const int32_t nv_next = cur.nv();
    const int32_t rnext = cur.ri;
    if (i + 1 < ntiles) {
      ld.issue(qg, rs, cur.ks, nv_next, smem + (slot ^ 1) * TB, tid, wave);
      ld.issue(dog, rs, cur.ks, nv_next, smem + 2 * TB + (slot ^ 1) * TB, tid, wave);
      issue_stats(cur.ks, smem + 4 * TB + (slot ^ 1) * SB);
      cur.advance(s_rng);
    }
    const char* qt = smem + slot * TB;
    const char* dot = smem + 2 * TB + slot * TB;
    const float* st = reinterpret_cast<const float*>(smem + 4 * TB + slot * SB);
    // Whether this lane's key sees the tile's query range (corresponding-LR
    // key tiles); a ragged tail needs no mask (its rows are zero).
    const bool sees = (kmask >> rcur) & 1;
    const uint64_t seen = __ballot(sees);
    const bool all_see = seen == ~uint64_t(0);  // uniform
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      if (seen == 0) break;  // no key of this wave sees the range (uniform)
      // S = Q K^T (B: K in registers) and dP = dO V^T (B: the wave's V rows)
      // as alternating MFMAs, their LDS operands kSLead slots ahead
      f32x16 s = f32x16{}, dp = f32x16{};
      {
        constexpr int kS = 2 * (D / 16);
        constexpr int kSLead = 1;
        bf16x8 oa[kSLead + 1], ob[kSLead + 1];
        const char* q0 = qt + mb * 32 * L::RB;
        const char* d0 = dot + mb * 32 * L::RB;
        auto sfetch = [&](int k) {
          const int i = k >> 1;
          if ((k & 1) == 0) {
            oa[k % (kSLead + 1)] = *reinterpret_cast<const bf16x8*>(q0 + lo.row[i]);
          } else {
            oa[k % (kSLead + 1)] = *reinterpret_cast<const bf16x8*>(d0 + lo.row[i]);
            ob[k % (kSLead + 1)] = *reinterpret_cast<const bf16x8*>(vblk + lo.row[i]);
          }
        };
#pragma unroll
        for (int k = 0; k < kSLead; ++k) sfetch(k);
#pragma unroll
        for (int k = 0; k < kS; ++k) {
          if (k + kSLead < kS) sfetch(k + kSLead);
          const int i = k >> 1;
          if ((k & 1) == 0)
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[k % (kSLead + 1)], kf[i], s, 0, 0, 0);
          else
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[k % (kSLead + 1)], ob[k % (kSLead + 1)], dp, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // P and dS of both 16-query chunks (registers 8cc .. 8cc+7) first, so
      // that S and dP are dead during the 16 MFMAs, whose operands then run
      // kLead reads ahead through a register ring
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2) {
          const int a = 2 * cc + a2;
          const int row0 = 32 * mb + 8 * a + 4 * g;  // query rows of registers 4a .. 4a+3
          const float4 l4 = *reinterpret_cast<const float4*>(st + row0);
          const float4 d4 = *reinterpret_cast<const float4*>(st + kRows + row0);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 4 * a + e;
            float pv = __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(fmaf(s[j], c2, -lv[e])), 0.f, 1.f);
            if (!all_see && !sees) pv = 0.f;
            pb[cc][4 * a2 + e] = __bf16(pv);
            dsb[cc][4 * a2 + e] = __bf16(pv * (dp[j] - dl[e]));
          }
        }
      }
      constexpr int kM = 4 * (D / 32);  // MFMAs: 2 chunks x D/32 dim tiles x (dV, dK)
      constexpr int kLead = 2;
      bf16x8 opnd[kLead + 1];
      auto fetch = [&](int k) {  // k = (cc * D/32 + t) * 2 + (0: dV from dO, 1: dK from Q)
        const int cc = k / (2 * (D / 32)), t = (k / 2) % (D / 32);
        opnd[k % (kLead + 1)] = tr_operand<D>((k & 1) ? qt : dot, t, 2 * mb + cc, lo);
      };
#pragma unroll
      for (int k = 0; k < kLead; ++k) fetch(k);
#pragma unroll
      for (int k = 0; k < kM; ++k) {
        if (k + kLead < kM) fetch(k + kLead);
        const int cc = k / (2 * (D / 32)), t = (k / 2) % (D / 32);
        if ((k & 1) == 0)
          dva[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[k % (kLead + 1)], pb[cc], dva[t], 0, 0, 0);
        else
          dka[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[k % (kLead + 1)], dsb[cc], dka[t], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    nv = nv_next;
    rcur = rnext;
    __builtin_amdgcn_s_waitcnt(0);  // this thread's loads of the next tile have landed
    __syncthreads();
  }
  char* const ost = smem + wave * 32 * L::RB;
  store_block<D>(dka, p.scale, ost, p.dk + hoff, rs, task.q0 + wave * 32, task.q1, lane);
  store_block<D>(dva, 1.0f, ost, p.dv + hoff, rs, task.q0 + wave * 32, task.q1, lane);
}

// prep on `s`; then the dQ pass on `s` and the dK/dV pass on the plan's
// second stream side by side (each fills the compute units the other's tail
// leaves idle; they read the same inputs and write different outputs), and
// `s` waits for both.  Stream capture is refused before anything is queued.
template <int D>
ug_status launch_bwd(ug_plan_t p, BwdParams bp, const __bf16* o, const float* lse, float* lse2, float* delta,
                     hipStream_t s, const char* fn) {
  ug_status st = ug::refuse_capture(s, fn);
  if (st != UG_OK) return st;
  const int32_t Lp = int32_t(p->stat_rows());
  const int32_t units = std::min(p->d.heads, kPrepHeads) * (D / 8);
  const unsigned prep_threads = unsigned(std::min(1024, (units + 63) / 64 * 64));
  const int64_t head_groups = (p->d.heads + kPrepHeads - 1) / kPrepHeads;
  const bool small = int64_t((Lp + kPrepRows - 1) / kPrepRows) * p->d.batch * head_groups < 2 * int64_t(p->cus);
  const int rows = small ? kPrepRowsSmall : kPrepRows;
  const dim3 prep_grid(unsigned((Lp + rows - 1) / rows), unsigned(p->d.batch), unsigned(head_groups));
  if (small)
    hipLaunchKernelGGL((bwd_prep_kernel<D, kPrepRowsSmall>), prep_grid, dim3(prep_threads), 0, s, o, bp.d_o, lse, lse2,
                       delta, int32_t(p->L), Lp, p->d.heads);
  else
    hipLaunchKernelGGL((bwd_prep_kernel<D, kPrepRows>), prep_grid, dim3(prep_threads), 0, s, o, bp.d_o, lse, lse2,
                       delta, int32_t(p->L), Lp, p->d.heads);
  bp.L = int32_t(p->L);
  bp.n_bh = p->d.batch * p->d.heads;
  BwdParams kq = bp;  // the dK/dV pass: the transposed (key-major) tables
  kq.tasks = p->d_ktasks;
  kq.ranges = p->d_kranges;
  kq.blocks = p->d_kblocks;
  kq.n_tasks = int32_t(p->ktasks.size());
  kq.mask_off = p->d_kmask_off;
  kq.masks = p->d_kmasks;
  bp.tasks = p->d_tasks;
  bp.ranges = p->d_ranges;
  bp.blocks = p->d_blocks;
  bp.n_tasks = int32_t(p->tasks.size());

  std::lock_guard<std::mutex> lock(p->bwd_mu);
  auto hip_fail = [&](const char* what) {
    return ug::fail(UG_ERR_HIP, std::string(fn) + ": " + what + " failed: " + hipGetErrorString(hipGetLastError()));
  };
  if (hipEventRecord(p->bwd_fork, s) != hipSuccess) return hip_fail("hipEventRecord");
  if (hipStreamWaitEvent(p->bwd_aux, p->bwd_fork, 0) != hipSuccess) return hip_fail("hipStreamWaitEvent");
  if (!p->blocks.empty()) {
    bp.queue_len = int32_t(p->blocks.size() / ug::kXcds);
    const unsigned grid = unsigned(std::min<size_t>(size_t(p->cus), p->blocks.size()));
    st = ug::launch_with_slot(p, s, fn, [&](int32_t* cursors) {
      bp.queue = cursors;
      hipLaunchKernelGGL((attn_bwd_dq_kernel<D>), dim3(grid), dim3(kThreads), 0, s, bp);
      return launch_status(fn);
    });
  }
  if (st == UG_OK && !p->kblocks.empty()) {
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D>), dim3(unsigned(p->kblocks.size())), dim3(kThreads), 0, p->bwd_aux,
                       kq);
    st = launch_status(fn);
  }
  // the join is queued whatever happened above, so `s` never runs ahead of
  // work already queued on the second stream
  if (hipEventRecord(p->bwd_join, p->bwd_aux) != hipSuccess) return hip_fail("hipEventRecord");
  if (hipStreamWaitEvent(s, p->bwd_join, 0) != hipSuccess) return hip_fail("hipStreamWaitEvent");
  return st;
}

// Scratch of ug_attn_bwd_noalloc: the per-row statistics (log2 LSE and
// Delta) that ug_attn_bwd keeps in the caller's workspace.  One copy per
// GPU, for the life of the process; host code uses the address that
// hipGetSymbolAddress returns for the current device, never the array's name.
constexpr size_t kBwdScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kBwdScratchBytes];
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kScratchDevices] = {};

// The scratch address on `device` (which must be current), looked up once.
ug_status scratch_on(int device, void** out) {
  if (device < 0 || device >= kScratchDevices)
    return ug::fail(UG_ERR_UNSUPPORTED, "ug_attn_bwd_noalloc: device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[device]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return ug::fail(UG_ERR_HIP, std::string("ug_attn_bwd_noalloc: hipGetSymbolAddress of the scratch failed: ") +
                                      hipGetErrorString(e));
    }
    g_scratch[device] = ptr;
  }
  *out = g_scratch[device];
  return UG_OK;
}

// The backward with its statistics in `workspace`, or (use_scratch) in the
// device's scratch, looked up once every argument has been checked.
ug_status bwd_common(ug_plan_t p, const void* q, const void* k, const void* v, const void* o, const void* d_o,
                     const float* lse, void* dq, void* dk, void* dv, void* workspace, bool use_scratch, void* stream,
                     const char* fn) {
  ug_status st = check_plan(p, fn);
  if (st != UG_OK) return st;
  if (p->d.dtype != UG_BF16) return ug::fail(UG_ERR_UNSUPPORTED, std::string(fn) + ": only bf16 plans are supported");
  if (p->d.head_dim != 64 && p->d.head_dim != 128)
    return ug::fail(UG_ERR_UNSUPPORTED, std::string(fn) + ": head_dim must be 64 or 128");
  const void* ins[] = {q, k, v, o, d_o};
  void* outs[] = {dq, dk, dv};
  for (const void* x : ins)
    if (!x || !aligned16(x)) return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": NULL or unaligned input tensor");
  for (const void* x : outs)
    if (!x || !aligned16(x)) return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": NULL or unaligned output tensor");
  if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": NULL or unaligned lse");
  const int64_t ws_bytes = p->bwd_workspace_bytes();
  if (use_scratch && ws_bytes > int64_t(kBwdScratchBytes))
    return ug::fail(UG_ERR_UNSUPPORTED, std::string(fn) + ": the plan needs " + std::to_string(ws_bytes) +
                                            " bytes of statistics, more than the " +
                                            std::to_string(kBwdScratchBytes) + "-byte scratch; use ug_attn_bwd");
  if (!use_scratch && (!workspace || !aligned16(workspace)))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": workspace must be a 16-byte aligned buffer of "
                                             "info.bwd_workspace_bytes bytes");
  const int64_t n = tensor_bytes(p);
  const int64_t nl = int64_t(p->d.batch) * p->d.heads * p->L * int64_t(sizeof(float));
  for (int a = 0; a < 3; ++a) {
    for (int c = a + 1; c < 3; ++c)
      if (overlap_ranges(outs[a], n, outs[c], n))
        return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": dq, dk and dv must not overlap");
    for (const void* x : ins)
      if (overlap_ranges(outs[a], n, x, n))
        return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": an output overlaps an input");
    if (overlap_ranges(outs[a], n, lse, nl) || overlap_ranges(outs[a], n, workspace, ws_bytes))
      return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": an output overlaps lse or the workspace");
  }
  for (const void* x : ins)
    if (overlap_ranges(workspace, ws_bytes, x, n))
      return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": the workspace overlaps an input");
  if (overlap_ranges(workspace, ws_bytes, lse, nl))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": the workspace overlaps lse");
  if (p->max_task_ranges > ug::kAttnMaxRanges || p->kmax_task_ranges > ug::kAttnMaxRanges)
    return ug::fail(UG_ERR_UNSUPPORTED, std::string(fn) + ": a tile has more row ranges than the kernels stage (" +
                                            std::to_string(ug::kAttnMaxRanges) + "); use a smaller radius");
  if (current_device() != p->device)
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": current device is not the plan's device");
  if (use_scratch) {  // a static region: it cannot overlap the caller's buffers
    st = scratch_on(p->device, &workspace);
    if (st != UG_OK) return st;
  }

  BwdParams bp{};
  bp.q = static_cast<const __bf16*>(q);
  bp.k = static_cast<const __bf16*>(k);
  bp.v = static_cast<const __bf16*>(v);
  bp.d_o = static_cast<const __bf16*>(d_o);
  bp.dq = static_cast<__bf16*>(dq);
  bp.dk = static_cast<__bf16*>(dk);
  bp.dv = static_cast<__bf16*>(dv);
  const int64_t stat_elems = int64_t(p->d.batch) * p->d.heads * p->stat_rows();
  float* lse2 = static_cast<float*>(workspace);
  float* delta = lse2 + stat_elems;
  bp.lse2 = lse2;
  bp.delta = delta;
  bp.row_stride = int64_t(p->d.heads) * p->d.head_dim;
  bp.batch_stride = p->L * bp.row_stride;
  bp.heads = p->d.heads;
  bp.Lp = int32_t(p->stat_rows());
  bp.scale = float(1.0 / std::sqrt(double(p->d.head_dim)));
  bp.scale_log2 = float(1.4426950408889634 / std::sqrt(double(p->d.head_dim)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const __bf16* ob = static_cast<const __bf16*>(o);
  if (p->d.head_dim == 128) return launch_bwd<128>(p, bp, ob, lse, lse2, delta, s, fn);
  return launch_bwd<64>(p, bp, ob, lse, lse2, delta, s, fn);
}

}  // namespace

extern "C" {

ug_status ug_attn_bwd(ug_plan_t p, const void* q, const void* k, const void* v, const void* o, const void* d_o,
                      const float* lse, void* dq, void* dk, void* dv, void* workspace, void* stream) {
  ug::clear_error();
  return bwd_common(p, q, k, v, o, d_o, lse, dq, dk, dv, workspace, false, stream, "ug_attn_bwd");
}

ug_status ug_attn_bwd_noalloc(ug_plan_t p, const void* q, const void* k, const void* v, const void* o,
                              const void* d_o, const float* lse, void* dq, void* dk, void* dv, void* stream) {
  ug::clear_error();
  return bwd_common(p, q, k, v, o, d_o, lse, dq, dk, dv, nullptr, true, stream, "ug_attn_bwd_noalloc");
}

}  // extern "C"

UG_BOUNDS_ACCESSOR(ug_debug_bounds_bwd)
