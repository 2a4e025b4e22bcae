// gfx950 kernels of the hierarchical local attention path and their C-ABI
// launchers: window-first permutation (and its inverse), in-place 2D axial
// RoPE, and the composite-masked block-sparse attention forward.
//
// Method: "UltraGen: Efficient Ultra-High-Resolution Image Generation with
// Hierarchical Local Attention" (papernotes.org notes, 关键设计 1-3; the
// gist.science summary, section 2.A-2.B).  The kernel design is our own for
// CDNA4; the FlashAttention-2 / SageAttention tile sizes the pages mention
// are not used.
//
// Tensor layout everywhere: [B, L, Hh, D] contiguous, D innermost, so one
// token's row of all heads is Hh*D contiguous elements.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <string>
#include <type_traits>

#include "common.hpp"

namespace {

using namespace ug::dev;
using ug::host::aligned16;
using ug::host::check_plan;
using ug::host::current_device;
using ug::host::launch_status;
using ug::host::overlap;
using ug::host::tensor_bytes;


// ---------------------------------------------------------------------------
// Row gather: dst row j <- src row map(j), whole token rows (all heads) at a
// time.  Text rows copy in place; HR row T+i copies from T + table[i]; LR
// row T+N+i copies from T+N+lr_table[i] (in place when lr_table is null).
// With the forward tables this is the window-first permutation, with the
// inverse tables the unpermutation.  Pure HBM
// streaming: every byte is read once and written once, so the accesses are
// non-temporal 16-byte vectors; each thread owns one 16-byte column of
// kGatherRows consecutive rows and has all of them in flight at once.
// ---------------------------------------------------------------------------
constexpr int kGatherRows = 2;  // token rows per workgroup (2 measured fastest of 1, 2, 4, 8, 16)

__global__ __launch_bounds__(1024) void row_gather_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                          int32_t L, int32_t T, int32_t N, int32_t units,
                                                          const int32_t* __restrict__ table,
                                                          const int32_t* __restrict__ lr_table) {
  const int64_t batch_units = int64_t(L) * units;
  src += blockIdx.y * batch_units;
  dst += blockIdx.y * batch_units;
  const int32_t row0 = blockIdx.x * kGatherRows;
  for (int32_t c = threadIdx.x; c < units; c += blockDim.x) {
    u32x4 v[kGatherRows];
#pragma unroll
    for (int r = 0; r < kGatherRows; ++r) {
      const int32_t j = row0 + r;
      if (j < L) {
        const int32_t s = (j < T) ? j : (j < T + N) ? T + table[j - T] : lr_table ? T + N + lr_table[j - T - N] : j;
        UG_CHECK(s >= 0 && s < L && (j < T) == (s < T) && (j >= T + N) == (s >= T + N), 4);
        v[r] = __builtin_nontemporal_load(src + int64_t(s) * units + c);
      }
    }
#pragma unroll
    for (int r = 0; r < kGatherRows; ++r) {
      const int32_t j = row0 + r;
      if (j < L) __builtin_nontemporal_store(v[r], dst + int64_t(j) * units + c);
    }
  }
}

// ---------------------------------------------------------------------------
// 2D axial RoPE, in place on permuted Q and K (关键设计 1-2).  Row j of the
// permuted sequence: HR slot j-T holds raster token perm[j-T] = (r, c); LR row
// T+N+i holds LR token (m, n) = (i / w, i % w) at position (rho*m, rho*n).
// Dims [0, D/2) turn by the row position, [D/2, D) by the column position;
// pair (2k, 2k+1) of a half turns by pos * omega_k, (cos, sin) from the
// plan's table cs[pos][k].  Each thread owns one 16-byte column (part of one
// head) of kRopeRows consecutive rows in both Q and K, all loads in flight at
// once; every byte is read and written once, with non-temporal accesses.
// ---------------------------------------------------------------------------
constexpr int kRopeRows = 2;  // token rows per workgroup (2 measured fastest of 1, 2, 4, 8, 16)

// (cos, sin) of the angle, or of its negation for the transpose (inverse)
// rotation that carries gradients back through the RoPE.
template <bool kInverse>
__device__ __forceinline__ float2 rot(float2 t) {
  if constexpr (kInverse) t.y = -t.y;
  return t;
}

template <typename T, bool kInverse>
__global__ __launch_bounds__(1024) void rope2d_kernel(T* __restrict__ q, T* __restrict__ k, int32_t L, int32_t T0,
                                                      int32_t N, int32_t W, int32_t lr_w, int32_t rho, int32_t heads,
                                                      int32_t D, const int32_t* __restrict__ perm,
                                                      const int32_t* __restrict__ lr_perm,
                                                      const float2* __restrict__ cs) {
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte vector (8 bf16 or 4 fp32)
  const int32_t units_per_head = D / E;
  const int32_t units = heads * units_per_head;
  const int32_t rows = L - T0;  // HR + LR rows
  const int32_t rr0 = blockIdx.x * kRopeRows;
  const int64_t boff = int64_t(blockIdx.y) * L * units;
  u32x4* const qv = reinterpret_cast<u32x4*>(q) + boff;
  u32x4* const kv = reinterpret_cast<u32x4*>(k) + boff;
  // (row, column) positions of this workgroup's rows
  int32_t pr[kRopeRows], pc[kRopeRows];
#pragma unroll
  for (int r = 0; r < kRopeRows; ++r) {
    const int32_t rr = min(rr0 + r, rows - 1);
    if (rr < N) {
      const int32_t idx = perm[rr];
      pr[r] = idx / W;
      pc[r] = idx - pr[r] * W;
    } else {
      const int32_t i = lr_perm ? lr_perm[rr - N] : rr - N;  // raster LR index
      const int32_t m = i / lr_w;
      pr[r] = rho * m;
      pc[r] = rho * (i - m * lr_w);
    }
  }
  for (int32_t c = threadIdx.x; c < units; c += blockDim.x) {
    const int32_t e0 = (c % units_per_head) * E;  // first dim of this vector
    const bool col = e0 >= D / 2;
    const int32_t k0 = (col ? e0 - D / 2 : e0) / 2;  // first pair index
    u32x4 qa[kRopeRows], ka[kRopeRows];
#pragma unroll
    for (int r = 0; r < kRopeRows; ++r) {
      if (rr0 + r < rows) {
        const int64_t off = int64_t(T0 + rr0 + r) * units + c;
        qa[r] = __builtin_nontemporal_load(qv + off);
        ka[r] = __builtin_nontemporal_load(kv + off);
      }
    }
#pragma unroll
    for (int r = 0; r < kRopeRows; ++r) {
      if (rr0 + r >= rows) continue;
      const float2* tab = cs + int64_t(col ? pc[r] : pr[r]) * (D / 4) + k0;
      if constexpr (std::is_same<T, float>::value) {
        float* x = reinterpret_cast<float*>(&qa[r]);
        float* y = reinterpret_cast<float*>(&ka[r]);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const float2 t = rot<kInverse>(tab[p]);
          const float a = x[2 * p], b = x[2 * p + 1];
          x[2 * p] = a * t.x - b * t.y;
          x[2 * p + 1] = a * t.y + b * t.x;
          const float a2 = y[2 * p], b2 = y[2 * p + 1];
          y[2 * p] = a2 * t.x - b2 * t.y;
          y[2 * p + 1] = a2 * t.y + b2 * t.x;
        }
      } else {
        bf16x8 x = *reinterpret_cast<bf16x8*>(&qa[r]);
        bf16x8 y = *reinterpret_cast<bf16x8*>(&ka[r]);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float2 t = rot<kInverse>(tab[p]);
          const float a = float(x[2 * p]), b = float(x[2 * p + 1]);
          x[2 * p] = __bf16(a * t.x - b * t.y);
          x[2 * p + 1] = __bf16(a * t.y + b * t.x);
          const float a2 = float(y[2 * p]), b2 = float(y[2 * p + 1]);
          y[2 * p] = __bf16(a2 * t.x - b2 * t.y);
          y[2 * p + 1] = __bf16(a2 * t.y + b2 * t.x);
        }
        qa[r] = *reinterpret_cast<u32x4*>(&x);
        ka[r] = *reinterpret_cast<u32x4*>(&y);
      }
      const int64_t off = int64_t(T0 + rr0 + r) * units + c;
      __builtin_nontemporal_store(qa[r], qv + off);
      __builtin_nontemporal_store(ka[r], kv + off);
    }
  }
}

// ---------------------------------------------------------------------------
// Fused window-first permutation + 2D axial RoPE of Q and K, and its
// transpose for the gradients.
//   forward (kBwd false): permuted row j reads raster row T0 + perm[j - T0]
//     (HR; LR through lr_perm) and rotates it by the position of that raster
//     row;
//   backward (kBwd true): raster row j reads permuted row T0 + inv[j - T0]
//     (HR; LR through lr_inv) and applies the transposed rotation of raster
//     row j's position.
// HR and LR rows are rotated exactly as rope2d_kernel does (same table, same
// fp32 arithmetic), so the result is bit-identical to permute followed by
// rope2d, or to rope2d's transpose followed by unpermute; text rows are
// copied.  One read and one write of Q and K instead of two of each.
// ---------------------------------------------------------------------------
template <typename T, bool kBwd>
__global__ __launch_bounds__(1024) void permute_rope_kernel(const T* __restrict__ qsrc, const T* __restrict__ ksrc,
                                                            T* __restrict__ qdst, T* __restrict__ kdst, int32_t L,
                                                            int32_t T0, int32_t N, int32_t W, int32_t lr_w,
                                                            int32_t rho, int32_t heads, int32_t D,
                                                            const int32_t* __restrict__ tab_hr,
                                                            const int32_t* __restrict__ tab_lr,
                                                            const float2* __restrict__ cs) {
  constexpr int E = 16 / sizeof(T);
  const int32_t units_per_head = D / E;
  const int32_t units = heads * units_per_head;
  const int32_t j0 = blockIdx.x * kRopeRows;
  const int64_t boff = int64_t(blockIdx.y) * L * units;
  const u32x4* const qs = reinterpret_cast<const u32x4*>(qsrc) + boff;
  const u32x4* const ks = reinterpret_cast<const u32x4*>(ksrc) + boff;
  u32x4* const qd = reinterpret_cast<u32x4*>(qdst) + boff;
  u32x4* const kd = reinterpret_cast<u32x4*>(kdst) + boff;
  int32_t src[kRopeRows], pr[kRopeRows], pc[kRopeRows];
#pragma unroll
  for (int r = 0; r < kRopeRows; ++r) {
    const int32_t j = min(j0 + r, L - 1);
    src[r] = j;
    pr[r] = -1;  // text: not rotated
    pc[r] = 0;
    if (j >= T0 && j < T0 + N) {
      const int32_t t = tab_hr[j - T0];
      UG_CHECK(t >= 0 && t < N, 4);
      const int32_t idx = kBwd ? j - T0 : t;  // raster HR index of the rotated row
      src[r] = T0 + t;
      pr[r] = idx / W;
      pc[r] = idx - pr[r] * W;
    } else if (j >= T0 + N) {
      const int32_t li = j - T0 - N;
      const int32_t t = tab_lr ? tab_lr[li] : li;
      UG_CHECK(t >= 0 && t < L - T0 - N, 4);
      const int32_t i = kBwd ? li : t;  // raster LR index of the rotated row
      src[r] = T0 + N + t;
      const int32_t m = i / lr_w;
      pr[r] = rho * m;
      pc[r] = rho * (i - m * lr_w);
    }
  }
  for (int32_t c = threadIdx.x; c < units; c += blockDim.x) {
    const int32_t e0 = (c % units_per_head) * E;
    const bool col = e0 >= D / 2;
    const int32_t k0 = (col ? e0 - D / 2 : e0) / 2;
    u32x4 qa[kRopeRows], ka[kRopeRows];
#pragma unroll
    for (int r = 0; r < kRopeRows; ++r) {
      if (j0 + r < L) {
        qa[r] = __builtin_nontemporal_load(qs + int64_t(src[r]) * units + c);
        ka[r] = __builtin_nontemporal_load(ks + int64_t(src[r]) * units + c);
      }
    }
#pragma unroll
    for (int r = 0; r < kRopeRows; ++r) {
      if (j0 + r >= L) continue;
      if (pr[r] >= 0) {
        const float2* tab = cs + int64_t(col ? pc[r] : pr[r]) * (D / 4) + k0;
        if constexpr (std::is_same<T, float>::value) {
          float* x = reinterpret_cast<float*>(&qa[r]);
          float* y = reinterpret_cast<float*>(&ka[r]);
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const float2 t = rot<kBwd>(tab[p]);
            const float a = x[2 * p], b = x[2 * p + 1];
            x[2 * p] = a * t.x - b * t.y;
            x[2 * p + 1] = a * t.y + b * t.x;
            const float a2 = y[2 * p], b2 = y[2 * p + 1];
            y[2 * p] = a2 * t.x - b2 * t.y;
            y[2 * p + 1] = a2 * t.y + b2 * t.x;
          }
        } else {
          bf16x8 x = *reinterpret_cast<bf16x8*>(&qa[r]);
          bf16x8 y = *reinterpret_cast<bf16x8*>(&ka[r]);
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const float2 t = rot<kBwd>(tab[p]);
            const float a = float(x[2 * p]), b = float(x[2 * p + 1]);
            x[2 * p] = __bf16(a * t.x - b * t.y);
            x[2 * p + 1] = __bf16(a * t.y + b * t.x);
            const float a2 = float(y[2 * p]), b2 = float(y[2 * p + 1]);
            y[2 * p] = __bf16(a2 * t.x - b2 * t.y);
            y[2 * p + 1] = __bf16(a2 * t.y + b2 * t.x);
          }
          qa[r] = *reinterpret_cast<u32x4*>(&x);
          ka[r] = *reinterpret_cast<u32x4*>(&y);
        }
      }
      const int64_t off = int64_t(j0 + r) * units + c;
      __builtin_nontemporal_store(qa[r], qd + off);
      __builtin_nontemporal_store(ka[r], kd + off);
    }
  }
}

// ---------------------------------------------------------------------------
// Composite-masked attention forward (关键设计 3 with the mask of 关键设计 2).
//
// One workgroup = one query tile (<= 256 permuted rows sharing one key set)
// of one (batch, head); 8 waves x 32 queries, two waves per SIMD.  The key
// set is a list of contiguous row ranges, walked in 64-key tiles that go
// straight from global memory into LDS (buffer_load_dwordx4 ... lds, no
// registers), one barrier per tile.
//
// Per wave and 64-key tile, with 32x32 MFMA tiles (lane l: column l%32,
// lane half g = l/32):
//   S^T = K Q^T    A = K rows from LDS, B = the wave's Q held in registers.
//                  Output lane l holds query l%32 and 16 keys
//                  8*(j/4) + 4*g + j%4 (j < 16) of each 32-key block, so a
//                  query's softmax statistics are lane-local except for one
//                  exchange between the two lane halves (v_permlane32_swap).
//   P = exp2(S*scale*log2e - m), m a softmax reference (fp32, log2 units).
//   O^T += V^T P^T A = V^T read from the [key][dim] V tile with the LDS
//                  transpose read ds_read_b64_tr_b16: in each 16-lane group,
//                  lane j gets dim j of four keys, so two reads give a lane
//                  the 8 keys its own S^T registers hold (keys 4g..4g+3 and
//                  8+4g..8+4g+3 of a 16-key chunk): B = P^T straight from
//                  the S^T registers, no shuffles.
// LDS rows are unpadded; 16-byte chunks are XOR-swizzled by row so the
// K-operand reads (32 rows, one chunk) and the transpose reads (4 rows,
// 64 bytes) are bank-conflict free.
//
// bf16 (v_mfma_f32_32x32x16_bf16), attn_item_bf16: a three-stage software
// pipeline.  Step i runs QK^T of tile i+1, the exponentials of tile i and PV
// of tile i-1 side by side, as one MFMA per slot with one or two weights of
// tile i per slot, so the VALU work is spread evenly over every MFMA (VALU
// instructions next to MFMAs cost MFMA time once a slot holds more than a
// few).  The softmax reference is not a running maximum: it starts 8 above
// the first tile's exact maximum and only moves when a later tile could hold
// large weights, which the row sum detects exactly: a lane's partial sum of
// its 32 weights of a tile is below 2^8 only if every weight is.  When some
// lane's partial sum reaches 2^8, the reference moves up by a whole number
// of octaves (so the rescaling of what was accumulated is exact), to 8 above
// the tile's maximum, and the tile's weights are recomputed before the next
// step uses them.  P is rounded to bf16 for the PV product, and the row sum
// is taken over the same rounded weights.
// fp32 (v_mfma_f32_32x32x2_f32), attn_item_f32: a two-stage pipeline (QK^T
// of tile i+1 beside the exponentials of tile i, then PV of tile i beside the
// maximum of tile i+1) with a running maximum moved only when a tile's
// maximum exceeds it by more than 8.
// The output goes through LDS so every row is written with full 16-byte
// stores.
// Persistent grid: one workgroup per CU takes query tiles from the plan's
// eight per-XCD queues (the workgroup order, XCD x's queue at items x,
// x + 8, ...) through an atomic cursor per queue, its own XCD's queue first,
// then the others'.  The XCDs run at different speeds (up to 4% per tile on
// the same work) and the hardware dispatches workgroups to them in lockstep,
// so a static one-tile-per-workgroup grid leaves CUs idle between tiles and
// at the end; taking tiles dynamically keeps every CU busy until the queues
// are empty.
// ---------------------------------------------------------------------------
constexpr int kAttnThreads = 512;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kKT = ug::kAttnKeyTile;  // 64

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t row_stride;    // elements between consecutive rows (Hh*D)
  int64_t batch_stride;  // elements between consecutive batches (L*Hh*D)
  int32_t heads;
  int32_t pad;
  const ug::Task* tasks;
  const ug::Range* ranges;
  const ug::Block* blocks;
  // the bf16 kernel's view of blocks[], read with uniform (scalar) loads
  // (load_item)
  __attribute__((address_space(4))) const ug::AttnItem* items;
  int32_t qlen[ug::kXcds];    // items of each XCD queue before its padding
  float scale_log2;      // log2(e) / sqrt(D)
  int32_t T, N;          // text rows, HR rows
  const int32_t* out_perm;     // non-null: write HR output row T+i to raster row T+out_perm[i]
  const int32_t* out_lr_perm;  // non-null (with out_perm): LR row T+N+i to T+N+out_lr_perm[i]
  float* lse;                  // non-null: natural-log LSE of each row, [batch*heads][lse_rows]
  int64_t lse_rows;
  int32_t* queue;     // this launch's cursor slot: 8 per-XCD queue cursors, then the finished-workgroup count
  int32_t queue_len;  // items per XCD queue (blocks / 8)
  int32_t L, n_tasks, n_bh;  // rows, tasks and batch*heads (index checks of the debug build)
};


template <typename T, int D>
struct AttnLds {
  static constexpr bool kBF = std::is_same<T, __bf16>::value;
  static constexpr int kEl16 = 16 / int(sizeof(T));  // elements per 16-B chunk
  static constexpr int kChunks = D / kEl16;           // chunks per row
  static_assert(kChunks == 8 || kChunks == 16 || kChunks == 32, "row must be 8, 16 or 32 chunks");
  static constexpr int kTileBytes = kKT * D * int(sizeof(T));
  static constexpr int kSlots = kTileBytes / 16;      // 16-B slots per tile
  static constexpr int kLoadsPerThread = kSlots / kAttnThreads;
  static_assert(kSlots % kAttnThreads == 0, "tile must split evenly over the workgroup");
  // K ring (2 tiles) + V ring (2 tiles); bf16 adds the prologue region
  // (the next item's K_0 and K_1)
  static constexpr int kTotalBytes = (kBF ? 6 : 4) * kTileBytes;
  static_assert(kAttnWaves * 32 * D * int(sizeof(T)) <= kTotalBytes, "output staging must fit");
  // physical chunk of logical chunk c in row r
  __device__ static __forceinline__ int k_swz(int r) {  // 16 consecutive rows -> 16 bank groups
    if constexpr (kChunks >= 16) return r & 15;
    else return (r >> 1) & 7;
  }
  __device__ static __forceinline__ int v_swz(int r) {  // 4 consecutive rows x 4 chunks -> 16 bank groups
    if constexpr (kChunks >= 16) return 4 * (r & 3);
    else return 4 * ((r >> 1) & 1);
  }
};



// Direct global->LDS loads of one 64-key tile (rows ks .. ks+63).  Slot
// s = i*512 + tid of the tile holds row s / kChunks, physical chunk
// s % kChunks, i.e. logical chunk (s % kChunks) ^ swz(row).  `off[i]` is the
// thread's byte offset of that chunk relative to row ks (constant over
// tiles).  The buffer descriptor covers the nv valid rows only, so in a
// ragged tile (nv < 64) the rows past the range read as zeros (their scores
// are masked and their P is 0) and no load leaves the key range; nv <= 0
// loads nothing but zeros.  The issue is branch-free.
template <typename T, int D, bool kIsV>
struct TileLoader {
  using Lds = AttnLds<T, D>;
  uint32_t off[Lds::kLoadsPerThread];
  __device__ __forceinline__ static int row_of(int i, int tid) { return (i * kAttnThreads + tid) / Lds::kChunks; }
  __device__ __forceinline__ static int lchunk_of(int i, int tid) {
    const int slot = i * kAttnThreads + tid;
    const int r = slot / Lds::kChunks;
    return (slot % Lds::kChunks) ^ (kIsV ? Lds::v_swz(r) : Lds::k_swz(r));
  }
  __device__ __forceinline__ void init(int64_t rs, int tid) {
#pragma unroll
    for (int i = 0; i < Lds::kLoadsPerThread; ++i)
      off[i] = uint32_t(row_of(i, tid) * rs * int64_t(sizeof(T)) + lchunk_of(i, tid) * 16);
  }
  __device__ __forceinline__ void issue(const T* __restrict__ src, int64_t rs, int32_t ks, int32_t nv, char* tile,
                                        int tid, int wave) const {
    const char* base = reinterpret_cast<const char*>(src + int64_t(ks) * rs);  // wave-uniform
    // uniform by construction; readfirstlane keeps the descriptor in scalar registers
    const int32_t bytes = __builtin_amdgcn_readfirstlane(max(nv, 0) * int32_t(rs) * int32_t(sizeof(T)));
#pragma unroll
    for (int i = 0; i < Lds::kLoadsPerThread; ++i)
      load_lds<16>(base, off[i], (lds_void*)(tile + (i * kAttnThreads + wave * 64) * 16), bytes);
    (void)tid;
  }
  // The thread's i-th 16-byte load of the tile at `base` (bytes as above).
  __device__ __forceinline__ void issue_one(int i, const char* base, int32_t bytes, char* tile, int wave) const {
    load_lds<16>(base, off[i], (lds_void*)(tile + (i * kAttnThreads + wave * 64) * 16), bytes);
  }
};

// S^T (two 32-key blocks) = K Q^T for one 64-key tile in LDS.  koff[i] is
// the lane's byte offset of its chunk for MFMA step i in row l%32.
template <typename T, int D, typename QReg, int KOFF>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[2], const char* ktile, const QReg* qf, const int (&koff)[KOFF]) {
  using Lds = AttnLds<T, D>;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const char* kb = ktile + mb * 32 * D * int(sizeof(T));
    if constexpr (Lds::kBF) {
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kb + koff[0]), qf[0],
                                                      f32x16{}, 0, 0, 0);
#pragma unroll
      for (int i = 1; i < D / 16; ++i)
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kb + koff[i]), qf[i],
                                                        s[mb], 0, 0, 0);
    } else {
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(*reinterpret_cast<const float*>(kb + koff[0]), qf[0], f32x16{},
                                                   0, 0, 0);
#pragma unroll
      for (int i = 1; i < D / 2; ++i)
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(*reinterpret_cast<const float*>(kb + koff[i]), qf[i], s[mb], 0,
                                                     0, 0);
    }
  }
}

typedef __attribute__((address_space(4))) const AttnParams* KArgs;
__device__ __forceinline__ KArgs kernel_args() { return opaque_args<AttnParams>(); }

// Work item `idx`'s record, by uniform loads through the constant address
// space (scalar loads: the index is wave-uniform).
__device__ __forceinline__ ug::AttnItem load_item(KArgs kp, int32_t idx) {
  typedef __attribute__((address_space(4))) const int32_t* CInt;
  const CInt src = reinterpret_cast<CInt>(kp->items + idx);
  ug::AttnItem r;
  int32_t* dst = reinterpret_cast<int32_t*>(&r);
#pragma unroll
  for (int k = 0; k < int(sizeof(ug::AttnItem) / 4); ++k) dst[k] = src[k];
  return r;
}

// One fp32 query tile (plan item `item`) of the attention.
template <int D>
__device__ __forceinline__ void attn_item_f32(KArgs kp, int32_t item, char* smem, ug::Range* s_rng) {
  using T = float;
  using Lds = AttnLds<T, D>;
  constexpr int TB = Lds::kTileBytes;
  // K ring at [0, 2*TB), V ring at [2*TB, 4*TB)

  UG_CHECK(item >= 0 && item < kp->queue_len * ug::kXcds, 0);
  const ug::Block blk = kp->blocks[item];
  UG_CHECK(blk.task >= 0 && blk.task < kp->n_tasks && blk.bh >= 0 && blk.bh < kp->n_bh, 0);
  const ug::Task task = kp->tasks[blk.task];
  UG_CHECK(task.q0 >= 0 && task.q0 < task.q1 && task.q1 <= kp->L && task.q1 - task.q0 <= ug::kAttnQueryTile, 1);
  const int32_t b = blk.bh / kp->heads, h = blk.bh - b * kp->heads;
  const int64_t hoff = int64_t(b) * kp->batch_stride + int64_t(h) * D;
  const T* __restrict__ qg = static_cast<const T*>(kp->q) + hoff;
  const T* __restrict__ kg = static_cast<const T*>(kp->k) + hoff;
  const T* __restrict__ vg = static_cast<const T*>(kp->v) + hoff;
  T* __restrict__ og = static_cast<T*>(kp->o) + hoff;
  const int64_t rs = kp->row_stride;

  const int tid = opaque_tid<kAttnThreads>();
  // wave index in a scalar register (the opaque tid hides that it is uniform),
  // masked so that alias analysis keeps its range
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (kAttnWaves - 1);
  const int l32 = lane & 31, g = lane >> 5;
  const int32_t qrow = task.q0 + wave * 32 + l32;
  const int32_t qload = qrow < task.q1 ? qrow : task.q1 - 1;
  const float c2 = kp->scale_log2;

  // The task's key ranges (at most ug::kAttnMaxRanges, checked at launch)
  // are staged in LDS (s_rng), so moving to the next range inside the tile
  // loop is an LDS read rather than a global load that would wait on the tile
  // loads in flight.
  const int32_t nr = task.r1 - task.r0;
  UG_CHECK(nr >= 1 && nr <= ug::kAttnMaxRanges, 1);
  if (tid < nr) {
    const ug::Range r = kp->ranges[task.r0 + tid];
    UG_CHECK(r.k0 >= 0 && r.k0 < r.k1 && r.k1 <= kp->L, 1);
    s_rng[tid] = r;
  }

  // The wave's queries as the B operand of S^T = K Q^T.
  constexpr int kQRegs = D / 2;
  float qf[kQRegs];
#pragma unroll
  for (int i = 0; i < kQRegs; ++i) qf[i] = qg[qload * rs + 2 * i + g];
  __syncthreads();  // s_rng is filled

  // number of 64-key tiles
  int32_t ntiles = 0;
  for (int32_t r = 0; r < nr; ++r) {
    const ug::Range rg = s_rng[r];
    ntiles += (rg.k1 - rg.k0 + kKT - 1) / kKT;
  }
  ntiles = __builtin_amdgcn_readfirstlane(ntiles);  // uniform: it feeds scalar buffer descriptors

  // Per-lane LDS byte offsets.  K operand of step i: row l32 (plus 32 per
  // block), element 2i + g.
  constexpr int RB = D * int(sizeof(T));  // bytes per LDS row
  int koff[kQRegs];
#pragma unroll
  for (int i = 0; i < kQRegs; ++i) {
    const int e = 2 * i + g;
    koff[i] = l32 * RB + (((e / 4) ^ Lds::k_swz(l32)) * 16) + (e % 4) * 4;
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
  float m2 = -INFINITY;  // running maximum, in log2 units (scaled)
  float lsum = 0.f;      // this lane half's share of the row sum

  TileCursor ck, cv;  // next K tile to load, next V tile to load
  ck.init(s_rng, 0, nr);
  cv = ck;
  TileLoader<T, D, false> kld;
  TileLoader<T, D, true> vld;
  kld.init(rs, tid);
  vld.init(rs, tid);

  // Scores of a freshly computed tile: mask a ragged tail (rare, uniform
  // branch) and return the tile maximum (both lane halves agree).
  auto mask_tail = [&](f32x16(&s)[2], int32_t nv) {
    const int lim = nv - 4 * g;  // key 8*(j/4) + 4g + j%4 of block mb is valid iff its offset < lim
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (mb * 32 + 8 * (j >> 2) + (j & 3) >= lim) s[mb][j] = -INFINITY;
  };
  auto tile_max = [&](const f32x16(&s)[2]) {
    float mx = s[0][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[mb][j]);
    return pair_max(mx);
  };
  // Move the running maximum when the new tile's maximum exceeds it by more
  // than 2^8 (log2 units), rescaling what has been accumulated so far.
  auto update_max = [&](float mx, bool valid) {
    const float mt = mx * c2;
    const bool need = valid && mt > m2 + 8.0f;
    if (__ballot(need)) {
      const float mnew = need ? mt : m2;
      const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
      m2 = mnew;
      lsum *= alpha;
#pragma unroll
      for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
    }
  };

  // prologue: K_0 -> K slot 0, K_1 -> K slot 1, V_0 -> V slot 0; S_0
  kld.issue(kg, rs, ck.ks, ck.nv(), smem, tid, wave);
  vld.issue(vg, rs, cv.ks, cv.nv(), smem + 2 * TB, tid, wave);
  const int32_t nv_cur = cv.nv();
  ck.advance(s_rng);
  cv.advance(s_rng);
  if (ntiles > 1) {
    kld.issue(kg, rs, ck.ks, ck.nv(), smem + TB, tid, wave);
    ck.advance(s_rng);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 sa[2], sb[2];
  qk_tile<T, D>(sa, smem, qf, koff);
  if (nv_cur < kKT) mask_tail(sa, nv_cur);
  update_max(tile_max(sa), true);
  __syncthreads();  // step 0 overwrites K slot 0 with K_2

  // One pipeline step on tile i, whose scores s_cur are masked and whose
  // maximum is already folded into m2:
  //   [A] exponentials of tile i (VALU)  ||  QK^T of tile i+1 (MFMA)
  //   [B] PV of tile i (MFMA)            ||  maximum of tile i+1 (VALU)
  // then the rare paths (ragged tail of tile i+1, moving the maximum).
  // PAR = i & 1 selects the ring slots at compile time.
  auto step = [&](int32_t i, auto par, f32x16(&s_cur)[2], f32x16(&s_next)[2]) {
    constexpr int PAR = decltype(par)::value;
    char* const k_next = smem + (PAR ? 0 : TB);            // holds K_{i+1}
    char* const v_cur = smem + 2 * TB + (PAR ? TB : 0);    // holds V_i
    const bool has_k = i + 2 < ntiles;
    const bool has_v = i + 1 < ntiles;
    const int32_t nv_next = has_v ? cv.nv() : kKT;
    if (has_k) {  // K_{i+2} replaces K_i
      kld.issue(kg, rs, ck.ks, ck.nv(), smem + (PAR ? TB : 0), tid, wave);
      ck.advance(s_rng);
    }
    if (has_v) {  // V_{i+1} replaces V_{i-1}
      vld.issue(vg, rs, cv.ks, nv_next, smem + 2 * TB + (PAR ? 0 : TB), tid, wave);
      cv.advance(s_rng);
    }

#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        s_cur[mb][j] = __builtin_amdgcn_exp2f(fmaf(s_cur[mb][j], c2, -m2));
        lsum += s_cur[mb][j];
      }
    qk_tile<T, D>(s_next, k_next, qf, koff);
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = mb * 32 + 8 * (j >> 2) + 4 * g + (j & 3);
          const int dim = 32 * t + l32;
          const float vv = *reinterpret_cast<const float*>(v_cur + key * RB +
                                                           (((dim / 4) ^ Lds::v_swz(key)) * 16) + (dim % 4) * 4);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv, s_cur[mb][j], acc[t], 0, 0, 0);
        }
    if (nv_next < kKT) mask_tail(s_next, nv_next);
    update_max(tile_max(s_next), has_v);

    __builtin_amdgcn_s_waitcnt(0);  // this thread's direct-to-LDS loads have landed
    __syncthreads();
  };

  for (int32_t i = 0; i < ntiles; i += 2) {
    step(i, std::integral_constant<int, 0>{}, sa, sb);
    if (i + 1 >= ntiles) break;
    step(i + 1, std::integral_constant<int, 1>{}, sb, sa);
  }

  // ---- epilogue: combine the lane halves' row sums, normalise, and write
  // the wave's 32 x D output block through LDS (swizzled rows) as full rows.
  kp = kernel_args();  // the epilogue's arguments are loaded here, not kept across the loop
  const float total = pair_sum(lsum);
  const float inv = 1.0f / total;
  UG_CHECK(!(kp->lse && g == 0 && qrow < task.q1) || qrow < kp->lse_rows, 3);
  if (kp->lse && g == 0 && qrow < task.q1)  // log(sum_j exp(s_j)) = (m2 + log2(total)) * ln 2
    kp->lse[int64_t(blk.bh) * kp->lse_rows + qrow] = (m2 + __log2f(total)) * 0.6931471805599453f;
  char* const ost = smem + wave * 32 * RB;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = t * 32 + 8 * q4 + 4 * g;  // 4 consecutive dims
      char* dst = ost + l32 * RB + (((d0 / Lds::kEl16) ^ Lds::k_swz(l32)) * 16) + (d0 % Lds::kEl16) * int(sizeof(T));
      *reinterpret_cast<float4*>(dst) = make_float4(acc[t][4 * q4 + 0] * inv, acc[t][4 * q4 + 1] * inv,
                                                    acc[t][4 * q4 + 2] * inv, acc[t][4 * q4 + 3] * inv);
    }
  // each wave reads back only its own block: LDS operations of one wave
  // complete in order, so no barrier is needed between the write and read.
  constexpr int rows_per_pass = 64 / Lds::kChunks;
  constexpr int kPasses = 32 / rows_per_pass;
  // Destination rows first, as branch-free table reads (rows past the tile
  // are clamped for the lookup and skipped at the store), so that all the
  // lookups are in flight together.
  int32_t orow[kPasses];
  if (kp->out_perm) {  // uniform
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
      const int32_t row = min(task.q0 + wave * 32 + pass * rows_per_pass + lane / Lds::kChunks, task.q1 - 1);
      const bool hr = row >= kp->T && row < kp->T + kp->N;
      const bool lr = row >= kp->T + kp->N && kp->out_lr_perm != nullptr;
      const int32_t* tab = lr ? kp->out_lr_perm : kp->out_perm;
      const int32_t idx = hr ? row - kp->T : lr ? row - kp->T - kp->N : 0;
      const int32_t v = tab[idx];
      orow[pass] = hr ? kp->T + v : lr ? kp->T + kp->N + v : row;
    }
  } else {
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass)
      orow[pass] = task.q0 + wave * 32 + pass * rows_per_pass + lane / Lds::kChunks;
  }
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int r = pass * rows_per_pass + lane / Lds::kChunks;
    const int cc = lane % Lds::kChunks;
    const uint4 val = *reinterpret_cast<const uint4*>(ost + r * RB + ((cc ^ Lds::k_swz(r)) * 16));
    if (task.q0 + wave * 32 + r < task.q1) {
      UG_CHECK(orow[pass] >= 0 && orow[pass] < kp->L, 3);
      *reinterpret_cast<uint4*>(og + int64_t(orow[pass]) * rs + cc * Lds::kEl16) = val;
    }
  }
}


// The next item's loads, issued before the item starts (at the kernel's
// start, and in the previous item's epilogue): its first two K tiles into
// the prologue region (K_0 at 4*TB, K_1 at 5*TB) and its key ranges into
// s_rng (wave 0, by direct-to-LDS dword loads; rows past the item's ranges
// read as zeros and are never used) ...
template <int D>
__device__ __forceinline__ void prefetch_keys(KArgs kp, const ug::AttnItem& it, char* smem, ug::Range* s_rng, int tid,
                                              int wave, int lane) {
  using T = __bf16;
  using Lds = AttnLds<T, D>;
  constexpr int TB = Lds::kTileBytes;
  UG_CHECK(it.bh >= 0 && it.bh < kp->n_bh && it.nr >= 1 && it.nr <= ug::kAttnMaxRanges, 0);
  UG_CHECK(it.ks0 >= 0 && it.nv0 >= 1 && it.nv0 <= kKT && it.ks0 + it.nv0 <= kp->L, 2);
  UG_CHECK(it.ks1 >= 0 && it.nv1 >= 0 && it.nv1 <= kKT && it.ks1 + it.nv1 <= kp->L, 2);
  const int32_t b = it.bh / kp->heads, h = it.bh - b * kp->heads;
  const int64_t rs = kp->row_stride;
  const T* __restrict__ kg = static_cast<const T*>(kp->k) + int64_t(b) * kp->batch_stride + int64_t(h) * D;
  TileLoader<T, D, false> kld;
  kld.init(rs, tid);
  kld.issue(kg, rs, it.ks0, it.nv0, smem + 4 * TB, tid, wave);
  kld.issue(kg, rs, it.ks1, it.nv1, smem + 5 * TB, tid, wave);
  if (wave == 0) {
    static_assert(ug::kAttnMaxRanges * sizeof(ug::Range) == 2 * 64 * 4, "two dword loads per lane stage the ranges");
    const char* rbase = reinterpret_cast<const char*>(kp->ranges + it.r0);
    const int32_t bytes = it.nr * int32_t(sizeof(ug::Range));
    load_lds<4>(rbase, uint32_t(4 * lane), (lds_void*)s_rng, bytes);
    load_lds<4>(rbase, uint32_t(256 + 4 * lane), (lds_void*)(reinterpret_cast<char*>(s_rng) + 256), bytes);
  }
}

// ... and each wave's 32 query rows into its own 32-row block of the K/V ring
// area (the block its output is staged in), with the K tiles' chunk swizzle,
// so the prologue reads the Q operand from LDS.  Rows past the item's end
// read as zeros (their outputs are never stored).
template <int D>
__device__ __forceinline__ void prefetch_queries(KArgs kp, const ug::AttnItem& it, char* smem, int wave, int lane) {
  using T = __bf16;
  using Lds = AttnLds<T, D>;
  constexpr int RB = D * 2;
  constexpr int kLoads = 32 * RB / 1024;  // 1 KB (64 lanes x 16 B) per load
  const int32_t b = it.bh / kp->heads, h = it.bh - b * kp->heads;
  const int64_t rs = kp->row_stride;
  const int32_t row0 = it.q0 + wave * 32;
  UG_CHECK(it.q0 >= 0 && it.q0 < it.q1 && it.q1 <= kp->L && it.q1 - it.q0 <= ug::kAttnQueryTile, 1);
  const T* __restrict__ qg = static_cast<const T*>(kp->q) + int64_t(b) * kp->batch_stride + int64_t(h) * D;
  const char* base = reinterpret_cast<const char*>(qg + int64_t(min(row0, it.q1)) * rs);
  const int32_t bytes =
      __builtin_amdgcn_readfirstlane(min(max(it.q1 - row0, 0), 32) * int32_t(rs) * int32_t(sizeof(T)));
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int slot = i * 64 + lane;
    const int r = slot / Lds::kChunks;
    const int lc = (slot % Lds::kChunks) ^ Lds::k_swz(r);
    load_lds<16>(base, uint32_t(r * rs * int64_t(sizeof(T)) + lc * 16), (lds_void*)(smem + wave * 32 * RB + i * 1024),
                 bytes);
  }
}

// One bf16 query tile (work item `it`) of the attention: the three-stage
// pipeline described above.  On entry the item's key ranges are in s_rng,
// its first two K tiles in the prologue region and each wave's queries in
// its block of the ring area (prefetch_keys, prefetch_queries); the
// epilogue publishes the next item in s_next_idx and issues its loads.
template <int D>
__device__ __forceinline__ void attn_item_bf16(KArgs kp, const ug::AttnItem& it, char* smem, ug::Range* s_rng,
                                               int32_t* s_next_idx) {
  using T = __bf16;
  using Lds = AttnLds<T, D>;
  constexpr int TB = Lds::kTileBytes;
  constexpr int kQRegs = D / 16;    // k-steps of one QK^T block
  constexpr int RB = D * 2;         // bytes per LDS row
  constexpr int kHalfSlots = D / 8;  // QK^T MFMAs (= PV MFMAs) per tile
  constexpr int kSlots = 2 * kHalfSlots;
  constexpr int kExpPerSlot = 32 / kSlots;  // weights of the lane's 32 per slot
  constexpr int kLead = 4;                  // operand reads run this many slots ahead
  constexpr float kHeadroom = 8.0f;         // octaves between the reference and the largest weight seen
  static_assert(kSlots * kExpPerSlot == 32, "32 weights per lane and tile");

  UG_CHECK(it.bh >= 0 && it.bh < kp->n_bh, 0);
  UG_CHECK(it.q0 >= 0 && it.q0 < it.q1 && it.q1 <= kp->L && it.q1 - it.q0 <= ug::kAttnQueryTile, 1);
  UG_CHECK(it.nr >= 1 && it.nr <= ug::kAttnMaxRanges && it.ntiles >= 1, 1);
  const int32_t b = it.bh / kp->heads, h = it.bh - b * kp->heads;
  const int64_t hoff = int64_t(b) * kp->batch_stride + int64_t(h) * D;
  const T* __restrict__ kg = static_cast<const T*>(kp->k) + hoff;
  const T* __restrict__ vg = static_cast<const T*>(kp->v) + hoff;
  T* __restrict__ og = static_cast<T*>(kp->o) + hoff;
  const int64_t rs = kp->row_stride;

  const int tid = opaque_tid<kAttnThreads>();
  // wave index in a scalar register (the opaque tid hides that it is uniform),
  // masked so that alias analysis keeps its range
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (kAttnWaves - 1);
  const int l32 = lane & 31, g = lane >> 5;
  const int32_t qrow = it.q0 + wave * 32 + l32;
  const float c2 = kp->scale_log2;
  const int32_t nr = it.nr;
  const int32_t ntiles = it.ntiles;

  // Per-lane LDS byte offsets.  K operand of k-step i: row l32 (plus 32 per
  // block), logical chunk of dims 16i + 8g.
  int koff[kQRegs];
#pragma unroll
  for (int i = 0; i < kQRegs; ++i) {
    const int lc = 2 * i + g;
    koff[i] = l32 * RB + ((lc ^ Lds::k_swz(l32)) * 16);
  }
  // V^T operand: for dim tile t, the lane's transpose-read address in 16-key
  // chunk c, half hh is row 16c + 8hh + vrow, dims 32t + vdim .. +3.
  const int vrow = 4 * g + ((lane & 15) >> 2);
  const int vdim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int voff[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    const int dim = 32 * t + vdim;
    voff[t] = vrow * RB + (((dim / 8) ^ Lds::v_swz(vrow)) * 16) + (dim % 8) * 2;
  }

  // The wave's queries as the B operand of S^T = K Q^T, from the wave's
  // block of the ring area (same row and chunk layout as a K tile).
  bf16x8 qf[kQRegs];
#pragma unroll
  for (int i = 0; i < kQRegs; ++i) qf[i] = *reinterpret_cast<const bf16x8*>(smem + wave * 32 * RB + koff[i]);

  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
  float mref;        // softmax reference, log2 units of the scaled logits
  float lsum = 0.f;  // this lane half's share of the row sum

  // K_0 and K_1 are already loaded, so the K cursor starts at tile 2.
  TileCursor ck, cv;  // next K tile to load, next V tile to load
  ck.init(s_rng, 0, nr);
  cv = ck;
  ck.advance(s_rng);
  ck.advance(s_rng);
  TileLoader<T, D, false> kld;
  TileLoader<T, D, true> vld;
  kld.init(rs, tid);
  vld.init(rs, tid);

  // Scores of keys past a ragged tile's end are masked.  The empty volatile
  // asm keeps the (rare, uniform) branch a branch.
  auto mask_tail = [&](f32x16(&s)[2], int32_t nv) {
    asm volatile("");
    const int lim = nv - 4 * g;  // key 8*(j/4) + 4g + j%4 of block mb is valid iff its offset < lim
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (mb * 32 + 8 * (j >> 2) + (j & 3) >= lim) s[mb][j] = -INFINITY;
  };
  auto tile_max = [&](const f32x16(&s)[2]) {
    float mx = s[0][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[mb][j]);
    return pair_max(mx);
  };
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  // Weight k (0..31) of the lane's scores of a tile: block k/16, register
  // k%16; weights 2m and 2m+1 form one packed pair of P chunk m/4.  The
  // volatile asm statements pin the work to its slot: without them the
  // compiler gathers it after the MFMAs, where nothing hides it.
  float e_hold = 0.f;
  bf16x2 pr_prev = {};  // the last packed pair, whose row-sum term is still to be added
  // The row sum takes the rounded weights, the ones that multiply V (a
  // dominant weight's rounding then cancels in the normalisation).  At
  // head_dim 128 a pair is split into two fp32 values by two bit operations
  // (a bf16 half moved into the high half of a word is that value) and
  // added; at head_dim 64, where the step has half as many MFMAs to hide
  // VALU work behind, one dot product with (1, 1) adds it, one pair late:
  // between the next pair's exponential and its pack, where it fills the
  // wait states those two would need (at head_dim 128 those waits are hidden
  // behind the MFMAs and the late order measured slower).  `first` starts
  // the sum (d enters as 0).
  constexpr bool kLateSum = D == 64;
  auto sum_pair = [&](float& d, bf16x2 pr, bool first) {
    if constexpr (D == 64) {
      const bf16x2 ones = {__bf16(1.0f), __bf16(1.0f)};
      d = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, first ? 0.0f : d, false);
    } else {
      const uint32_t u = __builtin_bit_cast(uint32_t, pr);
      const float x = __uint_as_float(u << 16) + __uint_as_float(u & 0xffff0000u);
      d = first ? x : d + x;
    }
    asm volatile("" : "+v"(d));
  };
  auto weight = [&](const f32x16(&s)[2], bf16x8(&p)[4], float& d, int k) {
    float e = __builtin_amdgcn_exp2f(fmaf(s[k >> 4][k & 15], c2, -mref));
    if ((k & 1) == 0) {
      e_hold = e;
      asm volatile("" : "+v"(e_hold));
    } else {
      if constexpr (kLateSum) {
        asm volatile("" : "+v"(e));
        if (k >= 3) sum_pair(d, pr_prev, k == 3);
      }
      bf16x2 pr = {__bf16(e_hold), __bf16(e)};
      asm volatile("" : "+v"(pr));
      p[k >> 3][(k & 7) - 1] = pr[0];
      p[k >> 3][k & 7] = pr[1];
      if constexpr (kLateSum) pr_prev = pr;
      else sum_pair(d, pr, k == 1);
    }
  };
  // the last pair's term, once all 32 weights of a tile are formed
  auto sum_last = [&](float& d) {
    if constexpr (kLateSum) sum_pair(d, pr_prev, false);
  };
  auto weights_all = [&](const f32x16(&s)[2], bf16x8(&p)[4], float& d) {
#pragma unroll
    for (int k = 0; k < 32; ++k) weight(s, p, d, k);
    sum_last(d);
  };
  // Some lane's weights of tile s may be large: move the reference up by a
  // whole number of octaves, to kHeadroom above the tile's maximum, rescale
  // what was accumulated (exactly: a power of two) and recompute the tile's
  // weights.  Rare and wave-uniform.
  auto settle = [&](const f32x16(&s)[2], bf16x8(&p)[4], float& d) {
    asm volatile("");
    const float mt = tile_max(s) * c2;
    const float shift = fmaxf(ceilf(mt - mref) + kHeadroom, 0.0f);
    mref += shift;
    const float alpha = __builtin_ldexpf(1.0f, -int(shift));
    lsum *= alpha;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
    d = 0.f;
    weights_all(s, p, d);
  };
  auto pv_all = [&](const bf16x8(&p)[4], const char* vt) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        const char* a0 = vt + voff[t] + (16 * c) * RB;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0 + 8 * RB));
        const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[c], acc[t], 0, 0, 0);
      }
    }
  };

  // prologue: S_0 from K_0 (prologue region); the reference is kHeadroom
  // above tile 0's maximum
  const int32_t nv0 = it.nv0;
  int32_t nv_pend = ntiles > 1 ? it.nv1 : kKT;  // rows of the K tile issued most recently (tile i+1 at step i)
  f32x16 sa[2], sb[2];
  bf16x8 pa[4], pb[4];
  qk_tile<T, D>(sa, smem + 4 * TB, qf, koff);
  if (nv0 < kKT) mask_tail(sa, nv0);
  mref = tile_max(sa) * c2 + kHeadroom;
  __syncthreads();  // step 0's loads overwrite the Q rows of waves 0, 1, 4 and 5 (K slot 0, V slot 0)

  // Loads of step i: K_{i+2} -> K slot i&1 (K_i was read in step i-1),
  // V_i -> V slot i&1 (V_{i-2} was read in step i-1).
  auto issue_loads = [&](int32_t i, int par) {
    int32_t nv = kKT;
    if (i + 2 < ntiles) {
      nv = ck.nv();
      kld.issue(kg, rs, ck.ks, nv, smem + (par ? TB : 0), tid, wave);
      ck.advance(s_rng);
    }
    if (i < ntiles) {
      vld.issue(vg, rs, cv.ks, cv.nv(), smem + 2 * TB + (par ? TB : 0), tid, wave);
      cv.advance(s_rng);
    }
    return nv;
  };

  // step 0: QK^T of tile 1 || weights of tile 0 (all below 2^-kHeadroom)
  {
    const int32_t nv_s = nv_pend;
    nv_pend = issue_loads(0, 0);
    float d = 0.f;
    weights_all(sa, pa, d);
    if (ntiles > 1) {
      qk_tile<T, D>(sb, smem + 5 * TB, qf, koff);
      if (nv_s < kKT) mask_tail(sb, nv_s);
    }
    lsum += d;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Step i in [1, ntiles): QK^T(i+1) || weights(i) || PV(i-1) as 2*(D/8)
  // slots of one MFMA each (even: QK^T, odd: PV), the operand reads kLead
  // slots ahead and 32/slots weights of tile i per slot.  The slots are
  // fenced, so the compiler keeps this interleave.  The last step
  // (i = ntiles - 1, `last`) has no tile i+1: its even slots hold weights
  // only, it loads no K tile, and one thread takes the cursor of the next
  // item, so that its atomic is in flight during the step.
  // The epilogue's first reads.  At the start of the last step (or of the
  // epilogue, for an item of one tile) thread 0 takes the own queue's cursor
  // for the next item, so the atomic is in flight during the step; once the
  // step's loads have landed (the cursor with them) every lane looks up the
  // permutation entries of its output rows (raster output: branch-free table
  // reads, rows past the tile clamped for the lookup and skipped at the
  // store), all in flight during the last PV.  The variables are declared
  // without values, so nothing of this is live across the tile loop.
  constexpr int rows_per_pass = 64 / Lds::kChunks;
  constexpr int kPasses = 32 / rows_per_pass;
  int32_t cnext;          // thread 0: the own queue's cursor for the next item
  int32_t oent[kPasses];  // raster output: the permutation entry of each output row
  auto take_cursor = [&]() {
    if (tid == 0) {
      KArgs ka = kernel_args();
      cnext = __hip_atomic_fetch_add(ka->queue + xcc_id(), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  auto out_row = [&](int pass) {  // the tile row of output pass `pass`, clamped into the tile
    return min(it.q0 + wave * 32 + pass * rows_per_pass + lane / Lds::kChunks, it.q1 - 1);
  };
  auto look_up_rows = [&]() {
    KArgs ka = kernel_args();
    const int32_t* perm = ka->out_perm;
    if (perm) {  // uniform
      const int32_t* lrp = ka->out_lr_perm;
      asm volatile("" : "+s"(perm), "+s"(lrp));  // two scalar pointers; the table is picked per lane
      const int32_t T0 = ka->T, N0 = ka->N;
#pragma unroll
      for (int pass = 0; pass < kPasses; ++pass) {
        const int32_t row = out_row(pass);
        const bool hr = row >= T0 && row < T0 + N0;
        const bool lr = row >= T0 + N0 && lrp != nullptr;
        const int32_t* tab = lr ? lrp : perm;
        oent[pass] = tab[hr ? row - T0 : lr ? row - T0 - N0 : 0];
      }
    }
  };

  // Step i in [1, ntiles - 1): QK^T(i+1) || weights(i) || PV(i-1) as 2*(D/8)
  // slots of one MFMA each (even: QK^T, odd: PV), the operand reads kLead
  // slots ahead and 32/slots weights of tile i per slot.  The slots are
  // fenced, so the compiler keeps this interleave.
  auto step = [&](int32_t i, auto par, f32x16(&s_cur)[2], f32x16(&s_nxt)[2], bf16x8(&p_cur)[4],
                  bf16x8(&p_nxt)[4]) {
    constexpr int PAR = decltype(par)::value;                   // i & 1
    const char* const k_next = smem + (PAR ? 0 : TB);           // K_{i+1}
    const char* const v_prev = smem + 2 * TB + (PAR ? 0 : TB);  // V_{i-1}
    const int32_t nv_s = nv_pend;                               // rows of tile i+1
    // The step's loads (K_{i+2} and V_i, as issue_loads) go out one at a time,
    // kLoadGap slots apart, rather than all at the step's start, where the
    // eight waves' loads and their first operand reads would meet.  With no
    // K_{i+2} the K loads read zero bytes (into the slot K_i left).
    const char* kbase = reinterpret_cast<const char*>(kg);
    int32_t kbytes = 0;
    nv_pend = kKT;
    if (i + 2 < ntiles) {
      nv_pend = ck.nv();
      kbase = reinterpret_cast<const char*>(kg + int64_t(ck.ks) * rs);
      kbytes = __builtin_amdgcn_readfirstlane(nv_pend * int32_t(rs) * int32_t(sizeof(T)));  // nv_pend >= 1
      ck.advance(s_rng);
    }
    const char* const vbase = reinterpret_cast<const char*>(vg + int64_t(cv.ks) * rs);
    // V_i exists (i < ntiles), so it has at least one row
    const int32_t vbytes = __builtin_amdgcn_readfirstlane(cv.nv() * int32_t(rs) * int32_t(sizeof(T)));
    cv.advance(s_rng);
    constexpr int kLPT = Lds::kLoadsPerThread;
    constexpr int kLoadGap = D == 64 ? 4 : 2;
    static_assert(kLoadGap * 2 * kLPT <= kSlots, "the loads fit in the step");
    auto load_at = [&](int k) {
      if (k % kLoadGap == 0 && k / kLoadGap < 2 * kLPT) {
        const int j = k / kLoadGap;
        if ((j & 1) == 0) kld.issue_one(j >> 1, kbase, kbytes, smem + (PAR ? TB : 0), wave);
        else vld.issue_one(j >> 1, vbase, vbytes, smem + 2 * TB + (PAR ? TB : 0), wave);
      }
    };
    bf16x8 opnd[kLead + 1];  // operand ring: slot k's A operand in opnd[k % (kLead + 1)]
    auto fetch = [&](int k) {
      const int j = k >> 1;
      if ((k & 1) == 0) {  // QK^T: K rows of block j / kQRegs, dims of k-step j % kQRegs
        opnd[k % (kLead + 1)] =
            *reinterpret_cast<const bf16x8*>(k_next + (j / kQRegs) * 32 * RB + koff[j % kQRegs]);
      } else {  // PV: V^T of 16-key chunk j / (D/32), dim tile j % (D/32)
        const char* a0 = v_prev + voff[j % (D / 32)] + (16 * (j / (D / 32))) * RB;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0 + 8 * RB));
        opnd[k % (kLead + 1)] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
#pragma unroll
    for (int k = 0; k < kLead; ++k) fetch(k);
    float d = 0.f;
#pragma unroll
    for (int k = 0; k < kSlots; ++k) {
      load_at(k);
      if (k + kLead < kSlots) fetch(k + kLead);
      const int j = k >> 1;
      if ((k & 1) == 0) {
        const int mb = j / kQRegs, ks = j % kQRegs;
        s_nxt[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[k % (kLead + 1)], qf[ks],
                                                            ks == 0 ? f32x16{} : s_nxt[mb], 0, 0, 0);
      } else {
        acc[j % (D / 32)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[k % (kLead + 1)], p_cur[j / (D / 32)],
                                                                    acc[j % (D / 32)], 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < kExpPerSlot; ++e) weight(s_cur, p_nxt, d, k * kExpPerSlot + e);
      __builtin_amdgcn_sched_barrier(0);
    }
    sum_last(d);
    if (nv_s < kKT) mask_tail(s_nxt, nv_s);  // uniform (scalar) condition
    if (__ballot(!(d < 256.0f))) settle(s_cur, p_nxt, d);
    lsum += d;
    __builtin_amdgcn_s_waitcnt(0);  // this thread's direct-to-LDS loads have landed
    __syncthreads();
  };

  // The last step (i = ntiles - 1): weights(i) || PV(i-1), with no tile i+1
  // and so no QK^T and no K load; the odd slots hold the PV MFMAs, every slot
  // its weights.  Its ring slots follow i's parity at run time (one form for
  // both parities): V_{i-1} is read from slot (i-1)&1 and V_i goes to slot i&1.
  auto last_step = [&](int32_t i, f32x16(&s_cur)[2], bf16x8(&p_cur)[4], bf16x8(&p_nxt)[4]) {
    take_cursor();
    const int32_t vpar = (i & 1) * TB;
    const char* const v_prev = smem + 3 * TB - vpar;  // V_{i-1}
    char* const v_dst = smem + 2 * TB + vpar;          // V_i
    const char* const vbase = reinterpret_cast<const char*>(vg + int64_t(cv.ks) * rs);
    const int32_t vbytes = __builtin_amdgcn_readfirstlane(cv.nv() * int32_t(rs) * int32_t(sizeof(T)));
    constexpr int kLPT = Lds::kLoadsPerThread;
    constexpr int kLoadGap = D == 64 ? 4 : 2;
    bf16x8 opnd[kLead + 1];
    auto fetch = [&](int k) {  // odd slots only
      const int j = k >> 1;
      const char* a0 = v_prev + voff[j % (D / 32)] + (16 * (j / (D / 32))) * RB;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0 + 8 * RB));
      opnd[k % (kLead + 1)] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
#pragma unroll
    for (int k = 1; k < kLead; k += 2) fetch(k);
    float d = 0.f;
#pragma unroll
    for (int k = 0; k < kSlots; ++k) {
      if (k % kLoadGap == 0 && k / kLoadGap < 2 * kLPT && (k / kLoadGap) % 2 == 1)
        vld.issue_one((k / kLoadGap) >> 1, vbase, vbytes, v_dst, wave);
      if (k + kLead < kSlots && ((k + kLead) & 1)) fetch(k + kLead);
      if (k & 1) {
        const int j = k >> 1;
        acc[j % (D / 32)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[k % (kLead + 1)], p_cur[j / (D / 32)],
                                                                    acc[j % (D / 32)], 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < kExpPerSlot; ++e) weight(s_cur, p_nxt, d, k * kExpPerSlot + e);
      __builtin_amdgcn_sched_barrier(0);
    }
    sum_last(d);
    if (__ballot(!(d < 256.0f))) settle(s_cur, p_nxt, d);
    lsum += d;
    __builtin_amdgcn_s_waitcnt(0);  // V_i, and the cursor, have landed
    look_up_rows();
    __syncthreads();
  };

  // Pairs of steps, so that the ring slots and register sets are fixed at
  // compile time; the loop has no exit between the two (an exit there keeps
  // both weight sets alive across the pair and spills).
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  // The pairs stop before the last step, which then runs in the even
  // form's registers: scores of the last tile in sa, weights of the tile
  // before it in pb; the last tile's weights land in pa.
  int32_t i = 1;
  for (; i + 2 < ntiles; i += 2) {
    step(i, P1{}, sb, sa, pa, pb);
    step(i + 1, P0{}, sa, sb, pb, pa);
  }
  if (i < ntiles) {
    if (i + 1 < ntiles) {  // two steps left: the odd one, then the last
      step(i, P1{}, sb, sa, pa, pb);
      ++i;
    } else {  // the last step is odd: its operands move to the even form's registers
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) sa[mb] = sb[mb];
#pragma unroll
      for (int c = 0; c < 4; ++c) pb[c] = pa[c];
    }
    last_step(i, sa, pb, pa);
  } else {  // one tile: its weights (step 0) are in pa, its V in slot 0
    take_cursor();
    look_up_rows();
  }

  // ---- epilogue: the last PV; combine the lane halves' row sums,
  // normalise, and write the wave's 32 x D output block through LDS
  // (swizzled rows) as full rows.  The next item is published at the
  // barrier that frees the LDS; its record is read while the output is
  // staged, and its loads go out after the output stores.
  kp = kernel_args();  // the epilogue's arguments are loaded here, not kept across the loop
  const int32_t x0 = xcc_id();
  pv_all(pa, smem + 2 * TB + ((ntiles - 1) & 1) * TB);  // the last tile's weights, its V in slot (ntiles-1)&1
  int32_t orow[kPasses];
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int32_t row = out_row(pass);
    if (kp->out_perm) {  // uniform
      const bool hr = row >= kp->T && row < kp->T + kp->N;
      const bool lr = row >= kp->T + kp->N && kp->out_lr_perm != nullptr;
      orow[pass] = hr ? kp->T + oent[pass] : lr ? kp->T + kp->N + oent[pass] : row;
    } else {
      orow[pass] = row;
    }
  }
  const float total = pair_sum(lsum);
  const float inv = 1.0f / total;
  UG_CHECK(!(kp->lse && g == 0 && qrow < it.q1) || qrow < kp->lse_rows, 3);
  if (kp->lse && g == 0 && qrow < it.q1)  // log(sum_j exp(s_j)) = (mref + log2(total)) * ln 2
    kp->lse[int64_t(it.bh) * kp->lse_rows + qrow] = (mref + __log2f(total)) * 0.6931471805599453f;
  // The next item: the cursor taken in the last step if it lies within the own queue's
  // items (past them the queue holds padding), else the usual search over
  // the queues (which moves the own queue's cursor once more, as a failed
  // grab does).
  if (tid == 0) {
    const int32_t next = cnext < kp->qlen[x0] ? cnext * ug::kXcds + x0
                                              : queue_grab(kp->queue, kp->queue_len, kp->blocks, x0);
    UG_CHECK(next < kp->queue_len * ug::kXcds, 0);
    *s_next_idx = next;
  }
  __syncthreads();  // every wave has read the last V tile; the next item is published
  const int32_t next = __builtin_amdgcn_readfirstlane(*s_next_idx);
  char* const ost = smem + wave * 32 * RB;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = t * 32 + 8 * q4 + 4 * g;  // 4 consecutive dims
      char* dst = ost + l32 * RB + (((d0 / Lds::kEl16) ^ Lds::k_swz(l32)) * 16) + (d0 % Lds::kEl16) * 2;
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = __bf16(acc[t][4 * q4 + e] * inv);
      *reinterpret_cast<bf16x4*>(dst) = w;
    }
  // each wave reads back only its own block: LDS operations of one wave
  // complete in order, so no barrier is needed between the write and read.
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int r = pass * rows_per_pass + lane / Lds::kChunks;
    const int cc = lane % Lds::kChunks;
    const uint4 val = *reinterpret_cast<const uint4*>(ost + r * RB + ((cc ^ Lds::k_swz(r)) * 16));
    if (it.q0 + wave * 32 + r < it.q1) {
      UG_CHECK(orow[pass] >= 0 && orow[pass] < kp->L, 3);
      *reinterpret_cast<uint4*>(og + int64_t(orow[pass]) * rs + cc * Lds::kEl16) = val;
    }
  }
  // The next item's first loads: its K_0, K_1 and ranges into the prologue
  // region and s_rng, and its queries into the wave's block once the wave's
  // reads of it have completed.
  if (next >= 0) {
    const ug::AttnItem nx = load_item(kp, next);
    prefetch_keys<D>(kp, nx, smem, s_rng, tid, wave, lane);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    prefetch_queries<D>(kp, nx, smem, wave, lane);
  }
}


template <typename T, int D>
__global__ __launch_bounds__(kAttnThreads) void attn_fwd_kernel(AttnParams p) {
  (void)p;  // read through kernel_args()
  using Lds = AttnLds<T, D>;
  __shared__ __attribute__((aligned(1024))) char smem[Lds::kTotalBytes];
  __shared__ ug::Range s_rng[ug::kAttnMaxRanges];
  if constexpr (std::is_same<T, __bf16>::value) {
    // The next item is published in s_next_idx, and its first loads are
    // issued, before it starts: here for the first item, in the previous
    // item's epilogue for the others.
    __shared__ int32_t s_next_idx;
    if (threadIdx.x == 0) {
      KArgs kp = kernel_args();
      s_next_idx = queue_grab(kp->queue, kp->queue_len, kp->blocks, xcc_id());
    }
    __syncthreads();
    {
      const int tid = opaque_tid<kAttnThreads>();
      const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (kAttnWaves - 1);
      const int32_t first = __builtin_amdgcn_readfirstlane(s_next_idx);
      if (first >= 0) {
        KArgs kp = kernel_args();
        const ug::AttnItem nx = load_item(kp, first);
        prefetch_keys<D>(kp, nx, smem, s_rng, tid, wave, lane);
        prefetch_queries<D>(kp, nx, smem, wave, lane);
      }
    }
    for (;;) {
      __builtin_amdgcn_s_waitcnt(0);  // this thread's loads of the item's ranges, K_0, K_1 and Q have landed
      __syncthreads();
      const int32_t idx = __builtin_amdgcn_readfirstlane(s_next_idx);
      if (idx < 0) break;
      KArgs kp = kernel_args();
      UG_CHECK(idx < kp->queue_len * ug::kXcds, 0);
      const ug::AttnItem it = load_item(kp, idx);
      attn_item_bf16<D>(kp, it, smem, s_rng, &s_next_idx);
    }
  } else {
    __shared__ int32_t s_item;
    if (threadIdx.x == 0) {
      KArgs kp = kernel_args();
      s_item = queue_grab(kp->queue, kp->queue_len, kp->blocks, xcc_id());
    }
    __syncthreads();
    for (;;) {
      const int32_t item = s_item;
      if (item < 0) break;
      attn_item_f32<D>(kernel_args(), item, smem, s_rng);
      __syncthreads();  // the next item reuses the LDS and s_item
      if (threadIdx.x == 0) {
        KArgs kp = kernel_args();
        s_item = queue_grab(kp->queue, kp->queue_len, kp->blocks, xcc_id());
      }
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) queue_finish(kernel_args()->queue);
}


ug_status gather(ug_plan_t p, const void* src, void* dst, const int32_t* table, const int32_t* lr_table,
                 hipStream_t s, const char* fn) {
  ug::clear_error();
  ug_status st = check_plan(p, fn);
  if (st != UG_OK) return st;
  if (!src || !dst) return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": NULL tensor");
  if (!aligned16(src) || !aligned16(dst))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": tensors must be 16-byte aligned");
  if (overlap(src, dst, tensor_bytes(p)))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": input and output overlap (out of place only)");
  if (current_device() != p->device)
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": current device is not the plan's device");
  const int32_t units = int32_t(int64_t(p->d.heads) * p->d.head_dim * (p->d.dtype == UG_BF16 ? 2 : 4) / 16);
  const dim3 grid(unsigned((p->L + kGatherRows - 1) / kGatherRows), unsigned(p->d.batch));
  const unsigned threads = unsigned(std::min<int64_t>(1024, (int64_t(units) + 63) / 64 * 64));
  hipLaunchKernelGGL(row_gather_kernel, grid, dim3(threads), 0, s, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), int32_t(p->L), int32_t(p->T), int32_t(p->N), units, table, lr_table);
  return launch_status(fn);
}

template <typename T, int D>
void launch_attn(ug_plan_t p, const AttnParams& ap, hipStream_t s) {
  const unsigned grid = unsigned(std::min<size_t>(size_t(p->cus), p->blocks.size()));
  hipLaunchKernelGGL((attn_fwd_kernel<T, D>), dim3(grid), dim3(kAttnThreads), 0, s, ap);
}

ug_status attn_common(ug_plan_t p, const void* q, const void* k, const void* v, void* o, float* lse,
                      void* workspace, void* stream, bool raster_out, const char* fn) {
  ug::clear_error();
  (void)workspace;
  ug_status st = check_plan(p, fn);
  if (st != UG_OK) return st;
  if (!q || !k || !v || !o) return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": NULL tensor");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": tensors must be 16-byte aligned");
  const int64_t n = tensor_bytes(p);
  if (overlap(o, q, n) || overlap(o, k, n) || overlap(o, v, n))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": o overlaps q, k or v");
  if (lse) {
    const int64_t nl = int64_t(p->d.batch) * p->d.heads * p->L * int64_t(sizeof(float));
    if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
      return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": lse must be 4-byte aligned");
    if (ug::host::overlap_ranges(lse, nl, o, n) || ug::host::overlap_ranges(lse, nl, q, n) ||
        ug::host::overlap_ranges(lse, nl, k, n) || ug::host::overlap_ranges(lse, nl, v, n))
      return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": lse overlaps a tensor");
  }
  if (current_device() != p->device)
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": current device is not the plan's device");
  if (p->max_task_ranges > ug::kAttnMaxRanges)
    return ug::fail(UG_ERR_UNSUPPORTED, std::string(fn) + ": a query tile has " + std::to_string(p->max_task_ranges) +
                                            " key ranges, more than the kernel stages (" +
                                            std::to_string(ug::kAttnMaxRanges) + "); use a smaller radius");
  if (p->blocks.empty()) return UG_OK;
  AttnParams ap{};
  ap.q = q;
  ap.k = k;
  ap.v = v;
  ap.o = o;
  ap.row_stride = int64_t(p->d.heads) * p->d.head_dim;
  ap.batch_stride = p->L * ap.row_stride;
  ap.heads = p->d.heads;
  ap.tasks = p->d_tasks;
  ap.ranges = p->d_ranges;
  ap.blocks = p->d_blocks;
  ap.items = reinterpret_cast<__attribute__((address_space(4))) const ug::AttnItem*>(
      reinterpret_cast<uintptr_t>(p->d_items));
  for (int x = 0; x < ug::kXcds; ++x) ap.qlen[x] = p->queue_items[x];
  ap.scale_log2 = float(1.4426950408889634 / std::sqrt(double(p->d.head_dim)));
  ap.T = int32_t(p->T);
  ap.N = int32_t(p->N);
  ap.out_perm = raster_out ? p->d_perm : nullptr;
  ap.out_lr_perm = raster_out ? p->d_lr_perm : nullptr;
  ap.lse = lse;
  ap.lse_rows = p->L;
  ap.queue_len = int32_t(p->blocks.size() / ug::kXcds);
  ap.L = int32_t(p->L);
  ap.n_tasks = int32_t(p->tasks.size());
  ap.n_bh = p->d.batch * p->d.heads;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = p->d.dtype == UG_BF16;
  return ug::launch_with_slot(p, s, fn, [&](int32_t* cursors) {
    ap.queue = cursors;
    if (bf && p->d.head_dim == 128)
      launch_attn<__bf16, 128>(p, ap, s);
    else if (bf && p->d.head_dim == 64)
      launch_attn<__bf16, 64>(p, ap, s);
    else if (!bf && p->d.head_dim == 128)
      launch_attn<float, 128>(p, ap, s);
    else
      launch_attn<float, 64>(p, ap, s);
    return launch_status(fn);
  });
}

template <bool kInverse>
ug_status rope_common(ug_plan_t p, void* q_perm, void* k_perm, void* stream, const char* fn) {
  ug::clear_error();
  ug_status st = check_plan(p, fn);
  if (st != UG_OK) return st;
  if (!q_perm || !k_perm) return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": NULL tensor");
  if (!aligned16(q_perm) || !aligned16(k_perm))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": tensors must be 16-byte aligned");
  if (overlap(q_perm, k_perm, tensor_bytes(p)))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": q and k overlap");
  if (current_device() != p->device)
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": current device is not the plan's device");
  const int64_t rows = p->N + p->Nlr;
  if (rows == 0) return UG_OK;
  const int E = p->d.dtype == UG_BF16 ? 8 : 4;
  const int64_t units = int64_t(p->d.heads) * p->d.head_dim / E;
  const dim3 grid(unsigned((rows + kRopeRows - 1) / kRopeRows), unsigned(p->d.batch));
  const unsigned threads = unsigned(std::min<int64_t>(1024, (units + 63) / 64 * 64));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float2* cs = reinterpret_cast<const float2*>(p->d_rope);
  const int32_t lr_w = std::max(p->d.lr_w, 1);
  if (p->d.dtype == UG_BF16)
    hipLaunchKernelGGL((rope2d_kernel<__bf16, kInverse>), grid, dim3(threads), 0, s, static_cast<__bf16*>(q_perm),
                       static_cast<__bf16*>(k_perm), int32_t(p->L), int32_t(p->T), int32_t(p->N), p->d.hr_w, lr_w,
                       p->d.rho, p->d.heads, p->d.head_dim, p->d_perm, p->d_lr_perm, cs);
  else
    hipLaunchKernelGGL((rope2d_kernel<float, kInverse>), grid, dim3(threads), 0, s, static_cast<float*>(q_perm),
                       static_cast<float*>(k_perm), int32_t(p->L), int32_t(p->T), int32_t(p->N), p->d.hr_w, lr_w,
                       p->d.rho, p->d.heads, p->d.head_dim, p->d_perm, p->d_lr_perm, cs);
  return launch_status(fn);
}

template <bool kBwd>
ug_status permute_rope_common(ug_plan_t p, const void* q_in, const void* k_in, void* q_out, void* k_out,
                              void* stream, const char* fn) {
  ug::clear_error();
  ug_status st = check_plan(p, fn);
  if (st != UG_OK) return st;
  if (!q_in || !k_in || !q_out || !k_out) return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": NULL tensor");
  if (!aligned16(q_in) || !aligned16(k_in) || !aligned16(q_out) || !aligned16(k_out))
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": tensors must be 16-byte aligned");
  const int64_t n = tensor_bytes(p);
  const void* ins[2] = {q_in, k_in};
  const void* outs[2] = {q_out, k_out};
  for (const void* a : outs)
    for (const void* b : ins)
      if (overlap(a, b, n)) return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": an output overlaps an input");
  if (overlap(q_out, k_out, n)) return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": the two outputs overlap");
  if (current_device() != p->device)
    return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": current device is not the plan's device");
  const int E = p->d.dtype == UG_BF16 ? 8 : 4;
  const int64_t units = int64_t(p->d.heads) * p->d.head_dim / E;
  const dim3 grid(unsigned((p->L + kRopeRows - 1) / kRopeRows), unsigned(p->d.batch));
  const unsigned threads = unsigned(std::min<int64_t>(1024, (units + 63) / 64 * 64));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float2* cs = reinterpret_cast<const float2*>(p->d_rope);
  const int32_t lr_w = std::max(p->d.lr_w, 1);
  const int32_t* tab_hr = kBwd ? p->d_inv : p->d_perm;
  const int32_t* tab_lr = kBwd ? p->d_lr_inv : p->d_lr_perm;
  if (p->d.dtype == UG_BF16)
    hipLaunchKernelGGL((permute_rope_kernel<__bf16, kBwd>), grid, dim3(threads), 0, s,
                       static_cast<const __bf16*>(q_in), static_cast<const __bf16*>(k_in), static_cast<__bf16*>(q_out),
                       static_cast<__bf16*>(k_out), int32_t(p->L), int32_t(p->T), int32_t(p->N), p->d.hr_w, lr_w,
                       p->d.rho, p->d.heads, p->d.head_dim, tab_hr, tab_lr, cs);
  else
    hipLaunchKernelGGL((permute_rope_kernel<float, kBwd>), grid, dim3(threads), 0, s, static_cast<const float*>(q_in),
                       static_cast<const float*>(k_in), static_cast<float*>(q_out), static_cast<float*>(k_out),
                       int32_t(p->L), int32_t(p->T), int32_t(p->N), p->d.hr_w, lr_w, p->d.rho, p->d.heads,
                       p->d.head_dim, tab_hr, tab_lr, cs);
  return launch_status(fn);
}

}  // namespace

extern "C" {

ug_status ug_permute(ug_plan_t p, const void* x_raster, void* x_perm, void* stream) {
  return gather(p, x_raster, x_perm, p ? p->d_perm : nullptr, p ? p->d_lr_perm : nullptr,
                static_cast<hipStream_t>(stream), "ug_permute");
}

ug_status ug_unpermute(ug_plan_t p, const void* x_perm, void* x_raster, void* stream) {
  return gather(p, x_perm, x_raster, p ? p->d_inv : nullptr, p ? p->d_lr_inv : nullptr,
                static_cast<hipStream_t>(stream), "ug_unpermute");
}

ug_status ug_rope2d(ug_plan_t p, void* q_perm, void* k_perm, void* stream) {
  return rope_common<false>(p, q_perm, k_perm, stream, "ug_rope2d");
}

ug_status ug_rope2d_bwd(ug_plan_t p, void* dq_perm, void* dk_perm, void* stream) {
  return rope_common<true>(p, dq_perm, dk_perm, stream, "ug_rope2d_bwd");
}

ug_status ug_attn_fwd(ug_plan_t p, const void* q, const void* k, const void* v, void* o, void* workspace,
                      void* stream) {
  return attn_common(p, q, k, v, o, nullptr, workspace, stream, false, "ug_attn_fwd");
}

ug_status ug_attn_fwd_raster(ug_plan_t p, const void* q, const void* k, const void* v, void* o_raster,
                             void* workspace, void* stream) {
  return attn_common(p, q, k, v, o_raster, nullptr, workspace, stream, true, "ug_attn_fwd_raster");
}

ug_status ug_attn_fwd_lse(ug_plan_t p, const void* q, const void* k, const void* v, void* o, float* lse,
                          void* workspace, void* stream) {
  if (!lse) {
    ug::clear_error();
    return ug::fail(UG_ERR_INVALID_ARGUMENT, "ug_attn_fwd_lse: NULL lse");
  }
  return attn_common(p, q, k, v, o, lse, workspace, stream, false, "ug_attn_fwd_lse");
}

ug_status ug_permute_rope(ug_plan_t p, const void* q_raster, const void* k_raster, void* q_perm, void* k_perm,
                          void* stream) {
  return permute_rope_common<false>(p, q_raster, k_raster, q_perm, k_perm, stream, "ug_permute_rope");
}

ug_status ug_permute_rope_bwd(ug_plan_t p, const void* dq_perm, const void* dk_perm, void* dq_raster,
                              void* dk_raster, void* stream) {
  return permute_rope_common<true>(p, dq_perm, dk_perm, dq_raster, dk_raster, stream, "ug_permute_rope_bwd");
}

}  // extern "C"

UG_BOUNDS_ACCESSOR(ug_debug_bounds_fwd)
