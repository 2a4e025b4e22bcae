// Definitions shared by the kernel files: vector types, lane-pair
// reductions, the key-range cursor, and the host-side argument checks of the
// launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "plan_internal.hpp"

// Debug build (compiled with -DUG_BOUNDS_CHECK into libultragen_debug.so):
// UG_CHECK(cond, bit) records a failed index check as bit `bit` of the
// translation unit's violation word instead of trapping, so a test can read
// the word back after its launches (ug_debug_bounds_*).  Bits:
//   0 work item, task or (batch, head) index outside its table
//   1 key or query range outside [0, L), inverted, or more ranges than staged
//   2 tile load window past the sequence
//   3 destination row of an output or statistics store outside its array
//   4 permutation-table value outside its range
//   5 warm start: LR patch index outside the staged patch, or a tensor index
//     outside the tensor
// In the release build the condition is not evaluated.
#ifdef UG_BOUNDS_CHECK
namespace {
__device__ uint32_t ug_bounds_word;
}
#define UG_CHECK(cond, bit)                                                                                     \
  do {                                                                                                          \
    if (!(cond)) __hip_atomic_fetch_or(&ug_bounds_word, 1u << (bit), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); \
  } while (0)
// extern "C" accessor of the word: copies it to *out, then clears it if asked
#define UG_BOUNDS_ACCESSOR(name)                                                                         \
  extern "C" ug_status name(uint32_t* out, int32_t clear) {                                              \
    if (!out) return ug::fail(UG_ERR_INVALID_ARGUMENT, #name ": out is NULL");                            \
    if (hipMemcpyFromSymbol(out, HIP_SYMBOL(ug_bounds_word), sizeof(uint32_t)) != hipSuccess)             \
      return ug::fail(UG_ERR_HIP, #name ": hipMemcpyFromSymbol failed");                                  \
    const uint32_t zero = 0;                                                                             \
    if (clear && hipMemcpyToSymbol(HIP_SYMBOL(ug_bounds_word), &zero, sizeof(uint32_t)) != hipSuccess)   \
      return ug::fail(UG_ERR_HIP, #name ": hipMemcpyToSymbol failed");                                    \
    return UG_OK;                                                                                        \
  }
#else
#define UG_CHECK(cond, bit) ((void)0)
#define UG_BOUNDS_ACCESSOR(name)
#endif

namespace ug {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Lane l and lane l^32 of a wave hold the two halves of one 32x32 MFMA
// column; these combine them (v_permlane32_swap).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Direct global->LDS load of 16 (or 4) bytes per lane, issued in its MUBUF
// form (buffer_load_dword{,x4} ... lds): lane l's bytes land at lds_base +
// size * l; the global address is row_base + voffset.  Same data movement as
// global_load_lds, but the compiler tracks the buffer form with the
// vector-memory counter only, whereas it counts the global form as an LDS
// event of unknown order, after which every LDS wait of the wave becomes a
// full drain.  The descriptor (raw, stride 0, 32-bit data format) is built
// from a wave-uniform base, so it lives in scalar registers.  Its bounds
// check also zero-fills the rows past a ragged tile's end.
constexpr int kBufferFlags = 0x00020000;

// Lanes whose voffset + size exceeds `bytes` read zeros instead (the buffer
// bounds check), which no lane can fault on.
template <int kSize>
__device__ __forceinline__ void load_lds(const void* row_base, uint32_t voffset, lds_void* lds_base,
                                         int32_t bytes = 0x7fffffff) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row_base), (short)0, bytes, kBufferFlags);
  static_assert(kSize == 16 || kSize == 4, "16- or 4-byte lanes");
  if constexpr (kSize == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds_base, 16, voffset, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds_base, 4, voffset, 0, 0, 0);
}

// Walks the 64-row tiles of a list of row ranges (key ranges of a query
// tile, or query ranges of a key tile), one range after another.
// The cursor is wave-uniform; the range bounds are read back with
// readfirstlane so the compiler knows it (they feed scalar buffer
// descriptors).
struct TileCursor {
  int32_t ri, r1, ks, k1;
  __device__ __forceinline__ void init(const ug::Range* ranges, int32_t r0, int32_t rend) {
    ri = r0;
    r1 = rend;
    const ug::Range r = ranges[r0];
    ks = __builtin_amdgcn_readfirstlane(r.k0);
    k1 = __builtin_amdgcn_readfirstlane(r.k1);
  }
  __device__ __forceinline__ int32_t nv() const { return min(ug::kAttnKeyTile, k1 - ks); }
  __device__ __forceinline__ void advance(const ug::Range* ranges) {
    ks += ug::kAttnKeyTile;
    if (ks >= k1 && ri + 1 < r1) {
      ++ri;
      const ug::Range r = ranges[ri];
      ks = __builtin_amdgcn_readfirstlane(r.k0);
      k1 = __builtin_amdgcn_readfirstlane(r.k1);
    }
  }
};

// Item loops of persistent kernels.  Kernel arguments read through an opaque
// pointer are loaded where they are used, once per item, instead of being
// hoisted out of the item loop and held in scalar registers across the tile
// loop.  The thread index is made opaque for the same reason (values derived
// from it and kept live across the tile loop make the compiler fall back to a
// serial LDS-read schedule); the mask gives its range back to alias analysis,
// which proves that tile loads in flight do not overlap the LDS being read.
// P must be the kernel's only explicit argument, taken by value: the AMDGPU
// ABI places the explicit arguments at the start of the argument segment.
template <typename P>
__device__ __forceinline__ __attribute__((address_space(4))) const P* opaque_args() {
  auto x = (__attribute__((address_space(4))) const P*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(x));
  return x;
}
template <int kThreads>
__device__ __forceinline__ int opaque_tid() {
  static_assert((kThreads & (kThreads - 1)) == 0, "power-of-two workgroup");
  int t = int(threadIdx.x);
  asm volatile("" : "+v"(t));
  return t & (kThreads - 1);
}

// Work queues of a persistent grid (one workgroup per CU).  The plan lays out
// eight per-XCD queues interleaved in one item array: item k * 8 + x is the
// k-th of XCD x's queue, and items with task < 0 pad the short queues.  A
// launch owns one cursor slot: queue[x] is the cursor of XCD x's queue,
// queue[8] the number of workgroups that have finished.  The cursors are
// agent-scope atomics, shared by the XCDs.
__device__ __forceinline__ int32_t xcc_id() {
  return int32_t(__builtin_amdgcn_s_getreg((31 << 11) | 20)) & (ug::kXcds - 1);  // HW_REG_XCC_ID
}
// Next item for a workgroup on XCD x0: its own XCD's queue first, then the
// others'; -1 when every queue is empty.  A cursor past the end of its queue
// or on a padding item means that queue is empty.
__device__ __forceinline__ int32_t queue_grab(int32_t* queue, int32_t queue_len, const ug::Block* items, int32_t x0) {
  for (int32_t k = 0; k < ug::kXcds; ++k) {
    const int32_t x = (x0 + k) & (ug::kXcds - 1);
    const int32_t c = __hip_atomic_fetch_add(queue + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (c < queue_len && items[c * ug::kXcds + x].task >= 0) return c * ug::kXcds + x;
  }
  return -1;
}
// Once per workgroup, after its last (failed) grab: the last workgroup to
// finish clears the slot for a later launch.  The finish count is acq_rel:
// each workgroup's grabs happen before its release, and the last one's
// acquire orders every workgroup's grabs before its clearing stores, so no
// cursor moves after it is cleared.
__device__ __forceinline__ void queue_finish(int32_t* queue) {
  if (__hip_atomic_fetch_add(queue + ug::kXcds, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
      int32_t(gridDim.x * gridDim.y * gridDim.z) - 1)
    for (int x = 0; x <= ug::kXcds; ++x) __hip_atomic_store(queue + x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dev

namespace host {

inline ug_status check_plan(ug_plan_t p, const char* fn) {
  if (!p) return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": plan is NULL");
  if (p->host_only) return ug::fail(UG_ERR_INVALID_ARGUMENT, std::string(fn) + ": plan was built host-only");
  return UG_OK;
}

inline bool aligned16(const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15u) == 0; }

inline int64_t tensor_bytes(ug_plan_t p) {
  return int64_t(p->d.batch) * p->L * p->d.heads * p->d.head_dim * (p->d.dtype == UG_BF16 ? 2 : 4);
}

inline bool overlap(const void* a, const void* b, int64_t n) {
  const auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + uintptr_t(n) && y < x + uintptr_t(n);
}

// [a, a + na) and [b, b + nb) share a byte
inline bool overlap_ranges(const void* a, int64_t na, const void* b, int64_t nb) {
  const auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + uintptr_t(nb) && y < x + uintptr_t(na);
}

inline ug_status launch_status(const char* fn) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return ug::fail(UG_ERR_HIP, std::string(fn) + ": launch failed: " + hipGetErrorString(e));
  return UG_OK;
}

inline int current_device() {
  int d = -1;
  if (hipGetDevice(&d) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  return d;
}

}  // namespace host
}  // namespace ug
